"""Build libgclip.so for gfx950 in-tree with hipcc.

Every HIP source is compiled with packed fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); hipcc's host pass warns
that it does not know the feature, which is harmless.

`python -m global_l2_norm_amd.build --phase-stamps` builds instead the
diagnostic library of include/gclip_stamps.h, with -DGCLIP_PHASE_STAMPS,
into _stamps/libgclip.so (the fused kernel then records its phase
timeline); the library itself is not touched.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgclip.so")
STAMPS_LIB = os.path.join(HERE, "_stamps", "libgclip.so")
SOURCES = ["gclip_api.cpp", "gclip_plan.cpp", "gclip_trace.cpp", "gclip_kernels.hip", "gclip_tensor.hip",
           "gclip_adamw.hip", "gclip_noalloc.hip", "gclip_ref.hip"]
ARCH = os.environ.get("GCLIP_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def compile_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", "-Wall", "-Wextra", "-Wno-unused-parameter", "-I", os.path.join(ROOT, "include")]


def _jobs() -> int:
    try:
        n = int(os.environ.get("MAX_JOBS", "0"))
    except ValueError:
        n = 0
    return max(1, min(n if n > 0 else (os.cpu_count() or 1), 16))


def build(verbose: bool = False, defines=(), lib_path: str = LIB) -> str:
    """Always recompile the library (the sources in parallel); return its
    path.  `defines` are extra -D flags (tuning sweeps); objects go to a
    _build folder beside lib_path."""
    odir = os.path.join(os.path.dirname(lib_path), "_build")
    os.makedirs(odir, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(odir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc()] + compile_flags() + [f"-D{d}" for d in defines] + ["-x", "hip", "-c",
                                                                             os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        errs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
        return src, obj, cmd, r.returncode, errs

    with ThreadPoolExecutor(max_workers=min(_jobs(), len(SOURCES))) as pool:
        results = list(pool.map(compile_one, SOURCES))
    objs = []
    for src, obj, cmd, rc, errs in results:
        if verbose:
            print(" ".join(cmd), flush=True)
        if rc != 0:
            sys.stderr.write(errs + "\n")
            raise RuntimeError(f"hipcc failed on {src}")
        if verbose and errs.strip():
            sys.stderr.write(errs + "\n")
        objs.append(obj)
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib_path)
    return lib_path


def build_phase_stamps(verbose: bool = False) -> str:
    """The diagnostic build of include/gclip_stamps.h."""
    return build(verbose=verbose, defines=("GCLIP_PHASE_STAMPS",), lib_path=STAMPS_LIB)


if __name__ == "__main__":
    if sys.argv[1:] == ["--phase-stamps"]:
        print(build_phase_stamps(verbose=True))
    elif sys.argv[1:]:
        sys.exit("usage: python -m global_l2_norm_amd.build [--phase-stamps]")
    else:
        print(build(verbose=True))
