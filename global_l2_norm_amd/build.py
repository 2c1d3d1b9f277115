"""Build libgclip.so for gfx950 in-tree with hipcc.

Every HIP source is compiled with packed fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); hipcc's host pass warns
that it does not know the feature, which is harmless.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgclip.so")
BENCH = os.path.join(HERE, "gclip_bench")
SOURCES = ["gclip_api.cpp", "gclip_plan.cpp", "gclip_trace.cpp", "gclip_kernels.hip", "gclip_tensor.hip",
           "gclip_adamw.hip"]
ARCH = os.environ.get("GCLIP_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def compile_flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
            "-packed-fp32-ops", "-Wall", "-Wextra", "-Wno-unused-parameter", "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False, defines=(), lib_path: str = LIB, bench_path: str = BENCH) -> str:
    """Always recompile the library and the native timing driver; return the
    library's path.  `defines` are extra -D flags (tuning sweeps)."""
    objs = []
    odir = os.path.join(HERE, "_build")
    os.makedirs(odir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(odir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc()] + compile_flags() + [f"-D{d}" for d in defines] + ["-x", "hip", "-c",
                                                                             os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        errs = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
        if r.returncode != 0:
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
    # native timing driver, linked to the library next to it
    libdir, libname = os.path.split(lib_path)
    tmpb = bench_path + ".tmp"
    cmd = [hipcc()] + compile_flags() + ["-x", "hip", os.path.join(CSRC, "gclip_bench.cpp"), "-x", "none",
                                         f"-L{libdir}", f"-l:{libname}", "-Wl,-rpath,$ORIGIN", "-o", tmpb]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write("\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l) + "\n")
        raise RuntimeError("hipcc failed on gclip_bench.cpp")
    os.replace(tmpb, bench_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose=True))
