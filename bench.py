"""Benchmark of the global L2-norm clipping path on one MI355X.

One step is one gclip_clip_ call (norm of the whole list, the decision, and
the in-place scale) over the ANDREA-120M-shaped fp32 gradient list (124
tensors, 92,248,320 elements, N(0, 1e-3^2): norm ~9.6 > max_norm 1.0, so every
step clips).  Between steps, outside the timed region, the gradients are
restored from a pristine device copy and a 2 GiB buffer is read so that no
cache holds the list (a read, so no dirty lines are left to drain into the
timed call).  Each step is bracketed by HIP events on the stream the kernels
run on; value = algorithmic bytes / mean event time, where the algorithmic
bytes are N*s read by the norm pass plus 2*N*s read and written by the scale
pass.  The same run times the library's reference kernels (include/
gclip_ref.h: a plain read and a plain in-place copy of the same number of
bytes, cold) for the attainable rate of those two passes, the same steps
warm (no flush), and the oracle on the host's cores.

Prints one JSON line.  Other modes:
  --config NAME        another synthetic set (synth.gradsets.CONFIGS)
  --path fused|split   force the kernel path
  --path adamw|amp     the clip fused into AdamW; the loss-scaled clip
  --path per_tensor    per-tensor clipping and per-tensor norms
  --path accum         the last microbatch's += fused with the norm pass
  --path ref           the reference kernels alone, at the workloads' sizes
  --profile-pass       a short run for rocprofv3 (no CPU baseline, plus a
                       calibration copy of known size for the PMC counters)
  --summarize-rocprof  turn rocprofv3 output into the summaries kept in
                       profiles/ (see the --help of that mode)
  --phase-stamps       the fused kernel's phase timeline, from the diagnostic
                       build of include/gclip_stamps.h (built first with
                       `python -m global_l2_norm_amd.build --phase-stamps`):
                       the same cold steps, then a table of when the median
                       and the last workgroup ended each phase
"""
import argparse
import glob
import hashlib
import re
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "clip_grad_norm GB/s and % of HBM peak, ANDREA-120M-shaped grads"
HBM_PEAK_GBPS = 8000.0
# The sources that decide what the measured kernels move: every kernel, the
# device walk, the host plan and workspace layout (chunk and block split,
# store kinds, claims) and the public headers.  A committed profile summary
# is used only while these hash to the value recorded in it.
KERNEL_SOURCES = sorted([os.path.join("global_l2_norm_amd", "csrc", f)
                         for f in os.listdir(os.path.join(ROOT, "global_l2_norm_amd", "csrc"))
                         if f.endswith((".hip", ".hpp", ".cpp"))] +
                        [os.path.join("include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                         if f.endswith(".h")])
PROFILES = os.path.join(ROOT, "profiles")
# byte sizes of the workloads' lists: 120M fp16, 120M fp32, twice that, and 1.3B bf16
REF_SIZES = [184_496_640, 368_993_280, 737_986_560, 2_622_365_696]
CPU_REPS = 5
WORKLOADS = {
    "andrea120m_f32": "ANDREA-120M-shaped fp32 gradient list: 124 tensors (tok_embed [8449,768], pos_embed "
                      "[1024,768], 12 blocks of W_Q/W_K/W_V/W_O [768,768], W_1 [768,3072], W_2 [3072,768], four "
                      "[768] norms, final norm 2x[768]), 92,248,320 elements, N(0,1e-3^2), max_norm 1.0",
}


CALIBRATION_BYTES = 369_000_000


def upload(arrays, dtype):
    """Host raw storage (float32 or uint16 bit patterns) to device tensors."""
    import numpy as np
    import torch
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    if dtype == "f32":
        return [torch.from_numpy(np.ascontiguousarray(a)).to("cuda") for a in arrays]
    return [torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(tdt) for a in arrays]


def _code_only(text):
    """A source file's code alone: comments dropped and spacing collapsed, so
    that a comment edit is not taken for a change of the measured kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(numel, esize, wrote):
    return numel * esize * (3 if wrote else 1)


def pmc_summary_path(kernels, config):
    return os.path.join(PROFILES, f"{kernels}__{config}__pmc.txt")


def _pmc_summary(kernels, config):
    """The key: value lines of a committed PMC summary, or None when it is
    missing or was taken on other kernel source."""
    path = pmc_summary_path(kernels, config)
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return kv


def read_traffic(kernels, config, kernel=None):
    """HBM bytes per step of the given kernel(s) ('a+b' for a two-kernel
    path) from the committed PMC summary -- or, with `kernel`, of that one
    kernel of the summary per launch -- or None when the summary is missing
    or was taken on other kernel source."""
    kv = _pmc_summary(kernels, config)
    if kv is None:
        return None
    try:
        if kernel is None:
            return int(float(kv["hbm_bytes_per_dispatch"]))
        fetch_cal = float(kv["fetch_calibration (counter bytes / copy bytes)"])
        write_cal = float(kv["write_calibration (counter bytes / copy bytes)"])
        return int(float(kv[f"fetch_kib_per_dispatch {kernel}"]) * 1024 / fetch_cal
                   + float(kv[f"write_kib_per_dispatch {kernel}"]) * 1024 / write_cal)
    except (KeyError, ValueError, ZeroDivisionError):
        return None


def traffic_fields(roofline, traffic, seconds):
    """Add the measured-traffic rate and fraction to a roofline object."""
    roofline["traffic"] = traffic
    if traffic is not None:
        roofline["traffic_gbps"] = round(traffic / seconds / 1e9, 1)
        roofline["traffic_frac"] = round(traffic / seconds / 1e9 / HBM_PEAK_GBPS, 4)
    return roofline


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def host_threads():
    """Threads for the oracle's threaded leg: the cores this process may run
    on, capped by OMP_NUM_THREADS where that is set (a machine's share of a
    shared host)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    try:
        cap = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        cap = 0
    return max(1, min(n, cap) if cap > 0 else n)


def oracle_rate(run, restore, nbytes, sample, reps=CPU_REPS):
    """The oracle timed on this host: the median of `reps` runs of run()
    (restore() before each, untimed); nbytes algorithmic bytes per run."""
    times = []
    for _ in range(reps):
        restore()
        t0 = time.perf_counter()
        run()
        times.append(time.perf_counter() - t0)
    sec = statistics.median(times)
    return {"value": round(nbytes / sec / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{sample}; median of {reps} reps, {sec:.2f} s each, single-threaded binary64 C",
            "cpu_model": cpu_model()}


def cpu_baseline(g, reps=CPU_REPS):
    """The oracle as it stands, on this host's cores, on the same workload:
    norm, decision and scale of the whole list, the median of `reps` runs
    with the list restored before each (untimed); on T threads (the list cut
    into T runs of consecutive elements, oracle.clip_sharded_) and on one
    thread (oracle.clip_)."""
    import oracle
    work = [a.copy() for a in g.arrays]
    esize = 4 if g.dtype == "f32" else 2

    def timed(threads):
        times, r = [], None
        for _ in range(reps):
            for w, a in zip(work, g.arrays):
                w[...] = a
            t0 = time.perf_counter()
            if threads == 1:
                r = oracle.clip_(work, g.dtype, g.max_norm, g.avg_factor, g.error_if_nonfinite)
            else:
                r = oracle.clip_sharded_(work, g.dtype, g.max_norm, g.avg_factor, g.error_if_nonfinite, threads)
            times.append(time.perf_counter() - t0)
        return statistics.median(times), r

    T = host_threads()
    sec1, r = timed(1)
    secT, _ = timed(T) if T > 1 else (sec1, r)
    wrote = not (r["skipped"] or r["scale"] == 1.0)
    alg = algorithmic_bytes(g.numel, esize, wrote)
    return {"value": round(alg / secT / 1e9, 3), "unit": "GB/s", "cores": T, "kind": "oracle",
            "sample": f"the whole {g.name} list ({g.numel} elements), norm+decision+scale, binary64 C; "
                      f"{T} threads over {T} runs of consecutive elements; median of {reps} reps, "
                      f"{secT:.3f} s each",
            "statistic": f"median of {reps}", "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(),
            "single_thread": {"value": round(alg / sec1 / 1e9, 3), "unit": "GB/s", "cores": 1,
                              "s_per_rep": round(sec1, 3)}}


def ref_times(nbytes, reps, flush, stream, copy_too=True):
    """Mean event time (ms) of the reference kernels over nbytes, cold: the
    plain read, the in-place copy and (copy_too) the copy to a second buffer."""
    import torch
    from global_l2_norm_amd import _lib
    n16 = (nbytes + 15) // 16 * 16
    src = torch.ones(n16 // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src) if copy_too else None
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    sp = stream.cuda_stream
    runs = {"read": lambda: _lib.lib.gclip_ref_read(src.data_ptr(), n16, sink.data_ptr(), sp),
            "in_place": lambda: _lib.lib.gclip_ref_copy(src.data_ptr(), src.data_ptr(), n16, sp)}
    if copy_too:
        runs["copy"] = lambda: _lib.lib.gclip_ref_copy(dst.data_ptr(), src.data_ptr(), n16, sp)
    out = {}
    for name, run in runs.items():
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps + 2)]
        for e0, e1 in evs:
            flush.sum()
            e0.record(stream)
            if run() != 0:
                raise RuntimeError(f"gclip_ref {name} failed")
            e1.record(stream)
        torch.cuda.synchronize()
        out[name] = statistics.fmean(e0.elapsed_time(e1) for e0, e1 in evs[2:])
    del src, dst
    return n16, out


def calibration_copy(flush):
    """For the PMC counters: an elementwise kernel that reads and writes
    exactly CALIBRATION_BYTES each (torch.neg), cold, three times."""
    import torch
    src = torch.full((CALIBRATION_BYTES // 4,), 3.0, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        flush.sum()
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="andrea120m_f32")
    ap.add_argument("--path", choices=["auto", "fused", "split", "adamw", "amp", "per_tensor", "accum", "ref"],
                    default="auto",
                    help="adamw: time the clip fused into an AdamW step (gclip_norm + gclip_adamw_step) "
                         "against gclip_clip_ followed by the same AdamW step; amp: time the loss-scaled "
                         "clip (gclip_clip_amp_) against gclip_clip_ with the same factor given by the host; "
                         "per_tensor: time the per-tensor clip (gclip_clip_per_tensor_) and the per-tensor "
                         "norms alone (gclip_tensor_norms); accum: time the last microbatch's += fused with the "
                         "clip (gclip_accumulate_clip_) on the four-microbatch list against torch's += followed "
                         "by gclip_clip_; ref: the reference read and copy kernels at the workloads' sizes")
    ap.add_argument("--no-flush", action="store_true", help="skip the cache flush between steps")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-pass", action="store_true",
                    help="a calibration copy of known size first (for PMC counters), then the run without the "
                         "CPU baseline")
    ap.add_argument("--summarize-rocprof", nargs="+", metavar="ARG",
                    help="KIND OUT DIR...: KIND is 'trace' (a --kernel-trace --stats output dir) or 'pmc' "
                         "(FETCH_SIZE dir, then WRITE_SIZE dir); OUT is the summary file to write, named "
                         "KERNEL[+KERNEL]__CONFIG__KIND.txt")
    ap.add_argument("--phase-stamps", action="store_true",
                    help="the fused kernel's phase timeline (needs the --phase-stamps build of the library)")
    ap.add_argument("--rocprof-command", action="append", default=[],
                    help="with --summarize-rocprof: the command that produced each output dir (repeatable)")
    a = ap.parse_args()

    if a.summarize_rocprof:
        return summarize(a.summarize_rocprof, a.rocprof_command)
    if a.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {a.gpus})",
              file=sys.stderr)
        return 2

    if a.phase_stamps:
        stamps_lib = os.path.join(ROOT, "global_l2_norm_amd", "_stamps", "libgclip.so")
        if not os.path.exists(stamps_lib):
            print("--phase-stamps needs the diagnostic build: python -m global_l2_norm_amd.build --phase-stamps",
                  file=sys.stderr)
            return 2
        os.environ["GCLIP_LIBRARY"] = stamps_lib
    import torch

    import global_l2_norm_amd as G
    from synth import gradsets as gs

    if not torch.cuda.is_available():
        print("bench.py needs the GPU", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    if a.profile_pass:
        a.no_cpu_baseline = True
    # read-only flush: a sum over an int64 view (no cast, so no temporaries
    # are written and no dirty lines are left to drain into the timed call)
    flush = torch.ones((2 << 30) // 8, dtype=torch.int64, device="cuda")
    if a.profile_pass:
        calibration_copy(flush)
    if a.path == "ref":
        return bench_ref(a, flush)
    if a.path == "accum":
        if a.phase_stamps:
            return bench_phases_accum(a, G, gs, flush)
        return bench_accum(a, G, gs, flush)
    g = gs.make(a.config)
    esize = 4 if g.dtype == "f32" else 2
    tensors = upload(g.arrays, g.dtype)
    pristine = [t.clone() for t in tensors]
    gl = G.GradList(tensors)
    if a.path == "adamw":
        return bench_adamw(a, G, g, tensors, pristine, flush, gl)
    if a.path == "amp":
        return bench_amp(a, G, g, tensors, pristine, flush, gl)
    if a.path == "per_tensor":
        if a.phase_stamps:
            return bench_phases_per_tensor(a, G, g, tensors, pristine, flush, gl)
        return bench_per_tensor(a, G, g, tensors, pristine, flush, gl)
    if a.phase_stamps:
        return bench_phases(a, G, g, tensors, pristine, flush, gl)
    if a.path != "auto":
        gl.set_path(G.GCLIP_PATH_FUSED if a.path == "fused" else G.GCLIP_PATH_SPLIT)
    info = gl.info()
    path_name = {1: "fused", 2: "split"}[info["path"]]
    stream = torch.cuda.current_stream()

    def restore(cold=True):
        for t, p in zip(tensors, pristine):
            t.copy_(p)
        if cold:
            flush.sum()

    def timed_steps(cold):
        for _ in range(a.warmup):
            restore(cold)
            gl.clip_(g.max_norm, g.avg_factor, g.error_if_nonfinite)
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(a.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(a.steps):
            restore(cold)
            ev[i][0].record(stream)
            gl.clip_(g.max_norm, g.avg_factor, g.error_if_nonfinite)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in ev], time.perf_counter() - t0

    ms, t_wall = timed_steps(not a.no_flush)
    st, r = gl.read(g.error_if_nonfinite)
    mean_ms = statistics.fmean(ms)
    wrote = not (r["skipped"] or r["scale"] == 1.0)
    alg = algorithmic_bytes(g.numel, esize, wrote)
    gbps = alg / (mean_ms * 1e-3) / 1e9
    # a list of one group (one worker) is clipped by one workgroup on the fused path
    one_group = info["n_workers"] == 1 and info["n_vectors"] <= 4096 and info["n_scalars"] <= info["worker_threads"]
    kernels = (("k_grad_clip_small" if one_group else "k_grad_clip_fused") if path_name == "fused"
               else "k_grad_norm_partial+k_grad_scale")
    traffic = read_traffic(kernels, a.config)
    roofline = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": kernels,
                "resident_bytes": info["resident_vectors"] * 16}
    # the rate of the bytes that actually crossed HBM, against the same peak
    traffic_fields(roofline, traffic, mean_ms * 1e-3)
    if not a.profile_pass:
        # attainable: the reference read of the list's bytes, plus (when the
        # step writes) the reference in-place copy of them, cold, same events
        nref, rt = ref_times(g.numel * esize, a.steps, flush, stream, copy_too=False)
        att_ms = rt["read"] + (rt["in_place"] if wrote else 0.0)
        roofline["attainable"] = round(alg / (att_ms * 1e-3) / 1e9, 1)
        roofline["frac_of_attainable"] = round(gbps / roofline["attainable"], 4)
        roofline["attainable_basis"] = (f"gclip_ref_read {rt['read'] * 1e3:.1f} us"
                                        + (f" + gclip_ref_copy in place {rt['in_place'] * 1e3:.1f} us" if wrote else "")
                                        + f" over {nref} bytes, cold")
    out = {
        "metric": METRIC if a.config == "andrea120m_f32" else f"clip_grad_norm GB/s and % of HBM peak, {a.config}",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(mean_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": g.dtype,
        "data": "synthetic",
        "config": {"workload": WORKLOADS.get(a.config, a.config), "name": a.config, "path": path_name,
                   "launches_per_step": 1 if path_name == "fused" else 2,
                   "n_tensors": len(g.arrays), "n_elements": g.numel, "algorithmic_bytes_per_step": alg,
                   "clipped": bool(r["clipped"]), "cache_state": "cold" if not a.no_flush else "after restore"},
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "elements_per_s": round(g.numel / (mean_ms * 1e-3), 1),
        "ms_per_step_median": round(statistics.median(ms), 5),
        "ms_per_step_min": round(min(ms), 5),
        "wall_s_timed_loop_incl_restore_and_flush": round(t_wall, 4),
        "roofline": roofline,
        "norm": r["norm"],
    }
    if not a.profile_pass and not a.no_flush:
        wms, _ = timed_steps(False)
        wmean = statistics.fmean(wms)
        out["warm"] = {"ms_per_step": round(wmean, 5), "value": round(alg / (wmean * 1e-3) / 1e9, 1),
                       "pct_hbm_peak": round(100.0 * alg / (wmean * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                       "note": "the same steps without the cache flush: the restore copy leaves part of the "
                               "list in the caches"}
    if st not in (0,) or r["status"] != 0:
        out["error"] = f"status {st}, device status {r['status']}"
    gl.close()
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(g)
    print(json.dumps(out), flush=True)
    return 0


XCDS = 8
PHASES = [(1, "sum chunks done"), (2, "block read into VGPRs and LDS"), (3, "decision seen"),
          (4, "block written back from VGPRs and LDS"), (5, "scale chunks done"), (6, "end")]
TENSOR_PHASES = [(1, "streamed run summed"), (2, "resident pieces read into VGPRs and LDS"),
                 (7, "pieces counted, completed tensors summed"), (3, "decision seen"),
                 (4, "resident pieces written"), (5, "claimed pieces scaled"), (6, "end")]


def bench_phases(a, G, g, tensors, pristine, flush, gl):
    """The fused clip's phase timeline (gclip_clip_ on the fused path)."""
    gl.set_path(G.GCLIP_PATH_FUSED)

    def prepare():
        for t, p in zip(tensors, pristine):
            t.copy_(p)
        if not a.no_flush:
            flush.sum()

    title = f"k_grad_clip_fused, {a.config} ({g.dtype}, {g.numel} elements)"
    rc = phase_timeline(a, G, gl.info()["n_workers"], prepare,
                        lambda: gl.clip_(g.max_norm, g.avg_factor, g.error_if_nonfinite),
                        lambda: gl.read(g.error_if_nonfinite), title)
    gl.close()
    return rc


def bench_phases_accum(a, G, gs, flush):
    """The fused += kernel's phase timeline (gclip_accumulate_clip_ on the
    four-microbatch list of --path accum)."""
    buf, last = gs.andrea120m_f32_accum4_parts()
    acc = upload(buf.arrays, "f32")
    contrib = upload(last.arrays, "f32")
    pristine = [t.clone() for t in acc]
    gl = G.GradList(acc)
    gl.set_path(G.GCLIP_PATH_FUSED)
    c = G.Contribution(gl, contrib)

    def prepare():
        for x, y in zip(acc, pristine):
            x.copy_(y)
        if not a.no_flush:
            flush.sum()

    title = f"k_accum_clip_fused, andrea120m_f32_accum4 (f32, {buf.numel} elements)"
    rc = phase_timeline(a, G, gl.info()["n_workers"], prepare, lambda: gl.accumulate_clip_(c, 1.0, buf.avg_factor),
                        gl.read, title)
    c.close()
    gl.close()
    return rc


def bench_phases_per_tensor(a, G, g, tensors, pristine, flush, gl):
    """The one-launch per-tensor clip's phase timeline (gclip_clip_per_tensor_
    on the fused path, at the per-tensor max_norm of --path per_tensor)."""
    gl.set_path(G.GCLIP_PATH_FUSED)

    def prepare():
        for t, p in zip(tensors, pristine):
            t.copy_(p)
        if not a.no_flush:
            flush.sum()

    title = f"k_tensor_clip_fused, {a.config} ({g.dtype}, {g.numel} elements), per-tensor max_norm {PER_TENSOR_MAX_NORM}"
    rc = phase_timeline(a, G, gl.info()["n_workers"], prepare,
                        lambda: gl.clip_per_tensor_(PER_TENSOR_MAX_NORM, g.avg_factor), gl.read, title,
                        phases=TENSOR_PHASES)
    gl.close()
    return rc


def phase_timeline(a, G, nw, prepare, launch, read, title, phases=PHASES):
    """Run prepare() (restore, flush) and launch() (one fused launch, timed
    with HIP events) warmup + steps times and print the launch's
    phase timeline: per step, every workgroup's stamps from the earliest
    workgroup start; per phase, the median over steps of the median
    workgroup and of the last one (a workgroup that handed its block back
    counts up to the block read)."""
    import ctypes

    import numpy as np
    import torch

    f = G._lib.lib.gclip_phase_stamps
    f.argtypes = [ctypes.POINTER(ctypes.c_uint64), ctypes.c_int32, ctypes.POINTER(ctypes.c_int64)]
    f.restype = ctypes.c_int32
    points = 8
    buf = np.zeros(nw * points, dtype=np.uint64)
    rate = ctypes.c_int64(0)
    per_step = []
    ev_ms = []
    stream = torch.cuda.current_stream()
    for i in range(a.warmup + a.steps):
        prepare()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        launch()
        e1.record(stream)
        torch.cuda.synchronize()
        st = f(buf.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), nw, ctypes.byref(rate))
        if st != 0:
            raise RuntimeError(f"gclip_phase_stamps: status {st}")
        if i < a.warmup:
            continue
        s = buf.reshape(nw, points).astype(np.int64)
        t0 = s[:, 0].min()
        row = {}
        for k, _ in phases:
            ok = s[:, k] >= s[:, 0]
            v = (s[ok, k] - t0) / rate.value * 1e6
            row[k] = (float(np.median(v)), float(v.max()), int(ok.sum())) if ok.any() else None
            # workgroups are dealt to the XCDs in turn: XCD of w = w % XCDS
            xcd = np.arange(nw)[ok] % XCDS
            row[("xcd", k)] = [float(np.median(v[xcd == x])) if (xcd == x).any() else float("nan")
                               for x in range(XCDS)]
        per_step.append(row)
        ev_ms.append(e0.elapsed_time(e1))
    st, r = read()
    print(f"# phase timeline of {title}, {a.steps} cold steps after {a.warmup} warm-up")
    print(f"# {nw} workgroups; wall clock {rate.value / 1e6:.0f} MHz; norm {r['norm']:.6g}, scale {r['scale']:.6g}, "
          f"handed back {r['handed_back']} (last step)")
    print(f"# event time per launch: median "
          f"{statistics.median(ev_ms) * 1e3:.1f} us")
    print(f"# kernel sources sha256/16: {kernel_source_hash()}")
    print("| phase (times from the first workgroup's start) | median workgroup | last workgroup | workgroups |")
    print("|---|---|---|---|")
    for k, name in phases:
        rows = [row[k] for row in per_step if row.get(k) is not None]
        if not rows:
            print(f"| {name} | — | — | 0 |")
            continue
        med = statistics.median(x[0] for x in rows)
        last = statistics.median(x[1] for x in rows)
        cnt = min(x[2] for x in rows)
        print(f"| {name} | {med:.1f} us | {last:.1f} us | {cnt} |")
    print("# each figure is the median over the steps of that step's median (or last) workgroup")
    print()
    print("| phase: median workgroup of each XCD (workgroup index mod 8) | "
          + " | ".join(f"XCD {x}" for x in range(XCDS)) + " |")
    print("|---|" + "---|" * XCDS)
    for k, name in phases:
        rows = [row[("xcd", k)] for row in per_step if row.get(k) is not None]
        if not rows:
            continue
        cells = [statistics.median(r_[x] for r_ in rows) for x in range(XCDS)]
        print(f"| {name} | " + " | ".join(f"{c:.1f}" for c in cells) + " |")
    return 0 if st == 0 and r["status"] == 0 else 1


def bench_ref(a, flush):
    """The reference kernels (include/gclip_ref.h) alone, cold, at the byte
    sizes of the workloads' lists: the attainable rates of a read pass and of
    a read + write pass (in place, and to a second buffer) on this device."""
    import torch
    stream = torch.cuda.current_stream()
    rows = []
    for nb in REF_SIZES:
        n16, rt = ref_times(nb, a.steps, flush, stream)
        rows.append({"bytes": n16,
                     "read_us": round(rt["read"] * 1e3, 2),
                     "read_gbps": round(n16 / (rt["read"] * 1e-3) / 1e9, 1),
                     "in_place_us": round(rt["in_place"] * 1e3, 2),
                     "in_place_gbps": round(2 * n16 / (rt["in_place"] * 1e-3) / 1e9, 1),
                     "copy_us": round(rt["copy"] * 1e3, 2),
                     "copy_gbps": round(2 * n16 / (rt["copy"] * 1e-3) / 1e9, 1)})
        torch.cuda.empty_cache()
    head = rows[1]
    out = {"metric": "attainable streaming GB/s, own reference kernels (read; read+write in place; copy)",
           "value": head["read_gbps"], "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": 2,
           "ms_per_step": round(head["read_us"] * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "u32x4", "data": "synthetic",
           "config": {"workload": "plain streaming over one flat buffer, cold (2 GiB read between reps)",
                      "kernels": "k_ref_read (128 KB per workgroup), k_ref_copy (32 KB per workgroup)"},
           "sizes": rows}
    print(json.dumps(out), flush=True)
    return 0


ADAMW_HP = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


def bench_adamw(a, G, g, grads, pristine, flush, gl):
    """The clip fused into AdamW: a step is gclip_norm over the gradients and
    one gclip_adamw_step (weights and both moments binary32, the gradient
    multiplied by the clip factor on load), against the separate form:
    gclip_clip_ writing the clipped gradient back, then the same AdamW step
    with factor 1.  Weights and moments are restored before every step, the
    caches flushed, and each step is timed with HIP events."""
    import torch
    n = g.numel
    esize = 4 if g.dtype == "f32" else 2
    gen = torch.Generator(device="cuda").manual_seed(12)
    params = [torch.randn(t.numel(), device="cuda", generator=gen) * 0.02 for t in grads]
    m = [torch.zeros(t.numel(), device="cuda") for t in grads]
    v = [torch.zeros(t.numel(), device="cuda") for t in grads]
    p0 = [x.clone() for x in params]
    opt = G.AdamWList(params, grads, m, v)
    stream = torch.cuda.current_stream()

    def restore():
        for x, y in zip(grads, pristine):
            x.copy_(y)
        for x, y in zip(params, p0):
            x.copy_(y)
        for x in m + v:
            x.zero_()
        if not a.no_flush:
            flush.sum()

    def run(fused, ev):
        restore()
        ev[0].record(stream)
        if fused:
            gl.norm(g.avg_factor)
        else:
            gl.clip_(g.max_norm, g.avg_factor)
        ev[1].record(stream)
        if fused:
            opt.step(gl, step=1, max_norm=g.max_norm, avg_factor=g.avg_factor, **ADAMW_HP)
        else:
            opt.step(gl, step=1, max_norm=math.inf, avg_factor=1.0, **ADAMW_HP)
        ev[2].record(stream)

    times = {}
    for fused in (True, False):
        for _ in range(a.warmup):
            run(fused, [torch.cuda.Event(enable_timing=True) for _ in range(3)])
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(a.steps)]
        for ev in evs:
            run(fused, ev)
        torch.cuda.synchronize()
        times[fused] = ([e[0].elapsed_time(e[2]) for e in evs], [e[1].elapsed_time(e[2]) for e in evs])
    opt.close()
    step_ms = statistics.fmean(times[True][0])
    adam_ms = statistics.fmean(times[True][1])
    sep_ms = statistics.fmean(times[False][0])
    adam_bytes = n * (esize + 3 * 4 + 3 * 4)  # read g, p, m, v; write p, m, v
    alg = n * esize + adam_bytes
    cpu = None
    if not a.no_cpu_baseline:
        import numpy as np

        import oracle
        k, tot = 0, 0
        while k < len(g.arrays) and tot + g.arrays[k].size <= 12_000_000:
            tot += g.arrays[k].size
            k += 1
        k = max(k, 1)
        rng = np.random.default_rng(12)
        sg = [x for x in g.arrays[:k]]
        sp = [(rng.standard_normal(x.size) * 0.02).astype(np.float32) for x in sg]
        sm = [np.zeros(x.size, np.float32) for x in sg]
        ns = sum(x.size for x in sg)
        cpu = oracle_rate(lambda: oracle.clip_adamw(sp, sg, sm, [x.copy() for x in sm], g.dtype, g.max_norm,
                                                    g.avg_factor, False, step=1, **ADAMW_HP),
                          lambda: None, ns * esize + ns * (esize + 24),
                          f"the first {k} tensors ({ns} elements): norm, decision, AdamW step")
    out = {
        "metric": "clip + AdamW step GB/s, ANDREA-120M-shaped fp32 weights, moments and grads",
        "value": round(alg / (step_ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(step_ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": g.dtype, "data": "synthetic",
        "config": {"workload": WORKLOADS.get(a.config, a.config) + "; AdamW lr 3e-4, betas (0.9, 0.95), "
                               "eps 1e-8, wd 0.1, step 1", "name": a.config, "path": "norm + adamw",
                   "launches_per_step": 2, "algorithmic_bytes_per_step": alg},
        "pct_hbm_peak": round(100.0 * alg / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
        "separate_ms_per_step": round(sep_ms, 5),
        "separate_algorithmic_bytes": 3 * n * esize + adam_bytes,
        "saved_vs_separate": round(1.0 - step_ms / sep_ms, 4),
        "roofline": traffic_fields(
            {"bound": "hbm", "achieved": round(adam_bytes / (adam_ms * 1e-3) / 1e9, 1), "peak": HBM_PEAK_GBPS,
             "unit": "GB/s", "frac": round(adam_bytes / (adam_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
             "kernel": "k_adamw_clip", "ms_per_launch": round(adam_ms, 5)},
            read_traffic("k_grad_norm_partial+k_adamw_clip", a.config, kernel="k_adamw_clip"), adam_ms * 1e-3),
        "step_traffic": read_traffic("k_grad_norm_partial+k_adamw_clip", a.config),
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)
    return 0


AMP_SCALE = 1024.0


def bench_amp(a, G, g, grads, pristine, flush, gl):
    """The loss-scaled clip: the list is read as gradients of a loss scaled by
    S = 1024, so a = 1 / (n S) is read on the device from the loss-scale
    state, and max_norm is divided by S so that the decision is that of the
    plain run; the loss-scale update follows on the same stream.  Against
    gclip_clip_ with the same factor given by the host.  Gradients and state
    are restored and the caches flushed before every step."""
    import torch
    n_mb = 1.0 / g.avg_factor
    max_norm = g.max_norm / AMP_SCALE
    amp = G.AmpState(grads[0].device, AMP_SCALE)
    stream = torch.cuda.current_stream()

    def restore():
        for x, y in zip(grads, pristine):
            x.copy_(y)
        amp.set(AMP_SCALE)
        if not a.no_flush:
            flush.sum()

    def run(loss_scaled, ev):
        restore()
        ev[0].record(stream)
        if loss_scaled:
            gl.clip_amp_(max_norm, n_mb, amp)
        else:
            gl.clip_(max_norm, g.avg_factor / AMP_SCALE, True)
        ev[1].record(stream)

    times = {}
    for loss_scaled in (True, False):
        for _ in range(a.warmup):
            run(loss_scaled, [torch.cuda.Event(enable_timing=True) for _ in range(2)])
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(a.steps)]
        for ev in evs:
            run(loss_scaled, ev)
        torch.cuda.synchronize()
        times[loss_scaled] = [e[0].elapsed_time(e[1]) for e in evs]
        st, r = gl.read()
        if loss_scaled:
            state = amp.read()
    esize = 4 if g.dtype == "f32" else 2
    wrote = not (r["skipped"] or r["scale"] == 1.0)
    alg = algorithmic_bytes(g.numel, esize, wrote)
    ms = statistics.fmean(times[True])
    plain_ms = statistics.fmean(times[False])
    gbps = alg / (ms * 1e-3) / 1e9
    out = {
        "metric": f"loss-scaled clip_grad_norm GB/s, {a.config}", "value": round(gbps, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": g.dtype, "data": "synthetic",
        "config": {"workload": WORKLOADS.get(a.config, a.config) + f"; read as scaled by S = {AMP_SCALE:g}, "
                               f"{n_mb:g} microbatch(es), max_norm {max_norm:g}", "name": a.config,
                   "path": {1: "fused", 2: "split"}[gl.info()["path"]],
                   "launches_per_step": 1 if gl.info()["path"] == G.GCLIP_PATH_FUSED else 3,
                   "algorithmic_bytes_per_step": alg, "clipped": bool(r["clipped"])},
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "host_factor_ms_per_step": round(plain_ms, 5),
        "loss_scale_overhead_ms": round(ms - plain_ms, 5),
        "state_after": {"scale": state[0], "growth_tracker": state[1], "found_inf": state[2]},
        "roofline": traffic_fields({"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                                    "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                                    "kernel": "k_grad_clip_fused"},
                                   read_traffic("k_grad_clip_fused", f"{a.config}_loss_scaled")
                                   if gl.info()["path"] == G.GCLIP_PATH_FUSED else None, ms * 1e-3),
    }
    if not a.no_cpu_baseline:
        import oracle
        work = [x.copy() for x in g.arrays]

        def restore_cpu():
            for w, x in zip(work, g.arrays):
                w[...] = x

        out["cpu_baseline"] = oracle_rate(lambda: oracle.clip_amp_(work, g.dtype, max_norm, n_mb, AMP_SCALE),
                                          restore_cpu, alg, f"the whole {a.config} list, loss-scaled clip")
    print(json.dumps(out), flush=True)
    return 0


def bench_accum(a, G, gs, flush):
    """The last microbatch's += fused with the clip (gclip_accumulate_clip_:
    one launch on the fused path, which keeps each worker's block of sums on
    chip across the decision), on the four-microbatch ANDREA-120M fp32 list:
    the buffer holds ((c0 + c1) + c2), the contribution is c3, a = 1/4,
    max_norm 1.0 (the average has norm ~4.8, so every step clips).  Also
    timed: the same call on the split path (the += with the norm, the
    per-tensor reduction, the scale pass), the += with the norm alone, and the
    separate form -- torch's += (torch._foreach_add_) then gclip_clip_.  The
    buffer is restored and the caches flushed before every step; every step
    is timed with HIP events."""
    import torch
    buf, last = gs.andrea120m_f32_accum4_parts()
    acc = upload(buf.arrays, "f32")
    contrib = upload(last.arrays, "f32")
    pristine = [t.clone() for t in acc]
    gl = G.GradList(acc)
    c = G.Contribution(gl, contrib)
    stream = torch.cuda.current_stream()
    n = buf.numel
    max_norm, avg = 1.0, buf.avg_factor

    def restore():
        for x, y in zip(acc, pristine):
            x.copy_(y)
        if not a.no_flush:
            flush.sum()

    def run(which, ev):
        restore()
        ev[0].record(stream)
        if which in ("fused", "three_kernels"):
            gl.accumulate_clip_(c, max_norm, avg)
        elif which == "norm_only":
            gl.accumulate_norm(c, avg)
        else:
            torch._foreach_add_(acc, contrib)
            gl.clip_(max_norm, avg)
        ev[1].record(stream)

    times = {}
    for which in ("fused", "norm_only", "three_kernels", "separate"):
        gl.set_path(G.GCLIP_PATH_SPLIT if which == "three_kernels" else G.GCLIP_PATH_AUTO)
        for _ in range(a.warmup):
            run(which, [torch.cuda.Event(enable_timing=True) for _ in range(2)])
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(a.steps)]
        for ev in evs:
            run(which, ev)
        torch.cuda.synchronize()
        times[which] = [e[0].elapsed_time(e[1]) for e in evs]
        if which == "fused":
            st, r = gl.read()
    c.close()
    gl.close()
    ms = statistics.fmean(times["fused"])
    acc_ms = statistics.fmean(times["norm_only"])
    three_ms = statistics.fmean(times["three_kernels"])
    sep_ms = statistics.fmean(times["separate"])
    alg = 5 * n * 4  # += reads the buffer and c3, writes the buffer; the scale pass reads and writes it
    acc_alg = 3 * n * 4
    gbps = alg / (ms * 1e-3) / 1e9
    out = {
        "metric": "last += fused with clip_grad_norm, GB/s, four-microbatch ANDREA-120M fp32",
        "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": WORKLOADS["andrea120m_f32"].replace(", N(0,1e-3^2), max_norm 1.0", "") +
                   "; buffer ((c0+c1)+c2) and contribution c3, each N(0,1e-3^2), a = 1/4, max_norm 1.0",
                   "name": "andrea120m_f32_accum4", "path": "fused", "launches_per_step": 1,
                   "algorithmic_bytes_per_step": alg,
                   "clipped": bool(r["clipped"]), "norm": r["norm"]},
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "accumulate_norm_ms": round(acc_ms, 5),
        "accumulate_norm_gbps": round(acc_alg / (acc_ms * 1e-3) / 1e9, 1),
        "three_kernels_ms_per_step": round(three_ms, 5),
        "separate_ms_per_step": round(sep_ms, 5),
        "separate_note": "torch._foreach_add_ then gclip_clip_ (fused kernel)",
        "saved_vs_separate": round(1.0 - ms / sep_ms, 4),
        "roofline": traffic_fields({"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                                    "frac": round(gbps / HBM_PEAK_GBPS, 4), "kernel": "k_accum_clip_fused"},
                                   read_traffic("k_accum_clip_fused", "andrea120m_f32_accum4_last"), ms * 1e-3),
        "status": st,
    }
    if not a.no_cpu_baseline:
        import oracle
        work = [x.copy() for x in buf.arrays]

        def restore_cpu():
            for w, x in zip(work, buf.arrays):
                w[...] = x

        out["cpu_baseline"] = oracle_rate(lambda: oracle.accumulate_clip_(work, last.arrays, "f32", max_norm, avg),
                                          restore_cpu, alg, "the whole four-microbatch list, last += and clip")
    print(json.dumps(out), flush=True)
    return 0


PER_TENSOR_MAX_NORM = 0.5


def bench_per_tensor(a, G, g, grads, pristine, flush, gl):
    """Per-tensor clipping (every tensor by its own norm) at max_norm 0.5,
    which clips the large matrices and leaves the norm vectors alone: in one
    launch (the fused path, timed as the step), and on the split path (two
    kernels; three with the stop switch); and the per-tensor norms alone.
    Gradients are restored and the caches flushed before every step; each
    step is timed with HIP events."""
    import torch
    stream = torch.cuda.current_stream()
    esize = 4 if g.dtype == "f32" else 2

    def restore():
        for x, y in zip(grads, pristine):
            x.copy_(y)
        if not a.no_flush:
            flush.sum()

    def run(which, ev):
        gl.set_path(G.GCLIP_PATH_SPLIT if which.startswith("split") else G.GCLIP_PATH_AUTO)
        restore()
        ev[0].record(stream)
        if which in ("clip", "split"):
            gl.clip_per_tensor_(PER_TENSOR_MAX_NORM, g.avg_factor)
        elif which in ("clip_stop", "split_stop"):
            # with the stop switch on (no NaN/Inf here, so the same work):
            # the reduction and decisions in a kernel of their own
            gl.clip_per_tensor_(PER_TENSOR_MAX_NORM, g.avg_factor, True)
        else:
            gl.tensor_norms(g.avg_factor)
        ev[1].record(stream)

    times = {}
    for which in ("clip", "clip_stop", "split", "split_stop", "norms"):
        for _ in range(a.warmup):
            run(which, [torch.cuda.Event(enable_timing=True) for _ in range(2)])
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(a.steps)]
        for ev in evs:
            run(which, ev)
        torch.cuda.synchronize()
        times[which] = [e[0].elapsed_time(e[1]) for e in evs]
        if which == "clip":
            st, r = gl.read()
            tr = gl.read_tensors()
            fused = gl.info()["path"] == G.GCLIP_PATH_FUSED
    numel = [t.numel() for t in grads]
    clipped_elems = sum(n for n, t in zip(numel, tr) if float(t["scale"]) != 1.0)
    alg = g.numel * esize + 2 * clipped_elems * esize
    ms = statistics.fmean(times["clip"])
    norm_ms = statistics.fmean(times["norms"])
    gbps = alg / (ms * 1e-3) / 1e9
    norm_gbps = g.numel * esize / (norm_ms * 1e-3) / 1e9
    pt_kernels = "k_tensor_clip_fused" if fused else "k_tensor_partial+k_tensor_clip"
    out = {
        "metric": f"per-tensor clip GB/s, {a.config}", "value": round(gbps, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": g.dtype, "data": "synthetic",
        "config": {"workload": WORKLOADS.get(a.config, a.config) + f"; per-tensor max_norm {PER_TENSOR_MAX_NORM}",
                   "name": a.config, "path": "fused" if fused else "split",
                   "launches_per_step": 1 if fused else 2, "algorithmic_bytes_per_step": alg,
                   "tensors_clipped": int(sum(int(t["clipped"]) for t in tr)), "n_tensors": len(grads),
                   "elements_written": clipped_elems},
        "pct_hbm_peak": round(100.0 * gbps / HBM_PEAK_GBPS, 2),
        "stop_switch_ms_per_step": round(statistics.fmean(times["clip_stop"]), 5),
        "stop_switch_note": "error_if_nonfinite=True" + (", the same one launch" if fused else
                                                          ": partial, decide, scale (three launches)"),
        "split_ms_per_step": round(statistics.fmean(times["split"]), 5),
        "split_stop_switch_ms_per_step": round(statistics.fmean(times["split_stop"]), 5),
        "split_note": "the split path: partial, then decide-and-scale per piece (two launches); with the stop "
                      "switch partial, decide, scale (three)",
        "tensor_norms_ms": round(norm_ms, 5),
        "tensor_norms_gbps": round(norm_gbps, 1),
        "tensor_norms_pct_hbm_peak": round(100.0 * norm_gbps / HBM_PEAK_GBPS, 2),
        "roofline": traffic_fields({"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                                    "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                                    "kernel": pt_kernels},
                                   read_traffic(pt_kernels, a.config), ms * 1e-3),
        "status": st,
    }
    if not a.profile_pass:
        # attainable: the reference read of the list, plus the reference
        # in-place copy of the share of it that the clip writes
        nref, rt = ref_times(g.numel * esize, a.steps, flush, stream, copy_too=False)
        wshare = clipped_elems / g.numel if g.numel else 0.0
        att_ms = rt["read"] + rt["in_place"] * wshare
        out["roofline"]["attainable"] = round(alg / (att_ms * 1e-3) / 1e9, 1)
        out["roofline"]["frac_of_attainable"] = round(gbps / out["roofline"]["attainable"], 4)
        out["roofline"]["attainable_basis"] = (f"gclip_ref_read {rt['read'] * 1e3:.1f} us + {wshare:.4f} x "
                                               f"gclip_ref_copy in place {rt['in_place'] * 1e3:.1f} us over "
                                               f"{nref} bytes, cold")
    if not a.no_cpu_baseline:
        import oracle
        work = [x.copy() for x in g.arrays]

        def restore_cpu():
            for w, x in zip(work, g.arrays):
                w[...] = x

        out["cpu_baseline"] = oracle_rate(lambda: oracle.clip_per_tensor_(work, g.dtype, PER_TENSOR_MAX_NORM,
                                                                          g.avg_factor),
                                          restore_cpu, alg, f"the whole {a.config} list, per-tensor clip")
    print(json.dumps(out), flush=True)
    return 0


def _stats_rows(d):
    import csv
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *kernel_stats.csv under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _counter_rows(d):
    import csv
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no *counter_collection.csv under {d}")
    with open(files[0]) as f:
        return list(csv.DictReader(f))


def _short_kernel(name):
    base = name.split("(")[0]
    for k in ("k_grad_clip_fused", "k_grad_clip_small", "k_grad_norm_partial", "k_grad_scale", "k_accum_clip_fused",
              "k_ref_read", "k_ref_copy"):
        if k in base:
            return base.replace("void ", "").strip()
    if "neg_kernel" in name:
        return "torch neg (elementwise, calibration copy)"
    if "reduce_kernel" in base:
        return "torch sum (reduce, cache flush)"
    if "direct_copy_kernel" in name:
        return "torch copy_ (elementwise, restore)"
    return base.replace("void ", "").strip()[-60:]


def summarize(args, commands):
    """Write a short text summary of rocprofv3 output into profiles/."""
    kind, out = args[0], args[1]
    dirs = args[2:]
    lines = ["# summary of rocprofv3 output, written by: python bench.py --summarize-rocprof " + " ".join(args)]
    for c in commands:
        lines.append(f"# profiled command: {c}")
    lines.append(f"kernel_source_sha256_16: {kernel_source_hash()}")
    if kind == "trace":
        rows = _stats_rows(dirs[0])
        lines.append("# rocprofv3 --kernel-trace --stats: per-kernel time (ns)")
        lines.append(f"{'kernel':62s} {'calls':>6s} {'avg_ns':>12s} {'min_ns':>12s} {'max_ns':>12s} {'pct':>6s}")
        for r in rows:
            short = _short_kernel(r.get("Name", ""))[:62]
            lines.append(f"{short:62s} {r.get('Calls', ''):>6s} {float(r.get('AverageNs', 0)):12.1f} "
                         f"{float(r.get('MinNs', 0)):12.1f} {float(r.get('MaxNs', 0)):12.1f} "
                         f"{float(r.get('Percentage', 0)):6.2f}")
        # this library's kernels per launch shape, from the per-dispatch trace:
        # one line per (kernel, grid), with the resources each launch held
        import csv
        files = glob.glob(os.path.join(dirs[0], "**", "*kernel_trace.csv"), recursive=True)
        if files:
            groups = {}
            for r in csv.DictReader(open(files[0])):
                name = r.get("Kernel_Name", "")
                if "gclip::" not in name:
                    continue
                key = (_short_kernel(name)[:52], int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"])),
                       int(r["Workgroup_Size_X"]), r.get("VGPR_Count", ""), r.get("Accum_VGPR_Count", ""),
                       r.get("LDS_Block_Size", ""), r.get("Scratch_Size", ""))
                groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
            lines.append("# per launch shape (from the per-dispatch trace): workgroups x lanes, VGPRs, AGPRs, LDS and "
                         "scratch bytes per workgroup")
            lines.append(f"{'kernel':52s} {'wgs':>7s} {'lanes':>5s} {'vgpr':>4s} {'agpr':>4s} {'lds':>7s} "
                         f"{'scr':>4s} {'calls':>5s} {'avg_ns':>11s} {'median_ns':>11s}")
            for key in sorted(groups):
                d = groups[key]
                lines.append(f"{key[0]:52s} {key[1]:7d} {key[2]:5d} {key[3]:>4s} {key[4]:>4s} {key[5]:>7s} "
                             f"{key[6]:>4s} {len(d):5d} {statistics.fmean(d):11.1f} {statistics.median(d):11.1f}")
    elif kind == "pmc":
        # the kernels are named by the summary file: KERNEL[+KERNEL]__CONFIG__pmc.txt
        kernels = os.path.basename(out).split("__")[0].split("+")
        per = {}
        for d, counter in zip(dirs, ("FETCH_SIZE", "WRITE_SIZE")):
            rows = _counter_rows(d)
            acc = {}
            for r in rows:
                if r.get("Counter_Name", "") != counter:
                    continue
                name = r.get("Kernel_Name", "")
                if "neg_kernel" in name or "k_calib_copy" in name:
                    key = "copy"
                else:
                    key = next((k for k in kernels if re.search(r"\b" + re.escape(k) + r"\b", name)), None)
                if key is None:
                    continue
                acc.setdefault(key, []).append(float(r["Counter_Value"]))
            per[counter] = {k: statistics.median(v) for k, v in acc.items()}
        missing = [k for k in kernels + ["copy"] for c in per if k not in per[c]]
        if missing:
            raise SystemExit(f"no counter rows for {sorted(set(missing))}")
        copy_bytes = CALIBRATION_BYTES
        f_cal = per["FETCH_SIZE"]["copy"] * 1024 / copy_bytes
        w_cal = per["WRITE_SIZE"]["copy"] * 1024 / copy_bytes
        lines += ["# rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE (KiB per dispatch, median over dispatches);",
                  "# each scaled by what the counter reads for a copy kernel that reads and writes",
                  f"# exactly {CALIBRATION_BYTES} bytes; a step of several kernels is their sum"]
        fetch = write = 0.0
        for k in kernels:
            lines += [f"fetch_kib_per_dispatch {k}: {per['FETCH_SIZE'][k]:.1f}",
                      f"write_kib_per_dispatch {k}: {per['WRITE_SIZE'][k]:.1f}"]
            fetch += per["FETCH_SIZE"][k] * 1024 / f_cal
            write += per["WRITE_SIZE"][k] * 1024 / w_cal
        lines += [f"fetch_kib_per_dispatch_copy: {per['FETCH_SIZE']['copy']:.1f}",
                  f"write_kib_per_dispatch_copy: {per['WRITE_SIZE']['copy']:.1f}",
                  f"fetch_calibration (counter bytes / copy bytes): {f_cal:.4f}",
                  f"write_calibration (counter bytes / copy bytes): {w_cal:.4f}",
                  f"hbm_fetch_bytes_per_dispatch: {fetch:.0f}",
                  f"hbm_write_bytes_per_dispatch: {write:.0f}",
                  f"hbm_bytes_per_dispatch: {fetch + write:.0f}"]
    else:
        raise SystemExit("kind must be 'trace' or 'pmc'")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


if __name__ == "__main__":
    sys.exit(main())
