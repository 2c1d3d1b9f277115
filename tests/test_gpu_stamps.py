"""The phase-timeline build of the fused kernels (include/gclip_stamps.h,
global_l2_norm_amd/_stamps/libgclip.so): bench.py --phase-stamps runs it in
a process of its own and prints, per phase, when the median and the last
workgroup ended it.  Every workgroup must have stamped every phase it
reaches, in phase order."""
import os
import re
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
STAMPS_LIB = os.path.join(ROOT, "global_l2_norm_amd", "_stamps", "libgclip.so")
PHASES = ["sum chunks done", "block read into VGPRs and LDS", "decision seen",
          "block written back from VGPRs and LDS", "scale chunks done", "end"]
TENSOR_PHASES = ["streamed run summed", "resident pieces read into VGPRs and LDS",
                 "pieces counted, completed tensors summed", "decision seen", "resident pieces written",
                 "claimed pieces scaled", "end"]


def _timeline(args):
    if not os.path.exists(STAMPS_LIB):
        pytest.skip("the --phase-stamps build is not there (python -m global_l2_norm_amd.build --phase-stamps)")
    print(f"phase timeline: bench.py --phase-stamps {' '.join(args)}", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--phase-stamps", *args],
                       cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]
    rows = {}
    for line in r.stdout.splitlines():
        m = re.match(r"\| ([A-Za-z ,]+) \| ([0-9.]+) us \| ([0-9.]+) us \| (\d+) \|", line)
        if m:
            rows[m.group(1)] = (float(m.group(2)), float(m.group(3)), int(m.group(4)))
    workers = int(re.search(r"# (\d+) workgroups", r.stdout).group(1))
    return rows, workers


@pytest.mark.parametrize("config", ["tiny_f32", "andrea120m_f16_spike"])
def test_phase_timeline_of_a_clipping_list(config):
    rows, workers = _timeline(["--config", config, "--steps", "3", "--warmup", "1"])
    assert list(rows) == PHASES, rows
    prev = (0.0, 0.0)
    for name in PHASES:
        med, last, n = rows[name]
        assert n == workers, (name, n, workers)
        assert 0.0 <= med <= last, (name, med, last)
        assert med >= prev[0] - 1e-9 and last >= prev[1] - 1e-9, (name, rows)
        prev = (med, last)


def test_phase_timeline_without_writes():
    """The no-write list decides factor 1: no workgroup writes its block or
    scales a chunk, so those two phases have no stamps."""
    rows, workers = _timeline(["--config", "andrea120m_f16_small", "--steps", "3", "--warmup", "1"])
    assert [n for n in PHASES if n in rows] == ["sum chunks done", "block read into VGPRs and LDS",
                                                  "decision seen", "end"], rows
    assert all(rows[n][2] == workers for n in rows)


def test_phase_timeline_of_the_per_tensor_clip():
    """The one-launch per-tensor clip stamps its own phases, in order."""
    rows, workers = _timeline(["--path", "per_tensor", "--config", "andrea120m_f16_spike", "--steps", "3",
                               "--warmup", "1"])
    assert list(rows) == TENSOR_PHASES, rows
    prev = (0.0, 0.0)
    for name in TENSOR_PHASES:
        med, last, n = rows[name]
        assert n == workers, (name, n, workers)
        assert 0.0 <= med <= last and med >= prev[0] - 1e-9 and last >= prev[1] - 1e-9, (name, rows)
        prev = (med, last)
