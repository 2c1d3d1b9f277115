"""Hot calls captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every launch leaves a list's workspace as it found it, so a captured call
can be replayed.  Each test captures one call, then replays it several times
with different gradient contents written between the replays (eager work and
synchronisations in between), and checks every replay bit for bit against
the same call made eagerly on the same contents -- so a replay that used the
decision of an earlier one, or a counter left behind, would show.  The
eager results themselves are checked against the oracle by the other tests;
here the first replay is also checked against it."""
import math

import numpy as np
import pytest

import oracle
from synth import gradsets as gs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("the gpu tests need an MI355X")
    import global_l2_norm_amd  # noqa: F401  (fails loudly when libgclip.so is missing)


def _G():
    import global_l2_norm_amd as G
    return G


def capture(call):
    """Warm up on a side stream, then capture call() into a graph."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    return g


def variants(rng, dtype, sizes, n=4):
    """Contents for successive replays: norms on both sides of max_norm 1.0,
    and (last) one with a NaN."""
    out = []
    for k, sigma in enumerate([1e-3, 1e-5, 3e-3, 1e-3][:n]):
        arrays = [gs.to_storage(rng.standard_normal(m) * sigma, dtype) for m in sizes]
        if k == n - 1:
            arrays[0][5] = gs.to_storage(np.array([math.nan]), dtype)[0]
        out.append(arrays)
    return out


SIZES = [3_000_001, 590_000, 768, 2_359_296, 1, 4_097]


def load(ts, arrays, dtype):
    for t, a in zip(ts, gu.upload(arrays, dtype)):
        t.copy_(a)


@pytest.mark.parametrize("path", ("fused", "split"))
@pytest.mark.parametrize("dtype", ("f32", "bf16"))
def test_clip_replays(dtype, path):
    import torch
    G = _G()
    rng = np.random.default_rng(4000)
    contents = variants(rng, dtype, SIZES)
    ts = gu.upload(contents[0], dtype)
    gl = G.GradList(ts)
    gl.set_path(G.GCLIP_PATH_FUSED if path == "fused" else G.GCLIP_PATH_SPLIT)
    g = capture(lambda: gl.clip_(1.0, 0.5, True))
    for rep in range(2):
        for k, arrays in enumerate(contents):
            load(ts, arrays, dtype)
            gl.clip_(1.0, 0.5, True)
            _, r_eager = gl.read(True)
            eager = gu.download(ts, dtype)
            load(ts, arrays, dtype)
            torch.cuda.synchronize()
            g.replay()
            _, r = gl.read(True)
            out = gu.download(ts, dtype)
            what = f"{dtype} {path} replay {rep}.{k}"
            gu.assert_bitwise_equal(out, eager, what)
            for key in ("sumsq", "norm", "scale", "nonfinite", "clipped", "skipped", "status"):
                assert r[key] == r_eager[key] or (isinstance(r[key], float) and math.isnan(r[key])
                                                  and math.isnan(r_eager[key])), (what, key)
            if rep == 0:
                ref = [a.copy() for a in arrays]
                ro = oracle.clip_(ref, dtype, 1.0, 0.5, True)
                assert r["skipped"] == ro["skipped"] and r["clipped"] == ro["clipped"], what
                if not ro["skipped"]:
                    gu.assert_elems_close(out, ref, dtype, what)
    gl.close()


@pytest.mark.parametrize("path", ("fused", "split"))
def test_per_tensor_and_accumulate_replays(path):
    import torch
    G = _G()
    rng = np.random.default_rng(4100)
    contents = variants(rng, "f32", SIZES, n=3)
    contrib = [gs.to_storage(rng.standard_normal(m) * 1e-3, "f32") for m in SIZES]
    ts = gu.upload(contents[0], "f32")
    tc = gu.upload(contrib, "f32")
    gl = G.GradList(ts)
    gl.set_path(G.GCLIP_PATH_FUSED if path == "fused" else G.GCLIP_PATH_SPLIT)
    c = G.Contribution(gl, tc)
    for name, call in (("per_tensor", lambda: gl.clip_per_tensor_(0.5, 1.0, False)),
                       ("per_tensor_stop", lambda: gl.clip_per_tensor_(0.5, 1.0, True)),
                       ("accumulate", lambda: gl.accumulate_clip_(c, 1.0, 0.5, False))):
        g = capture(call)
        for k, arrays in enumerate(contents):
            load(ts, arrays, "f32")
            call()
            eager = gu.download(ts, "f32")
            _, r_eager = gl.read()
            load(ts, arrays, "f32")
            torch.cuda.synchronize()
            g.replay()
            out = gu.download(ts, "f32")
            _, r = gl.read()
            gu.assert_bitwise_equal_but_nan(out, eager, "f32", f"{name} replay {k}")
            assert r["clipped"] == r_eager["clipped"] and r["nonfinite"] == r_eager["nonfinite"], (name, k)
            assert r["skipped"] == r_eager["skipped"], (name, k)
            if name == "per_tensor_stop" and r["nonfinite"]:
                assert r["skipped"], (name, k)
                gu.assert_bitwise_equal_but_nan(out, arrays, "f32", f"{name} replay {k}: stopped, nothing written")
    gu.assert_bitwise_equal(gu.download(tc, "f32"), contrib, "contribution only read")
    c.close()
    gl.close()


def test_loss_scaled_replays_follow_the_state():
    """The loss-scale state lives in device memory: successive replays see
    the state the previous one left, as successive eager calls would."""
    import torch
    G = _G()
    rng = np.random.default_rng(4200)
    sizes = [70_001, 4_096 * 10 + 3]
    ts = gu.upload([np.zeros(m, np.uint16) for m in sizes], "f16")
    gl = G.GradList(ts)
    amp = G.AmpState(ts[0].device, 1024.0, 2.0, 0.5, 2)
    g = capture(lambda: gl.clip_amp_(0.5, 1.0, amp))
    amp.set(1024.0, 0)
    scale, tracker = 1024.0, 0
    for step in range(7):
        arrays = [gs.to_storage(rng.standard_normal(m) * 1e-3 * scale, "f16") for m in sizes]
        if step == 3:
            arrays[1][17] = gs.to_storage(np.array([math.inf]), "f16")[0]
        load(ts, arrays, "f16")
        torch.cuda.synchronize()
        g.replay()
        out = gu.download(ts, "f16")
        sc, tr, fi = amp.read()
        ref = [a.copy() for a in arrays]
        ro = oracle.clip_amp_(ref, "f16", 0.5, 1.0, scale, tracker, 2.0, 0.5, 2)
        assert fi == ro["found_inf"] and sc == ro["loss_scale"] and tr == ro["growth_tracker"], step
        if ro["skipped"] or ro["scale"] == 1.0:
            gu.assert_bitwise_equal(out, arrays, f"step {step} untouched")
        else:
            gu.assert_elems_close(out, ref, "f16", f"step {step}")
        scale, tracker = ro["loss_scale"], ro["growth_tracker"]
    assert scale != 1024.0
    gl.close()
