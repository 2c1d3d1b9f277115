"""GPU parity of the loss-scaled steps (gclip_norm_amp, gclip_clip_amp_,
gclip_adamw_step_amp), through the C ABI, against the oracle.

The averaging factor is a = 1 / (n S), with the binary32 loss scale S read on
the device; the clip tolerances are those of the plain path (norm relative
1e-5, fp32 elements relative 1e-5, fp16/bf16 elements 1 ulp), the AdamW
tolerances those of the optimizer tests.  The loss-scale state (scale,
count of clean steps, found-inf flag) must match the oracle's bit for bit
after every step, and a found-inf step must leave the gradients (and the
weights and moments) bitwise unchanged."""
import math

import numpy as np
import pytest

import oracle
from synth import gradsets as gs
from tests import gpu_util as gu
from tests.test_gpu_adamw import HP, assert_adamw_close

pytestmark = pytest.mark.gpu

PATHS = ("fused", "split")
DTYPES = ("f32", "f16", "bf16")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("the gpu tests need an MI355X")
    import global_l2_norm_amd  # noqa: F401  (fails loudly when libgclip.so is missing)


def _G():
    import global_l2_norm_amd as G
    return G


def make_list(tensors, path):
    G = _G()
    gl = G.GradList(tensors)
    gl.set_path(G.GCLIP_PATH_FUSED if path == "fused" else G.GCLIP_PATH_SPLIT)
    return gl


def check_clip_amp(arrays, dtype, max_norm, n, scale, tracker, growth, backoff, interval, path, what,
                   gl=None, ts=None, amp=None):
    """One gclip_clip_amp_ on the GPU against oracle.clip_amp_ (state included)."""
    G = _G()
    own = gl is None
    if own:
        ts = gu.upload(arrays, dtype)
        gl = make_list(ts, path)
    if amp is None:
        amp = G.AmpState(ts[0].device if ts else "cuda", scale, growth, backoff, interval)
        amp.set(scale, tracker)
    gl.clip_amp_(max_norm, n, amp)
    st, r = gl.read()
    out = gu.download(ts, dtype)
    sc, tr, fi = amp.read()
    ref = [a.copy() for a in arrays]
    ro = oracle.clip_amp_(ref, dtype, max_norm, n, scale, tracker, growth, backoff, interval)
    assert r["status"] == 0, what
    assert fi == ro["found_inf"] == r["nonfinite"], what
    assert np.float32(sc).tobytes() == np.float32(ro["loss_scale"]).tobytes(), (what, sc, ro["loss_scale"])
    assert tr == ro["growth_tracker"], (what, tr, ro["growth_tracker"])
    if not math.isnan(ro["norm"]):
        gu.assert_norm_close(r["norm"], ro["norm"], what)
        assert r["clipped"] == ro["clipped"], what
    assert r["skipped"] == ro["skipped"], what
    if ro["skipped"] or ro["scale"] == 1.0:
        gu.assert_bitwise_equal(out, arrays, what + " (must be untouched)")
    else:
        gu.assert_elems_close(out, ref, dtype, what)
    if own:
        gl.close()
    return r, ro, out


# ------------------------------------------------------------------ worked example
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_unscale_before_clip_6_8(dtype, path):
    """[6, 8] scaled by S = 1024, clipped at 5: the unscaled [3, 4], exactly."""
    a = [gs.to_storage(np.array([6.0 * 1024, 8.0 * 1024]), dtype)]
    r, ro, out = check_clip_amp(a, dtype, 5.0, 1.0, 1024.0, 0, 2.0, 0.5, 2000, path, f"6_8 {dtype} {path}")
    assert r["norm"] == 10.0 and r["clipped"] and not r["nonfinite"]
    assert np.array_equal(gu.values(out[0], dtype), [3.0, 4.0])


def test_norm_amp_matches_avg_factor():
    """gclip_norm_amp(n, S) gives the norm of gclip_norm with a = 1 / (n S)."""
    G = _G()
    rng = np.random.default_rng(71)
    arrays = [gs.to_storage(rng.standard_normal(k) * 300.0, "f16") for k in (4096 * 9 + 17, 70_001, 5)]
    ts = gu.upload(arrays, "f16")
    gl = G.GradList(ts)
    amp = G.AmpState(ts[0].device, 8192.0)
    gl.norm_amp(3.0, amp)
    _, r = gl.read()
    ro = oracle.clip_([a.copy() for a in arrays], "f16", 1e30, oracle.amp_avg(3.0, 8192.0))
    gu.assert_norm_close(r["norm"], ro["norm"], "norm_amp")
    assert amp.read() == (8192.0, 0, False)  # the norm alone leaves the state as it is
    gu.assert_bitwise_equal(gu.download(ts, "f16"), arrays, "norm_amp reads only")
    gl.close()


# ------------------------------------------------------------------ a run of loss-scaled steps
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype", ("f16", "bf16"))
def test_step_sequence(dtype, path):
    """Twelve steps over one list (several tiles and a ragged tail): the
    gradients of each step are drawn at the current loss scale, some steps
    hold a NaN or Inf; the state must follow the oracle's bit for bit."""
    G = _G()
    rng = np.random.default_rng(1000 + DTYPES.index(dtype) * 10 + PATHS.index(path))
    sizes = [512 * 1024 + 3, 33, 4096 * 40 + 1000, 1, 250_000]
    growth, backoff, interval = 2.0, 0.5, 3
    scale, tracker = 2.0 ** 12, 0
    ts = gu.upload([np.zeros(k, gs.storage_dtype(dtype)) for k in sizes], dtype)
    gl = make_list(ts, path)
    amp = G.AmpState(ts[0].device, scale, growth, backoff, interval)
    bad_steps = {4: math.inf, 7: math.nan, 8: -math.inf}
    for step in range(12):
        sigma = 1e-3 * scale  # scaled gradients: the loss was multiplied by S
        arrays = [gs.to_storage(rng.standard_normal(k) * sigma, dtype) for k in sizes]
        if step in bad_steps:
            t = int(rng.integers(0, len(sizes)))
            arrays[t][int(rng.integers(0, sizes[t]))] = gs.to_storage(np.array([bad_steps[step]]), dtype)[0]
        for dst, a in zip(ts, gu.upload(arrays, dtype)):
            dst.copy_(a)
        r, ro, _ = check_clip_amp(arrays, dtype, 0.5, 2.0, scale, tracker, growth, backoff, interval, path,
                                  f"{dtype} {path} step {step}", gl=gl, ts=ts, amp=amp)
        assert ro["found_inf"] == (step in bad_steps)
        scale, tracker = ro["loss_scale"], ro["growth_tracker"]
    assert scale != 2.0 ** 12  # the run both grew and backed off the scale
    gl.close()


@pytest.mark.parametrize("path", PATHS)
def test_growth_that_overflows_is_not_taken(path):
    big = float(np.float32(1.5 * 2.0 ** 127))
    a = [gs.to_storage(np.linspace(-1.0, 1.0, 5000) * 1e30, "f32")]
    check_clip_amp(a, "f32", 1.0, 1.0, big, 0, 2.0, 0.5, 1, path, f"overflow {path}")


@pytest.mark.parametrize("path", PATHS)
def test_invalid_scale_in_state_writes_nothing(path):
    """A state whose scale is not positive and finite counts as found-inf."""
    G = _G()
    a = [gs.to_storage(np.arange(1.0, 2001.0), "f32")]
    for bad in (0.0, -4.0, math.inf, math.nan):
        ts = gu.upload(a, "f32")
        gl = make_list(ts, path)
        amp = G.AmpState(ts[0].device, bad)
        gl.clip_amp_(1.0, 1.0, amp)
        st, r = gl.read()
        _, tr, fi = amp.read()
        assert fi and r["nonfinite"] and r["skipped"] and tr == 0, bad
        gu.assert_bitwise_equal(gu.download(ts, "f32"), a, f"scale {bad}")
        gl.close()


# ------------------------------------------------------------------ full size
@pytest.mark.parametrize("path", PATHS)
def test_andrea120m_f16_loss_scaled(path):
    """The ANDREA-120M fp16 list read as gradients scaled by S = 1024, two
    microbatches (unscaled norm ~0.145), clipped at 0.1; then the same list
    with one NaN: found-inf, nothing written, the scale halves."""
    g = gs.andrea120m_f16_spike()
    check_clip_amp(g.arrays, "f16", 0.1, 2.0, 1024.0, 7, 2.0, 0.5, 2000, path, f"andrea f16 amp {path}")
    gs.inject_nan(g, "h11.W_2", 123_457)
    r, ro, _ = check_clip_amp(g.arrays, "f16", 0.1, 2.0, 1024.0, 7, 2.0, 0.5, 2000, path,
                              f"andrea f16 amp nan {path}")
    assert ro["found_inf"] and ro["loss_scale"] == 512.0 and ro["growth_tracker"] == 0


# ------------------------------------------------------------------ AdamW on the unscaled, clipped gradient
def _adam_case(rng, sizes, dtype, scale, bad=None):
    params = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in sizes]
    m = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for n in sizes]
    v = [(rng.random(n) * 1e-6).astype(np.float32) for n in sizes]
    grads = [gs.to_storage(rng.standard_normal(n) * 1e-2 * scale, dtype) for n in sizes]
    if bad is not None:
        grads[-1][len(grads[-1]) // 2] = gs.to_storage(np.array([bad]), dtype)[0]
    return params, grads, m, v


@pytest.mark.parametrize("bad", (None, math.inf))
@pytest.mark.parametrize("dtype", DTYPES)
def test_adamw_step_amp(dtype, bad):
    import torch
    G = _G()
    rng = np.random.default_rng(300 + DTYPES.index(dtype))
    sizes = [4096 * 5 + 7, 130_000, 3]
    scale, tracker, n, max_norm, step = 512.0, 2, 4.0, 0.05, 3
    params, grads, m, v = _adam_case(rng, sizes, dtype, scale, bad)
    dev = [torch.from_numpy(x.copy()).to("cuda") for x in params], gu.upload(grads, dtype), \
        [torch.from_numpy(x.copy()).to("cuda") for x in m], [torch.from_numpy(x.copy()).to("cuda") for x in v]
    tp, tg, tm, tv = dev
    gl = G.GradList(tg)
    opt = G.AdamWList(tp, tg, tm, tv)
    amp = G.AmpState(tg[0].device, scale, 2.0, 0.5, 3)
    amp.set(scale, tracker)
    gl.norm_amp(n, amp)
    opt.step_amp(gl, amp, step=step, max_norm=max_norm, n_microbatches=n, **HP)
    st, r = gl.read()
    out = tuple([t.cpu().numpy() for t in group] for group in (tp, tm, tv))
    sc, tr, fi = amp.read()
    avg = oracle.amp_avg(n, scale)
    ro, ref = oracle.clip_adamw(params, grads, m, v, dtype, max_norm, avg, True, step=step, **HP)
    esc, etr = oracle.amp_update(scale, tracker, ro["nonfinite"], 2.0, 0.5, 3)
    assert fi == ro["nonfinite"] == (bad is not None)
    assert np.float32(sc).tobytes() == np.float32(esc).tobytes() and tr == etr
    gu.assert_bitwise_equal(gu.download(tg, dtype), grads, "gradients are only read")
    if ro["skipped"]:
        for a, b in zip(out, (params, m, v)):
            gu.assert_bitwise_equal(a, b, "found-inf: nothing written")
    else:
        gu.assert_norm_close(r["norm"], ro["norm"], "adamw amp norm")
        assert r["clipped"] == ro["clipped"]
        assert_adamw_close(out, ref, (params, m, v), grads, dtype, ro["scale"], HP, step, f"adamw amp {dtype}")
    opt.close()
    gl.close()


# ------------------------------------------------------------------ argument checks
def test_invalid_arguments():
    import torch
    G = _G()
    ts = gu.upload([np.ones(10, np.float32)], "f32")
    gl = G.GradList(ts)
    amp = G.AmpState(ts[0].device, 1024.0)
    for kw in (dict(growth_factor=0.5), dict(growth_factor=math.inf), dict(backoff_factor=0.0),
               dict(backoff_factor=1.5), dict(backoff_factor=math.nan), dict(growth_interval=0)):
        p = dict(growth_factor=2.0, backoff_factor=0.5, growth_interval=10)
        p.update(kw)
        with pytest.raises(G.GclipError):
            G.gclip_clip_amp_(gl.handle, 1.0, 1.0, amp.d_state, p["growth_factor"], p["backoff_factor"],
                              p["growth_interval"], gl.d_result, torch.cuda.current_stream().cuda_stream)
    for n in (0.0, -1.0, math.inf, math.nan):
        with pytest.raises(G.GclipError):
            gl.clip_amp_(1.0, n, amp)
        with pytest.raises(G.GclipError):
            gl.norm_amp(n, amp)
    with pytest.raises(G.GclipError):
        G.gclip_norm_amp(gl.handle, 1.0, 0, gl.d_result, torch.cuda.current_stream().cuda_stream)
    with pytest.raises(G.GclipError):
        G.gclip_clip_amp_(gl.handle, 1.0, 1.0, amp.d_state + 2, 2.0, 0.5, 10, gl.d_result,
                          torch.cuda.current_stream().cuda_stream)
    # nothing ran: the gradients and the state are as they were
    gu.assert_bitwise_equal(gu.download(ts, "f32"), [np.ones(10, np.float32)], "rejected calls write nothing")
    assert amp.read() == (1024.0, 0, False)
    gl.close()
