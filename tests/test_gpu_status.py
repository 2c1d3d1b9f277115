"""A failed gathering wait stops whatever follows on the same result block.

gclip_accumulate_norm, and the split path of gclip_accumulate_clip_, reduce
the per-tensor sums in one gathering workgroup whose wait is bounded.  With
that bound cut to nothing (gclip_set_gather_wait(0): a limit on the kernel's
own wait, set from the host, so every kernel still ends normally) it gives
up in most calls and reports GCLIP_DEVICE_WAIT_TIMEOUT in the result block.
The block's sumsq and nonfinite are then not this call's.  The scale pass and
the optimizer step that read the block must not act on them: they write no
gradient and take no step, and gclip_result_read returns GCLIP_EDEVICE.

Before every such call the same block is left clean by a plain norm pass
(finite norm above the threshold, no NaN), so acting on the stale figures
would scale the sums or step the weights; with a NaN in the contribution it
would also let the NaN reach the weights past the stop switch.  Calls that
do not give up are checked against the oracle as usual."""
import math

import numpy as np
import pytest

import oracle
from synth import gradsets as gs
from tests import gpu_util as gu
from tests.test_gpu_adamw import HP, assert_adamw_close

pytestmark = pytest.mark.gpu

REPS = 4
# calls beyond REPS, at most, until one has given up waiting (each call does
# so or not by a race between the gathering workgroup and the others)
MAX_REPS = 12
# many one-element tensors keep the gathering workgroup waiting for the
# others' sums; the 4M-element tensor gives a norm of ~20, well above c = 1
SIZES = [5] + [1] * 1500 + [4_000_001] + [300] * 200 + [0]
NAN_AT = 7  # one of the one-element tensors


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("the gpu tests need an MI355X")
    import global_l2_norm_amd  # noqa: F401  (fails loudly when libgclip.so is missing)


def _G():
    import global_l2_norm_amd as G
    return G


def _lists(seed, nan):
    rng = np.random.default_rng(seed)
    acc = [gs.to_storage(rng.standard_normal(n) * 1e-2, "f32") for n in SIZES]
    contrib = [gs.to_storage(rng.standard_normal(n) * 1e-2, "f32") for n in SIZES]
    if nan:
        contrib[NAN_AT] = contrib[NAN_AT].copy()
        contrib[NAN_AT][0] = np.float32("nan")
    summed = [a.copy() for a in acc]
    oracle.accumulate_(summed, contrib, "f32")
    return acc, contrib, summed


def _reload(ts, arrays):
    import torch
    for t, a in zip(ts, arrays):
        if a.size:
            t.copy_(torch.from_numpy(a))


@pytest.mark.parametrize("nan", (False, True))
def test_split_accumulate_clip_after_gather_timeout(nan):
    G = _G()
    from global_l2_norm_amd import _lib
    acc, contrib, summed = _lists(5100 + nan, nan)
    clipped = [a.copy() for a in summed]
    ro = oracle.clip_(clipped, "f32", 1.0, 1.0, True)
    assert ro["nonfinite"] == nan and (ro["skipped"] or ro["clipped"])
    ta, tc = gu.upload(acc, "f32"), gu.upload(contrib, "f32")
    gl = G.GradList(ta)
    gl.set_path(G.GCLIP_PATH_SPLIT)
    c = G.Contribution(gl, tc)
    timeouts = 0
    calls = 0
    for rep in range(MAX_REPS):
        if rep >= REPS and timeouts:
            break
        calls += 1
        _reload(ta, acc)
        gl.norm(1.0)  # a clean block: the pristine buffer's norm, no NaN
        try:
            G.gclip_set_gather_wait(0)
            gl.accumulate_clip_(c, 1.0, 1.0, True)
        finally:
            G.gclip_set_gather_wait(-1)
        st, r = gl.read(True)
        out = gu.download(ta, "f32")
        what = f"nan={nan} rep {rep}"
        if r["status"] == G.GCLIP_DEVICE_WAIT_TIMEOUT:
            timeouts += 1
            assert st == _lib.GCLIP_EDEVICE, what
            gu.assert_bitwise_equal_but_nan(out, summed, "f32", what + ": the sums written, nothing scaled")
        else:
            assert r["status"] == 0, (what, r)
            if nan:
                assert st == _lib.GCLIP_ENONFINITE and r["skipped"], (what, r)
                gu.assert_bitwise_equal_but_nan(out, summed, "f32", what + ": stopped")
            else:
                assert st == _lib.GCLIP_OK and r["clipped"], (what, r)
                gu.assert_elems_close(out, clipped, "f32", what + ": clipped")
    c.close()
    gl.close()
    print(f"{timeouts} of {calls} calls gave up waiting")
    assert timeouts >= 1


@pytest.mark.parametrize("loss_scaled", (False, True))
@pytest.mark.parametrize("nan", (False, True))
def test_adamw_after_gather_timeout(nan, loss_scaled):
    """gclip_accumulate_norm then gclip_adamw_step (or its loss-scaled form,
    whose loss-scale state must not move either when the norm failed)."""
    import torch
    G = _G()
    from global_l2_norm_amd import _lib
    acc, contrib, summed = _lists(5200 + 2 * nan + loss_scaled, nan)
    rng = np.random.default_rng(5300)
    params = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in SIZES]
    m = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for n in SIZES]
    v = [(rng.random(n) * 1e-6).astype(np.float32) for n in SIZES]
    ta, tc = gu.upload(acc, "f32"), gu.upload(contrib, "f32")
    tp, tm, tv = (gu.upload(x, "f32") for x in (params, m, v))
    gl = G.GradList(ta)
    c = G.Contribution(gl, tc)
    opt = G.AdamWList(tp, ta, tm, tv)
    amp = G.AmpState(ta[0].device, 1.0) if loss_scaled else None
    ro, ref = oracle.clip_adamw(params, summed, m, v, "f32", 1.0, 1.0, True, step=1, **HP)
    timeouts = 0
    calls = 0
    for rep in range(MAX_REPS):
        if rep >= REPS and timeouts:
            break
        calls += 1
        for ts, arrays in ((ta, acc), (tp, params), (tm, m), (tv, v)):
            _reload(ts, arrays)
        if amp is not None:
            amp.set(1.0, 5)
        gl.norm(1.0)  # a clean block: the pristine buffer's norm, no NaN
        try:
            G.gclip_set_gather_wait(0)
            gl.accumulate_norm(c, 1.0)
        finally:
            G.gclip_set_gather_wait(-1)
        if amp is None:
            opt.step(gl, step=1, max_norm=1.0, avg_factor=1.0, error_if_nonfinite=True, **HP)
        else:
            opt.step_amp(gl, amp, step=1, max_norm=1.0, n_microbatches=1.0, **HP)
        st, r = gl.read(True)
        out = tuple(gu.download(x, "f32") for x in (tp, tm, tv))
        gu.assert_bitwise_equal_but_nan(gu.download(ta, "f32"), summed, "f32", f"rep {rep}: the += itself")
        state = amp.read() if amp is not None else None
        what = f"nan={nan} loss_scaled={loss_scaled} rep {rep}"
        if r["status"] == G.GCLIP_DEVICE_WAIT_TIMEOUT:
            timeouts += 1
            assert st == _lib.GCLIP_EDEVICE, what
            for a, b in zip(out, (params, m, v)):
                gu.assert_bitwise_equal(a, b, what + ": no step taken")
            if amp is not None:
                assert state == (1.0, 5, False), (what, state)
        else:
            assert r["status"] == 0, (what, r)
            assert bool(r["nonfinite"]) == nan and bool(r["skipped"]) == nan, (what, r)
            if nan:
                assert st == _lib.GCLIP_ENONFINITE, what
                for a, b in zip(out, (params, m, v)):
                    gu.assert_bitwise_equal(a, b, what + ": stopped")
            else:
                assert st == _lib.GCLIP_OK and r["clipped"], (what, r)
                gu.assert_norm_close(r["norm"], ro["norm"], what)
                assert_adamw_close(out, ref, (params, m, v), summed, "f32", ro["scale"], HP, 1, what)
            if amp is not None:
                assert state == ((0.5, 0, True) if nan else (1.0, 6, False)), (what, state)
    opt.close()
    c.close()
    gl.close()
    del tp, tm, tv
    torch.cuda.empty_cache()
    print(f"{timeouts} of {calls} calls gave up waiting")
    assert timeouts >= 1
