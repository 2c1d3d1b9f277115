"""A seeded random sweep over every clipping entry point, against the oracle.

Each case draws a list (1 to 12 tensors of 0 to ~2M elements, log-uniform,
some placed as views at odd element offsets), a storage format, a threshold
kept away from the norm (and from every tensor's norm for the per-tensor
clip) by more than the tolerance, an averaging factor, the stop switch and,
now and then, a NaN or Inf; then one call -- the clip on either path, norm
then scale, the per-tensor clip, the += with the clip on either path, or the
loss-scaled clip -- checked against the oracle to the usual tolerances."""
import math

import numpy as np
import pytest

import oracle
from synth import gradsets as gs
from tests import gpu_util as gu
from tests.test_gpu_accum import odd_offsets, views_at

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "f16", "bf16")
CALLS = ("clip_fused", "clip_split", "norm_scale", "per_tensor", "accum_fused", "accum_split", "amp",
         "per_tensor_split")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("the gpu tests need an MI355X")
    import global_l2_norm_amd  # noqa: F401  (fails loudly when libgclip.so is missing)


def _G():
    import global_l2_norm_amd as G
    return G


def draw_list(rng, dtype):
    n = int(rng.integers(1, 13))
    sizes = [0 if rng.random() < 0.1 else int(np.exp(rng.uniform(0, np.log(2e6)))) for _ in range(n)]
    sigma = float(np.exp(rng.uniform(np.log(1e-4), np.log(3.0 if dtype == "f16" else 30.0))))
    return [gs.to_storage(rng.standard_normal(m) * sigma, dtype) for m in sizes]


def inject(rng, arrays, dtype):
    live = [k for k, a in enumerate(arrays) if a.size]
    if not live:
        return False
    k = int(rng.choice(live))
    arrays[k][int(rng.integers(0, arrays[k].size))] = gs.to_storage(
        np.array([float(rng.choice([math.nan, math.inf, -math.inf]))]), dtype)[0]
    return True


def threshold(rng, norms):
    """A threshold log-uniform around the largest finite norm, more than 1e-4
    (relative) away from every norm given."""
    finite = [x for x in norms if math.isfinite(x) and x > 0]
    centre = max(finite) if finite else 1.0
    for _ in range(200):
        c = centre * float(np.exp(rng.uniform(-1.5, 1.0)))
        if all(not math.isfinite(x) or abs(x - c) > 1e-4 * c for x in norms):
            return c
    raise AssertionError("no threshold off the norms")


def upload(rng, arrays, dtype, as_views):
    if as_views and arrays:
        offs = odd_offsets(rng, arrays)
        buf, ts = views_at(arrays, dtype, offs)
        return ts, buf, offs
    return gu.upload(arrays, dtype), None, None


@pytest.mark.parametrize("case", range(150))
def test_random_case(case):
    import torch
    G = _G()
    rng = np.random.default_rng(7000 + case)
    dtype = DTYPES[case % 3]
    call = CALLS[(case // 3) % len(CALLS)]
    arrays = draw_list(rng, dtype)
    bad = rng.random() < 0.25 and inject(rng, arrays, dtype)
    err = bool(rng.random() < 0.5)
    avg = float(rng.choice([1.0, 0.5, 0.25, 1.0 / 3.0]))
    as_views = bool(rng.random() < 0.4)
    what = f"case {case}: {call} {dtype} sizes {[a.size for a in arrays]} avg {avg} err {err} bad {bad}"
    print(what, flush=True)
    ts, buf, offs = upload(rng, arrays, dtype, as_views)
    gl = G.GradList(ts)
    if call in ("clip_split", "norm_scale", "accum_split", "per_tensor_split"):
        gl.set_path(G.GCLIP_PATH_SPLIT)

    if call in ("clip_fused", "clip_split", "norm_scale", "amp"):
        if call == "amp":
            scale = float(rng.choice([1.0, 256.0, 65536.0]))
            n_mb = 1.0 / avg
            a_eff = oracle.amp_avg(n_mb, scale)
        else:
            a_eff = avg
        s_ref, _ = oracle.sumsq([a.copy() for a in arrays], dtype, a_eff)
        c = threshold(rng, [math.sqrt(s_ref)])
        if call == "amp":
            amp = G.AmpState(ts[0].device if ts else "cuda", scale, 2.0, 0.5, 3)
            gl.clip_amp_(c, n_mb, amp)
            err = True
        elif call == "norm_scale":
            gl.norm(avg)
            gl.scale(c, avg, err)
        else:
            gl.clip_(c, avg, err)
        st, r = gl.read(err)
        ref = [a.copy() for a in arrays]
        ro = oracle.clip_(ref, dtype, c, a_eff, err)
        if call == "amp":
            sc, tr, fi = amp.read()
            esc, etr = oracle.amp_update(scale, 0, ro["nonfinite"], 2.0, 0.5, 3)
            assert fi == ro["nonfinite"] and sc == esc and tr == etr, what
    elif call in ("per_tensor", "per_tensor_split"):
        norms = [math.sqrt(x) for x in oracle.tensor_sumsq(arrays, dtype, avg)]
        c = threshold(rng, norms)
        gl.clip_per_tensor_(c, avg, err)
        st, r = gl.read(err)
        ref = [a.copy() for a in arrays]
        ro = oracle.clip_per_tensor_(ref, dtype, c, avg, err)
        tr = gl.read_tensors()
        for k, t in enumerate(ro["tensors"]):
            assert bool(tr[k]["nonfinite"]) == t["nonfinite"], (what, k)
            if not math.isnan(t["norm"]):
                gu.assert_norm_close(float(tr[k]["norm"]), t["norm"], f"{what} tensor {k}")
                assert bool(tr[k]["clipped"]) == t["clipped"], (what, k)
    else:  # the += with the clip
        contrib = [gs.to_storage(gu.values(a, dtype) * float(rng.uniform(-1.2, 1.2)) +
                                 rng.standard_normal(a.size) * 1e-3, dtype) for a in arrays]
        if as_views and arrays:
            bc, tc = views_at(contrib, dtype, offs)
        else:
            bc, tc = None, gu.upload(contrib, dtype)
        summed = [a.copy() for a in arrays]
        oracle.accumulate_(summed, contrib, dtype)
        s_ref, _ = oracle.sumsq([x.copy() for x in summed], dtype, avg)
        c = threshold(rng, [math.sqrt(s_ref)])
        cb = G.Contribution(gl, tc)
        gl.accumulate_clip_(cb, c, avg, err)
        st, r = gl.read(err)
        ref = [a.copy() for a in arrays]
        ro = oracle.accumulate_clip_(ref, contrib, dtype, c, avg, err)
        gu.assert_bitwise_equal(gu.download(tc, dtype), contrib, what + " (contribution only read)")
        cb.close()
        arrays = summed  # what an unscaled call leaves behind

    out = gu.download(ts, dtype)
    assert r["status"] == 0, what
    assert r["nonfinite"] == ro["nonfinite"] and r["skipped"] == ro["skipped"], what
    if not math.isnan(ro["norm"]):
        gu.assert_norm_close(r["norm"], ro["norm"], what)
        assert r["clipped"] == ro["clipped"], what
    if call in ("per_tensor", "per_tensor_split"):
        for k, (o, rr, a, t) in enumerate(zip(out, ref, arrays, ro["tensors"])):
            if ro["skipped"] or t["scale"] == 1.0:
                gu.assert_bitwise_equal_but_nan([o], [a], dtype, f"{what} tensor {k} untouched")
            else:
                gu.assert_elems_close([o], [rr], dtype, f"{what} tensor {k}")
    elif ro["skipped"] or ro["scale"] == 1.0:
        gu.assert_bitwise_equal_but_nan(out, arrays, dtype, what + " (nothing scaled)")
    else:
        gu.assert_elems_close(out, ref, dtype, what)
    if buf is not None:
        mask = torch.ones(buf.numel(), dtype=torch.bool, device="cuda")
        for v in ts:
            mask[v.storage_offset():v.storage_offset() + v.numel()] = False
        assert int(torch.count_nonzero(buf[mask].float())) == 0, what + " (padding written)"
    gl.close()
