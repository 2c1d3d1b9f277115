"""Maximum sizes: one tensor of more than 2^31 elements and 4 GiB, and
lists of more than 1 GiB (fp32 and fp16) through the one-launch += with the
clip.

The 4.3 GB bf16 tensor exercises 64-bit byte offsets in every walk, the
nontemporal-store variants (lists of 1 GiB and more), and the per-tensor
reduction over more partials than it stages in LDS at once (~65,500
pieces, six windows).  Every output element is compared with the oracle's
(the oracle's reference is computed once per list and compared tensor by
tensor); the norms against the oracle's sums over every element."""
import math

import numpy as np
import pytest

import oracle
from synth import gradsets as gs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

BIG = (1 << 31) + 1027


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("the gpu tests need an MI355X")
    import global_l2_norm_amd  # noqa: F401  (fails loudly when libgclip.so is missing)


def _G():
    import global_l2_norm_amd as G
    return G


def check_all(ref, ts, dtype, what, before=None):
    """Every element of the device tensors ts against the oracle's ref, one
    tensor at a time; on a mismatch the message shows the first bad elements
    and, if given, what the tensor held before the call."""
    for k, (rf, t) in enumerate(zip(ref, ts)):
        got = gu.download([t], dtype)[0]
        try:
            gu.assert_elems_close([got], [rf], dtype, f"{what}: tensor {k}")
        except AssertionError as e:
            idx = np.flatnonzero(gu.elem_mismatches(got, rf, dtype))[:6]
            rows = [f"[{int(i)}] got {gu.values(got[i:i + 1], dtype)[0]!r} want {gu.values(rf[i:i + 1], dtype)[0]!r}"
                    + (f" before {gu.values(before[k][i:i + 1], dtype)[0]!r}" if before is not None else "")
                    for i in idx]
            raise AssertionError(f"{e}; " + "; ".join(rows)) from None
        del got


@pytest.fixture(scope="module")
def big_list():
    rng = np.random.default_rng(9000)
    arrays = [gs.bf16_bits(BIG, 9001), gs.to_storage(rng.standard_normal(5) * 1e-2, "bf16"),
              gs.to_storage(rng.standard_normal(70_001) * 1e-2, "bf16")]
    per = oracle.tensor_sumsq(arrays, "bf16")
    return arrays, per


@pytest.mark.timeout(900)
def test_over_4gib_tensor(big_list):
    import torch
    G = _G()
    arrays, per = big_list
    s_ref = float(np.sum(per))
    n_ref = math.sqrt(s_ref)
    ts = gu.upload(arrays, "bf16")
    pristine = [t.clone() for t in ts]
    gl = G.GradList(ts)
    assert gl.info()["n_bytes"] > (1 << 32)
    s, clipped, _ = oracle.decide(n_ref, False, 1.0)
    assert clipped
    ref = [a.copy() for a in arrays]
    oracle.scale_(ref, "bf16", s)
    for path in ("fused", "split"):
        for t, p in zip(ts, pristine):
            t.copy_(p)
        gl.set_path(G.GCLIP_PATH_FUSED if path == "fused" else G.GCLIP_PATH_SPLIT)
        gl.clip_(1.0)
        st, r = gl.read()
        assert st == 0 and r["status"] == 0 and r["clipped"] and not r["nonfinite"], (path, r)
        gu.assert_norm_close(r["norm"], n_ref, f"4 GiB {path}")
        check_all(ref, ts, "bf16", f"4 GiB clip {path}")
    del ref
    # every tensor by its own norm: ~65,500 pieces, staged in several windows
    for t, p in zip(ts, pristine):
        t.copy_(p)
    gl.clip_per_tensor_(0.05)
    st, r = gl.read()
    tr = gl.read_tensors()
    ref = [a.copy() for a in arrays]
    for k, ps in enumerate(per):
        gu.assert_norm_close(float(tr[k]["sumsq"]), ps, f"4 GiB per-tensor sumsq {k}")
        sk, ck, _ = oracle.decide(math.sqrt(ps), False, 0.05)
        assert bool(tr[k]["clipped"]) == ck, k
        oracle.scale_(ref[k:k + 1], "bf16", sk)
    check_all(ref, ts, "bf16", "4 GiB per-tensor clip")
    del ref
    gl.close()
    del pristine
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("dtype", ("f32", "f16"))
def test_over_1gib_accumulate_fused(dtype):
    """The one-launch += with the clip on a list of more than 1 GiB (its
    nontemporal-store variant): every element against the oracle's sums
    scaled by its decision.  Its scaling pass reads sums that other
    workgroups, on other XCDs, wrote in its summing pass: a missing release
    or acquire between the two shows here as stale elements."""
    import torch
    G = _G()
    if dtype == "f32":
        rng = np.random.default_rng(9100)
        sizes = [200_000_003, 100_000_001, 7]
        acc = [gs.to_storage(rng.standard_normal(n) * 1e-3, "f32") for n in sizes]
        contrib = [gs.to_storage(rng.standard_normal(n) * 1e-3, "f32") for n in sizes]
    else:
        sizes = [420_000_003, 130_000_001, 9]
        acc = [gs.f16_bits(n, 9200 + k) for k, n in enumerate(sizes)]
        contrib = [gs.f16_bits(n, 9300 + k) for k, n in enumerate(sizes)]
    ta, tc = gu.upload(acc, dtype), gu.upload(contrib, dtype)
    gl = G.GradList(ta)
    assert gl.info()["n_bytes"] >= (1 << 30)
    c = G.Contribution(gl, tc)
    gl.accumulate_clip_(c, 1.0, 0.5)
    st, r = gl.read()
    summed = [a.copy() for a in acc]
    oracle.accumulate_(summed, contrib, dtype)
    s_ref, nf = oracle.sumsq(summed, dtype, 0.5)
    n_ref = math.sqrt(s_ref)
    s, clipped, _ = oracle.decide(n_ref, nf, 1.0, 0.5)
    assert clipped and r["clipped"] and st == 0
    gu.assert_norm_close(r["norm"], n_ref, f"1 GiB += {dtype}")
    oracle.scale_(summed, dtype, s)
    check_all(summed, ta, dtype, f"1 GiB += with the clip, {dtype}", before=acc)
    c.close()
    gl.close()
    del ta, tc
    torch.cuda.empty_cache()
