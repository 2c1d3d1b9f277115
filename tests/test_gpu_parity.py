"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Tolerances: the global norm within relative 1e-5 of the oracle's for every
format; clipped fp32 elements within relative 1e-5 (exact zero where the
oracle's is zero); clipped fp16/bf16 elements within 1 ulp of the storage
format; the non-finite flag exactly; untouched gradients bitwise.  Every
case runs on both kernel paths (one fused cooperative kernel, and the split
pair) unless it says otherwise.
"""
import math

import numpy as np
import pytest

import oracle
from synth import gradsets as gs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

PATHS = ("fused", "split")


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


def gpu_clip(arrays, dtype, max_norm, avg=1.0, err=False, path="fused", call="clip", views=None):
    """Upload, clip on the GPU, download.  call='clip' uses gclip_clip_,
    call='two' uses gclip_norm followed by gclip_scale."""
    ts = views if views is not None else gu.upload(arrays, dtype)
    gl = make_list(ts, path)
    if call == "clip":
        gl.clip_(max_norm, avg, err)
    else:
        gl.norm(avg)
        gl.scale(max_norm, avg, err)
    st, r = gl.read(err)
    out = gu.download(ts, dtype)
    gl.close()
    return st, r, out


def oracle_clip(arrays, dtype, max_norm, avg=1.0, err=False):
    ref = [a.copy() for a in arrays]
    r = oracle.clip_(ref, dtype, max_norm, avg, err)
    return r, ref


def check_against_oracle(arrays, dtype, max_norm, avg=1.0, err=False, path="fused", call="clip", what=""):
    st, r, out = gpu_clip(arrays, dtype, max_norm, avg, err, path, call)
    ro, ref = oracle_clip(arrays, dtype, max_norm, avg, err)
    assert r["status"] == 0
    assert r["nonfinite"] == ro["nonfinite"], what
    gu.assert_norm_close(r["norm"], ro["norm"], what)
    if not math.isnan(ro["norm"]):
        assert r["clipped"] == ro["clipped"], what
    assert r["skipped"] == ro["skipped"], what
    if ro["skipped"] or ro["scale"] == 1.0:
        gu.assert_bitwise_equal(out, arrays, what + " (must be untouched)")
    else:
        gu.assert_elems_close(out, ref, dtype, what)
    return st, r, ro, out


# ------------------------------------------------------------------ the pages' worked examples
@pytest.mark.parametrize("call", ["clip", "two"])
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_worked_example_6_8(dtype, path, call):
    """[6, 8] at threshold 5 becomes exactly [3, 4] (glossary page)."""
    a = [gs.to_storage(np.array([6.0, 8.0]), dtype)]
    st, r, out = gpu_clip(a, dtype, 5.0, path=path, call=call)
    assert st == 0 and r["norm"] == 10.0 and r["scale"] == 0.5 and r["clipped"] and r["decided"]
    assert list(gu.values(out[0], dtype)) == [3.0, 4.0]


@pytest.mark.parametrize("path", PATHS)
def test_accumulate_then_clip(path):
    """10 and -9 sum to 1, which survives a clip at 5; each clipped alone
    gives 5 and -5 (glossary page, 'Order changes the result')."""
    outs = []
    for v in (10.0, -9.0, 1.0):
        _, r, out = gpu_clip([np.array([v], dtype=np.float32)], "f32", 5.0, path=path)
        outs.append(float(out[0][0]))
    assert outs == [5.0, -5.0, 1.0]
    assert outs[0] + outs[1] == 0.0


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_tie_writes_nothing(dtype, path):
    """norm == max_norm passes unchanged (grad clip lesson, 'Math')."""
    a = [gs.to_storage(np.array([3.0, 4.0]), dtype)]
    st, r, out = gpu_clip(a, dtype, 5.0, path=path)
    assert not r["clipped"] and r["scale"] == 1.0 and r["norm"] == 5.0
    gu.assert_bitwise_equal(out, a)


# ------------------------------------------------------------------ small and ragged lists
@pytest.mark.parametrize("call", ["clip", "two"])
@pytest.mark.parametrize("path", PATHS)
def test_tiny_config(path, call):
    g = gs.tiny_f32()
    check_against_oracle(g.arrays, "f32", 1.0, path=path, call=call, what="tiny")


def ragged_arrays(rng, dtype, big=False):
    sizes = [1, 2, 3, 5, 7, 63, 255, 256, 257, 1000, 1023, 4096 + 7, 65_537, 300_001]
    if big:
        sizes += [3_000_017, 1_048_576]
    numels = [int(rng.choice(sizes)) for _ in range(int(rng.integers(3, 25)))]
    return [gs.to_storage(rng.standard_normal(n) * float(rng.choice([1e-3, 1.0, 30.0])), dtype) for n in numels]


def upload_as_views(arrays, dtype, rng):
    """Each tensor a view at an odd element offset inside one device buffer."""
    import torch
    offs, total = [], 0
    for a in arrays:
        total += int(rng.integers(1, 8))
        offs.append(total)
        total += a.size
    buf = torch.zeros(total + 8, dtype=gu.torch_dtype(dtype), device="cuda")
    views = []
    for a, o in zip(arrays, offs):
        v = buf[o:o + a.size]
        v.copy_(gu.upload([a], dtype)[0])
        views.append(v)
    return buf, views


@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_ragged_lists_misaligned_views(dtype, path, seed):
    rng = np.random.default_rng(1000 + seed)
    arrays = ragged_arrays(rng, dtype, big=seed >= 2)
    c = float(rng.choice([0.5, 2.0, 1e9]))
    buf, views = upload_as_views(arrays, dtype, rng)
    st, r, out = gpu_clip(arrays, dtype, c, path=path, views=views)
    ro, ref = oracle_clip(arrays, dtype, c)
    gu.assert_norm_close(r["norm"], ro["norm"], "ragged")
    assert r["clipped"] == ro["clipped"]
    if ro["clipped"]:
        gu.assert_elems_close(out, ref, dtype, "ragged")
    else:
        gu.assert_bitwise_equal(out, arrays, "ragged, not clipped")
    # the padding between views is never written
    import torch
    mask = torch.ones(buf.numel(), dtype=torch.bool, device="cuda")
    for v in views:
        o = v.storage_offset()
        mask[o:o + v.numel()] = False
    assert int(torch.count_nonzero(buf[mask].float())) == 0


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_medium_list_streams_past_the_resident_part(dtype):
    """Shares large enough that the fused kernel also re-reads part of them."""
    rng = np.random.default_rng(77)
    n_total = 40_000_000 if dtype == "f32" else 80_000_000
    sizes = [n_total // 2 + 13, n_total // 3 + 1, n_total - n_total // 2 - n_total // 3 - 14]
    arrays = [gs.to_storage(rng.standard_normal(n) * 1e-3, dtype) for n in sizes]
    for path in PATHS:
        check_against_oracle(arrays, dtype, 1.0, path=path, what=f"medium {dtype} {path}")


@pytest.mark.parametrize("path", PATHS)
def test_many_tiny_tensors(path):
    rng = np.random.default_rng(5)
    arrays = [gs.to_storage(rng.standard_normal(1), "bf16") for _ in range(4096)]
    arrays += [gs.to_storage(rng.standard_normal(7) * 0.1, "bf16") for _ in range(500)]
    arrays += [gs.to_storage(rng.standard_normal(2048) * 0.01, "bf16") for _ in range(50)]
    check_against_oracle(arrays, "bf16", 1.0, path=path, what="many tiny")


# ------------------------------------------------------------------ the full configurations
@pytest.fixture(scope="module")
def c2():
    return gs.andrea120m_f32()


@pytest.mark.parametrize("path", PATHS)
def test_andrea120m_f32(c2, path):
    st, r, ro, out = check_against_oracle(c2.arrays, "f32", c2.max_norm, path=path, what="andrea120m f32")
    assert r["clipped"] and abs(r["norm"] - 9.605) < 0.01
    # the kernels sum each vector's squares in fp32 (at most 7 roundings of
    # 2^-24, all terms positive) and add those partials in binary64; the oracle
    # sums sequentially in binary64, within (N - 1) * 2^-53 of the exact sum
    assert abs(r["sumsq"] - ro["sumsq"]) <= (8 * 2.0 ** -24 + c2.numel * 2.0 ** -53) * ro["sumsq"]


@pytest.mark.parametrize("path", PATHS)
def test_andrea120m_f16_spike(path):
    g = gs.andrea120m_f16_spike()
    st, r, ro, out = check_against_oracle(g.arrays, "f16", g.max_norm, path=path, what="andrea120m f16 spike")
    assert r["clipped"] and 290 < r["norm"] < 305


@pytest.mark.parametrize("path", PATHS)
def test_andrea120m_f16_small_writes_nothing(path):
    g = gs.andrea120m_f16_small()
    st, r, ro, out = check_against_oracle(g.arrays, "f16", g.max_norm, path=path, what="andrea120m f16 small")
    assert not r["clipped"] and r["scale"] == 1.0 and 0.09 < r["norm"] < 0.1


@pytest.mark.parametrize("path", PATHS)
def test_andrea120m_f32_accum4(path):
    g = gs.andrea120m_f32_accum4()
    st, r, ro, out = check_against_oracle(g.arrays, "f32", g.max_norm, avg=g.avg_factor, path=path,
                                          what="andrea120m accum4")
    assert r["clipped"] and abs(r["norm"] - 4.802) < 0.01


@pytest.fixture(scope="module")
def c5():
    return gs.gpt1p3b_bf16()


@pytest.fixture(scope="module")
def c5_clipped(c5):
    """The oracle's clip of the whole 1.3B list, computed once for both paths."""
    ref = [a.copy() for a in c5.arrays]
    ro = oracle.clip_(ref, "bf16", c5.max_norm)
    return ro, ref


@pytest.mark.timeout(900)
@pytest.mark.parametrize("path", PATHS)
def test_gpt1p3b_bf16(c5, c5_clipped, path):
    """The 2.6 GB list (nontemporal stores): every one of its 1.3B elements
    against the oracle's, within 1 ulp of bf16."""
    ro, ref = c5_clipped
    st, r, out = gpu_clip(c5.arrays, "bf16", c5.max_norm, path=path)
    s_ref, nf, n_ref = ro["sumsq"], ro["nonfinite"], ro["norm"]
    assert not nf and not r["nonfinite"] and r["status"] == 0
    gu.assert_norm_close(r["norm"], n_ref, "gpt1p3b")
    assert abs(r["sumsq"] - s_ref) <= (8 * 2.0 ** -24 + c5.numel * 2.0 ** -53) * s_ref
    s = ro["scale"]
    assert ro["clipped"] and r["clipped"] and abs(r["scale"] - s) <= (8 * 2.0 ** -24 + c5.numel * 2.0 ** -53) * s
    gu.assert_elems_close(out, ref, "bf16", f"gpt1p3b {path}")


@pytest.mark.timeout(900)
def test_gpt1p3b_bf16_paths_agree_bitwise(c5):
    """On the 2.6 GB list, whose sum chunks come in two sizes (weighted by
    XCD), the fused kernel and the split norm kernel add the same partials
    in the same order: the same sum, norm and factor to the bit, and the
    same bits in every element."""
    runs = [gpu_clip(c5.arrays, "bf16", c5.max_norm, path=path) for path in PATHS]
    (_, rf, of), (_, rs, os_) = runs
    for k in ("sumsq", "norm", "scale", "clipped", "nonfinite", "status"):
        assert rf[k] == rs[k], k
    gu.assert_bitwise_equal(of, os_, "gpt1p3b fused vs split")


def with_value(g, tensor, index, bits):
    arrays = list(g.arrays)
    t = g.names.index(tensor)
    arrays[t] = arrays[t].copy()
    arrays[t][index] = bits
    return arrays


@pytest.mark.timeout(900)
def test_gpt1p3b_bf16_nan(c5):
    """One NaN in block 23's W_2: the flag is set exactly; with the stop
    switch nothing is written, without it NaN > c is false and (a = 1)
    nothing is written either."""
    G = _G()
    arrays = with_value(c5, gs.NAN_TENSOR, gs.NAN_INDEX, 0x7FC0)
    s_ref, nf = oracle.sumsq(arrays, "bf16")
    assert nf and math.isnan(s_ref)
    for path in PATHS:
        for err in (True, False):
            st, r, out = gpu_clip(arrays, "bf16", 1.0, err=err, path=path)
            assert r["nonfinite"] and math.isnan(r["norm"]) and not r["clipped"]
            assert r["skipped"] == err
            assert st == (G._lib.GCLIP_ENONFINITE if err else G._lib.GCLIP_OK)
            gu.assert_bitwise_equal(out, arrays, f"nan err={err} {path}")


@pytest.mark.timeout(900)
def test_gpt1p3b_bf16_nan_in_last_scalar_and_inf_in_embed(c5):
    arrays = with_value(c5, "scalar4095", 0, 0x7FC0)
    st, r, out = gpu_clip(arrays, "bf16", 1.0, err=True)
    assert r["nonfinite"] and r["skipped"]
    gu.assert_bitwise_equal(out, arrays, "nan in the last one-element tensor")
    n_embed = c5.arrays[0].size
    for bits in (0x7F80, 0xFF80):  # +Inf, -Inf in the tail element of embed
        arrays = with_value(c5, "embed", n_embed - 1, bits)
        st, r, out = gpu_clip(arrays, "bf16", 1.0, err=False)
        assert r["nonfinite"] and r["norm"] == math.inf and r["clipped"] and r["scale"] == 0.0
        ro, ref = oracle_clip(arrays, "bf16", 1.0)
        assert ro["norm"] == math.inf and ro["scale"] == 0.0
        del arrays
        gu.assert_elems_close(out, ref, "bf16", f"inf {bits:#x} in embed: every element")
        assert np.isnan(gu.values(out[0][-1:], "bf16")[0])
        del out, ref


# ------------------------------------------------------------------ non-finite elements, small
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_nonfinite_positions(dtype, path):
    rng = np.random.default_rng(9)
    base = [gs.to_storage(rng.standard_normal(n) * 0.5, dtype) for n in (3, 5000, 257, 1)]
    bad_bits = {"f32": [np.float32("nan"), np.float32("inf"), np.float32("-inf")],
                "f16": [0x7E00, 0x7C00, 0xFC00], "bf16": [0x7FC0, 0x7F80, 0xFF80]}[dtype]
    for t, i in ((0, 0), (1, 2500), (1, 4999), (2, 256), (3, 0)):
        for bits in bad_bits:
            arrays = [a.copy() for a in base]
            arrays[t][i] = bits
            for err in (True, False):
                check_against_oracle(arrays, dtype, 1.0, err=err, path=path, what=f"nonfinite t{t} i{i} err{err}")


# ------------------------------------------------------------------ determinism and metamorphic checks
def test_bitwise_repeatable_and_paths_agree(c2):
    G = _G()
    runs = []
    for path in ("fused", "fused", "split", "split"):
        st, r, out = gpu_clip(c2.arrays, "f32", 1.0, path=path)
        runs.append((r, out))
    for r, out in runs[1:]:
        gu.assert_bitwise_equal(out, runs[0][1], "run to run / path to path")
        for k in ("sumsq", "norm", "scale", "clipped", "nonfinite"):
            assert r[k] == runs[0][0][k], k
    # gclip_norm alone gives the same bits as the fused path's norm
    ts = gu.upload(c2.arrays, "f32")
    gl = G.GradList(ts)
    gl.norm(1.0)
    _, rn = gl.read()
    gl.close()
    assert rn["sumsq"] == runs[0][0]["sumsq"] and not rn["decided"]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_power_of_two_scaling_is_exact(dtype):
    rng = np.random.default_rng(11)
    arrays = [gs.to_storage(rng.standard_normal(n) * 0.25, dtype) for n in (100_000, 777, 3)]
    _, r0, _ = gpu_clip(arrays, dtype, 1e30)
    scaled = [gs.to_storage(gu.values(a, dtype) * 4.0, dtype) for a in arrays]
    _, r1, _ = gpu_clip(scaled, dtype, 1e30)
    assert r1["sumsq"] == 16.0 * r0["sumsq"] and r1["norm"] == 4.0 * r0["norm"]


@pytest.mark.parametrize("path", PATHS)
def test_permuted_list_same_norm_and_elements(c2, path):
    """The ANDREA-120M list in another tensor order (a fixed random
    permutation): the norm is the same sum in another order, so it agrees
    with the original order's within the accumulation bound, the decision is
    the same, and every element matches the oracle (and the original run's
    element for the same tensor, within the element tolerance)."""
    rng = np.random.default_rng(4242)
    perm = rng.permutation(len(c2.arrays))
    arrays = [c2.arrays[i] for i in perm]
    st0, r0, out0 = gpu_clip(c2.arrays, "f32", c2.max_norm, path=path)
    st1, r1, ro, out1 = check_against_oracle(arrays, "f32", c2.max_norm, path=path, what=f"permuted {path}")
    bound = 2 * (8 * 2.0 ** -24 + c2.numel * 2.0 ** -53)
    assert abs(r1["sumsq"] - r0["sumsq"]) <= bound * r0["sumsq"]
    assert abs(r1["norm"] - r0["norm"]) <= 1e-5 * r0["norm"]
    assert r1["clipped"] == r0["clipped"]
    gu.assert_elems_close([out1[k] for k in np.argsort(perm)], out0, "f32", f"permuted vs original {path}")


@pytest.mark.parametrize("path", PATHS)
def test_concatenated_list_same_norm_and_elements(c2, path):
    """The same 92.2M values as one tensor (the list concatenated): one
    segment and no tensor boundaries, the same norm within the accumulation
    bound, and every element within tolerance of the per-tensor run's."""
    flat = [np.concatenate(c2.arrays)]
    st0, r0, out0 = gpu_clip(c2.arrays, "f32", c2.max_norm, path=path)
    st1, r1, ro, out1 = check_against_oracle(flat, "f32", c2.max_norm, path=path, what=f"concatenated {path}")
    bound = 2 * (8 * 2.0 ** -24 + c2.numel * 2.0 ** -53)
    assert abs(r1["sumsq"] - r0["sumsq"]) <= bound * r0["sumsq"]
    assert r1["clipped"] == r0["clipped"]
    gu.assert_elems_close(out1, [np.concatenate(out0)], "f32", f"concatenated vs list {path}")


def test_scale_with_caller_supplied_sumsq():
    """gclip_scale decides from the sumsq in the result block, e.g. one
    summed over several ranks: a block claiming 4x the local sumsq doubles
    the norm the decision sees."""
    import torch
    G = _G()
    rng = np.random.default_rng(12)
    arrays = [gs.to_storage(rng.standard_normal(1000), "f32")]
    local_sumsq, _ = oracle.sumsq(arrays, "f32")
    ts = gu.upload(arrays, "f32")
    gl = G.GradList(ts)
    blk = G.GclipResult()
    blk.sumsq = 4.0 * local_sumsq
    host = torch.frombuffer(bytearray(bytes(blk)), dtype=torch.uint8)
    gl.result.copy_(host)
    gl.scale(1.0, 1.0, False)
    st, r = gl.read()
    out = gu.download(ts, "f32")
    gl.close()
    s, clipped, _ = oracle.decide(2.0 * math.sqrt(local_sumsq), False, 1.0)
    assert r["clipped"] and abs(r["scale"] - s) <= 1e-15 * s  # the block's sumsq was given exactly
    ref = [arrays[0].copy()]
    oracle.scale_(ref, "f32", s)
    gu.assert_elems_close(out, ref, "f32", "external sumsq")


# ------------------------------------------------------------------ lists of one group
# A list whose vectors fit in one group of steps (512 lanes x 8 = 4,096
# vectors of 16 bytes) with at most one single element per lane gets a plan
# with one worker, and the fused path clips it in one workgroup with no
# grid-wide decision; the split path runs its two kernels on the same plan.
# Both must give the same bits, and the oracle's values.
ONE_GROUP_CASES = [
    ("tiny", "f32", [2, 64 * 64, 128, 33 * 17, 1], True),
    ("6_8", "f32", [2], True),
    ("4096 vectors f32", "f32", [16384], True),
    ("4097 vectors f32", "f32", [16388], False),
    ("4096 vectors bf16", "bf16", [32768], True),
    ("512 single elements", "f16", [1] * 512, True),
    ("513 single elements", "f16", [1] * 513, False),
    ("mixed", "bf16", [3, 1000, 63, 20000, 5], True),
]


@pytest.mark.parametrize("case", range(len(ONE_GROUP_CASES)))
def test_one_group_lists(case):
    import torch
    name, dtype, numels, one = ONE_GROUP_CASES[case]
    rng = np.random.default_rng(900 + case)
    arrays = [gs.to_storage(rng.standard_normal(n), dtype) for n in numels]
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    norm = oracle.clip_([a.copy() for a in arrays], dtype, 1e30)["norm"]
    for max_norm, err, bad in ((0.5 * norm, False, False), (2.0 * norm, False, False), (0.5 * norm, True, True),
                               (0.5 * norm, False, True)):
        cur = [a.copy() for a in arrays]
        if bad:
            cur[-1][-1] = gs.to_storage(np.array([math.nan]), dtype)[0]
        what = f"{name} max_norm {max_norm:.4g} err {err} nan {bad}"
        outs = {}
        for path in PATHS:
            ts = gu.upload(cur, dtype)
            gl = make_list(ts, path)
            assert gl.info()["n_workers"] == (1 if one else ncu), what
            gl.clip_(max_norm, 1.0, err)
            st, r = gl.read(err)
            outs[path] = (r, gu.download(ts, dtype))
            gl.close()
        (rf, of), (rs, os_) = outs["fused"], outs["split"]
        gu.assert_bitwise_equal(of, os_, what + " (fused vs split)")
        for k in ("clipped", "skipped", "nonfinite"):
            assert rf[k] == rs[k], (what, k)
        if not bad:
            assert rf["sumsq"] == rs["sumsq"] and rf["scale"] == rs["scale"], what
        check_against_oracle(cur, dtype, max_norm, err=err, path="fused", what=what)


# ------------------------------------------------------------------ edge cases
@pytest.mark.parametrize("path", PATHS)
def test_empty_list(path):
    G = _G()
    gl = make_list([], path)
    gl.clip_(1.0)
    st, r = gl.read()
    gl.close()
    assert st == 0 and r["norm"] == 0.0 and not r["clipped"] and r["scale"] == 1.0


@pytest.mark.parametrize("path", PATHS)
def test_zero_size_tensors_and_infinite_threshold(path):
    import torch
    rng = np.random.default_rng(13)
    arrays = [np.zeros(0, dtype=np.float32), gs.to_storage(rng.standard_normal(999) * 3, "f32"),
              np.zeros(0, dtype=np.float32)]
    check_against_oracle(arrays, "f32", 1.0, path=path, what="zero-size")
    st, r, out = gpu_clip(arrays, "f32", math.inf, path=path)
    assert not r["clipped"]
    gu.assert_bitwise_equal(out, arrays)


def test_averaging_without_clip_still_writes():
    rng = np.random.default_rng(14)
    arrays = [gs.to_storage(rng.standard_normal(5000) * 1e-3, "f32")]
    for path in PATHS:
        st, r, ro, out = check_against_oracle(arrays, "f32", 1e6, avg=0.25, path=path, what="average only")
        assert not r["clipped"] and r["scale"] == 0.25


def test_invalid_arguments_enqueue_nothing():
    G = _G()
    arrays = [np.array([6.0, 8.0], dtype=np.float32)]
    ts = gu.upload(arrays, "f32")
    gl = G.GradList(ts)
    for bad in (float("nan"), 0.0, -1.0):
        with pytest.raises(G.GclipError):
            gl.clip_(bad)
    for bad in (0.0, -0.5, float("inf"), float("nan")):
        with pytest.raises(G.GclipError):
            gl.clip_(5.0, avg_factor=bad)
    import torch
    torch.cuda.synchronize()
    assert list(gu.values(gu.download(ts, "f32")[0], "f32")) == [6.0, 8.0]
    gl.close()


@pytest.mark.parametrize("path", PATHS)
def test_one_list_reused_on_new_data(path):
    """One list (one workspace) over calls on changing data, alternating the
    entry points: every call sees its own data only."""
    import torch
    rng = np.random.default_rng(21)
    sizes = (3_000_001, 1_000_003, 4099, 7)
    arrays = [gs.to_storage(rng.standard_normal(n) * 1e-3, "f32") for n in sizes]
    ts = gu.upload(arrays, "f32")
    gl = make_list(ts, path)
    for k in range(6):
        new = [gs.to_storage(rng.standard_normal(n) * 10.0 ** rng.uniform(-4, -1), "f32") for n in sizes]
        for t, a in zip(ts, new):
            t.copy_(torch.from_numpy(a).to("cuda"))
        if k % 2 == 0:
            gl.clip_(1.0)
        else:
            gl.norm(1.0)
            gl.scale(1.0)
        st, r = gl.read()
        out = gu.download(ts, "f32")
        ro, ref = oracle_clip(new, "f32", 1.0)
        gu.assert_norm_close(r["norm"], ro["norm"], f"call {k}")
        assert r["clipped"] == ro["clipped"]
        if ro["clipped"]:
            gu.assert_elems_close(out, ref, "f32", f"call {k}")
        else:
            gu.assert_bitwise_equal(out, new, f"call {k}")
    gl.close()


# ------------------------------------------------------------------ the fused kernel's bounded wait
def _clip_with_wait(arrays, dtype, max_norm, wait_us, err=False, calls=1):
    G = _G()
    ts = gu.upload(arrays, dtype)
    gl = make_list(ts, "fused")
    gl.set_wait(wait_us)
    res = []
    for _ in range(calls):
        gl.clip_(max_norm, 1.0, err)
        res.append(gl.read(err))
    out = gu.download(ts, dtype)
    gl.close()
    return res, out


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_handed_back_blocks_give_the_same_bits(dtype):
    """With no wait at all, every workgroup but the deciding one hands its
    block back; the blocks are then scaled from memory by others, with the
    same result as the split path and the oracle."""
    rng = np.random.default_rng(31)
    arrays = ragged_arrays(rng, dtype, big=True)
    arrays.append(gs.to_storage(rng.standard_normal(6_000_001) * 1e-3, dtype))
    [(st, r)], out = _clip_with_wait(arrays, dtype, 0.5, 0)
    assert st == 0 and r["status"] == 0
    assert r["handed_back"] >= 1, r
    _, r_split, out_split = gpu_clip(arrays, dtype, 0.5, path="split")
    gu.assert_bitwise_equal(out, out_split, f"hand-back {dtype} vs split")
    assert r["sumsq"] == r_split["sumsq"] and r["scale"] == r_split["scale"]
    ro, ref = oracle_clip(arrays, dtype, 0.5)
    gu.assert_norm_close(r["norm"], ro["norm"], "hand-back")
    assert r["clipped"] == ro["clipped"] == 1
    gu.assert_elems_close(out, ref, dtype, f"hand-back {dtype}")


@pytest.mark.parametrize("dtype,n_total", [("f32", 60_000_000), ("bf16", 120_000_000), ("f32", 43_500_000)])
def test_handed_back_with_a_streamed_region(dtype, n_total):
    """A list larger than what the fused kernel keeps on chip: besides the
    blocks, every worker that hands back leaves the two scale chunks of the
    streamed region it takes without a claim to whoever takes the block
    over.  The 240 MB lists have more than two scale chunks per worker, the
    174 MB one between one and two (some workers have no second chunk)."""
    rng = np.random.default_rng(34)
    sizes = [n_total // 2 + 7, n_total // 4 + 3, n_total - n_total // 2 - n_total // 4 - 10]
    arrays = [gs.to_storage(rng.standard_normal(n) * 1e-3, dtype) for n in sizes]
    [(st, r)], out = _clip_with_wait(arrays, dtype, 1.0, 0)
    assert st == 0 and r["status"] == 0 and r["handed_back"] >= 1, r
    _, r_split, out_split = gpu_clip(arrays, dtype, 1.0, path="split")
    assert r["sumsq"] == r_split["sumsq"] and r["scale"] == r_split["scale"] and r["clipped"]
    gu.assert_bitwise_equal(out, out_split, f"hand-back with streamed region {dtype} vs split")


def test_hand_back_then_normal_wait_on_one_list():
    """The block states are cleared after a launch with hand-backs: the next
    calls on the same list (no wait, then the default wait) each scale
    exactly once."""
    import torch
    G = _G()
    rng = np.random.default_rng(32)
    arrays = [gs.to_storage(rng.standard_normal(n) * 1e-2, "f32") for n in (5_000_003, 777_777, 4099, 3)]
    ts = gu.upload(arrays, "f32")
    gl = make_list(ts, "fused")
    cur = [a.copy() for a in arrays]
    for k, wait in enumerate((0, 0, 1000, 0, 1000)):
        gl.set_wait(wait)
        gl.clip_(1.0)
        st, r = gl.read()
        ro, ref = oracle_clip(cur, "f32", 1.0)
        out = gu.download(ts, "f32")
        gu.assert_norm_close(r["norm"], ro["norm"], f"call {k}")
        if ro["clipped"]:
            gu.assert_elems_close(out, ref, "f32", f"call {k}")
        # next call starts from a fresh random draw so that it clips again
        cur = [gs.to_storage(rng.standard_normal(a.size) * 1e-2, "f32") for a in arrays]
        for t, a in zip(ts, cur):
            t.copy_(torch.from_numpy(a).to("cuda"))
    gl.close()


@pytest.mark.parametrize("err", [True, False])
def test_hand_back_with_nothing_to_write(err):
    """A NaN with error_if_nonfinite (skip) and a norm under the threshold
    (factor 1) write nothing, also when blocks were handed back."""
    rng = np.random.default_rng(33)
    arrays = [gs.to_storage(rng.standard_normal(n) * 1e-3, "bf16") for n in (4_000_000, 12345, 5)]
    if err:
        arrays[0][1_999_999] = 0x7fc0  # bf16 NaN
    [(st, r)], out = _clip_with_wait(arrays, "bf16", 1e30, 0, err=err)
    gu.assert_bitwise_equal(out, arrays, "nothing written")
    assert r["skipped"] == (1 if err else 0) and r["scale"] == 1.0


def test_set_wait_rejects_out_of_range():
    G = _G()
    ts = gu.upload([np.ones(100, dtype=np.float32)], "f32")
    gl = G.GradList(ts)
    for bad in (-1, 60_000_001):
        with pytest.raises(G.GclipError):
            gl.set_wait(bad)
    gl.set_wait(0)
    gl.set_wait(60_000_000)
    gl.close()
