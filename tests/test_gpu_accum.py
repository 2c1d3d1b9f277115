"""GPU parity of the last microbatch's += fused with the norm pass
(gclip_accumulate_norm, gclip_accumulate_clip_), through the C ABI, against
the oracle's += followed by its clip.

The accumulated buffer must equal the oracle's bit for bit: the += is the
storage format's own correctly rounded addition on both sides.  The norm,
and the clipped values of gclip_accumulate_clip_, follow the tolerances of
the global path (norm relative 1e-5; fp32 elements relative 1e-5, fp16/bf16
elements 1 ulp); the non-finite flag exactly; the contribution is only read."""
import math

import numpy as np
import pytest

import oracle
from synth import gradsets as gs
from tests import gpu_util as gu
from tests.test_gpu_parity import ragged_arrays

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "f16", "bf16")
PATHS = ("fused", "split")  # one launch, or the += with the norm then the scale pass


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("the gpu tests need an MI355X")
    import global_l2_norm_amd  # noqa: F401  (fails loudly when libgclip.so is missing)


def _G():
    import global_l2_norm_amd as G
    return G


def views_at(arrays, dtype, offsets):
    """Each array a view at the given element offset inside one device buffer."""
    import torch
    total = (offsets[-1] + arrays[-1].size + 8) if arrays else 8
    buf = torch.zeros(total, dtype=gu.torch_dtype(dtype), device="cuda")
    views = []
    for a, o in zip(arrays, offsets):
        v = buf[o:o + a.size]
        if a.size:
            v.copy_(gu.upload([a], dtype)[0])
        views.append(v)
    return buf, views


def odd_offsets(rng, arrays):
    offs, total = [], 0
    for a in arrays:
        total += int(rng.integers(1, 8))
        offs.append(total)
        total += a.size
    return offs


def gpu_accumulate(acc, contrib, dtype, call, max_norm=1.0, avg=1.0, err=False, offsets=None, per_tensor=False,
                   path="fused", wait_us=None):
    G = _G()
    if offsets is None:
        ta, tg = gu.upload(acc, dtype), gu.upload(contrib, dtype)
        keep = None
    else:
        ba, ta = views_at(acc, dtype, offsets)
        bg, tg = views_at(contrib, dtype, offsets)
        keep = (ba, bg)
    gl = G.GradList(ta)
    gl.set_path(G.GCLIP_PATH_FUSED if path == "fused" else G.GCLIP_PATH_SPLIT)
    if wait_us is not None:
        gl.set_wait(wait_us)
    c = G.Contribution(gl, tg)
    if call == "norm":
        gl.accumulate_norm(c, avg, per_tensor=per_tensor)
    else:
        gl.accumulate_clip_(c, max_norm, avg, err)
    st, r = gl.read(err)
    tr = gl.read_tensors() if per_tensor else None
    out, g_after = gu.download(ta, dtype), gu.download(tg, dtype)
    c.close()
    gl.close()
    del keep
    return st, r, out, g_after, tr


def check_accumulate(acc, contrib, dtype, max_norm=1.0, avg=1.0, err=False, offsets=None, what="", path="fused"):
    # the += with the norm
    st, r, out, g_after, tr = gpu_accumulate(acc, contrib, dtype, "norm", avg=avg, offsets=offsets,
                                             per_tensor=True)
    ref = [a.copy() for a in acc]
    oracle.accumulate_(ref, contrib, dtype)
    gu.assert_bitwise_equal_but_nan(out, ref, dtype, what + " (the += itself)")
    gu.assert_bitwise_equal(g_after, contrib, what + " (contribution only read)")
    s, nf = oracle.sumsq(ref, dtype, avg)
    assert r["nonfinite"] == nf and not r["decided"], what
    gu.assert_norm_close(r["norm"], math.sqrt(s), what)
    for k, ps in enumerate(oracle.tensor_sumsq(ref, dtype, avg)):
        gu.assert_norm_close(float(tr[k]["sumsq"]), ps, f"{what} tensor {k}")
    # the += with the clip
    st, r, out, g_after, _ = gpu_accumulate(acc, contrib, dtype, "clip", max_norm, avg, err, offsets, path=path)
    what = f"{what} ({path})"
    gu.assert_bitwise_equal(g_after, contrib, what + " (contribution only read)")
    ref = [a.copy() for a in acc]
    ro = oracle.accumulate_clip_(ref, contrib, dtype, max_norm, avg, err)
    summed = [a.copy() for a in acc]
    oracle.accumulate_(summed, contrib, dtype)
    assert r["nonfinite"] == ro["nonfinite"] and r["skipped"] == ro["skipped"], what
    if not math.isnan(ro["norm"]):
        gu.assert_norm_close(r["norm"], ro["norm"], what)
        assert r["clipped"] == ro["clipped"], what
    if ro["skipped"] or ro["scale"] == 1.0:
        gu.assert_bitwise_equal_but_nan(out, summed, dtype, what + " (sum written, nothing scaled)")
    else:
        gu.assert_elems_close(out, ref, dtype, what + " (clipped sum)")
    return r, ro


@pytest.mark.parametrize("dtype", DTYPES)
def test_order_example(dtype):
    """Glossary page, "Order changes the result": 10 and -9 are summed to 1
    first, and the clip of the sum at 5 keeps it."""
    acc, g = [gs.to_storage(np.array([10.0]), dtype)], [gs.to_storage(np.array([-9.0]), dtype)]
    r, ro = check_accumulate(acc, g, dtype, max_norm=5.0, what=f"order {dtype}")
    assert r["norm"] == 1.0 and not r["clipped"]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("dtype", DTYPES)
def test_ragged_lists(dtype, seed, path):
    """Tensors of 1 .. 3M elements; seeds 1 and 3 as views at odd element
    offsets (single elements at both ends of each vector run)."""
    rng = np.random.default_rng(3000 + seed)
    acc = ragged_arrays(rng, dtype, big=seed >= 2)
    # a multiple of the buffer plus noise: factors near -1 cancel most digits
    contrib = [gs.to_storage(gu.values(a, dtype) * float(rng.uniform(-1.5, 1.5)) + rng.standard_normal(a.size) * 1e-3,
                             dtype) for a in acc]
    avg = [1.0, 0.25, 0.5, 1.0 / 3.0][seed]
    s, _ = oracle.sumsq([x.copy() for x in acc], dtype, avg)
    offsets = odd_offsets(rng, acc) if seed % 2 else None
    check_accumulate(acc, contrib, dtype, max_norm=0.5 * math.sqrt(s) + 1e-3, avg=avg, offsets=offsets,
                     what=f"ragged {dtype} seed {seed}", path=path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("err", (False, True))
@pytest.mark.parametrize("dtype", DTYPES)
def test_special_values(dtype, err, path):
    """Overflow to Inf, Inf - Inf, subnormals, exact cancellation, signed
    zeros, a NaN; with the stop switch the sum is still written but not
    scaled."""
    big = {"f32": 3.0e38, "f16": 60000.0, "bf16": 3.0e38}[dtype]
    tiny = {"f32": 1e-40, "f16": 3e-6, "bf16": 1e-39}[dtype]
    rng = np.random.default_rng(3100)
    n = 4096 * 3 + 5
    a = rng.standard_normal(n)
    g = rng.standard_normal(n)
    pairs = [(big, big), (math.inf, -math.inf), (tiny, tiny), (tiny, -tiny), (7.0, -7.0), (-0.0, -0.0),
             (math.nan, 1.0), (-big, -big)]
    for k, (x, y) in enumerate(pairs):
        a[100 * k + 3], g[100 * k + 3] = x, y
    acc, contrib = [gs.to_storage(a, dtype)], [gs.to_storage(g, dtype)]
    r, ro = check_accumulate(acc, contrib, dtype, max_norm=1.0, err=err, what=f"special {dtype} err={err}",
                             path=path)
    assert r["nonfinite"] and r["skipped"] == err


def test_four_microbatches_then_clip():
    """((c0 + c1) + c2) + c3 with every += on the GPU, the last fused with
    the clip at a = 1/4: the oracle's buffer and clip."""
    G = _G()
    rng = np.random.default_rng(3200)
    sizes = [4096 * 17 + 3, 1000, 3, 70_001]
    cs = [[gs.to_storage(rng.standard_normal(n) * 1e-3, "f32") for n in sizes] for _ in range(4)]
    ta = gu.upload(cs[0], "f32")
    gl = G.GradList(ta)
    contribs = []
    for k in range(1, 4):
        tg = gu.upload(cs[k], "f32")
        contribs.append((G.Contribution(gl, tg), tg))
    for c, _ in contribs[:2]:
        gl.accumulate_norm(c)
    gl.accumulate_clip_(contribs[2][0], 1e-3, 0.25)
    st, r = gl.read()
    out = gu.download(ta, "f32")
    ref = [x.copy() for x in cs[0]]
    oracle.accumulate_(ref, cs[1], "f32")
    oracle.accumulate_(ref, cs[2], "f32")
    ro = oracle.accumulate_clip_(ref, cs[3], "f32", 1e-3, 0.25)
    gu.assert_norm_close(r["norm"], ro["norm"], "four microbatches")
    assert r["clipped"] and ro["clipped"]
    gu.assert_elems_close(out, ref, "f32", "four microbatches")
    for c, _ in contribs:
        c.close()
    gl.close()


def test_adamw_after_accumulate_norm():
    """The last += with the norm, then the optimizer step on the clipped sum."""
    import torch
    from tests.test_gpu_adamw import HP, assert_adamw_close
    G = _G()
    rng = np.random.default_rng(3300)
    sizes = [4096 * 9 + 1, 513, 20_000]
    acc = [gs.to_storage(rng.standard_normal(n) * 1e-2, "f32") for n in sizes]
    contrib = [gs.to_storage(rng.standard_normal(n) * 1e-2, "f32") for n in sizes]
    params = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in sizes]
    m = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for n in sizes]
    v = [(rng.random(n) * 1e-6).astype(np.float32) for n in sizes]
    ta, tg = gu.upload(acc, "f32"), gu.upload(contrib, "f32")
    tp, tm, tv = ([torch.from_numpy(x.copy()).cuda() for x in grp] for grp in (params, m, v))
    gl = G.GradList(ta)
    c = G.Contribution(gl, tg)
    opt = G.AdamWList(tp, ta, tm, tv)
    gl.accumulate_norm(c, 0.5)
    opt.step(gl, step=2, max_norm=0.1, avg_factor=0.5, **HP)
    st, r = gl.read()
    out = tuple([t.cpu().numpy() for t in grp] for grp in (tp, tm, tv))
    summed = [x.copy() for x in acc]
    oracle.accumulate_(summed, contrib, "f32")
    ro, ref = oracle.clip_adamw(params, summed, m, v, "f32", 0.1, 0.5, False, step=2, **HP)
    gu.assert_bitwise_equal(gu.download(ta, "f32"), summed, "the += itself")
    gu.assert_norm_close(r["norm"], ro["norm"], "norm")
    assert_adamw_close(out, ref, (params, m, v), summed, "f32", ro["scale"], HP, 2, "adamw after +=")
    opt.close()
    c.close()
    gl.close()


def test_invalid_contributions():
    import torch
    G = _G()
    acc = [np.ones(100, np.float32), np.ones(37, np.float32)]
    ta = gu.upload(acc, "f32")
    gl = G.GradList(ta)
    other = G.GradList(gu.upload(acc, "f32"))
    buf = torch.zeros(200, dtype=torch.float32, device="cuda")
    with pytest.raises(G.GclipError):  # misaligned: 4 bytes off the list's alignment
        G.gclip_contrib_create(gl.handle, [buf[1:101].data_ptr(), buf[120:157].data_ptr()])
    with pytest.raises(G.GclipError):  # the list's own tensors
        G.gclip_contrib_create(gl.handle, [ta[0].data_ptr(), ta[1].data_ptr()])
    with pytest.raises(G.GclipError):  # two contribution tensors overlap
        G.gclip_contrib_create(gl.handle, [buf[0:100].data_ptr(), buf[64:101].data_ptr()])
    with pytest.raises(G.GclipError):  # NULL
        G.gclip_contrib_create(gl.handle, [0, buf[120:157].data_ptr()])
    c = G.Contribution(other, gu.upload(acc, "f32"))
    with pytest.raises(G.GclipError):  # registered for another list
        gl.accumulate_norm(c)
    with pytest.raises(G.GclipError):
        gl.accumulate_clip_(c, 1.0)
    c.close()
    gu.assert_bitwise_equal(gu.download(ta, "f32"), acc, "rejected calls write nothing")
    other.close()
    gl.close()


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("cfg", ("andrea120m_f32", "andrea120m_f16_spike"))
def test_andrea120m(cfg, path):
    """The 124-tensor list plus a second draw of it, averaged by 1/2, clipped
    at 1.0 (the fp32 sum has norm ~6.8, so it clips)."""
    g = gs.make(cfg)
    h = gs.make(cfg, seed=11)
    check_accumulate(g.arrays, h.arrays, g.dtype, max_norm=1.0, avg=0.5, what=cfg, path=path)


# ------------------------------------------------------------------ the fused kernel's hand-backs with the +=
@pytest.mark.parametrize("dtype", ("f32", "bf16"))
def test_handed_back_blocks_with_the_accumulate(dtype):
    """With no wait at all nearly every workgroup hands its block back before
    writing it; whoever takes a block over reads it with its contribution,
    adds, scales and writes it.  A list larger than the on-chip share, so
    that the streamed region's chunks are handed over too.  Bit for bit the
    result of the same call with the normal wait."""
    rng = np.random.default_rng(3400)
    n_total = 35_000_000 if dtype == "f32" else 70_000_000
    sizes = [n_total // 2 + 5, n_total - n_total // 2 - 5]
    acc = [gs.to_storage(rng.standard_normal(n) * 1e-3, dtype) for n in sizes]
    contrib = [gs.to_storage(rng.standard_normal(n) * 1e-3, dtype) for n in sizes]
    st, r0, out0, _, _ = gpu_accumulate(acc, contrib, dtype, "clip", 1.0, 0.5, False, path="fused")
    st, r, out, g_after, _ = gpu_accumulate(acc, contrib, dtype, "clip", 1.0, 0.5, False, path="fused", wait_us=0)
    assert r["handed_back"] >= 1 and r0["handed_back"] == 0, (r, r0)
    assert r["sumsq"] == r0["sumsq"] and r["scale"] == r0["scale"] and r["clipped"]
    gu.assert_bitwise_equal(out, out0, f"hand-back with += {dtype}")
    gu.assert_bitwise_equal(g_after, contrib, "contribution only read")
    ref = [a.copy() for a in acc]
    ro = oracle.accumulate_clip_(ref, contrib, dtype, 1.0, 0.5)
    gu.assert_norm_close(r["norm"], ro["norm"], "hand-back with +=")
    gu.assert_elems_close(out, ref, dtype, f"hand-back with += {dtype}")


@pytest.mark.parametrize("bad", (math.nan, None))
def test_handed_back_blocks_write_the_sum_when_nothing_is_scaled(bad):
    """Stop switch (a NaN) or factor 1 (norm under max_norm): nothing is
    scaled, but the += is still written, by whoever holds each block."""
    rng = np.random.default_rng(3500)
    sizes = [30_000_001, 4_000_000, 7]
    acc = [gs.to_storage(rng.standard_normal(n) * 1e-4, "f32") for n in sizes]
    contrib = [gs.to_storage(rng.standard_normal(n) * 1e-4, "f32") for n in sizes]
    if bad is not None:
        contrib[1][123] = np.float32(bad)
    st, r, out, _, _ = gpu_accumulate(acc, contrib, "f32", "clip", 1e30, 1.0, True, path="fused", wait_us=0)
    assert r["handed_back"] >= 1
    assert r["skipped"] == (bad is not None) and r["scale"] == 1.0
    summed = [a.copy() for a in acc]
    oracle.accumulate_(summed, contrib, "f32")
    gu.assert_bitwise_equal_but_nan(out, summed, "f32", "sum written, nothing scaled")
