"""GPU parity of the per-tensor calls (gclip_tensor_norms, gclip_clip_per_tensor_),
through the C ABI, against the oracle's per-tensor clip -- the per-tensor
clip on both paths: one launch (the fused path, a list's default) and two or
three kernels (the split path), which must also agree bit for bit.

Tolerances are those of the global path: every tensor's norm and the list's
within relative 1e-5 of the oracle's; clipped fp32 elements within relative
1e-5, fp16/bf16 elements within 1 ulp; the per-tensor clipped and nonfinite
flags exactly; tensors the oracle leaves alone bitwise unchanged.  Random
thresholds are kept away from every tensor's norm by more than the norm
tolerance, so that no decision is a near-tie."""
import math

import numpy as np
import pytest

import oracle
from synth import gradsets as gs
from tests import gpu_util as gu
from tests.test_gpu_parity import ragged_arrays, upload_as_views

pytestmark = pytest.mark.gpu

DTYPES = ("f32", "f16", "bf16")
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


def set_path(gl, path):
    G = _G()
    gl.set_path(G.GCLIP_PATH_FUSED if path == "fused" else G.GCLIP_PATH_SPLIT)


def gpu_per_tensor(arrays, dtype, max_norm, avg=1.0, err=False, views=None, path="fused"):
    ts = views if views is not None else gu.upload(arrays, dtype)
    gl = _G().GradList(ts)
    set_path(gl, path)
    gl.clip_per_tensor_(max_norm, avg, err)
    st, r = gl.read(err)
    tr = gl.read_tensors()
    out = gu.download(ts, dtype)
    gl.close()
    return st, r, tr, out


def check_tensor_figures(tr, ro, what):
    assert len(tr) == len(ro["tensors"]), what
    for k, (g, o) in enumerate(zip(tr, ro["tensors"])):
        assert bool(g["nonfinite"]) == o["nonfinite"], (what, k)
        gu.assert_norm_close(float(g["norm"]), o["norm"], f"{what} tensor {k}")
        gu.assert_norm_close(float(g["sumsq"]), o["sumsq"], f"{what} tensor {k} sumsq")
        if not math.isnan(o["norm"]):
            assert bool(g["clipped"]) == o["clipped"], (what, k)
            if o["scale"] == 1.0:
                assert float(g["scale"]) == 1.0, (what, k)
            else:
                assert abs(float(g["scale"]) - o["scale"]) <= 1e-5 * abs(o["scale"]), (what, k)


def check_per_tensor(arrays, dtype, max_norm, avg=1.0, err=False, views=None, what="", path="fused"):
    st, r, tr, out = gpu_per_tensor(arrays, dtype, max_norm, avg, err, views, path)
    what = f"{what} ({path})"
    ref = [a.copy() for a in arrays]
    ro = oracle.clip_per_tensor_(ref, dtype, max_norm, avg, err)
    assert r["status"] == 0, what
    assert r["nonfinite"] == ro["nonfinite"] and r["skipped"] == ro["skipped"], what
    gu.assert_norm_close(r["norm"], ro["norm"], what)
    assert r["clipped"] == ro["clipped"] and r["scale"] == 1.0, what
    check_tensor_figures(tr, ro, what)
    for k, (g, o, a) in enumerate(zip(out, ref, arrays)):
        if ro["skipped"] or ro["tensors"][k]["scale"] == 1.0:
            gu.assert_bitwise_equal([g], [a], f"{what} tensor {k} (must be untouched)")
        else:
            gu.assert_elems_close([g], [o], dtype, f"{what} tensor {k}")
    return r, ro, tr, out


def _threshold_off_ties(rng, arrays, dtype, avg=1.0):
    norms = [math.sqrt(s) for s in oracle.tensor_sumsq(arrays, dtype, avg)]
    for _ in range(100):
        c = float(np.exp(rng.uniform(np.log(1e-3), np.log(1e3))))
        if all(abs(n - c) > 1e-4 * c for n in norms):
            return c
    raise AssertionError("no threshold away from every norm")


# ------------------------------------------------------------------ the page's contrast
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_contrast_6_8_and_small(dtype, path):
    """[6, 8] and [0.3, 0.4] at c = 1: [0.6, 0.8] and the second unchanged."""
    a = [gs.to_storage(np.array([6.0, 8.0]), dtype), gs.to_storage(np.array([0.3, 0.4]), dtype)]
    r, ro, tr, out = check_per_tensor(a, dtype, 1.0, what=f"contrast {dtype}", path=path)
    assert float(tr[0]["norm"]) == 10.0 and tr[0]["clipped"] and not tr[1]["clipped"]
    assert np.array_equal(out[0], gs.to_storage(np.array([0.6, 0.8]), dtype))


# ------------------------------------------------------------------ ragged lists
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("err", (False, True))
@pytest.mark.parametrize("seed", range(4))
@pytest.mark.parametrize("dtype", DTYPES)
def test_ragged_lists_misaligned_views(dtype, seed, err, path):
    """Tensors of 1 .. 3M elements at odd element offsets (single elements at
    both ends of each vector run), several pieces per big tensor; in one
    launch, and on the split path without the stop switch (two kernels) and
    with it (three)."""
    rng = np.random.default_rng(2000 + seed)
    arrays = ragged_arrays(rng, dtype, big=seed >= 2)
    avg = [1.0, 0.25, 1.0, 1.0 / 3.0][seed]
    c = _threshold_off_ties(rng, arrays, dtype, avg)
    buf, views = upload_as_views(arrays, dtype, rng)
    check_per_tensor(arrays, dtype, c, avg, err=err, views=views, what=f"ragged {dtype} seed {seed} err {err}",
                     path=path)
    import torch
    mask = torch.ones(buf.numel(), dtype=torch.bool, device="cuda")
    for v in views:
        o = v.storage_offset()
        mask[o:o + v.numel()] = False
    assert int(torch.count_nonzero(buf[mask].float())) == 0, "padding between views written"


@pytest.mark.parametrize("dtype", DTYPES)
def test_tensor_norms_then_global_scale(dtype):
    """gclip_tensor_norms + gclip_scale is the global clip with per-tensor
    figures: the list's norm and the written values as gclip_clip_'s."""
    rng = np.random.default_rng(2100)
    arrays = ragged_arrays(rng, dtype, big=True)
    ts = gu.upload(arrays, dtype)
    gl = _G().GradList(ts)
    gl.tensor_norms(0.5)
    st, r0 = gl.read()
    tr = gl.read_tensors()
    assert not r0["decided"]
    gu.assert_bitwise_equal(gu.download(ts, dtype), arrays, "norms only: nothing written")
    per = oracle.tensor_sumsq(arrays, dtype, 0.5)
    for k, s in enumerate(per):
        gu.assert_norm_close(float(tr[k]["sumsq"]), s, f"tensor {k}")
        assert float(tr[k]["scale"]) == 1.0 and not tr[k]["clipped"]
    ro_ = oracle.clip_([a.copy() for a in arrays], dtype, 1e30, 0.5)
    gu.assert_norm_close(r0["norm"], ro_["norm"], "list norm")
    c = 0.5 * ro_["norm"]
    gl.scale(c, 0.5)
    st, r = gl.read()
    out = gu.download(ts, dtype)
    ref = [a.copy() for a in arrays]
    ro = oracle.clip_(ref, dtype, c, 0.5)
    assert r["clipped"] and ro["clipped"]
    gu.assert_elems_close(out, ref, dtype, "global scale after per-tensor norms")
    gl.close()


# ------------------------------------------------------------------ non-finite, empty, repeatability
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("err", (False, True))
@pytest.mark.parametrize("dtype", DTYPES)
def test_nonfinite(dtype, err, path):
    rng = np.random.default_rng(2200)
    arrays = [gs.to_storage(rng.standard_normal(n) * 3.0, dtype) for n in (5000, 70_001, 33, 4096 * 8)]
    arrays[1][12_345] = gs.to_storage(np.array([math.nan]), dtype)[0]
    arrays[3][7] = gs.to_storage(np.array([-math.inf]), dtype)[0]
    r, ro, tr, out = check_per_tensor(arrays, dtype, 1.0, err=err, what=f"nonfinite {dtype} err={err}", path=path)
    assert r["nonfinite"] and list(tr["nonfinite"]) == [0, 1, 0, 1]
    assert r["skipped"] == err


@pytest.mark.parametrize("path", PATHS)
def test_empty_lists_and_tensors(path):
    G = _G()
    import torch
    for arrays in ([], [np.zeros(0, np.float32)], [np.zeros(0, np.float32), np.ones(3, np.float32) * 2.0,
                                                    np.zeros(0, np.float32)]):
        ts = gu.upload(arrays, "f32") if arrays else []
        gl = G.GradList(ts)
        set_path(gl, path)
        gl.clip_per_tensor_(1.0)
        st, r = gl.read()
        tr = gl.read_tensors()
        ro = oracle.clip_per_tensor_([a.copy() for a in arrays], "f32", 1.0)
        gu.assert_norm_close(r["norm"], ro["norm"], "empty")
        assert len(tr) == len(arrays)
        check_tensor_figures(tr, ro, "empty")
        gl.close()
    torch.cuda.synchronize()


def test_repeatable_bits():
    rng = np.random.default_rng(2300)
    arrays = ragged_arrays(rng, "f32", big=True)
    ts = gu.upload(arrays, "f32")
    gl = _G().GradList(ts)
    runs = []
    for _ in range(3):
        gl.tensor_norms()
        st, r = gl.read()
        runs.append((r["sumsq"], gl.read_tensors()["sumsq"].tobytes()))
    assert runs[0] == runs[1] == runs[2]
    gl.close()


def test_invalid_arguments():
    import torch
    G = _G()
    ts = gu.upload([np.ones(10, np.float32)], "f32")
    gl = G.GradList(ts)
    s = torch.cuda.current_stream().cuda_stream
    for bad in (0, gl.tensor_results.data_ptr() + 4):
        with pytest.raises(G.GclipError):
            G.gclip_tensor_norms(gl.handle, 1.0, bad, gl.d_result, s)
        with pytest.raises(G.GclipError):
            G.gclip_clip_per_tensor_(gl.handle, 1.0, 1.0, False, bad, gl.d_result, s)
    for c, a in ((0.0, 1.0), (math.nan, 1.0), (1.0, 0.0), (1.0, math.inf)):
        with pytest.raises(G.GclipError):
            gl.clip_per_tensor_(c, a)
    gu.assert_bitwise_equal(gu.download(ts, "f32"), [np.ones(10, np.float32)], "rejected calls write nothing")
    gl.close()


# ------------------------------------------------------------------ full size
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("err", (False, True))
@pytest.mark.parametrize("dtype_cfg", ("andrea120m_f32", "andrea120m_f16_spike"))
def test_andrea120m(dtype_cfg, err, path):
    """The 124-tensor list at c = 0.5: the big matrices are clipped, the norm
    vectors are not (their norms are ~0.03)."""
    g = gs.make(dtype_cfg)
    r, ro, tr, out = check_per_tensor(g.arrays, g.dtype, 0.5, err=err, what=f"{dtype_cfg} err {err}", path=path)
    flags = [t["clipped"] for t in ro["tensors"]]
    assert any(flags) and not all(flags)


# ------------------------------------------------------------------ two kernels: every piece decides for its tensor
def _reload(ts, arrays, dtype):
    for t, a in zip(ts, gu.upload(arrays, dtype)):
        t.copy_(a)


def _check_call(gl, ts, arrays, ref, ro, dtype, what, complete=True):
    """One call's outputs against the oracle's; the list's figures too when
    the result block is complete."""
    st, r = gl.read()
    tr = gl.read_tensors()
    out = gu.download(ts, dtype)
    if complete:
        assert st == 0 and r["status"] == 0, (what, r)
        gu.assert_norm_close(r["norm"], ro["norm"], what)
        assert r["clipped"] == ro["clipped"] and r["nonfinite"] == ro["nonfinite"] and not r["skipped"], what
    check_tensor_figures(tr, ro, what)
    for k, (g, o, a) in enumerate(zip(out, ref, arrays)):
        if ro["tensors"][k]["scale"] == 1.0:
            gu.assert_bitwise_equal([g], [a], f"{what} tensor {k} (must be untouched)")
        else:
            gu.assert_elems_close([g], [o], dtype, f"{what} tensor {k}")
    return st, r, tr, out


@pytest.mark.parametrize("dtype", DTYPES)
def test_two_kernel_clip_many_tensors_repeated(dtype):
    """Without the stop switch every piece sums its own tensor's partials and
    decides; the first piece of each tensor publishes the tensor's sum and
    workgroup 0 gathers the list's figures.  A list of 2,300 tensors (two
    big ones, empty ones, 2,000 single elements, 300 short runs), three calls
    in a row on one list -- the publication count must be back at zero after
    each -- every call against the oracle, and the same bits every time."""
    rng = np.random.default_rng(2600)
    sizes = [1_000_003, 0] + [1] * 2000 + [0, 3_000_001] + [int(n) for n in rng.integers(2, 200, size=300)] + [0]
    arrays = [gs.to_storage(rng.standard_normal(n) * 1e-2, dtype) for n in sizes]
    # the two big tensors' norms are ~5 and ~8.7 at a = 0.5, the others' at most ~0.1
    c = 1.0
    assert all(abs(math.sqrt(x) - c) > 1e-3 for x in oracle.tensor_sumsq(arrays, dtype, 0.5))
    ref = [a.copy() for a in arrays]
    ro = oracle.clip_per_tensor_(ref, dtype, c, 0.5, False)
    assert any(t["clipped"] for t in ro["tensors"]) and not all(t["clipped"] for t in ro["tensors"])
    ts = gu.upload(arrays, dtype)
    gl = _G().GradList(ts)
    set_path(gl, "split")
    runs = []
    for rep in range(3):
        _reload(ts, arrays, dtype)
        gl.clip_per_tensor_(c, 0.5, False)
        st, r, tr, out = _check_call(gl, ts, arrays, ref, ro, dtype, f"many tensors {dtype} call {rep}")
        runs.append((r["sumsq"], tr.tobytes(), b"".join(o.tobytes() for o in out)))
    assert runs[0] == runs[1] == runs[2]
    gl.close()


# calls with no gathering wait before one must have given up (each one does
# so or not by a race)
WAIT0_CALLS = 12


def test_gather_wait_timeout_is_reported_and_recovers():
    """With the gathering workgroup's wait cut to nothing (a bound on the
    kernel's own wait, set from the host) it gives up before the other
    tensors have published: the result block says so
    (GCLIP_DEVICE_WAIT_TIMEOUT, and gclip_result_read returns GCLIP_EDEVICE),
    every tensor is still decided, scaled and given its figures, and later
    calls with the normal wait are complete again (the counts of the
    abandoned wait were taken back).  Whether one call gives up is a race
    between the gathering workgroup and the others, so the calls go on (at
    most WAIT0_CALLS) until one has."""
    G = _G()
    from global_l2_norm_amd import _lib
    rng = np.random.default_rng(2700)
    sizes = [5] + [1] * 1500 + [4_000_001] + [300] * 200 + [0]
    arrays = [gs.to_storage(rng.standard_normal(n) * 1e-2, "f32") for n in sizes]
    c = 1.0  # clips the 4M-element tensor (norm ~20), none of the others (at most ~0.2)
    assert all(abs(math.sqrt(x) - c) > 1e-3 for x in oracle.tensor_sumsq(arrays, "f32"))
    ref = [a.copy() for a in arrays]
    ro = oracle.clip_per_tensor_(ref, "f32", c)
    assert any(t["clipped"] for t in ro["tensors"]) and not all(t["clipped"] for t in ro["tensors"])
    ts = gu.upload(arrays, "f32")
    gl = G.GradList(ts)
    set_path(gl, "split")  # the two-kernel form's gathering wait
    timeouts = 0
    try:
        G.gclip_set_gather_wait(0)
        for rep in range(WAIT0_CALLS):
            _reload(ts, arrays, "f32")
            gl.clip_per_tensor_(c)
            st, r = gl.read()
            assert r["status"] in (0, G.GCLIP_DEVICE_WAIT_TIMEOUT), r
            if r["status"]:
                timeouts += 1
                assert st == _lib.GCLIP_EDEVICE
            _check_call(gl, ts, arrays, ref, ro, "f32", f"wait 0, call {rep}", complete=r["status"] == 0)
            if rep >= 2 and timeouts:
                break
    finally:
        G.gclip_set_gather_wait(-1)
    print(f"{timeouts} of {rep + 1} calls gave up waiting")
    assert timeouts >= 1
    for rep in range(2):
        _reload(ts, arrays, "f32")
        gl.clip_per_tensor_(c)
        _check_call(gl, ts, arrays, ref, ro, "f32", f"normal wait, call {rep}")
    gl.close()


def test_gather_wait_timeout_with_the_stop_switch_writes_nothing():
    """With the stop switch the decisions are gathered before the scale
    kernel runs; when the gathering wait gives up, the stop decision has not
    been taken, so nothing may be written: the scale kernel reads the failure
    in the result block.  Later calls with the normal wait clip as the
    oracle does.  The calls with no wait go on (at most WAIT0_CALLS) until
    one has given up."""
    G = _G()
    from global_l2_norm_amd import _lib
    rng = np.random.default_rng(2800)
    sizes = [5] + [1] * 1500 + [4_000_001] + [300] * 200 + [0]
    arrays = [gs.to_storage(rng.standard_normal(n) * 1e-2, "f32") for n in sizes]
    c = 1.0
    assert all(abs(math.sqrt(x) - c) > 1e-3 for x in oracle.tensor_sumsq(arrays, "f32"))
    ref = [a.copy() for a in arrays]
    ro = oracle.clip_per_tensor_(ref, "f32", c, 1.0, True)
    ts = gu.upload(arrays, "f32")
    gl = G.GradList(ts)
    set_path(gl, "split")  # the three-kernel form's gathering wait
    timeouts = 0
    try:
        G.gclip_set_gather_wait(0)
        for rep in range(WAIT0_CALLS):
            _reload(ts, arrays, "f32")
            gl.clip_per_tensor_(c, 1.0, True)
            st, r = gl.read(True)
            assert r["status"] in (0, G.GCLIP_DEVICE_WAIT_TIMEOUT), r
            if r["status"]:
                timeouts += 1
                assert st == _lib.GCLIP_EDEVICE
                gu.assert_bitwise_equal(gu.download(ts, "f32"), arrays, f"gave up, call {rep}: nothing written")
            else:
                _check_call(gl, ts, arrays, ref, ro, "f32", f"stop switch, wait 0, call {rep}")
            if rep >= 2 and timeouts:
                break
    finally:
        G.gclip_set_gather_wait(-1)
    print(f"{timeouts} of {rep + 1} calls gave up waiting")
    assert timeouts >= 1
    for rep in range(2):
        _reload(ts, arrays, "f32")
        gl.clip_per_tensor_(c, 1.0, True)
        _check_call(gl, ts, arrays, ref, ro, "f32", f"stop switch, normal wait, call {rep}")
    gl.close()


def test_gather_wait_bounds():
    G = _G()
    with pytest.raises(G.GclipError):
        G.gclip_set_gather_wait(61 * 1000 * 1000)
    G.gclip_set_gather_wait(-1)


# ------------------------------------------------------------------ one launch against the split path, bit for bit
def _both_paths(arrays, dtype, max_norm, avg, err, wait_us=None):
    """The one-launch clip and the split path on the same input: every
    written bit, every figure and the result block's figures must agree."""
    got = {}
    for path in PATHS:
        ts = gu.upload(arrays, dtype)
        gl = _G().GradList(ts)
        set_path(gl, path)
        if wait_us is not None and path == "fused":
            gl.set_wait(wait_us)
        gl.clip_per_tensor_(max_norm, avg, err)
        st, r = gl.read(err)
        got[path] = (st, r, gl.read_tensors(), gu.download(ts, dtype))
        gl.close()
    (sf, rf, tf, of), (ss, rs, tsp, osp) = got["fused"], got["split"]
    what = f"{dtype} {[a.size for a in arrays][:6]}... avg {avg} err {err} wait {wait_us}"
    assert sf == ss and rf["status"] == rs["status"] == 0, (what, rf, rs)
    for key in ("sumsq", "norm", "nonfinite", "clipped", "skipped", "scale", "decided"):
        same = rf[key] == rs[key] or (isinstance(rf[key], float) and math.isnan(rf[key]) and math.isnan(rs[key]))
        assert same, (what, key, rf[key], rs[key])
    assert tf.tobytes() == tsp.tobytes(), what
    gu.assert_bitwise_equal(of, osp, f"one launch vs split, {what}")
    return rf


@pytest.mark.parametrize("err", (False, True))
@pytest.mark.parametrize("dtype", DTYPES)
def test_one_launch_equals_split_bitwise(dtype, err):
    """Ragged lists (one with a streamed region: more pieces than the
    workers keep on chip), many small tensors, a NaN with and without the
    stop switch: the one-launch clip writes what the split path writes."""
    rng = np.random.default_rng(2900)
    for big in (False, True):
        arrays = ragged_arrays(rng, dtype, big=big)
        _both_paths(arrays, dtype, _threshold_off_ties(rng, arrays, dtype, 0.5), 0.5, err)
    sizes = [3_000_001, 0] + [1] * 700 + [int(n) for n in rng.integers(2, 5000, size=300)] + [9_000_000, 0]
    arrays = [gs.to_storage(rng.standard_normal(n) * 1e-2, dtype) for n in sizes]
    _both_paths(arrays, dtype, 0.05, 1.0, err)
    arrays[705][1] = gs.to_storage(np.array([math.nan]), dtype)[0]  # a tensor of 2 .. 4999 elements
    r = _both_paths(arrays, dtype, 0.05, 1.0, err)
    assert r["nonfinite"] and r["skipped"] == err


def test_one_launch_hand_back_equals_split():
    """With no wait at the decision every workgroup but the deciding one
    hands its resident pieces back (and the two streamed pieces it takes
    without a claim); they are scaled from memory with the same bits."""
    rng = np.random.default_rng(2950)
    sizes = [20_000_003, 7, 1, 0] + [int(n) for n in rng.integers(1, 70_000, size=200)] + [15_000_000]
    arrays = [gs.to_storage(rng.standard_normal(n) * 1e-2, "f32") for n in sizes]
    _both_paths(arrays, "f32", 0.5, 1.0, False, wait_us=0)
    ts = gu.upload(arrays, "f32")
    gl = _G().GradList(ts)
    gl.set_wait(0)
    gl.clip_per_tensor_(0.5)
    st, r = gl.read()
    assert st == 0 and r["handed_back"] >= 1, r
    gl.close()


@pytest.mark.parametrize("dtype", DTYPES)
def test_one_launch_many_tensors_repeated(dtype):
    """Three calls in a row on one list of 2,300 tensors: the tensors'
    counters and factor slots must be back to empty after each (a stale
    factor would scale the next call by the previous one's), every call
    against the oracle and the split path, the same bits every time."""
    rng = np.random.default_rng(2600)
    sizes = [1_000_003, 0] + [1] * 2000 + [0, 3_000_001] + [int(n) for n in rng.integers(2, 200, size=300)] + [0]
    arrays = [gs.to_storage(rng.standard_normal(n) * 1e-2, dtype) for n in sizes]
    c = 1.0
    assert all(abs(math.sqrt(x) - c) > 1e-3 for x in oracle.tensor_sumsq(arrays, dtype, 0.5))
    ref = [a.copy() for a in arrays]
    ro = oracle.clip_per_tensor_(ref, dtype, c, 0.5, False)
    ts = gu.upload(arrays, dtype)
    gl = _G().GradList(ts)
    set_path(gl, "fused")
    runs = []
    for rep in range(3):
        # a different input in between, so that stale state would show
        _reload(ts, [a[::-1].copy() for a in arrays], dtype)
        gl.clip_per_tensor_(0.3, 1.0, False)
        _reload(ts, arrays, dtype)
        gl.clip_per_tensor_(c, 0.5, False)
        st, r, tr, out = _check_call(gl, ts, arrays, ref, ro, dtype, f"one launch, many tensors {dtype} call {rep}")
        runs.append((r["sumsq"], tr.tobytes(), b"".join(o.tobytes() for o in out)))
    assert runs[0] == runs[1] == runs[2]
    gl.close()
    _both_paths(arrays, dtype, c, 0.5, False)
