"""gclip_clip_noalloc_, through the C ABI: the clip with its table and
workspace in the library's static device array instead of an allocation.

Each call must give the result block and the gradients of gclip_clip_ over a
list created from the same pointers (the same kernels on the same table, so
bit for bit), which the parity tests tie to the oracle; the norm is checked
against the oracle here too.  Two calls in a row share the array: the second,
on a smaller list, must not see anything of the first.  A list whose table
does not fit is rejected with GCLIP_ERANGE before anything is enqueued."""
import ctypes
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


def _noalloc(ts, dtype_code, max_norm, avg=1.0, err=False):
    """gclip_clip_noalloc_ on device tensors ts; returns (status, device result block)."""
    import torch
    from global_l2_norm_amd import _lib
    n = len(ts)
    ptrs = (ctypes.c_void_p * max(n, 1))(*[t.data_ptr() for t in ts])
    numels = (ctypes.c_int64 * max(n, 1))(*[t.numel() for t in ts])
    res = torch.zeros(64, dtype=torch.uint8, device="cuda")
    st = _lib.lib.gclip_clip_noalloc_(ptrs, numels, n, dtype_code, max_norm, avg, int(err), res.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream)
    return st, res


def _read(res):
    from global_l2_norm_amd import _lib
    import torch
    torch.cuda.synchronize()
    raw = bytes(res.cpu().numpy())
    return _lib.GclipResult.from_buffer_copy(raw).as_dict()


def _check_against_list(arrays, dtype, max_norm, avg=1.0, err=False, what=""):
    import torch
    G = __import__("global_l2_norm_amd")
    code = {"f32": G.GCLIP_F32, "f16": G.GCLIP_F16, "bf16": G.GCLIP_BF16}[dtype]
    ta = gu.upload(arrays, dtype)
    tb = gu.upload(arrays, dtype)
    st, res = _noalloc(ta, code, max_norm, avg, err)
    assert st == 0, (what, st)
    r_na = _read(res)
    gl = G.GradList(tb)
    gl.clip_(max_norm, avg, err)
    st_l, r_l = gl.read(err)
    gl.close()
    for k in ("sumsq", "norm", "scale", "max_norm", "nonfinite", "clipped", "skipped", "decided", "status"):
        a, b = r_na[k], r_l[k]
        assert a == b or (isinstance(a, float) and math.isnan(a) and math.isnan(b)), (what, k, a, b)
    gu.assert_bitwise_equal(gu.download(ta, dtype), gu.download(tb, dtype), what + ": gradients")
    s_ref, nf = oracle.sumsq(arrays, dtype, avg)
    gu.assert_norm_close(r_na["norm"], math.sqrt(s_ref), what)
    del ta, tb
    torch.cuda.empty_cache()
    return r_na


def test_two_calls_in_a_row_second_smaller():
    """The 120M fp32 list (its table and partials fill much of the array),
    then a small ragged bf16 list with odd-sized tensors and single
    elements, then the big one again."""
    big = gs.andrea120m_f32()
    r = _check_against_list(big.arrays, "f32", big.max_norm, what="andrea120m f32, first call")
    assert r["clipped"] and abs(r["norm"] - 9.605) < 0.01
    rng = np.random.default_rng(7100)
    small = [gs.to_storage(rng.standard_normal(n) * 0.05, "bf16") for n in (1, 3, 4097, 70_001, 9, 1_000_003, 2)]
    r = _check_against_list(small, "bf16", 1.0, what="small bf16, second call")
    assert r["clipped"]
    r = _check_against_list(small, "bf16", 1e9, avg=0.25, what="small bf16, averaging only")
    assert not r["clipped"] and r["scale"] == 0.25
    r = _check_against_list(big.arrays, "f32", big.max_norm, what="andrea120m f32, third call")
    assert r["clipped"]


def test_nonfinite_and_empty():
    rng = np.random.default_rng(7200)
    arrays = [gs.to_storage(rng.standard_normal(n), "f16") for n in (5000, 17)]
    arrays[0][123] = 0x7E00  # NaN
    r = _check_against_list(arrays, "f16", 1.0, err=True, what="nan, stop switch")
    assert r["nonfinite"] and r["skipped"]
    r = _check_against_list([], "f32", 1.0, what="empty list")
    assert r["norm"] == 0.0 and not r["clipped"]


def test_too_large_for_the_scratch_is_rejected():
    """600,000 one-element tensors (views into one buffer) need 8 bytes of
    table each, past the 4 MiB array: GCLIP_ERANGE, and nothing is
    written."""
    import torch
    from global_l2_norm_amd import _lib
    n = 600_000
    buf = torch.arange(n, dtype=torch.float32, device="cuda")
    before = buf.cpu().numpy().copy()
    ptrs = (ctypes.c_void_p * n)(*[buf.data_ptr() + 4 * i for i in range(n)])
    numels = (ctypes.c_int64 * n)(*([1] * n))
    res = torch.full((64,), 7, dtype=torch.uint8, device="cuda")
    st = _lib.lib.gclip_clip_noalloc_(ptrs, numels, n, 0, 1.0, 1.0, 0, res.data_ptr(),
                                      torch.cuda.current_stream().cuda_stream)
    assert st == _lib.GCLIP_ERANGE
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy(), before)
    assert bool((res == 7).all())
    # bad arguments, also before anything is enqueued
    one = (ctypes.c_void_p * 1)(buf.data_ptr())
    cnt = (ctypes.c_int64 * 1)(4)
    stream = torch.cuda.current_stream().cuda_stream
    assert _lib.lib.gclip_clip_noalloc_(one, cnt, 1, 0, 0.0, 1.0, 0, res.data_ptr(), stream) == _lib.GCLIP_EINVAL
    assert _lib.lib.gclip_clip_noalloc_(one, cnt, 1, 0, 1.0, float("nan"), 0, res.data_ptr(), stream) == \
        _lib.GCLIP_EINVAL
    assert _lib.lib.gclip_clip_noalloc_(one, cnt, 1, 9, 1.0, 1.0, 0, res.data_ptr(), stream) == _lib.GCLIP_EDTYPE
    assert _lib.lib.gclip_clip_noalloc_(one, cnt, 1, 0, 1.0, 1.0, 0, None, stream) == _lib.GCLIP_EINVAL
    torch.cuda.synchronize()
    assert np.array_equal(buf.cpu().numpy(), before)
