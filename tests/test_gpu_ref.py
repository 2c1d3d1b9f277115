"""The attainable-bandwidth reference kernels (include/gclip_ref.h) on the
GPU: the copy moves every byte (to another buffer, and in place, where it
must leave the bytes as they were) and the read leaves its sink alone."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("the gpu tests need an MI355X")
    import global_l2_norm_amd  # noqa: F401  (fails loudly when libgclip.so is missing)


@pytest.mark.parametrize("nbytes", [16, 32 * 1024 + 48, 50_000_016])
def test_copy_and_in_place(nbytes):
    import torch
    from global_l2_norm_amd import _lib
    n = nbytes // 4
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (n + 8,), dtype=torch.int32, device="cuda")
    dst = torch.zeros(n + 8, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    assert _lib.lib.gclip_ref_copy(dst.data_ptr(), src.data_ptr(), nbytes, stream) == _lib.GCLIP_OK
    before = src.clone()
    assert _lib.lib.gclip_ref_copy(src.data_ptr(), src.data_ptr(), nbytes, stream) == _lib.GCLIP_OK
    sink = torch.full((4,), 7, dtype=torch.int32, device="cuda")
    assert _lib.lib.gclip_ref_read(src.data_ptr(), nbytes, sink.data_ptr(), stream) == _lib.GCLIP_OK
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src[:n]) and bool((dst[n:] == 0).all())
    assert torch.equal(src, before)
    assert bool((sink == 7).all())
