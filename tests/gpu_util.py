"""Helpers for the GPU parity tests: upload raw storage to device tensors,
download it back, and compare with the oracle to the stated tolerances."""
import numpy as np

TOL_NORM = 1e-5   # relative, GPU norm vs oracle norm (all formats)
TOL_F32 = 1e-5    # relative, clipped fp32 elements
TOL_ULP16 = 1     # ulps of the storage format, clipped fp16 / bf16 elements


def torch_dtype(dtype):
    import torch
    return {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def upload(arrays, dtype, device="cuda"):
    import torch
    out = []
    for a in arrays:
        if dtype == "f32":
            out.append(torch.from_numpy(np.ascontiguousarray(a)).to(device))
        else:
            out.append(torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch_dtype(dtype)))
    return out


def download(tensors, dtype):
    import torch
    if dtype == "f32":
        return [t.detach().cpu().numpy().copy() for t in tensors]
    return [t.detach().view(torch.int16).cpu().numpy().view(np.uint16).copy() for t in tensors]


def values(a, dtype):
    if dtype == "f32":
        return a.astype(np.float64)
    if dtype == "f16":
        return a.view(np.float16).astype(np.float64)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ordered16(b):
    b = b.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def elem_mismatches(gpu, ref, dtype):
    """Boolean mask of elements outside tolerance (NaN matches NaN)."""
    gv, rv = values(gpu, dtype), values(ref, dtype)
    gn, rn = np.isnan(gv), np.isnan(rv)
    if dtype == "f32":
        with np.errstate(invalid="ignore"):
            bad = ~(np.abs(gv - rv) <= TOL_F32 * np.abs(rv))
            bad &= ~((gv == rv) | (np.isinf(rv) & (gv == rv)))
    else:
        bad = np.abs(ordered16(gpu) - ordered16(ref)) > TOL_ULP16
    bad |= gn != rn
    bad &= ~(gn & rn)
    return bad


def _bits(a):
    return a.view(np.uint32 if a.itemsize == 4 else np.uint16)


def assert_elems_close(gpu_list, ref_list, dtype, what=""):
    """Every element of every tensor within tolerance.  Elements whose bits
    equal the oracle's pass at once; only the others go through the
    tolerance test, so lists of several GB compare in seconds."""
    nbad, first = 0, None
    for t, (g, r) in enumerate(zip(gpu_list, ref_list)):
        assert g.shape == r.shape
        g1, r1 = g.reshape(-1), r.reshape(-1)
        idx = np.flatnonzero(_bits(g1) != _bits(r1))
        if idx.size == 0:
            continue
        bad = elem_mismatches(g1[idx], r1[idx], dtype)
        k = int(bad.sum())
        if k and first is None:
            i = int(idx[np.argmax(bad)])
            first = (t, i, values(g1[i:i + 1], dtype)[0], values(r1[i:i + 1], dtype)[0])
        nbad += k
    assert nbad == 0, f"{what}: {nbad} elements outside tolerance, first (tensor, index, gpu, oracle) = {first}"


def assert_bitwise_equal(a_list, b_list, what=""):
    for t, (a, b) in enumerate(zip(a_list, b_list)):
        if a.tobytes() != b.tobytes():
            ua = a.view(np.uint32 if a.itemsize == 4 else np.uint16)
            ub = b.view(np.uint32 if b.itemsize == 4 else np.uint16)
            bad = np.flatnonzero(ua != ub)[:6]
            raise AssertionError(f"{what}: tensor {t} differs at {bad.size}+ places, first (index, got bits, "
                                 f"expected bits): {[(int(i), hex(int(ua[i])), hex(int(ub[i]))) for i in bad]}")


def assert_norm_close(gpu_norm, ref_norm, what=""):
    if np.isnan(ref_norm):
        assert np.isnan(gpu_norm), what
        return
    if np.isinf(ref_norm):
        assert gpu_norm == ref_norm, what
        return
    assert abs(gpu_norm - ref_norm) <= TOL_NORM * abs(ref_norm) + (0.0 if ref_norm else 0.0), \
        f"{what}: gpu norm {gpu_norm!r} vs oracle {ref_norm!r}"


def assert_bitwise_equal_but_nan(a_list, b_list, dtype, what=""):
    """Bit for bit, except that a NaN matches any NaN: IEEE 754 leaves the
    sign and payload of a NaN an operation returns to the implementation."""
    for t, (a, b) in enumerate(zip(a_list, b_list)):
        na, nb = np.isnan(values(a, dtype)), np.isnan(values(b, dtype))
        assert np.array_equal(na, nb), f"{what}: tensor {t}: NaN at different places"
        assert_bitwise_equal([a[~na]], [b[~nb]], f"{what} (tensor {t}, NaNs aside)")
