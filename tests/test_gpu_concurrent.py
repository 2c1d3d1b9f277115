"""Two fused launches at once, on two streams, on two lists; and two
per-tensor clips at once.

The fused kernel is an ordinary launch: it needs one workgroup per compute
unit resident to decide without waiting, and it gets that only when nothing
else runs.  With two such launches in flight they take compute units from
each other; a workgroup that waits longer than the list's bound at the
decision hands its block back and leaves, so both launches finish, and each
list must come out exactly as when it is clipped alone (the split path's
bits)."""
import numpy as np
import pytest

from synth import gradsets as gs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("the gpu tests need an MI355X")
    import global_l2_norm_amd  # noqa: F401  (fails loudly when libgclip.so is missing)


def _G():
    import global_l2_norm_amd as G
    return G


def _alone(arrays, dtype, max_norm):
    G = _G()
    ts = gu.upload(arrays, dtype)
    gl = G.GradList(ts)
    gl.set_path(G.GCLIP_PATH_SPLIT)
    gl.clip_(max_norm)
    st, r = gl.read()
    out = gu.download(ts, dtype)
    gl.close()
    return r, out


@pytest.mark.parametrize("wait_us", (0, 200, 1000))
def test_two_fused_launches_at_once(wait_us):
    import torch
    G = _G()
    rng = np.random.default_rng(4300)
    a = [gs.to_storage(rng.standard_normal(n) * 1e-3, "f32") for n in (40_000_003, 9_000_001, 5)]
    b = [gs.to_storage(rng.standard_normal(n) * 1e-3, "bf16") for n in (50_000_001, 30_000_000, 77)]
    ra, out_a = _alone(a, "f32", 1.0)
    rb, out_b = _alone(b, "bf16", 1.0)
    ta, tb = gu.upload(a, "f32"), gu.upload(b, "bf16")
    pa, pb = [t.clone() for t in ta], [t.clone() for t in tb]
    la, lb = G.GradList(ta), G.GradList(tb)
    for gl in (la, lb):
        gl.set_path(G.GCLIP_PATH_FUSED)
        gl.set_wait(wait_us)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    handed = 0
    for rep in range(3):
        for t, p in zip(ta + tb, pa + pb):
            t.copy_(p)
        torch.cuda.synchronize()
        la.clip_(1.0, stream=s1)
        lb.clip_(1.0, stream=s2)
        st1, r1 = la.read(stream=s1)
        st2, r2 = lb.read(stream=s2)
        assert st1 == 0 and st2 == 0 and r1["status"] == 0 and r2["status"] == 0, (rep, r1, r2)
        handed += r1["handed_back"] + r2["handed_back"]
        assert r1["sumsq"] == ra["sumsq"] and r1["scale"] == ra["scale"], rep
        assert r2["sumsq"] == rb["sumsq"] and r2["scale"] == rb["scale"], rep
        gu.assert_bitwise_equal(gu.download(ta, "f32"), out_a, f"list a, repeat {rep}")
        gu.assert_bitwise_equal(gu.download(tb, "bf16"), out_b, f"list b, repeat {rep}")
    print(f"wait {wait_us} us: {handed} blocks handed back over 3 repeats")
    la.close()
    lb.close()


def _set_path(gl, path):
    G = _G()
    gl.set_path(G.GCLIP_PATH_FUSED if path == "fused" else G.GCLIP_PATH_SPLIT)


def _per_tensor_alone(arrays, dtype, max_norm, path):
    G = _G()
    ts = gu.upload(arrays, dtype)
    gl = G.GradList(ts)
    _set_path(gl, path)
    gl.clip_per_tensor_(max_norm)
    st, r = gl.read()
    tr = gl.read_tensors()
    out = gu.download(ts, dtype)
    gl.close()
    return r, tr, out


@pytest.mark.parametrize("path", ("fused", "split"))
def test_two_per_tensor_clips_at_once(path):
    """Two per-tensor clips at once on two streams, each taking compute units
    from the other: in one launch every workgroup waits for the decisions
    (and hands its pieces back when it waits too long); in two kernels the
    second kernel's workgroup 0 waits for every tensor's sum.  Both lists
    must come out exactly as when clipped alone."""
    import torch
    G = _G()
    rng = np.random.default_rng(4400)
    a = [gs.to_storage(rng.standard_normal(n) * 1e-3, "f32") for n in (30_000_003, 1, 5_000_001) + (77,) * 500]
    b = [gs.to_storage(rng.standard_normal(n) * 1e-3, "bf16") for n in (40_000_001, 3) + (1,) * 800 + (20_000_000,)]
    ra, tra, out_a = _per_tensor_alone(a, "f32", 1.0, path)
    rb, trb, out_b = _per_tensor_alone(b, "bf16", 1.0, path)
    ta, tb = gu.upload(a, "f32"), gu.upload(b, "bf16")
    pa, pb = [t.clone() for t in ta], [t.clone() for t in tb]
    la, lb = G.GradList(ta), G.GradList(tb)
    _set_path(la, path)
    _set_path(lb, path)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for rep in range(3):
        for t, p in zip(ta + tb, pa + pb):
            t.copy_(p)
        torch.cuda.synchronize()
        la.clip_per_tensor_(1.0, stream=s1)
        lb.clip_per_tensor_(1.0, stream=s2)
        st1, r1 = la.read(stream=s1)
        st2, r2 = lb.read(stream=s2)
        assert st1 == 0 and st2 == 0 and r1["status"] == 0 and r2["status"] == 0, (rep, r1, r2)
        assert r1["sumsq"] == ra["sumsq"] and r2["sumsq"] == rb["sumsq"], rep
        assert la.read_tensors().tobytes() == tra.tobytes() and lb.read_tensors().tobytes() == trb.tobytes(), rep
        gu.assert_bitwise_equal(gu.download(ta, "f32"), out_a, f"list a, repeat {rep}")
        gu.assert_bitwise_equal(gu.download(tb, "bf16"), out_b, f"list b, repeat {rep}")
    la.close()
    lb.close()
