"""GPU parity of the optimizer step on the clipped gradient (gclip_norm, then
gclip_adamw_step), through the C ABI, against the oracle's clip followed by
AdamW in binary64.

Tolerances, from the kernel's binary32 arithmetic:
- moments: the GPU forms s * g, its square and two products and one sum in
  binary32, a few roundings of 2^-24 of the terms' magnitudes; the tests allow
  1e-6 of (b1 |m| + (1 - b1) |g|) for m and of (b2 v + (1 - b2) g^2) for v;
- weights: the result is rounded to binary32 next to the decay product
  (2^-22 of |p|), and the update u = mhat / (sqrt(vhat) + eps) carries the
  moments' errors through the division and the square root, plus its own
  roundings (1e-6 of |u|); both are bounded to first order, element by
  element, because the decay and the update can cancel.
The non-finite stop leaves weights and moments bitwise unchanged."""
import math

import numpy as np
import pytest

import oracle
from synth import gradsets as gs
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

HP = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("the gpu tests need an MI355X")
    import global_l2_norm_amd  # noqa: F401  (fails loudly when libgclip.so is missing)


def _G():
    import global_l2_norm_amd as G
    return G


def _to_dev(arrays):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda") for a in arrays]


def _from_dev(ts):
    return [t.detach().cpu().numpy().copy() for t in ts]


def gpu_clip_adamw(params, grads, m, v, dtype, max_norm, avg=1.0, err=False, step=1, hp=HP, dev=None):
    """Upload (or reuse device tensors), run norm + AdamW step, download."""
    G = _G()
    if dev is None:
        dev = (_to_dev(params), gu.upload(grads, dtype), _to_dev(m), _to_dev(v))
    tp, tg, tm, tv = dev
    gl = G.GradList(tg)
    opt = G.AdamWList(tp, tg, tm, tv)
    gl.norm(avg)
    opt.step(gl, step=step, max_norm=max_norm, avg_factor=avg, error_if_nonfinite=err, **hp)
    st, r = gl.read(err)
    out = (_from_dev(tp), _from_dev(tm), _from_dev(tv))
    g_after = gu.download(tg, dtype)
    opt.close()
    gl.close()
    return st, r, out, g_after


def assert_adamw_close(out, ref, old, grads, dtype, s, hp, step, what=""):
    """First-order error bounds of the binary32 update (see the header)."""
    (pg, mg, vg), (pr, mr, vr), (po, mo, vo) = out, ref, old
    b1, b2, lr, wd, eps = hp["beta1"], hp["beta2"], hp["lr"], hp["weight_decay"], hp["eps"]
    bc1, bc2 = 1 - b1 ** step, 1 - b2 ** step
    for k in range(len(pr)):
        g = s * gu.values(grads[k], dtype)
        p_old, m_old, v_old = (np.asarray(x, np.float64) for x in (po[k], mo[k], vo[k]))
        tol_m = 1e-6 * (b1 * np.abs(m_old) + (1 - b1) * np.abs(g)) + 1e-37
        tol_v = 1e-6 * (b2 * v_old + (1 - b2) * g * g) + 1e-37
        den = np.sqrt(vr[k] / bc2) + eps
        u = (mr[k] / bc1) / den
        # the update u = mhat / (sqrt(vhat) + eps): the moments' errors carried
        # through (|sqrt(a) - sqrt(b)| <= sqrt(|a - b|)), plus the roundings of
        # the square root, the division and the step constants
        tol_u = tol_m / (bc1 * den) + np.abs(u) * np.sqrt(tol_v / bc2) / den + 1e-6 * np.abs(u)
        tol_p = 2.0 ** -22 * np.abs(pr[k]) + lr * (2 * tol_u + 1e-6 * wd * np.abs(p_old)) + 1e-37
        for name, gpu, rf, tol in (("m", mg[k], mr[k], tol_m), ("v", vg[k], vr[k], tol_v),
                                   ("p", pg[k], pr[k], tol_p)):
            d = np.abs(gpu.astype(np.float64) - rf)
            bad = np.flatnonzero(~(d <= tol))
            assert bad.size == 0, (f"{what} tensor {k} {name}: {bad.size} of {d.size} off, first at {bad[0]}: "
                                   f"gpu {gpu[bad[0]]!r} ref {rf[bad[0]]!r} tol {tol[bad[0]]!r}")


def check_step(params, grads, m, v, dtype, max_norm, avg=1.0, err=False, step=1, hp=HP, what=""):
    st, r, out, g_after = gpu_clip_adamw(params, grads, m, v, dtype, max_norm, avg, err, step, hp)
    ro, ref = oracle.clip_adamw(params, grads, m, v, dtype, max_norm, avg, err, step=step, **hp)
    gu.assert_bitwise_equal(g_after, grads, what + " (gradients are only read)")
    assert r["nonfinite"] == ro["nonfinite"] and r["skipped"] == ro["skipped"], what
    if not math.isnan(ro["norm"]):
        gu.assert_norm_close(r["norm"], ro["norm"], what)
        assert r["clipped"] == ro["clipped"], what
    if ro["skipped"]:
        for a, b in zip(out, (params, m, v)):
            gu.assert_bitwise_equal(a, b, what + " (skipped: nothing written)")
    else:
        assert_adamw_close(out, ref, (params, m, v), grads, dtype, ro["scale"], hp, step, what)
    return r, ro, out


def _state(rng, sizes, warm=True):
    params = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in sizes]
    if not warm:
        z = [np.zeros(n, np.float32) for n in sizes]
        return params, z, [x.copy() for x in z]
    m = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for n in sizes]
    v = [(rng.random(n) * 1e-6).astype(np.float32) for n in sizes]
    return params, m, v


# ------------------------------------------------------------------ worked example and small lists
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_adamw_after_worked_example(dtype):
    """[6, 8] clipped at 5 is [3, 4]: the moments see (1 - b1) [3, 4]."""
    params = [np.array([1.0, -1.0], np.float32)]
    z = [np.zeros(2, np.float32)]
    grads = [gs.to_storage(np.array([6.0, 8.0]), dtype)]
    r, ro, (pg, mg, vg) = check_step(params, grads, z, [z[0].copy()], dtype, 5.0, what="[6,8]")
    assert r["clipped"] and r["scale"] == 0.5
    assert np.allclose(mg[0], (1 - HP["beta1"]) * np.array([3.0, 4.0]), rtol=1e-6)


@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_adamw_ragged_lists_several_steps(dtype, seed):
    """Ragged lists (pieces of every size, tensor tails of 1-3 elements),
    three steps with fresh gradients, the GPU's state fed back each step."""
    import torch
    rng = np.random.default_rng(400 + seed)
    sizes = [int(rng.choice([1, 2, 3, 5, 7, 63, 255, 257, 1000, 4099, 8191, 8192, 8193, 70_001, 300_003]))
             for _ in range(int(rng.integers(3, 20)))]
    params, m, v = _state(rng, sizes, warm=bool(seed % 2))
    tp, tm, tv = _to_dev(params), _to_dev(m), _to_dev(v)
    for step in range(1, 4):
        grads = [gs.to_storage(rng.standard_normal(n) * float(rng.choice([1e-3, 0.3, 5.0])), dtype) for n in sizes]
        tg = gu.upload(grads, dtype)
        old = (_from_dev(tp), _from_dev(tm), _from_dev(tv))
        st, r, out, _ = gpu_clip_adamw(None, None, None, None, dtype, 1.0, step=step, dev=(tp, tg, tm, tv))
        ro, ref = oracle.clip_adamw(old[0], grads, old[1], old[2], dtype, 1.0, step=step, **HP)
        assert r["clipped"] == ro["clipped"]
        assert_adamw_close(out, ref, old, grads, dtype, ro["scale"], HP, step, f"{dtype} seed {seed} step {step}")
        torch.cuda.synchronize()


def test_adamw_misaligned_views_take_the_element_path():
    """Views starting at odd elements (no 16-byte alignment) use the
    element-by-element path and must agree just the same."""
    import torch
    rng = np.random.default_rng(410)
    sizes = [1001, 77, 4099]
    params, m, v = _state(rng, sizes)
    grads = [gs.to_storage(rng.standard_normal(n) * 0.1, "bf16") for n in sizes]

    def views(arrays, dtype):
        outs = []
        for a in arrays:
            if dtype == "f32":
                base = torch.zeros(a.size + 3, dtype=torch.float32, device="cuda")
                base[1:1 + a.size] = torch.from_numpy(a).to("cuda")
            else:
                base = torch.zeros(a.size + 3, dtype=torch.bfloat16, device="cuda")
                base[1:1 + a.size] = torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
            outs.append(base[1:1 + a.size])
        return outs

    dev = (views(params, "f32"), views(grads, "bf16"), views(m, "f32"), views(v, "f32"))
    st, r, out, _ = gpu_clip_adamw(None, None, None, None, "bf16", 1.0, step=4, dev=dev)
    ro, ref = oracle.clip_adamw(params, grads, m, v, "bf16", 1.0, step=4, **HP)
    assert_adamw_close(out, ref, (params, m, v), grads, "bf16", ro["scale"], HP, 4, "misaligned views")


@pytest.mark.parametrize("err", [True, False])
def test_adamw_nonfinite(err):
    """A NaN with the stop switch leaves weights and moments bitwise as they
    were; without it, IEEE arithmetic decides (NaN norm: no clip)."""
    rng = np.random.default_rng(420)
    sizes = [5000, 33]
    params, m, v = _state(rng, sizes)
    grads = [gs.to_storage(rng.standard_normal(n) * 0.1, "f32") for n in sizes]
    grads[0][1234] = np.nan
    if err:
        check_step(params, grads, m, v, "f32", 1.0, err=True, step=2, what="NaN stop")
    else:
        st, r, out, _ = gpu_clip_adamw(params, grads, m, v, "f32", 1.0, err=False, step=2)
        assert r["nonfinite"] and not r["skipped"] and not r["clipped"]
        ro, ref = oracle.clip_adamw(params, grads, m, v, "f32", 1.0, step=2, **HP)
        # the NaN element turns NaN in both; every other element agrees
        for k in range(2):
            for gpu, rf in zip((out[0][k], out[1][k], out[2][k]), (ref[0][k], ref[1][k], ref[2][k])):
                assert np.array_equal(np.isnan(gpu), np.isnan(rf))


def test_adamw_with_averaging():
    """avg_factor a: the moments see a * coef * g."""
    rng = np.random.default_rng(430)
    sizes = [20000, 513]
    params, m, v = _state(rng, sizes)
    grads = [gs.to_storage(rng.standard_normal(n) * 0.02, "f32") for n in sizes]
    r, ro, _ = check_step(params, grads, m, v, "f32", 1.0, avg=0.25, step=7, what="avg 1/4")
    assert abs(r["scale"] - ro["scale"]) <= 1e-6 * ro["scale"]


def test_adamw_andrea120m():
    """The whole ANDREA-120M list (fp32 gradients), one step from zero moments."""
    g = gs.andrea120m_f32()
    rng = np.random.default_rng(440)
    sizes = [a.size for a in g.arrays]
    params = [(rng.standard_normal(n) * 0.02).astype(np.float32) for n in sizes]
    z = [np.zeros(n, np.float32) for n in sizes]
    r, ro, _ = check_step(params, g.arrays, z, [x.copy() for x in z], "f32", g.max_norm, step=1,
                          what="andrea120m")
    assert r["clipped"]


def test_adamw_bitwise_repeatable():
    rng = np.random.default_rng(450)
    sizes = [100_000, 77]
    params, m, v = _state(rng, sizes)
    grads = [gs.to_storage(rng.standard_normal(n) * 0.1, "f16") for n in sizes]
    outs = [gpu_clip_adamw(params, grads, m, v, "f16", 1.0, step=3)[2] for _ in range(2)]
    for a, b in zip(outs[0], outs[1]):
        gu.assert_bitwise_equal(a, b, "run to run")


def test_adamw_invalid_arguments():
    import torch
    G = _G()
    t = [torch.zeros(64, dtype=torch.float32, device="cuda") for _ in range(4)]
    with pytest.raises(G.GclipError):  # the weights are also the gradient: overlapping ranges
        G.AdamWList([t[0]], [t[0]], [t[2]], [t[3]])
    opt = G.AdamWList([t[0]], [t[1]], [t[2]], [t[3]])
    gl = G.GradList([t[1]])
    for bad in (dict(lr=-1.0), dict(beta1=1.0), dict(beta2=-0.1), dict(eps=0.0), dict(weight_decay=-1.0),
                dict(step=0)):
        kw = dict(HP, step=1)
        kw.update(bad)
        with pytest.raises(G.GclipError):
            opt.step(gl, max_norm=1.0, **kw)
    opt.close()
    gl.close()
