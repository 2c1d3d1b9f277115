"""Pins for the CPU oracle: checks against what the pages and the mathematics
fix, none of which retypes the oracle's own formula.

Every pin takes an ``oracle.Oracle`` handle so the same pins can be run
against deliberately broken builds of the oracle (tests/test_oracle_mutants.py).
Values are decoded here with numpy / torch / struct, never with the oracle's
own decoder.
"""
import json
import math
import os
import struct
from fractions import Fraction

import numpy as np

from synth import gradsets as gs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
DTYPES = ("f32", "f16", "bf16")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- decoding helpers (library routines)
def values(a: np.ndarray, dtype: str) -> np.ndarray:
    """binary64 values of raw storage, through numpy's own conversions."""
    if dtype == "f32":
        return a.astype(np.float64)
    if dtype == "f16":
        return a.view(np.float16).astype(np.float64)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def struct_value(bits: int, dtype: str) -> float:
    """One value through Python's struct module (IEEE binary16/binary32)."""
    if dtype == "f32":
        return struct.unpack("<f", struct.pack("<I", int(bits)))[0]
    if dtype == "f16":
        return struct.unpack("<e", struct.pack("<H", int(bits)))[0]
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def raw_bits(a: np.ndarray, dtype: str) -> np.ndarray:
    return a.view(np.uint32) if dtype == "f32" else a.view(np.uint16)


def ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the storage format at |v| (upper neighbour)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    if dtype == "f32":
        return np.spacing(v.astype(np.float32)).astype(np.float64)
    if dtype == "f16":
        return np.spacing(v.astype(np.float16)).astype(np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    e = np.maximum(e, -126.0)
    return np.exp2(e - 7.0)


def lib_round(x64: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage of x64 rounded to nearest-even by numpy (f32, f16)."""
    if dtype == "f32":
        return np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f16":
        return np.asarray(x64, dtype=np.float64).astype(np.float16).view(np.uint16)
    raise ValueError("numpy has no bfloat16")


def store(vals, dtype):
    return gs.to_storage(np.asarray(vals, dtype=np.float64), dtype)


# ---------------------------------------------------------------- the pins
def pin_worked_6_8(o):
    """[6, 8] with threshold 5 has norm 10 and becomes [3, 4] (glossary page,
    'Shorten the arrow, keep the direction'); exact in every storage format."""
    gd = golden("worked_6_8.json")
    for dt in DTYPES:
        arrs = [store(gd["g"], dt)]
        r = o.clip_(arrs, dt, gd["max_norm"])
        assert r["norm"] == gd["norm"], (dt, r)
        assert r["clipped"] and not r["nonfinite"] and not r["skipped"], (dt, r)
        assert r["scale"] == gd["max_norm"] / gd["norm"], (dt, r)
        assert list(values(arrs[0], dt)) == gd["clipped"], (dt, values(arrs[0], dt))


def pin_not_per_coordinate(o):
    """Norm clipping keeps the direction; clipping each coordinate to [-5, 5]
    would give [5, 5] with norm about 7.07 (glossary page)."""
    gd = golden("worked_6_8.json")
    a = [store(gd["g"], "f32")]
    o.clip_(a, "f32", gd["max_norm"])
    out = values(a[0], "f32")
    per_coord = np.clip(np.array(gd["g"]), -gd["max_norm"], gd["max_norm"])
    assert list(per_coord) == gd["per_coordinate_clipped"]
    assert abs(np.linalg.norm(per_coord) - gd["per_coordinate_norm_approx"]) < 5e-3
    assert not np.array_equal(out, per_coord)
    assert np.linalg.norm(out) == gd["max_norm"]
    # same direction: out is a positive multiple of g
    g = np.array(gd["g"])
    assert abs(out[0] * g[1] - out[1] * g[0]) == 0.0 and out[0] / g[0] > 0


def pin_sgd_step_length(o):
    """Plain SGD with lr 0.1: the clipped step has length 0.5 instead of 1."""
    gd = golden("worked_6_8.json")
    a = [store(gd["g"], "f32")]
    o.clip_(a, "f32", gd["max_norm"])
    lr = gd["sgd_lr"]
    assert abs(np.linalg.norm(-lr * values(a[0], "f32")) - gd["sgd_step_length_clipped"]) < 1e-12
    assert abs(np.linalg.norm(-lr * np.array(gd["g"])) - gd["sgd_step_length_unclipped"]) < 1e-12


def pin_accumulate_then_clip(o):
    """10 and -9 add up to 1, which a clip at 5 keeps; clipping each first gives
    5 and -5, summing to 0 (glossary page, 'Order changes the result').  On a
    one-element list norm clipping and value clipping coincide."""
    gd = golden("accumulate_then_clip.json")
    c = gd["max_norm"]
    clipped_each = []
    for v in gd["contributions"]:
        a = [store([v], "f32")]
        o.clip_(a, "f32", c)
        clipped_each.append(float(values(a[0], "f32")[0]))
    assert clipped_each == gd["clipped_contributions"]
    assert sum(clipped_each) == gd["sum_of_clipped"]
    acc = np.float32(gd["contributions"][0]) + np.float32(gd["contributions"][1])
    a = [np.array([acc], dtype=np.float32)]
    r = o.clip_(a, "f32", c)
    assert float(a[0][0]) == gd["clip_of_sum"] and not r["clipped"] and r["norm"] == gd["sum"]


def pin_tie_passes_unchanged(o):
    """norm == max_norm passes unchanged (grad-clip lesson 'Math': '<=' passes;
    glossary page uses '<=' too); just below the norm it clips."""
    for dt in DTYPES:
        a = [store([3.0, 4.0], dt)]
        before = a[0].copy()
        r = o.clip_(a, dt, 5.0)
        assert not r["clipped"] and r["scale"] == 1.0, (dt, r)
        assert np.array_equal(raw_bits(a[0], dt), raw_bits(before, dt))
    a = [store([3.0, 4.0], "f32")]
    r = o.clip_(a, "f32", 5.0 * (1 - 2.0 ** -30))
    assert r["clipped"] and r["scale"] < 1.0


def pin_below_threshold_bitwise(o):
    """norm <= max_norm: every byte of every tensor is left as it was."""
    rng = np.random.default_rng(11)
    for dt in DTYPES:
        for _ in range(5):
            g = gs.random_list(rng, dt, max_tensors=5, max_numel=40)
            norm = math.sqrt(sum(float(np.sum(values(x, dt) ** 2)) for x in g.arrays))
            before = [x.copy() for x in g.arrays]
            r = o.clip_(g.arrays, dt, max(2.0 * norm, 1e-30))
            assert not r["clipped"]
            for x, y in zip(g.arrays, before):
                assert np.array_equal(raw_bits(x, dt), raw_bits(y, dt))


def pin_post_clip_norm(o):
    """After a clip the global norm is max_norm (grad-clip lesson 'Math'), up
    to the rounding of each stored output: |‖out‖ - c| <= sqrt(sum ulp(out)^2)."""
    rng = np.random.default_rng(12)
    for dt in DTYPES:
        for c in (1.0, 0.37, 5.0):
            g = gs.random_list(rng, dt, max_tensors=6, max_numel=50, sigma=3.0)
            if not g.arrays or sum(x.size for x in g.arrays) == 0:
                continue
            r = o.clip_(g.arrays, dt, c)
            if not r["clipped"]:
                continue
            outv = np.concatenate([values(x, dt) for x in g.arrays])
            bound = math.sqrt(float(np.sum(ulp(outv, dt) ** 2))) + 1e-14 * c
            assert abs(np.linalg.norm(outv) - c) <= bound, (dt, c, np.linalg.norm(outv), bound)


def pin_single_global_factor(o):
    """One factor for every element of every tensor (grad-clip lesson, 'Two
    variants'): each output is g*s rounded once to nearest-even (numpy's
    rounding for f32/f16; a half-ulp bound for bf16)."""
    rng = np.random.default_rng(13)
    for dt in DTYPES:
        g = gs.random_list(rng, dt, max_tensors=6, max_numel=50, sigma=2.0)
        g.arrays.append(store(rng.standard_normal(64) * 4.0, dt))
        inp = [values(x, dt) for x in g.arrays]
        r = o.clip_(g.arrays, dt, 0.5)
        assert r["clipped"]
        s = r["scale"]
        for x, v in zip(g.arrays, inp):
            if dt in ("f32", "f16"):
                assert np.array_equal(raw_bits(x, dt), raw_bits(lib_round(v * s, dt), dt)), dt
            else:
                out = values(x, dt)
                assert np.all(np.abs(out - v * s) <= 0.5 * ulp(v * s, dt) * 1.0000001), dt


def pin_joint_norm_library(o):
    """The norm covers all tensors jointly (glossary page on clip_grad_norm_):
    sumsq == sum over tensors of numpy.linalg.norm(t)^2, and per-tensor sums
    match numpy tensor by tensor."""
    rng = np.random.default_rng(14)
    for dt in DTYPES:
        arrs = [store(rng.standard_normal(n) * sd, dt) for n, sd in ((1000, 1.0), (37, 0.01), (1, 5.0), (513, 2.0))]
        s, nf = o.sumsq(arrs, dt)
        ref = sum(np.linalg.norm(values(x, dt)) ** 2 for x in arrs)
        assert not nf and abs(s - ref) <= 1e-12 * ref, (dt, s, ref)
        per = o.tensor_sumsq(arrs, dt)
        for p, x in zip(per, arrs):
            q = np.linalg.norm(values(x, dt)) ** 2
            assert abs(p - q) <= 1e-12 * q
        # a single tensor reduces to the library 2-norm
        r = o.clip_([arrs[0].copy()], dt, 1e9)
        assert abs(r["norm"] - np.linalg.norm(values(arrs[0], dt))) <= 1e-13 * r["norm"]


def pin_bruteforce_exact(o):
    """Tiny random lists: math.fsum of the exact squares (values decoded by
    struct) is the correctly rounded sum; Fraction decides S > c^2 exactly."""
    rng = np.random.default_rng(15)
    for dt in DTYPES:
        for trial in range(30):
            sigma = [1.0, 1e-3, 1e-6, 300.0][trial % 4] if dt != "f16" else [1.0, 1e-3, 1e-6, 30.0][trial % 4]
            g = gs.random_list(rng, dt, max_tensors=5, max_numel=50, sigma=sigma)
            a = [0.25, 1.0, 1.0 / 3.0][trial % 3]
            vals = [struct_value(b, dt) for x in g.arrays for b in raw_bits(x, dt)]
            exact = sum((Fraction(a) * Fraction(v)) ** 2 for v in vals) if vals else Fraction(0)
            s, nf = o.sumsq(g.arrays, dt, a)
            assert not nf
            n = max(len(vals), 1)
            assert abs(Fraction(s) - exact) <= Fraction(n + 2) * Fraction(2.0 ** -52) * exact, (dt, s, float(exact))
            fs = math.fsum((a * v) ** 2 for v in vals) if a != 1.0 / 3.0 else None
            if fs is not None:
                assert abs(s - fs) <= n * 2.0 ** -53 * fs
            # exact decision; skip near-ties the rounding of S could flip
            for c in (0.5, 1.0, 3.0, 40.0):
                c2 = Fraction(c) ** 2
                if exact != 0 and abs(exact - c2) <= Fraction(1, 10 ** 9) * c2:
                    continue
                arrs = [x.copy() for x in g.arrays]
                r = o.clip_(arrs, dt, c, a)
                assert r["clipped"] == (exact > c2), (dt, c, float(exact))


def pin_decode_library(o):
    """Every fp16 and bf16 bit pattern, and many fp32 ones, decode to the same
    value as numpy's / torch's conversion (NaN to NaN)."""
    import torch
    allbits = np.arange(65536, dtype=np.uint32)
    ref16 = allbits.astype(np.uint16).view(np.float16).astype(np.float64)
    refbf = torch.from_numpy(allbits.astype(np.uint16).view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    rng = np.random.default_rng(16)
    f32bits = np.concatenate([rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32),
                              np.array([0, 1, 0x7F800000, 0xFF800000, 0x7FC00000, 0x80000001, 0x00800000, 0x7F7FFFFF],
                                       dtype=np.uint32)])
    with np.errstate(invalid="ignore"):
        ref32 = f32bits.view(np.float32).astype(np.float64)
    for dt, bits, ref in (("f16", allbits, ref16), ("bf16", allbits, refbf), ("f32", f32bits, ref32)):
        got = np.array([o.decode_bits(int(b), dt) for b in bits])
        same = (got == ref) | (np.isnan(got) & np.isnan(ref))
        assert np.all(same), (dt, bits[~same][:5])
        sign_ok = np.signbit(got[ref == 0]) == np.signbit(ref[ref == 0])
        assert np.all(sign_ok), dt


def _encode_cases(rng, dt):
    emin, mb, emax = {"f32": (-126, 23, 127), "f16": (-14, 10, 15), "bf16": (-126, 7, 127)}[dt]
    xs = list(rng.standard_normal(3000) * np.exp2(rng.integers(emin - mb - 2, emax + 2, 3000)))
    # exact midpoints between neighbours (ties) and values just off them
    for _ in range(1500):
        e = int(rng.integers(emin - 1, emax))
        m = int(rng.integers(0, 2 ** mb))
        q = max(e, emin) - mb
        mid = (2 ** mb + m + 0.5) * 2.0 ** q if e >= emin else (m + 0.5) * 2.0 ** q
        xs += [mid, -mid, math.nextafter(mid, 0), math.nextafter(mid, math.inf)]
    top = (2.0 - 2.0 ** -mb) * 2.0 ** emax
    xs += [top, top * (1 + 2.0 ** -(mb + 2)), top * (1 + 2.0 ** -(mb + 1)), 2.0 ** (emin - mb - 1),
           2.0 ** (emin - mb - 1) * 1.5, 2.0 ** (emin - mb), 0.0, -0.0, math.inf, -math.inf, 1e300, -1e-300]
    return np.array(xs, dtype=np.float64)


def pin_encode_library(o):
    """Round-to-nearest-even into each format agrees with numpy (binary64 to
    float32 / float16) and with torch (float32 to bfloat16), including ties,
    subnormals, overflow, signed zero, infinities and NaN."""
    import torch
    rng = np.random.default_rng(17)
    for dt in ("f32", "f16"):
        xs = _encode_cases(rng, dt)
        with np.errstate(over="ignore"):
            ref = raw_bits(lib_round(xs, dt), dt).astype(np.int64)
        got = np.array([o.encode(float(x), dt) for x in xs], dtype=np.int64)
        assert np.array_equal(got, ref), (dt, xs[got != ref][:5], got[got != ref][:5], ref[got != ref][:5])
    with np.errstate(over="ignore"):
        xs = _encode_cases(rng, "bf16").astype(np.float32)  # float32 inputs: torch rounds float32 -> bf16 once
    xs = xs[np.isfinite(xs) | np.isinf(xs)]
    ref = torch.from_numpy(xs).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).astype(np.int64)
    got = np.array([o.encode(float(x), "bf16") for x in xs], dtype=np.int64)
    assert np.array_equal(got, ref), (xs[got != ref][:5], got[got != ref][:5], ref[got != ref][:5])
    for dt in DTYPES:
        nan_bits = o.encode(float("nan"), dt)
        assert math.isnan(struct_value(nan_bits, dt))


def pin_nonfinite(o):
    """A NaN or +-Inf anywhere sets the flag; with error_if_nonfinite the
    update is stopped (glossary page: nothing is written); without it plain
    IEEE arithmetic decides: NaN > c is false (nothing clipped), an infinite
    norm gives the factor c/Inf = 0."""
    rng = np.random.default_rng(18)
    for dt in DTYPES:
        for where in ("first", "middle", "last"):
            for bad in (math.nan, math.inf, -math.inf):
                arrs = [store(rng.standard_normal(5), dt), store(rng.standard_normal(7), dt)]
                t, i = {"first": (0, 0), "middle": (1, 3), "last": (1, 6)}[where]
                arrs[t][i] = store([bad], dt)[0]
                before = [x.copy() for x in arrs]
                r = o.clip_(arrs, dt, 1.0, 1.0, True)
                assert r["nonfinite"] and r["skipped"], (dt, where, bad, r)
                for x, y in zip(arrs, before):
                    assert np.array_equal(raw_bits(x, dt), raw_bits(y, dt))
                arrs = [y.copy() for y in before]
                r = o.clip_(arrs, dt, 1.0, 1.0, False)
                assert r["nonfinite"] and not r["skipped"]
                if math.isnan(bad):
                    assert math.isnan(r["norm"]) and not r["clipped"] and r["scale"] == 1.0
                    for x, y in zip(arrs, before):
                        assert np.array_equal(raw_bits(x, dt), raw_bits(y, dt))
                else:
                    assert r["norm"] == math.inf and r["clipped"] and r["scale"] == 0.0
                    for x, y in zip(arrs, before):
                        vx, vy = values(x, dt), values(y, dt)
                        fin = np.isfinite(vy)
                        assert np.all(vx[fin] == 0.0) and np.array_equal(np.signbit(vx[fin]), np.signbit(vy[fin]))
                        assert np.all(np.isnan(vx[~fin]))
    # all finite: flag clear
    r = o.clip_([store([1e30, -1e30], "f32")], "f32", 1.0)
    assert not r["nonfinite"]


def pin_avg_factor(o):
    """Averaging by 1/n_microbatches precedes the norm (backprop lesson,
    'Accumulation across microbatches'; glossary page, 'Order changes the
    result'): the norm of a*g is a times the norm of g, and with a = 1/4 the
    fused factor equals averaging first, then clipping, bit for bit."""
    rng = np.random.default_rng(19)
    for dt in DTYPES:
        arrs = [store(rng.standard_normal(n) * 0.3, dt) for n in (100, 7, 33)]
        s1, _ = o.sumsq(arrs, dt, 1.0)
        s4, _ = o.sumsq(arrs, dt, 0.25)
        assert s4 == s1 / 16.0
        s3, _ = o.sumsq(arrs, dt, 1.0 / 3.0)
        assert abs(s3 - s1 / 9.0) <= 1e-14 * s1
        fused = [x.copy() for x in arrs]
        r = o.clip_(fused, dt, 0.5, 0.25)
        assert r["clipped"] and abs(r["norm"] - math.sqrt(s1) / 4.0) <= 1e-15 * r["norm"]
        twostep = [x.copy() for x in arrs]
        o.scale_(twostep, dt, 0.25)
        r2 = o.clip_(twostep, dt, 0.5, 1.0)
        for x, y in zip(fused, twostep):
            assert np.array_equal(raw_bits(x, dt), raw_bits(y, dt)), dt
        # averaging without a clip still writes a*g
        arrs2 = [x.copy() for x in arrs]
        r3 = o.clip_(arrs2, dt, 1e6, 0.25)
        assert not r3["clipped"] and r3["scale"] == 0.25
        for x, y in zip(arrs2, arrs):
            assert np.array_equal(values(x, dt), values(y, dt) * 0.25)


def pin_scale_invariance(o):
    """norm(2^k g) == 2^k norm(g) exactly (power-of-two scaling is exact away
    from overflow and underflow)."""
    rng = np.random.default_rng(20)
    for dt in DTYPES:
        v = rng.standard_normal(300)
        base = [store(v, dt)]
        s0, _ = o.sumsq(base, dt)
        for k in (-3, 2, 5):
            sk, _ = o.sumsq([store(values(base[0], dt) * 2.0 ** k, dt)], dt)
            assert sk == s0 * 4.0 ** k, (dt, k)


def pin_empty_and_zero_size(o):
    """An empty list has norm 0 and writes nothing; zero-size tensors add nothing."""
    r = o.clip_([], "f32", 1.0)
    assert r["norm"] == 0.0 and not r["clipped"] and not r["nonfinite"]
    rng = np.random.default_rng(21)
    for dt in DTYPES:
        a = store(rng.standard_normal(40) * 2, dt)
        z = store([], dt)
        r1 = o.clip_([a.copy()], dt, 1.0)
        arrs = [z.copy(), a.copy(), z.copy()]
        r2 = o.clip_(arrs, dt, 1.0)
        assert r1["sumsq"] == r2["sumsq"] and r1["scale"] == r2["scale"]


def pin_infinite_threshold(o):
    """max_norm = +inf never clips."""
    a = [store([1e30, 3.0], "f32")]
    r = o.clip_(a, "f32", math.inf)
    assert not r["clipped"] and r["scale"] == 1.0


# ------------------------------------------------------------------ AdamW after the clip
# Grad clip lesson, "Order matters: Pre-Adam": AdamW's moments see the
# clipped gradient.  The update is AdamW as published (decoupled weight decay,
# bias-corrected moments); these pins fix it against closed forms of the
# algorithm and against torch.optim.AdamW run in float64 on the CPU.
HP = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def _f32(x):
    return np.asarray(x, dtype=np.float32)


def pin_adamw_first_step(o):
    """From zero moments, step 1: m' = (1 - b1) g, v' = (1 - b2) g^2, the
    bias-corrected moments are g and g^2, so the step is g / (|g| + eps)."""
    rng = np.random.default_rng(30)
    for dt in DTYPES:
        g = store(rng.standard_normal(50) * 0.1, dt)
        gv = values(g, dt)
        p = _f32(rng.standard_normal(50))
        z = np.zeros(50, np.float32)
        s = 0.75
        pn, mn, vn = o.adamw(p, g, z, z, dt, s, step=1, **HP)
        gs = s * gv
        assert np.allclose(mn, (1 - HP["beta1"]) * gs, rtol=1e-15, atol=0)
        assert np.allclose(vn, (1 - HP["beta2"]) * gs * gs, rtol=1e-15, atol=0)
        p64 = p.astype(np.float64)
        want = p64 - HP["lr"] * (gs / (np.abs(gs) + HP["eps"]) + HP["weight_decay"] * p64)
        assert np.allclose(pn, want, rtol=1e-14, atol=1e-18)


def pin_adamw_decay_only(o):
    """A zero gradient on zero moments leaves only the decoupled decay:
    p' = p (1 - lr wd)."""
    p = _f32(np.linspace(-2, 2, 9))
    z = np.zeros(9, np.float32)
    pn, mn, vn = o.adamw(p, z, z, z, "f32", 1.0, step=3, **HP)
    assert np.all(mn == 0) and np.all(vn == 0)
    assert np.allclose(pn, p.astype(np.float64) * (1 - HP["lr"] * HP["weight_decay"]), rtol=1e-15, atol=0)


def pin_adamw_constant_gradient(o):
    """With the same gradient every step from zero moments, m_t = (1 - b1^t) g
    and v_t = (1 - b2^t) g^2 (a geometric sum), so the bias-corrected moments
    are exactly g and g^2 at every step."""
    g = _f32([0.5, -0.25, 2.0, -3.0])
    p = _f32([1.0, 1.0, -1.0, 0.5])
    m = np.zeros(4, np.float32)
    v = np.zeros(4, np.float32)
    b1, b2 = HP["beta1"], HP["beta2"]
    for t in range(1, 7):
        pn, mn, vn = o.adamw(p, g, m, v, "f32", 1.0, step=t, **HP)
        assert np.allclose(mn, (1 - b1 ** t) * g.astype(np.float64), rtol=1e-6)
        assert np.allclose(vn, (1 - b2 ** t) * g.astype(np.float64) ** 2, rtol=1e-6)
        g64 = g.astype(np.float64)
        step = g64 / (np.abs(g64) + HP["eps"])
        assert np.allclose(pn, p.astype(np.float64) * (1 - HP["lr"] * HP["weight_decay"]) - HP["lr"] * step,
                           rtol=1e-9)
        p, m, v = _f32(pn), _f32(mn), _f32(vn)


def pin_adamw_matches_torch(o):
    """Several steps with changing gradients against torch.optim.AdamW in
    float64 (same binary32 state fed to both at every step)."""
    import torch
    rng = np.random.default_rng(31)
    n = 64
    p = _f32(rng.standard_normal(n))
    m = np.zeros(n, np.float32)
    v = np.zeros(n, np.float32)
    hp = dict(lr=3e-4, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    for t in range(1, 6):
        g = store(rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 0), "f32")
        s = float(rng.uniform(0.2, 1.0))
        pn, mn, vn = o.adamw(p, g, m, v, "f32", s, step=t, **hp)
        tp = torch.nn.Parameter(torch.from_numpy(p.astype(np.float64)))
        opt = torch.optim.AdamW([tp], lr=hp["lr"], betas=(hp["beta1"], hp["beta2"]), eps=hp["eps"],
                                weight_decay=hp["weight_decay"], foreach=False)
        tp.grad = torch.from_numpy(g.astype(np.float64) * s)
        opt.state[tp] = {"step": torch.tensor(float(t - 1)), "exp_avg": torch.from_numpy(m.astype(np.float64)),
                         "exp_avg_sq": torch.from_numpy(v.astype(np.float64))}
        opt.step()
        st = opt.state[tp]
        assert np.allclose(pn, tp.detach().numpy(), rtol=1e-12, atol=1e-15), t
        assert np.allclose(mn, st["exp_avg"].numpy(), rtol=1e-12, atol=1e-18), t
        assert np.allclose(vn, st["exp_avg_sq"].numpy(), rtol=1e-12, atol=1e-20), t
        p, m, v = _f32(pn), _f32(mn), _f32(vn)


def pin_adamw_after_clip(o):
    """The moments see the clipped gradient: [6, 8] clipped at 5 gives
    [3, 4] (glossary page worked example), so m' = (1 - b1) [3, 4]; with a
    NaN and the stop switch on nothing changes at all."""
    p = _f32([1.0, -1.0])
    z = np.zeros(2, np.float32)
    res, (pn, mn, vn) = o.clip_adamw([p], [_f32([6.0, 8.0])], [z], [z], "f32", 5.0, step=1, **HP)
    assert res["clipped"] and res["scale"] == 0.5
    assert np.array_equal(mn[0], (1 - HP["beta1"]) * np.array([3.0, 4.0]))
    res, (pn, mn, vn) = o.clip_adamw([p], [_f32([np.nan, 8.0])], [z], [z], "f32", 5.0, 1.0, True, step=1, **HP)
    assert res["skipped"] and np.array_equal(pn[0], p) and np.all(mn[0] == 0) and np.all(vn[0] == 0)


# ------------------------------------------------------------------ loss scaling (AMP)
def pin_amp_unscale_before_clip(o):
    """Glossary page, "Order changes the result": with loss scaling, unscale
    first so that the threshold applies to the true gradient.  [6, 8] scaled
    by S = 1024 and clipped at 5 must come out as [3, 4] (unscaled); clipping
    the scaled gradient first and unscaling after would give [3, 4] / 1024."""
    for dt in DTYPES:
        a = [store([6.0 * 1024, 8.0 * 1024], dt)]
        r = o.clip_amp_(a, dt, 5.0, 1.0, 1024.0)
        assert r["norm"] == 10.0 and r["clipped"] and not r["found_inf"]
        assert np.array_equal(values(a[0], dt), [3.0, 4.0]), (dt, values(a[0], dt))
    # with n microbatches the factor is 1 / (n S)
    assert o.amp_avg(4.0, 65536.0) == 1.0 / (4.0 * 65536.0)
    assert o.amp_avg(3.0, 1000.0) == 1.0 / 3000.0


def pin_amp_found_inf_writes_nothing(o):
    """A NaN or Inf in the scaled gradients is found-inf: nothing is written
    and the scale backs off."""
    for bad in (math.nan, math.inf):
        a = [store([1.0, bad, 3.0], "f16")]
        before = raw_bits(a[0], "f16").copy()
        r = o.clip_amp_(a, "f16", 1.0, 2.0, 256.0, tracker=5, growth=2.0, backoff=0.5, interval=10)
        assert r["found_inf"] and r["skipped"] and r["loss_scale"] == 128.0 and r["growth_tracker"] == 0
        assert np.array_equal(raw_bits(a[0], "f16"), before)


def pin_amp_update_closed_form(o):
    """Clean steps grow the scale by growth every interval steps; a found-inf
    step backs it off and restarts the count; a growth that would overflow
    binary32 is not taken."""
    sc, tr = 1024.0, 0
    for k in range(1, 11):
        sc, tr = o.amp_update(sc, tr, False, 2.0, 0.5, 4)
        assert sc == 1024.0 * 2.0 ** (k // 4) and tr == k % 4, (k, sc, tr)
    sc, tr = o.amp_update(sc, tr, True, 2.0, 0.5, 4)
    assert sc == 2048.0 and tr == 0
    big = float(np.float32(1.5 * 2.0 ** 127))
    sc, tr = o.amp_update(big, 0, False, 2.0, 0.5, 1)
    assert sc == big and tr == 0


def pin_amp_update_matches_torch(o):
    """Against torch's own loss-scale update, bit for bit, over a random
    sequence of clean and found-inf steps and non-power-of-two factors."""
    import torch
    rng = np.random.default_rng(40)
    for growth, backoff, interval in ((2.0, 0.5, 3), (1.5, 0.7, 2), (3.0, 0.25, 5)):
        ts = torch.tensor([777.0], dtype=torch.float32)
        tt = torch.tensor([0], dtype=torch.int32)
        sc, tr = 777.0, 0
        for _ in range(40):
            inf = bool(rng.random() < 0.2)
            torch._amp_update_scale_(ts, tt, torch.tensor([1.0 if inf else 0.0]), growth, backoff, interval)
            sc, tr = o.amp_update(sc, tr, inf, growth, backoff, interval)
            assert sc == float(ts.item()) and tr == int(tt.item()), (growth, backoff, interval, sc, ts.item())


# ---------------------------------------------------------------- the last microbatch's +=
def pin_accumulate_library(o):
    """One += is the IEEE addition of the storage format: bit for bit the same
    as numpy's float32 and float16 additions and torch's bfloat16 addition,
    over random values of many magnitudes and the special cases (overflow to
    Inf, Inf - Inf, subnormals, x + (-x) = +0, -0 + -0 = -0)."""
    import torch
    rng = np.random.default_rng(70)
    special = {"f32": [3.0e38, 3.0e38, -0.0, -0.0, 1e-45, -1e-45, math.inf, -math.inf, 7.0, -7.0, 1e-40, 2e-40],
               "f16": [60000.0, 60000.0, -0.0, -0.0, 6e-8, -6e-8, math.inf, -math.inf, 7.0, -7.0, 3e-6, 1e-6],
               "bf16": [3.0e38, 3.0e38, -0.0, -0.0, 1e-39, -1e-39, math.inf, -math.inf, 7.0, -7.0, 5e-39, 1e-40]}
    for dt in DTYPES:
        lo, hi = (-17.0, 10.5) if dt == "f16" else (-30.0, 30.0)  # inside the format's range
        mags = np.exp(rng.uniform(lo, hi, 4000)) * rng.choice([-1.0, 1.0], 4000)
        x = store(np.concatenate([mags, special[dt][0::2]]), dt)
        y = store(np.concatenate([rng.permutation(mags) * rng.uniform(0.0, 2.0, 4000), special[dt][1::2]]), dt)
        acc = [x.copy()]
        o.accumulate_(acc, [y], dt)
        with np.errstate(over="ignore", invalid="ignore"):
            if dt == "f32":
                ref = (x + y).view(np.uint32)
            elif dt == "f16":
                ref = (x.view(np.float16) + y.view(np.float16)).view(np.uint16)
            else:
                tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
                ty = torch.from_numpy(y.view(np.int16)).view(torch.bfloat16)
                ref = (tx + ty).view(torch.int16).numpy().view(np.uint16)
        got = raw_bits(acc[0], dt)
        nan = np.isnan(values(acc[0], dt))
        assert np.array_equal(nan, np.isnan(values(ref if dt != "f32" else ref.view(np.float32), dt))), dt
        assert np.array_equal(got[~nan], np.asarray(ref)[~nan]), (dt, np.flatnonzero(got[~nan] != ref[~nan])[:5])


def pin_accumulate_four_microbatches(o):
    """Four contributions added in order, ((c0 + c1) + c2) + c3, give numpy's
    float32 sums bit for bit; the norm of the average (a = 1/4) of the buffer
    is the library norm of 0.25 times it."""
    rng = np.random.default_rng(71)
    sizes = (1000, 3, 517)
    cs = [[store(rng.standard_normal(n) * 1e-3, "f32") for n in sizes] for _ in range(4)]
    acc = [c.copy() for c in cs[0]]
    for k in range(1, 4):
        o.accumulate_(acc, cs[k], "f32")
    for t in range(len(sizes)):
        ref = ((cs[0][t] + cs[1][t]) + cs[2][t]) + cs[3][t]
        assert np.array_equal(acc[t].view(np.uint32), ref.view(np.uint32)), t
    before = [a.copy() for a in cs[0]]
    for k in range(1, 3):
        o.accumulate_(before, cs[k], "f32")
    r = o.accumulate_clip_(before, cs[3], "f32", 1e30, 0.25)
    ref_norm = math.sqrt(sum(np.linalg.norm(0.25 * a.astype(np.float64)) ** 2 for a in acc))
    assert abs(r["norm"] - ref_norm) <= 1e-13 * ref_norm
    # the clip at 1e30 does not clip, but the averaging by 1/4 is written back (exact in binary32 here)
    assert all(np.array_equal(x, y * np.float32(0.25)) for x, y in zip(before, acc))


def pin_accumulate_then_clip_golden(o):
    """Glossary page, "Order changes the result": 10 and -9 are accumulated to
    1 first, and the clip of the sum at 5 keeps it."""
    gd = golden("accumulate_then_clip.json")
    for dt in DTYPES:
        acc = [store([gd["contributions"][0]], dt)]
        r = o.accumulate_clip_(acc, [store([gd["contributions"][1]], dt)], dt, gd["max_norm"])
        assert values(acc[0], dt)[0] == gd["clip_of_sum"] and r["norm"] == gd["sum"] and not r["clipped"]


# ---------------------------------------------------------------- per-tensor clipping
def pin_per_tensor_contrast(o):
    """Grad clip lesson, "Two variants: Per-Tensor or Global": each tensor is
    clipped by its own norm.  [6, 8] and [0.3, 0.4] at c = 1: the first
    (norm 10) becomes [0.6, 0.8], the second (norm 0.5) passes unchanged, so
    the ratio of the two norms goes from 20 to 2 (the distortion the page
    names); the global clip keeps the ratio and shrinks both."""
    for dt in DTYPES:
        a = [store([6.0, 8.0], dt), store([0.3, 0.4], dt)]
        second = raw_bits(a[1], dt).copy()
        r = o.clip_per_tensor_(a, dt, 1.0)
        t0, t1 = r["tensors"]
        assert t0["norm"] == 10.0 and t0["clipped"] and t0["scale"] == 0.1
        assert not t1["clipped"] and t1["scale"] == 1.0
        assert abs(t1["norm"] - math.hypot(values(store([0.3], dt), dt)[0], values(store([0.4], dt), dt)[0])) \
            <= 1e-15
        assert np.array_equal(raw_bits(a[1], dt), second)
        assert np.array_equal(raw_bits(a[0], dt), raw_bits(store([0.6, 0.8], dt), dt)), (dt, values(a[0], dt))
        assert r["clipped"] and not r["skipped"] and not r["nonfinite"]
        assert abs(r["norm"] - math.sqrt(100.0 + t1["sumsq"])) <= 1e-14 * r["norm"]
        g = [store([6.0, 8.0], dt), store([0.3, 0.4], dt)]
        o.clip_(g, dt, 1.0)
        ratio_global = np.linalg.norm(values(g[0], dt)) / np.linalg.norm(values(g[1], dt))
        ratio_tensor = np.linalg.norm(values(a[0], dt)) / np.linalg.norm(values(a[1], dt))
        assert abs(ratio_global - 20.0) < 0.2 and abs(ratio_tensor - 2.0) < 0.02, (ratio_global, ratio_tensor)


def pin_per_tensor_library(o):
    """Per-tensor norms against numpy.linalg.norm tensor by tensor (so the
    tensor boundaries are right), the list norm against the joint norm, and
    the clipped values against torch.nn.utils.clip_grad_norm_ applied to
    each tensor alone in float64: torch divides by norm + 1e-6, so a clipped
    tensor may differ by that relative amount, an unclipped one not at all."""
    import torch
    rng = np.random.default_rng(60)
    for dt in DTYPES:
        sizes_sd = ((1000, 1.0), (37, 0.01), (1, 5.0), (513, 0.03), (0, 1.0), (200, 0.5))
        arrs = [store(rng.standard_normal(n) * sd, dt) for n, sd in sizes_sd]
        before = [values(x, dt) for x in arrs]
        c = 1.0
        r = o.clip_per_tensor_(arrs, dt, c)
        joint = math.sqrt(sum(np.linalg.norm(v) ** 2 for v in before))
        assert abs(r["norm"] - joint) <= 1e-13 * joint
        for k, (t, v, x) in enumerate(zip(r["tensors"], before, arrs)):
            nrm = float(np.linalg.norm(v))
            assert abs(t["norm"] - nrm) <= 1e-13 * max(nrm, 1e-300), (dt, k)
            assert t["clipped"] == (nrm > c), (dt, k)
            prm = torch.nn.Parameter(torch.zeros(v.size, dtype=torch.float64))
            prm.grad = torch.from_numpy(v.copy())
            torch.nn.utils.clip_grad_norm_([prm], c)
            ref = prm.grad.numpy()
            got = values(x, dt)
            if not t["clipped"]:
                assert np.array_equal(raw_bits(x, dt), raw_bits(store(v, dt), dt)), (dt, k)
            else:
                tol = (2e-6 / nrm) * np.abs(ref) + ulp(ref, dt)
                assert np.all(np.abs(got - ref) <= tol), (dt, k)
                # after the clip the tensor's norm is c, up to the storage rounding
                post = float(np.linalg.norm(got))
                assert abs(post - c) <= 4 * float(ulp(np.array([1.0]), dt)[0]) * c, (dt, k, post)


def pin_per_tensor_single_is_global(o):
    """A one-tensor list: per-tensor and global clipping are the same
    operation, bit for bit, also with averaging."""
    rng = np.random.default_rng(61)
    for dt in DTYPES:
        for n, sd, c, a in ((700, 1.0, 5.0, 1.0), (700, 1.0, 50.0, 0.25), (33, 0.1, 0.2, 1.0 / 3.0)):
            x = store(rng.standard_normal(n) * sd, dt)
            g, t = [x.copy()], [x.copy()]
            rg = o.clip_(g, dt, c, a)
            rt = o.clip_per_tensor_(t, dt, c, a)
            assert np.array_equal(raw_bits(g[0], dt), raw_bits(t[0], dt)), (dt, n, c, a)
            assert rt["tensors"][0]["scale"] == rg["scale"] and rt["tensors"][0]["norm"] == rg["norm"]


def pin_per_tensor_nonfinite(o):
    """With the stop switch a NaN/Inf anywhere stops the whole update (no
    tensor written); without it, the other tensors are clipped as usual and
    the tensor with the NaN keeps its values (NaN > c is false)."""
    for dt in DTYPES:
        lst = [[3.0, 4.0], [math.nan, 1.0], [30.0, 40.0], []]
        a = [store(v, dt) for v in lst]
        before = [raw_bits(x, dt).copy() for x in a]
        r = o.clip_per_tensor_(a, dt, 1.0, 1.0, True)
        assert r["skipped"] and r["nonfinite"] and all(t["scale"] == 1.0 for t in r["tensors"])
        assert all(np.array_equal(raw_bits(x, dt), b) for x, b in zip(a, before))
        r = o.clip_per_tensor_(a, dt, 1.0, 1.0, False)
        assert not r["skipped"] and r["nonfinite"]
        assert [t["nonfinite"] for t in r["tensors"]] == [False, True, False, False]
        assert [t["clipped"] for t in r["tensors"]] == [True, False, True, False]
        assert np.array_equal(raw_bits(a[0], dt), raw_bits(store([0.6, 0.8], dt), dt))
        assert np.array_equal(raw_bits(a[2], dt), raw_bits(store([0.6, 0.8], dt), dt))
        assert np.array_equal(raw_bits(a[1], dt), before[1])
        assert r["tensors"][3]["norm"] == 0.0 and r["tensors"][3]["scale"] == 1.0


ALL_PINS = [pin_worked_6_8, pin_not_per_coordinate, pin_sgd_step_length, pin_accumulate_then_clip,
            pin_tie_passes_unchanged, pin_below_threshold_bitwise, pin_post_clip_norm, pin_single_global_factor,
            pin_joint_norm_library, pin_bruteforce_exact, pin_decode_library, pin_encode_library, pin_nonfinite,
            pin_avg_factor, pin_scale_invariance, pin_empty_and_zero_size, pin_infinite_threshold,
            pin_adamw_first_step, pin_adamw_decay_only, pin_adamw_constant_gradient, pin_adamw_matches_torch,
            pin_adamw_after_clip, pin_amp_unscale_before_clip, pin_amp_found_inf_writes_nothing,
            pin_amp_update_closed_form, pin_amp_update_matches_torch, pin_per_tensor_contrast,
            pin_per_tensor_library, pin_per_tensor_single_is_global, pin_per_tensor_nonfinite,
            pin_accumulate_library, pin_accumulate_four_microbatches, pin_accumulate_then_clip_golden]
