"""The CPU oracle against its pins (the pages' worked examples, closed forms,
library routines and exact brute force).  CPU only."""
import math

import numpy as np
import pytest

import oracle
from synth import gradsets as gs
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.default())


def _stat_check(g, sigma2_of):
    """E[S] = sum_t n_t sigma_t^2 and Var[S] = sum_t 2 n_t sigma_t^4 for
    normal draws; the oracle's S must sit within 6 standard deviations."""
    s, nf = oracle.sumsq(g.arrays, g.dtype, g.avg_factor)
    mean = sum(a.size * sigma2_of(i) for i, a in enumerate(g.arrays)) * g.avg_factor ** 2
    sd = math.sqrt(sum(2 * a.size * sigma2_of(i) ** 2 for i, a in enumerate(g.arrays))) * g.avg_factor ** 2
    assert not nf
    assert abs(s - mean) <= 6 * sd + 1e-3 * mean, (g.name, s, mean, sd)
    return s


def test_statistics_tiny():
    g = gs.tiny_f32()
    assert g.numel == 4788
    s = _stat_check(g, lambda t: 1.0)
    assert 60 < math.sqrt(s) < 79


@pytest.mark.slow
def test_statistics_andrea120m_f32():
    g = gs.andrea120m_f32()
    assert g.numel == 92_248_320 and len(g.arrays) == 124
    s = _stat_check(g, lambda t: 1e-6)
    assert abs(math.sqrt(s) - 9.605) < 0.01


@pytest.mark.slow
def test_statistics_andrea120m_f16_small():
    g = gs.andrea120m_f16_small()
    # fp16 storage rounds N(0, 1e-5^2) draws (mostly subnormal); allow 1% for that
    s, nf = oracle.sumsq(g.arrays, g.dtype)
    assert not nf and abs(math.sqrt(s) - 0.0960) < 0.0015


def test_shapes_match_the_pages():
    a = gs.shapes_andrea120m()
    assert len(a) == 124
    assert sum(int(np.prod(s)) for _, s in a) == 92_248_320
    b = gs.shapes_gpt1p3b()
    assert len(b) == 4289
    assert sum(int(np.prod(s)) for _, s in b) == 1_311_182_848
    assert sum(int(np.prod(s)) for _, s in gs.shapes_tiny()) == 4788


@pytest.mark.parametrize("threads", [1, 2, 7, 16])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_sharded_leg_matches_the_sequential_oracle(dtype, threads):
    """The CPU baseline's threaded leg: its sum lies within N 2^-53 (relative)
    of the sequential oracle's -- both add the same exact binary64 squares,
    in another order -- it takes the same decision, and every element is the
    oracle's own rounding of g * s for the factor it decided; one thread is
    the sequential oracle bit for bit."""
    rng = np.random.default_rng(600 + threads)
    arrays = [gs.to_storage(rng.standard_normal(n) * 0.3, dtype) for n in (1, 5, 4097, 70_001, 3, 250_000)]
    n = sum(a.size for a in arrays)
    seq = [a.copy() for a in arrays]
    rs = oracle.clip_(seq, dtype, 1.0, 0.5)
    par = [a.copy() for a in arrays]
    rp = oracle.clip_sharded_(par, dtype, 1.0, 0.5, threads=threads)
    assert abs(rp["sumsq"] - rs["sumsq"]) <= n * 2.0 ** -53 * rs["sumsq"]
    assert rp["clipped"] == rs["clipped"] and rp["nonfinite"] == rs["nonfinite"]
    ref = [a.copy() for a in arrays]
    oracle.scale_(ref, dtype, rp["scale"])
    for a, b in zip(par, ref):
        assert a.tobytes() == b.tobytes()
    if threads == 1:
        assert rp["sumsq"] == rs["sumsq"] and rp["scale"] == rs["scale"]
        for a, b in zip(par, seq):
            assert a.tobytes() == b.tobytes()
    runs = oracle.shards(arrays, threads)
    assert len(runs) == threads and sum(v.size for r in runs for v in r) == n
    assert max(sum(v.size for v in r) for r in runs) - min(sum(v.size for v in r) for r in runs) <= 1
