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
