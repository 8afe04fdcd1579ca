"""Pins of the oracle's quantiser (Eq. 2) and grid (Eq. 3) against closed forms,
invariants and a brute-force nearest-level search. CPU only."""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import fsq_oracle as orc
from oracle import bruteforce as bf

H, D = 7.5075, 0.5


def closed_form_thresholds():
    """Level k -> k+1 switch points of Eq. 2, by inverting it on paper:
    u~ = k + 1/2  <=>  tanh(u + atanh(D/H)) = (k + 1/2 + D) / H
                  <=>  u = atanh((k + 1/2 + D) / H) - atanh(D / H),  k = -8..6."""
    return np.array([math.atanh((k + 0.5 + D) / H) - math.atanh(D / H) for k in range(-8, 7)])


def test_constants_match_pages(golden_dir):
    import json, os
    g = json.load(open(os.path.join(golden_dir, "page_byte_facts.json")))["fsq_constants_L16"]
    assert orc.H_BOUND == g["h"] and orc.DELTA == g["delta"]
    assert orc.LEVELS == g["levels"] and orc.BITS == g["bits"]
    assert 2 ** orc.BITS == orc.LEVELS


def test_thresholds_closed_form_values():
    u = closed_form_thresholds()
    # symmetric structure: thresholds for (k+1) = -j and +j average to -atanh(D/H)
    for j in range(1, 8):
        lo = math.atanh(-j / H) - math.atanh(D / H)
        hi = math.atanh(j / H) - math.atanh(D / H)
        assert lo + hi == pytest.approx(-2 * math.atanh(D / H), abs=1e-15)
    assert np.all(np.diff(u) > 0)
    # level -1 -> 0 switches at -atanh(D/H) < 0 and 0 -> 1 at atanh(1/H) - atanh(D/H) > 0,
    # so u = 0 lies inside the level-0 cell
    assert u[7] == pytest.approx(-math.atanh(D / H), abs=1e-15)
    assert u[7] < 0 < u[8]


@pytest.mark.parametrize("k", range(-8, 7))
def test_level_switches_at_closed_form_threshold(k):
    u = closed_form_thresholds()[k + 8]
    assert orc.fsq_levels(u - 1e-9) == k
    assert orc.fsq_levels(u + 1e-9) == k + 1


def test_levels_equal_threshold_count_on_many_points():
    g = np.random.Generator(np.random.PCG64(7))
    u = np.concatenate([g.normal(0, 1.5, 400_000), g.uniform(-6, 6, 100_000)])
    thr = closed_form_thresholds()
    lv_closed = np.searchsorted(thr, u, side="right") - 8
    assert np.array_equal(orc.fsq_levels(u), lv_closed)


def test_invariants():
    u = np.linspace(-20, 20, 200_001)
    c = orc.fsq_codes(u)
    assert c.dtype == np.uint8 and c.min() == 0 and c.max() == 15
    assert set(np.unique(c).tolist()) == set(range(16))     # all 16 levels reached
    assert np.all(np.diff(c.astype(int)) >= 0)              # monotone
    assert orc.fsq_codes(0.0) == 8                           # u = 0 -> level 0 exactly
    assert orc.fsq_bound(0.0) == pytest.approx(0.0, abs=1e-15)
    assert orc.fsq_codes(1e6) == 15 and orc.fsq_codes(-1e6) == 0
    # range of the bound: (-h - delta, h - delta)
    assert orc.fsq_bound(50.0) == pytest.approx(H - D) and orc.fsq_bound(-50.0) == pytest.approx(-H - D)


def test_grid_size_is_product_of_levels():
    """Eq. 3: |C| = prod L_i = 16^G. For G = 2 and 3, sweep a dense grid of u and
    count the distinct code vectors reached."""
    t = np.linspace(-4, 4, 161)        # step 0.05 < the narrowest cell (about 0.13)
    for G in (2, 3):
        axes = np.meshgrid(*([t] * G), indexing="ij")
        U = np.stack([a.ravel() for a in axes], axis=1)
        codes = orc.fsq_codes(U)
        keys = np.zeros(len(codes), dtype=np.int64)
        for i in range(G):
            keys = keys * 16 + codes[:, i]
        assert len(np.unique(keys)) == 16 ** G


@settings(max_examples=300, deadline=None)
@given(st.floats(min_value=-8, max_value=8, allow_nan=False))
def test_bruteforce_nearest_level_matches(u):
    assert orc.fsq_levels(u) == bf.quantise_scalar(u)


def test_encode_is_projection_then_quantise():
    g = np.random.Generator(np.random.PCG64(3))
    x = g.standard_normal((50, 32))
    E = g.standard_normal((6, 32)) / math.sqrt(32)
    codes = orc.encode(x, E)
    # brute force: each coordinate is an explicit dot product then a nearest-level search
    for t in range(50):
        for i in range(6):
            u = sum(x[t, c] * E[i, c] for c in range(32))
            assert codes[t, i] == bf.quantise_scalar(u) + 8


# --------------------------------------------------------------- mutants
@pytest.mark.parametrize("mutant", ["floor", "no_delta", "sign_offset", "h_off"])
def test_pins_catch_planted_mistakes(mutant, monkeypatch):
    """Plant a plausible mistake in the oracle's bound and check that the
    closed-form threshold pin no longer holds."""
    def bad_bound(u, h=H, delta=D):
        u = np.asarray(u, dtype=np.float64)
        if mutant == "no_delta":
            return h * np.tanh(u + math.atanh(delta / h))
        if mutant == "sign_offset":
            return h * np.tanh(u - math.atanh(delta / h)) - delta
        if mutant == "h_off":
            return 7.5 * np.tanh(u + math.atanh(delta / 7.5)) - delta
        return h * np.tanh(u + math.atanh(delta / h)) - delta

    if mutant == "floor":
        monkeypatch.setattr(orc, "fsq_levels", lambda u: np.floor(orc.fsq_bound(u)).astype(np.int64))
    else:
        monkeypatch.setattr(orc, "fsq_bound", bad_bound)
    thr = closed_form_thresholds()
    bad = 0
    for k in range(-8, 7):
        if orc.fsq_levels(thr[k + 8] - 1e-9) != k or orc.fsq_levels(thr[k + 8] + 1e-9) != k + 1:
            bad += 1
    assert bad > 0
