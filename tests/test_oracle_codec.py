"""Pins of the oracle's coordinate codec (VFlash paper §2.3; §3.1 "Base
VLM"): 2D image coordinates normalised to 0..1000 and 3D coordinates
quantised uniformly over a range map onto the 1,001 coordinate tokens, and
fixed-width sign + five-digit fields hold integers."""
import numpy as np
import pytest

from oracle import fpd_oracle as O

BASE = 150_000
PLUS, MINUS, D0, FILL = 151_003, 151_004, 151_005, 151_015


def test_2d_normalised_grid_is_the_identity_on_integers():
    v = np.arange(0, 1001, dtype=np.float64)
    t = O.coords_to_tokens(v, BASE)
    assert np.array_equal(t, BASE + np.arange(1001))
    assert np.array_equal(O.tokens_to_coords(t, BASE), v)


@pytest.mark.parametrize("lo,hi", [(0.0, 1000.0), (-50.0, 50.0), (-3.7, 81.25), (0.0, 1.0)])
def test_every_token_round_trips(lo, hi):
    t = BASE + np.arange(1001)
    assert np.array_equal(O.coords_to_tokens(O.tokens_to_coords(t, BASE, lo, hi), BASE, lo, hi), t)


@pytest.mark.parametrize("lo,hi", [(0.0, 1000.0), (-50.0, 50.0), (-3.7, 81.25)])
def test_decode_of_encode_is_within_half_a_bin(lo, hi):
    x = np.random.default_rng(1).uniform(lo, hi, 20_000)
    err = np.abs(O.tokens_to_coords(O.coords_to_tokens(x, BASE, lo, hi), BASE, lo, hi) - x)
    assert err.max() <= 0.5 * (hi - lo) / 1000 * (1 + 1e-12)


def test_rounding_clamping_and_invalid_values():
    t = O.coords_to_tokens([500.5, 501.5, 499.5, -0.4, -7.0, 1000.4, 3000.0, np.nan], BASE)
    assert t.tolist() == [BASE + 500, BASE + 502, BASE + 500, BASE, BASE, BASE + 1000, BASE + 1000, -1]
    v = O.tokens_to_coords([BASE - 1, BASE + 1001, 7, BASE + 3], BASE)
    assert np.isnan(v[:3]).all() and v[3] == 3.0


def test_field_examples():
    f = O.ints_to_fields([42, -7, 0, 99_999, 10_000, -99_999, 305], PLUS, MINUS, D0, FILL)
    assert f[0].tolist() == [PLUS, FILL, FILL, FILL, D0 + 4, D0 + 2]
    assert f[1].tolist() == [MINUS, FILL, FILL, FILL, FILL, D0 + 7]
    assert f[2].tolist() == [PLUS, FILL, FILL, FILL, FILL, D0]
    assert f[3].tolist() == [PLUS] + [D0 + 9] * 5
    assert f[4].tolist() == [PLUS, D0 + 1, D0, D0, D0, D0]
    assert f[5].tolist() == [MINUS] + [D0 + 9] * 5
    assert f[6].tolist() == [PLUS, FILL, FILL, D0 + 3, D0, D0 + 5]
    assert O.ints_to_fields([100_000, -123_456], PLUS, MINUS, D0, FILL).tolist() == [[-1] * 6] * 2


def test_fields_round_trip_and_satisfy_the_validator_rule():
    n = np.concatenate([np.arange(-1200, 1200), np.random.default_rng(2).integers(-99_999, 100_000, 3000)])
    f = O.ints_to_fields(n, PLUS, MINUS, D0, FILL)
    digits = set(range(D0, D0 + 10))
    assert all(O._field_first_bad(r[1:], FILL, digits) == -1 for r in f)
    vals, ok = O.fields_to_ints(f, PLUS, MINUS, D0, FILL)
    assert ok.all() and np.array_equal(vals, n)


def test_malformed_fields_are_invalid():
    bad = [
        [PLUS, D0 + 1, FILL, D0, D0, D0],      # FILL after a digit
        [PLUS, FILL, FILL, FILL, FILL, FILL],  # no digit at all
        [D0, FILL, FILL, FILL, FILL, D0],      # digit in the sign slot
        [MINUS, FILL, BASE, FILL, FILL, D0],   # foreign id
    ]
    vals, ok = O.fields_to_ints(bad, PLUS, MINUS, D0, FILL)
    assert not ok.any() and not vals.any()
