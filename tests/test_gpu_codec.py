"""GPU parity of the coordinate codec (VFlash paper §2.3 "Token
representation"; §3.1 "Base VLM"): the four codec kernels through the C ABI
against the float64 oracle, bit-exact on every output (token ids, the
float64 bin values, the integer fields and their validity flags).

Inputs are seeded and synthetic: uniform values over and past each range,
the float32 values nearest every bin midpoint (the ties the rounding rule
decides), infinities and NaN; integers across and past the five-digit field
width; fields that the oracle wrote, then corrupted at random positions."""
import numpy as np
import pytest
import torch

from oracle import fpd_oracle as O
from tests.gpu_cases import progress, small_ids

pytestmark = pytest.mark.gpu

IDS = small_ids(4099)
RANGES = [(0.0, 1000.0), (-51.2, 51.2), (-3.0, 17.5)]   # 2D image range; two 3D ranges


def _fpd():
    from block_draft_decoding_amd import fpd
    return fpd


def _coord_values(lo, hi, n, seed):
    rng = np.random.default_rng(seed)
    w = (hi - lo) / 1000.0
    span = hi - lo
    parts = [
        rng.uniform(lo - 0.02 * span, hi + 0.02 * span, n).astype(np.float32),
        (lo + (np.arange(-2, 1003) + 0.5) * w).astype(np.float32),        # nearest float32 to every midpoint
        (lo + np.arange(-2, 1003) * w).astype(np.float32),                # bin centres
        np.array([lo, hi, np.nextafter(np.float32(lo), np.float32(-np.inf)),
                  np.nextafter(np.float32(hi), np.float32(np.inf)), np.inf, -np.inf, np.nan, -np.nan,
                  3.4e38, -3.4e38, 0.0, -0.0], np.float32),
    ]
    if lo == 0.0 and hi == 1000.0:
        parts.append(np.arange(0, 1000, dtype=np.float32) + np.float32(0.5))   # exact ties: even bins win
    x = np.concatenate(parts)
    return x[rng.permutation(x.size)]


@pytest.mark.parametrize("lo,hi", RANGES)
def test_coords_to_tokens_bit_exact(lo, hi):
    fpd = _fpd()
    x = _coord_values(lo, hi, 300_001, seed=int(1000 * (hi - lo)) % 9973)
    progress(f"[codec c2t] lo={lo} hi={hi} n={x.size}")
    xd = torch.from_numpy(x).cuda()
    out = torch.full((x.size,), 7, dtype=torch.int32, device="cuda")
    fpd.fpd_coords_to_tokens(xd, out, IDS["coord_base"], lo, hi)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = O.coords_to_tokens(x, IDS["coord_base"], lo, hi)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, (bad.size, x[bad[:5]], got[bad[:5]], want[bad[:5]])
    assert set(np.unique(got)) <= set(range(IDS["coord_base"], IDS["coord_base"] + 1001)) | {-1}


@pytest.mark.parametrize("lo,hi", RANGES)
def test_tokens_to_coords_bit_exact(lo, hi):
    fpd = _fpd()
    rng = np.random.default_rng(17)
    cb = IDS["coord_base"]
    t = np.concatenate([rng.integers(cb - 40, cb + 1040, 200_003), np.arange(cb - 3, cb + 1004),
                        [np.iinfo(np.int32).min, np.iinfo(np.int32).max, 0, -1]]).astype(np.int32)
    progress(f"[codec t2c] lo={lo} hi={hi} n={t.size}")
    out = torch.zeros(t.size, dtype=torch.float64, device="cuda")
    fpd.fpd_tokens_to_coords(torch.from_numpy(t).cuda(), out, cb, lo, hi)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = O.tokens_to_coords(t, cb, lo, hi)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok].view(np.int64), want[ok].view(np.int64))


@pytest.mark.parametrize("lo,hi", RANGES)
def test_every_token_survives_a_round_trip_on_device(lo, hi):
    fpd = _fpd()
    cb = IDS["coord_base"]
    t = torch.arange(cb, cb + 1001, dtype=torch.int32, device="cuda")
    v = torch.empty(1001, dtype=torch.float64, device="cuda")
    fpd.fpd_tokens_to_coords(t, v, cb, lo, hi)
    back = torch.empty_like(t)
    fpd.fpd_coords_to_tokens(v.float().contiguous(), back, cb, lo, hi)
    torch.cuda.synchronize()
    assert torch.equal(back, t)


def test_ints_to_fields_bit_exact():
    fpd = _fpd()
    rng = np.random.default_rng(23)
    edges = [0, 1, -1, 9, -9, 10, -10, 99, 100, 9999, 10000, -10000, 99999, -99999, 100000, -100000,
             np.iinfo(np.int32).max, np.iinfo(np.int32).min]
    v = np.concatenate([rng.integers(-120_000, 120_001, 250_007), rng.integers(-99, 100, 1000), edges]).astype(np.int32)
    progress(f"[codec i2f] n={v.size}")
    out = torch.zeros((v.size, 6), dtype=torch.int32, device="cuda")
    fpd.fpd_ints_to_fields(torch.from_numpy(v).cuda(), out, IDS["plus_id"], IDS["minus_id"], IDS["digit0_id"],
                           IDS["fill_id"])
    torch.cuda.synchronize()
    want = O.ints_to_fields(v, IDS["plus_id"], IDS["minus_id"], IDS["digit0_id"], IDS["fill_id"])
    assert np.array_equal(out.cpu().numpy(), want)


def test_fields_to_ints_bit_exact_on_clean_and_corrupted_fields():
    fpd = _fpd()
    rng = np.random.default_rng(29)
    ids = (IDS["plus_id"], IDS["minus_id"], IDS["digit0_id"], IDS["fill_id"])
    v = rng.integers(-99_999, 100_000, 120_011).astype(np.int32)
    f = O.ints_to_fields(v, *ids)
    # corrupt about half of the fields at one to three random positions with tokens from the field
    # alphabet and a few outside it
    alphabet = np.array([ids[0], ids[1], ids[3], IDS["delim_id"], IDS["coord_base"], 0] +
                        list(range(ids[2], ids[2] + 10)), np.int32)
    bad_rows = rng.random(f.shape[0]) < 0.5
    for k in range(3):
        rows = np.nonzero(bad_rows & (rng.random(f.shape[0]) < 0.7 ** k))[0]
        cols = rng.integers(0, 6, rows.size)
        f[rows, cols] = alphabet[rng.integers(0, alphabet.size, rows.size)]
    progress(f"[codec f2i] n={f.shape[0]}")
    vals = torch.full((f.shape[0],), 5, dtype=torch.int32, device="cuda")
    valid = torch.full((f.shape[0],), 5, dtype=torch.int32, device="cuda")
    fpd.fpd_fields_to_ints(torch.from_numpy(np.ascontiguousarray(f)).cuda(), vals, valid, *ids)
    torch.cuda.synchronize()
    wv, wok = O.fields_to_ints(f, *ids)
    assert np.array_equal(valid.cpu().numpy(), wok)
    assert np.array_equal(vals.cpu().numpy(), wv)
    assert 0.3 < wok.mean() < 0.8          # both outcomes are exercised


def test_empty_calls_do_nothing():
    fpd = _fpd()
    e32 = torch.empty(0, dtype=torch.int32, device="cuda")
    fpd.fpd_coords_to_tokens(torch.empty(0, device="cuda"), e32, 0)
    fpd.fpd_tokens_to_coords(e32, torch.empty(0, dtype=torch.float64, device="cuda"), 0)
    fpd.fpd_ints_to_fields(e32, torch.empty((0, 6), dtype=torch.int32, device="cuda"), 1, 2, 3, 4)
    fpd.fpd_fields_to_ints(torch.empty((0, 6), dtype=torch.int32, device="cuda"), e32, e32.clone(), 1, 2, 3, 4)
    torch.cuda.synchronize()
