"""Pins for the oracle's E4M3FN codec (CPU only).

The codec is pinned against things other than itself: the OCP spec's spot
values (golden fixture), PyTorch's own float8_e4m3fn conversion (a library
routine), a brute-force nearest search, exact midpoints, saturation and NaN.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _finite_codes():
    return [c for c in range(256) if c not in (0x7F, 0xFF)]


def test_spot_values_match_spec():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_spot_values.json")))
    tab = e4m3.decode_table()
    for k, v in g["values"].items():
        c = int(k, 16)
        assert tab[c] == v, k
        assert np.signbit(tab[c]) == np.signbit(v), k
    for k in g["nan_codes"]:
        assert np.isnan(tab[int(k, 16)])
    assert np.isnan(tab).sum() == 2


def test_table_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = e4m3.decode_table()
    fin = ~np.isnan(ref)
    assert np.array_equal(np.isnan(tab), np.isnan(ref))
    assert np.array_equal(tab[fin], ref[fin])
    assert np.array_equal(np.signbit(tab[fin]), np.signbit(ref[fin]))


def test_table_monotone_and_symmetric():
    tab = e4m3.decode_table()
    pos = tab[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert pos[-1] == 448.0
    assert np.array_equal(-tab[0x80:0xFF], pos)


def test_round_trip_every_finite_code():
    tab = e4m3.decode_table()
    codes = np.array(_finite_codes(), dtype=np.uint8)
    vals = tab[codes].astype(np.float32)
    assert np.array_equal(e4m3.encode(vals), codes)


def _brute_force(x32: np.ndarray) -> np.ndarray:
    """Nearest finite code by exhaustive search, ties to the even code, clamp to ±448."""
    tab = e4m3.decode_table()
    codes = np.array([c for c in range(0x7F)], dtype=np.int64)  # non-negative finite
    vals = tab[codes]
    out = np.empty(x32.shape, dtype=np.uint8)
    a = np.minimum(np.abs(x32.astype(np.float64)), 448.0)
    dist = np.abs(a[:, None] - vals[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    # among tied candidates take the even code
    even = cand & ((codes[None, :] & 1) == 0)
    pick = np.where(even.any(axis=1), even.argmax(axis=1), cand.argmax(axis=1))
    out[:] = codes[pick].astype(np.uint8)
    out |= (np.signbit(x32).astype(np.uint8) << 7)
    return out


@pytest.mark.parametrize("scale", [1.0, 0.37, 2.0 ** -7, 1.0 / 448.0, 5.5e-3, 3.0])
def test_encoder_vs_brute_force_all_bf16(scale):
    bits = np.arange(65536, dtype=np.uint32)
    x = (bits << np.uint32(16)).view(np.float32)
    x = x[np.isfinite(x)]
    with np.errstate(over="ignore"):
        y = (x / np.float32(scale)).astype(np.float32)
    y = y[np.isfinite(y)]
    for chunk in np.array_split(y, 16):
        assert np.array_equal(e4m3.encode(chunk), _brute_force(chunk))


def test_encoder_vs_torch_in_range():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(200_000).astype(np.float32) * 100,
        rng.standard_normal(200_000).astype(np.float32) * 1e-2,
        (rng.random(100_000).astype(np.float32) * 2 - 1) * 463.0,
    ])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode(x), ref)


def test_midpoints_round_to_even_and_neighbours_round_to_nearest():
    tab = e4m3.decode_table()
    pos = tab[:0x7F]
    for c in range(0x7E):
        lo, hi = pos[c], pos[c + 1]
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2  # exact
        even = c if c % 2 == 0 else c + 1
        assert e4m3.encode(np.array([mid]))[0] == even
        up = np.nextafter(mid, np.float32(np.inf), dtype=np.float32)
        dn = np.nextafter(mid, np.float32(0), dtype=np.float32)
        assert e4m3.encode(np.array([up]))[0] == c + 1
        assert e4m3.encode(np.array([dn]))[0] == c
        assert e4m3.encode(np.array([-mid]))[0] == (even | 0x80)


def test_saturation_nan_and_signed_zero():
    x = np.array([448.0, 449.0, 463.9, 464.0, 1e6, np.inf, -1e6, -np.inf], dtype=np.float32)
    assert list(e4m3.encode(x)) == [0x7E] * 6 + [0xFE] * 2
    n = np.array([np.nan, -np.nan], dtype=np.float32)
    n[1] = -np.abs(n[1])
    assert list(e4m3.encode(n)) == [0x7F, 0xFF]
    z = np.array([0.0, -0.0, -1e-30, 1e-30, 2.0 ** -10, -(2.0 ** -10)], dtype=np.float32)
    # 2^-10 is the midpoint between 0 and the smallest subnormal: ties to even (0)
    assert list(e4m3.encode(z)) == [0x00, 0x80, 0x80, 0x00, 0x00, 0x80]


def test_quantisation_error_bound():
    """Relative error <= 2^-4 on normals, absolute <= 2^-10 on subnormals."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(100_000) * rng.choice([1e-3, 1e-1, 1, 50], 100_000)).astype(np.float32)
    x = np.clip(x, -448, 448)
    v = e4m3.decode(e4m3.encode(x))
    a = np.abs(x.astype(np.float64))
    err = np.abs(v - x)
    normal = a >= 2.0 ** -6
    assert np.all(err[normal] <= a[normal] * 2.0 ** -4 + 1e-300)
    assert np.all(err[~normal] <= 2.0 ** -10)
