"""Pins for the oracle's float8_e4m3fn codec (CPU only).

The codec is pinned against a library routine (torch's CPU float8_e4m3fn cast, exhaustively over
every binary32 bit pattern) and against brute-force nearest-value search, not against itself.
"""
import numpy as np
import pytest
import torch

import oracle

ALL_CODES = np.arange(256, dtype=np.uint8)
FINITE_CODES = ALL_CODES[(ALL_CODES & 0x7F) != 0x7F]


def test_decode_matches_torch_for_every_code():
    ours = oracle.e4m3_decode(ALL_CODES)
    ref = torch.from_numpy(ALL_CODES.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = (ALL_CODES & 0x7F) == 0x7F
    assert np.all(np.isnan(ours[nan])) and np.all(np.isnan(ref[nan]))
    assert np.array_equal(ours[~nan], ref[~nan])
    # signs of zero survive
    assert np.signbit(ours[0x80]) and not np.signbit(ours[0x00])


def test_format_constants():
    # largest finite 448 (0x7E), smallest normal 2^-6 (0x08), smallest subnormal 2^-9 (0x01)
    assert oracle.e4m3_decode(np.array([0x7E]))[0] == 448.0
    assert oracle.e4m3_decode(np.array([0x08]))[0] == 2.0 ** -6
    assert oracle.e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9
    assert oracle.e4m3_decode(np.array([0xFE]))[0] == -448.0


def test_roundtrip_every_finite_code():
    vals = oracle.e4m3_decode(FINITE_CODES).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), FINITE_CODES)


def test_encode_is_nearest_ties_to_even_bruteforce():
    """Random fp32 in [-448, 448] plus every midpoint between neighbouring codes: the code must be a
    nearest representable value, and at an exact midpoint the one with an even mantissa."""
    g = np.random.Generator(np.random.PCG64(7))
    v = np.concatenate([
        g.uniform(-448, 448, 20000),
        g.standard_normal(20000) * np.exp2(g.integers(-14, 8, 20000)),
    ]).astype(np.float32)
    pos = np.sort(oracle.e4m3_decode(FINITE_CODES[FINITE_CODES < 0x80]))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, -mids]).astype(np.float32)
    codes = oracle.e4m3_encode(v)
    table_codes = FINITE_CODES.astype(np.int64)
    table_vals = oracle.e4m3_decode(FINITE_CODES)
    dist = np.abs(v.astype(np.float64)[:, None] - table_vals[None, :])
    best = dist.min(axis=1)
    got = np.abs(v.astype(np.float64) - oracle.e4m3_decode(codes))
    assert np.array_equal(got, best)
    # ties: among the nearest candidates, the chosen code has an even mantissa field
    n_near = (dist == best[:, None]).sum(axis=1)
    tie = n_near > 1
    nonzero_tie = tie & (best > 0)
    assert nonzero_tie.sum() > 100
    assert np.all((codes[nonzero_tie] & 1) == 0)
    # sign is kept, also when the result is zero
    assert np.array_equal(np.signbit(oracle.e4m3_decode(codes)), np.signbit(v))
    del table_codes


def test_encode_saturates():
    v = np.array([448.0, 449.0, 463.9, 464.0, 500.0, 3.0e38, -1e30, -448.5], dtype=np.float32)
    assert list(oracle.e4m3_encode(v)) == [0x7E] * 6 + [0xFE, 0xFE]


@pytest.mark.parametrize("chunk", range(64))
def test_encode_exhaustive_vs_torch(chunk):
    """All 2^32 binary32 patterns (64 chunks of 2^26): the oracle's saturating encoder equals torch's
    RNE cast applied after clamping to +-448 (torch turns overflow into NaN instead of saturating).
    NaN inputs are outside the contract and skipped."""
    n = 1 << 26
    first = chunk * n
    ours = oracle.e4m3_encode_bits(first, n)
    bits = np.arange(first, first + n, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    ok = ~np.isnan(f)
    fc = np.clip(f, np.float32(-448), np.float32(448))
    ref = torch.from_numpy(fc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.nonzero((ours != ref) & ok)[0]
    assert bad.size == 0, f"first mismatch at bits {hex(first + int(bad[0]))}"
