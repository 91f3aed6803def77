"""Pins for the oracle's number-format conversions.

The oracle writes bf16 and fp16 rounding from the format definitions; these
tests hold them to independent library routines (torch's CPU fp32->bf16 cast,
numpy's fp32->fp16 cast), exhaustively over all 16-bit inputs for widening and
over every low half-word of many high half-words for narrowing, which covers
every tie, every carry into the exponent and the overflow to infinity.
"""
import numpy as np
import pytest
import torch

import oracle


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_widen_exhaustive():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = oracle.bf16_to_f32(h)
    ref = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_bf16_round_matches_torch_on_every_low_half():
    g = np.random.default_rng(7)
    highs = np.concatenate([
        g.integers(0, 1 << 16, size=200, dtype=np.uint32),
        np.array([0x0000, 0x8000, 0x0001, 0x007F, 0x0080, 0x3F80, 0x3F81,
                  0x7F7F, 0xFF7F, 0x7F80, 0xFF80, 0x7FC0, 0x4000, 0xC000], np.uint32)])
    low = np.arange(1 << 16, dtype=np.uint32)
    bits = ((highs[:, None] << 16) | low[None, :]).reshape(-1)
    x = bits.view(np.float32)
    mine = oracle.f32_to_bf16(x)
    ref = _torch_bf16_bits(x)
    nan = np.isnan(x)
    # NaN payloads are not graded: both sides must give a NaN
    assert np.all((mine[nan] & 0x7F80) == 0x7F80) and np.all((mine[nan] & 0x7F) != 0)
    assert np.array_equal(mine[~nan], ref[~nan])


@pytest.mark.parametrize("value,expect", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),            # exact tie, kept part even -> down
    (1.0 + 3 * 2.0 ** -8, 0x3F82),        # exact tie, kept part odd -> up
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),
    (-2.5, 0xC020),
    (3.3895313892515355e38, 0x7F7F),      # max finite bf16 is exact
    (float.fromhex("0x1.ffp127"), 0x7F80),      # tie above max, kept part odd -> inf
    (float.fromhex("0x1.ff8p127"), 0x7F80),     # above the tie -> inf
    (float.fromhex("0x1.fefffep127"), 0x7F7F),   # just below the tie to inf
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (float.fromhex("0x1p-133"), 0x0001),  # bf16 subnormal kept
])
def test_bf16_round_closed_forms(value, expect):
    assert int(oracle.f32_to_bf16(np.array([value], np.float32))[0]) == expect


def test_f16_widen_exhaustive():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = oracle.f16_to_f32(h)
    ref = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_round_matches_numpy():
    g = np.random.default_rng(11)
    # exponents around the binary16 range, every low half-word of a few values
    highs = np.concatenate([
        g.integers(0x3000, 0x4800, size=60, dtype=np.uint32),   # |x| ~ 2^-31 .. 2^17
        g.integers(0xB000, 0xC800, size=60, dtype=np.uint32),
        np.array([0x3380, 0x3800, 0x3880, 0x477F, 0x4780, 0x0000, 0x7F80, 0x7FC0,
                  0x33FF, 0x3400, 0x387F], np.uint32)])
    low = np.arange(1 << 16, dtype=np.uint32)
    bits = ((highs[:, None] << 16) | low[None, :]).reshape(-1)
    x = bits.view(np.float32)
    mine = oracle.f32_to_f16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.all((mine[nan] & 0x7C00) == 0x7C00) and np.all((mine[nan] & 0x3FF) != 0)
    assert np.array_equal(mine[~nan], ref[~nan])


@pytest.mark.parametrize("value,expect", [
    (65504.0, 0x7BFF),
    (65519.99, 0x7BFF),
    (65520.0, 0x7C00),          # tie at the top rounds to even -> overflow
    (2.0 ** -24, 0x0001),
    (2.0 ** -25, 0x0000),       # tie to even at the smallest subnormal
    (3 * 2.0 ** -25, 0x0002),
    (2.0 ** -14 - 2.0 ** -25, 0x0400),   # rounds up into the smallest normal
    (-1.5, 0xBE00),
])
def test_f16_round_closed_forms(value, expect):
    assert int(oracle.f32_to_f16(np.array([value], np.float32))[0]) == expect


# ---------------------------------------------- binary64 -> bfloat16 (one rounding)

def _bf16_grid_f64() -> np.ndarray:
    """Every non-negative finite bf16 value in pattern order (0x0000 .. 0x7F7F),
    widened by torch, plus 2^128 standing for +inf (pattern 0x7F80, an even
    significand): the set a correctly rounded conversion must choose from."""
    pats = np.arange(0x7F80, dtype=np.uint32).astype(np.uint16)
    vals = torch.from_numpy(pats.view(np.int16)).view(torch.bfloat16).double().numpy()
    return np.concatenate([vals, [2.0 ** 128]])


def _nearest_even_by_search(v: np.ndarray) -> np.ndarray:
    """Round each double to bf16 by searching the value grid: the nearest grid
    point, ties to the even pattern.  The distances are exact in fp64 (the two
    neighbours lie within a factor of two of v, or one of them is 0)."""
    grid = _bf16_grid_f64()
    a = np.abs(v)
    out = np.empty(v.shape, np.uint16)
    big = a >= 2.0 ** 128
    k = np.searchsorted(grid, a[~big], side="right") - 1
    lo, hi = grid[k], grid[np.minimum(k + 1, grid.size - 1)]
    dlo, dhi = a[~big] - lo, hi - a[~big]
    pick = np.where(dlo < dhi, k, np.where(dhi < dlo, k + 1, np.where(k % 2 == 0, k, k + 1)))
    out[~big] = pick.astype(np.uint16)
    out[big] = 0x7F80
    return out | np.where(np.signbit(v), 0x8000, 0).astype(np.uint16)


def test_f64_to_bf16_matches_a_search_of_the_value_grid():
    g = np.random.default_rng(13)
    grid = _bf16_grid_f64()
    # random magnitudes over the whole bf16 range, subnormals included
    v = [np.ldexp(g.random(100_000) + 0.5, g.integers(-140, 130, size=100_000))]
    # every tie between neighbours, and a hair above and below each
    mid = (grid[:-1] + grid[1:]) / 2
    pick = mid[g.choice(mid.size, 20_000, replace=False)]
    v += [pick, pick * (1 + 2.0 ** -45), pick * (1 - 2.0 ** -45)]
    # values just off every bf16 value (the sticky bits below fp32 precision)
    b = grid[g.choice(grid.size - 1, 20_000, replace=False)]
    v += [b * (1 + 2.0 ** -30), b * (1 - 2.0 ** -30)]
    v = np.concatenate(v)
    v = np.concatenate([v, -v])
    assert np.array_equal(oracle.f64_to_bf16(v), _nearest_even_by_search(v))


@pytest.mark.parametrize("value,expect", [
    (1.0 + 2.0 ** -8, 0x3F80),                  # exact tie, kept part even -> down
    (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),     # above the tie (through fp32: 0x3F80)
    (1.0 + 3 * 2.0 ** -8, 0x3F82),              # tie, kept part odd -> up
    (-(1.0 + 2.0 ** -8 + 2.0 ** -40), 0xBF81),
    (float.fromhex("0x1.fep127"), 0x7F7F),      # max finite bf16
    (float.fromhex("0x1.ffp127"), 0x7F80),      # tie above max -> inf
    (float.fromhex("0x1.fefffffffp127"), 0x7F7F),
    (2.0 ** -133, 0x0001),                      # smallest subnormal
    (2.0 ** -134, 0x0000),                      # tie to even at zero
    (3 * 2.0 ** -134, 0x0002),
    (float("inf"), 0x7F80), (-float("inf"), 0xFF80), (-0.0, 0x8000), (0.0, 0x0000),
])
def test_f64_to_bf16_closed_forms(value, expect):
    assert int(oracle.f64_to_bf16(np.array([value]))[0]) == expect


def test_f64_to_bf16_nan_stays_nan():
    h = int(oracle.f64_to_bf16(np.array([float("nan")]))[0])
    assert (h & 0x7F80) == 0x7F80 and (h & 0x7F) != 0
