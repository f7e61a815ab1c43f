"""Pins of the oracle's scalar conversions against host library casts and closed forms.

Each oracle conversion is written from the format's definition (nearest value, ties to the even
significand, gradual underflow). These tests hold it against something else:
  * bf16  : torch CPU float32 -> bfloat16 cast (nearest-even)
  * f16   : numpy float32 -> float16 cast (nearest-even, overflow to inf)
  * E4M3  : torch CPU float32 -> float8_e4m3fn cast (nearest-even) on [0, 448], and the 256-code
            decode table written from the format's closed form
  * E2M1  : an independent threshold formulation of nearest-even onto {0,.5,1,1.5,2,3,4,6}

The default sweeps cover every rounding decision class (each exponent and upper significand
pattern, with the discarded bits at 0, 1, just below/at/above the half-way point and all ones)
plus random fill; KVQ_EXHAUSTIVE=1 runs the full 2^32 sweeps.
"""

import numpy as np
import pytest
import torch

import oracle


def _torch_bf16(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _is_nan(x: np.ndarray) -> np.ndarray:
    return np.isnan(x)


def _structured(upper_bits: int, low_set) -> np.ndarray:
    """All (upper pattern, low pattern) pairs: upper = the top `upper_bits` of the word."""
    low_bits = 32 - upper_bits
    up = np.arange(1 << upper_bits, dtype=np.uint64) << np.uint64(low_bits)
    low = np.asarray(sorted(set(int(v) & ((1 << low_bits) - 1) for v in low_set)), dtype=np.uint64)
    return (up[:, None] | low[None, :]).reshape(-1).astype(np.uint32)


def test_bf16_matches_torch_every_decision_class():
    rng = np.random.default_rng(0)
    low = [0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000] + list(rng.integers(0, 1 << 16, 8))
    bits = _structured(16, low)
    x = bits.view(np.float32)
    keep = ~_is_nan(x)
    x = x[keep]
    np.testing.assert_array_equal(oracle.f32_to_bf16(x), _torch_bf16(x))


def test_bf16_ties_and_overflow_examples():
    one = np.float32(1.0)
    # 1 + 2^-8 is exactly half-way between bf16 1.0 and 1 + 2^-7: ties to even -> 1.0
    x = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 3.40e38, -0.0, 2.0 ** -133, 2.0 ** -134], np.float32)
    got = oracle.f32_to_bf16(x)
    assert got[0] == 0x3F80 and got[1] == 0x3F82
    assert got[2] == 0x7F80  # above the largest finite bf16 (3.3895e38) by more than half an ulp -> +inf
    assert got[3] == 0x8000  # signed zero kept
    assert got[4] == 0x0001  # smallest bf16 subnormal
    assert got[5] == 0x0000  # half of it: tie to even -> +0
    assert one == oracle.bf16_to_f32(np.array([0x3F80], np.uint16))[0]


def test_f16_matches_numpy_every_decision_class():
    rng = np.random.default_rng(1)
    low13 = [0, 1, 0xFFF, 0x1000, 0x1001, 0x1FFF, 0x800, 0x1800] + list(rng.integers(0, 1 << 13, 4))
    bits = _structured(19, low13)
    x = bits.view(np.float32)
    x = x[~_is_nan(x)]
    ref = x.astype(np.float16).view(np.uint16)
    np.testing.assert_array_equal(oracle.f32_to_f16(x), ref)


def test_f16_decode_all_codes():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = codes.view(np.float16).astype(np.float32)
    got = np.array([oracle.f16_to_f32(int(c)) for c in codes[::1]], np.float32)
    fin = np.isfinite(ref)
    np.testing.assert_array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))
    assert np.all(np.isinf(got[np.isinf(ref)]))


def _torch_e4m3(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_on_0_448():
    # every binary32 in [0, 448] whose discarded significand bits (20 of them for normal
    # targets) sit on a decision class; subnormal E4M3 targets are covered because the upper
    # 12 bits of the word are swept in full
    rng = np.random.default_rng(2)
    low20 = [0, 1, 0x7FFFF, 0x80000, 0x80001, 0xFFFFF, 0x40000, 0xC0000] + list(rng.integers(0, 1 << 20, 8))
    bits = _structured(12, low20)
    x = bits.view(np.float32)
    x = x[(x >= 0) & (x <= 448)]
    x = np.concatenate([x, rng.uniform(0, 448, 1 << 18).astype(np.float32),
                        (rng.uniform(0, 2.0 ** -6, 1 << 16)).astype(np.float32)])
    np.testing.assert_array_equal(oracle.f32_to_e4m3(x), _torch_e4m3(x))


def test_e4m3_decode_closed_form_all_codes():
    for b in range(256):
        s = -1.0 if b & 0x80 else 1.0
        E, M = (b >> 3) & 15, b & 7
        got = oracle.e4m3_to_f32(b)
        if E == 15 and M == 7:
            assert np.isnan(got)
            continue
        want = s * (M / 8.0 * 2.0 ** -6 if E == 0 else (1 + M / 8.0) * 2.0 ** (E - 7))
        assert got == want and np.signbit(got) == (s < 0), b
    # and against torch's own decode
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = np.array([oracle.e4m3_to_f32(int(c)) for c in codes], np.float32)
    fin = ~np.isnan(ref)
    np.testing.assert_array_equal(got[fin].view(np.uint32), ref[fin].view(np.uint32))


def test_e4m3_named_values():
    x = np.array([448.0, 460.0, 2.0 ** -10, 3 * 2.0 ** -11, 2.0 ** -9, 1.0, 224.0, 0.0], np.float32)
    got = oracle.f32_to_e4m3(x)
    assert list(got) == [0x7E, 0x7E, 0x00, 0x01, 0x01, 0x38, 0x76, 0x00]


E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def _e2m1_thresholds(m: np.ndarray) -> np.ndarray:
    """Independent formulation: nearest-even by comparison with the seven midpoints. A value
    exactly on a midpoint goes to the neighbour with the even code: the midpoints 0.25, 1.25,
    2.5, 5 belong to the lower neighbour and 0.75, 1.75, 3.5 to the upper one."""
    m = np.minimum(np.abs(m.astype(np.float64)), 6.0)
    c = ((m > 0.25).astype(np.uint8) + (m >= 0.75) + (m > 1.25) + (m >= 1.75) + (m > 2.5) + (m >= 3.5) + (m > 5.0))
    return c.astype(np.uint8)


def test_e2m1_grid_decode_table():
    for c in range(16):
        v = oracle.e2m1_to_f32(c)
        want = (-1 if c & 8 else 1) * E2M1[c & 7]
        assert v == want and np.signbit(v) == bool(c & 8)


def test_e2m1_encode_against_threshold_formulation():
    rng = np.random.default_rng(3)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] + E2M1, np.float32)
    steps = np.arange(-2000, 2001)
    around = []
    for m in mids:  # 2000 ulps either side of every midpoint and grid value
        u = m.view(np.uint32).astype(np.int64) + steps
        around.append(u[u >= 0].astype(np.uint32).view(np.float32))
    sweep = np.arange(0, 0x41000001, 97, dtype=np.uint32).view(np.float32)  # every 97th float in [0, 8]
    q = np.concatenate(around + [sweep, rng.uniform(0, 8, 1 << 20).astype(np.float32)])
    q = q[np.isfinite(q)]
    got = oracle.e2m1_encode(q)
    np.testing.assert_array_equal(got & 7, _e2m1_thresholds(q))
    assert np.all((got & 8) == 0)
    neg = -q
    gotn = oracle.e2m1_encode(neg)
    np.testing.assert_array_equal(gotn & 7, _e2m1_thresholds(q))
    assert np.all((gotn & 8) == 8)  # sign from the value, including -0.0


def test_e2m1_midpoints_named():
    q = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 100.0, -0.0, 0.0, -0.1], np.float32)
    assert list(oracle.e2m1_encode(q)) == [0, 2, 2, 4, 4, 6, 6, 7, 8, 0, 8]
    # one ulp either side of a midpoint leaves the tie
    up = np.nextafter(np.float32(0.25), np.float32(1))
    dn = np.nextafter(np.float32(0.75), np.float32(0))
    assert list(oracle.e2m1_encode(np.array([up, dn], np.float32))) == [1, 1]


@pytest.mark.exhaustive
def test_bf16_f16_exhaustive_2e32():
    step = 1 << 26
    for lo in range(0, 1 << 32, step):
        bits = np.arange(lo, lo + step, dtype=np.uint64).astype(np.uint32)
        x = bits.view(np.float32)
        x = x[~np.isnan(x)]
        np.testing.assert_array_equal(oracle.f32_to_bf16(x), _torch_bf16(x))
        np.testing.assert_array_equal(oracle.f32_to_f16(x), x.astype(np.float16).view(np.uint16))


@pytest.mark.exhaustive
def test_e4m3_exhaustive_0_448():
    top = int(np.float32(448).view(np.uint32))
    step = 1 << 26
    for lo in range(0, top + 1, step):
        bits = np.arange(lo, min(lo + step, top + 1), dtype=np.uint64).astype(np.uint32)
        x = bits.view(np.float32)
        np.testing.assert_array_equal(oracle.f32_to_e4m3(x), _torch_e4m3(x))


@pytest.mark.exhaustive
def test_e2m1_exhaustive_nonnegative():
    step = 1 << 26
    for lo in range(0, 0x7F800000, step):
        bits = np.arange(lo, min(lo + step, 0x7F800000), dtype=np.uint64).astype(np.uint32)
        q = bits.view(np.float32)
        np.testing.assert_array_equal(oracle.e2m1_encode(q), _e2m1_thresholds(q))
