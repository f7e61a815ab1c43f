"""Pins of the oracle's NVFP4 codec (CPU only).

What pins it:
  * closed cases: a tensor built from E2M1 grid values with amax 6 has g = 448, block scale 448
    (E4M3 0x7E), decode scale exactly 1, and round-trips exactly; a block with amax 3 in the same
    tensor gets block scale 224 (0x76), decode scale 1/2; all-zero and empty tensors give g = 1
    and zero codes (with the sign of the input zero);
  * the global multiplier: 2688 / amax, amax = 0 -> 1, overflow -> FLT_MAX;
  * the tiny-scale path: a tensor with amax ~1e-35 whose small blocks have a decode scale below
    the binary32 normal range, so 1 / s_dec overflows and the direct division is taken; the
    decode error there stays within the block bound;
  * the group axis per kind (K blocks over 16 tokens, V over 16 channels) and low-first nibbles;
  * invariants on seeded data: |x - x_hat| within half an E2M1 gap times s_dec (plus output
    rounding), the sign of every code equals the sign of its input, the block that holds the
    tensor amax gets the top E4M3 scale;
  * the pages' loose error magnitude for N(0,1) data (context only).
"""

import numpy as np
import pytest

import oracle
from workloads import bf16_bits, bf16_to_f32, c2_tensors, tiny_tensor

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def nibbles(codes, D):
    out = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(*codes.shape[:-1], -1)
    return out[..., :D]


def e2m1_value(c):
    c = np.asarray(c)
    v = GRID[c & 7]
    return np.where(c & 8, -v, v)


def e4m3_value(b):
    return np.array([oracle.e4m3_to_f32(int(v)) for v in np.asarray(b).ravel()]).reshape(np.shape(b))


@pytest.mark.parametrize("kind", ["key", "value"])
def test_grid_tensor_round_trips_exactly(kind):
    rng = np.random.default_rng(0)
    T, H, D = 64, 2, 32
    codes = rng.integers(0, 16, (T, H, D))
    x64 = e2m1_value(codes).astype(np.float64)
    # every 16-block (along the kind's axis) holds a +6 so that each block amax is 6
    if kind == "key":
        x64[::16] = 6.0
    else:
        x64[:, :, ::16] = 6.0
    x = bf16_bits(x64)
    p = oracle.pack(x, kind, "nvfp4")
    assert p.global_scale[0] == np.float32(448.0)
    assert np.all(p.meta0 == 0x7E)
    want = codes.copy()
    if kind == "key":
        want[::16] = 7
    else:
        want[:, :, ::16] = 7
    # -0.0 inputs keep the sign bit: code 8 stays 8
    np.testing.assert_array_equal(nibbles(p.codes, D), want)
    np.testing.assert_array_equal(oracle.unpack(p), x)


def test_half_amax_block():
    # V blocks: first block amax 6, second block amax 3 -> scale 224 (0x76), s_dec = 1/2
    x64 = np.zeros((1, 1, 32))
    x64[0, 0, 0] = 6.0
    x64[0, 0, 16:] = [3.0, 1.5, 0.75, -3.0, 0.25, 0.5, 2.25, 1.0, 0, 0, 0, 0, 0, 0, 0, 0]
    p = oracle.pack(bf16_bits(x64), "value", "nvfp4")
    assert p.global_scale[0] == 448.0
    assert list(p.meta0[0, 0]) == [0x7E, 0x76]
    c = nibbles(p.codes, 32)[0, 0, 16:24]
    # q = x / (1/2): 6 -> 7, 3 -> 5, 1.5 -> 3, -6 -> 15, 0.5 -> 1, 1 -> 2, 4.5 -> 4 (tie to even), 2 -> 4
    assert list(c) == [7, 5, 3, 15, 1, 2, 6, 4]


def test_global_multiplier():
    assert oracle.nvfp4_global(6.0) == np.float32(448.0)
    assert oracle.nvfp4_global(0.0) == 1.0
    assert oracle.nvfp4_global(1e-40) == np.finfo(np.float32).max
    assert oracle.nvfp4_global(3.0) == np.float32(2688.0) / np.float32(3.0)


@pytest.mark.parametrize("kind", ["key", "value"])
def test_zero_and_empty(kind):
    x = bf16_bits(np.zeros((20, 2, 20)))
    x[3, 1, 5] = 0x8000  # one -0.0
    p = oracle.pack(x, kind, "nvfp4")
    assert p.global_scale[0] == 1.0 and np.all(p.meta0 == 0)
    c = nibbles(p.codes, 20)
    assert c[3, 1, 5] == 8 and np.count_nonzero(c) == 1
    np.testing.assert_array_equal(oracle.unpack(p), x)
    e = oracle.pack(np.zeros((0, 2, 20), np.uint16), kind, "nvfp4")
    assert e.global_scale[0] == 1.0 and e.codes.size == 0


@pytest.mark.parametrize("kind", ["key", "value"])
def test_tiny_scale_fallback_path(kind):
    x = tiny_tensor()
    p = oracle.pack(x, kind, "nvfp4")
    g = np.float32(p.global_scale[0])
    sf = e4m3_value(p.meta0).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        s_dec = sf / g
        r = np.float32(1.0) / s_dec
    fallback = np.isinf(r) & (sf > 0)
    assert fallback.sum() > 0, "no block took the direct-division path"
    # decode error per block stays within one E2M1 top gap (1.0) times s_dec, plus bf16 rounding
    xf = bf16_to_f32(x).astype(np.float64)
    y = bf16_to_f32(oracle.unpack(p)).astype(np.float64)
    if kind == "key":
        sd = np.repeat(s_dec.astype(np.float64), 16, axis=0)[: x.shape[0]]
    else:
        sd = np.repeat(s_dec.astype(np.float64), 16, axis=2)[..., : x.shape[2]]
    bf16_sub_ulp = 2.0 ** -133
    assert np.all(np.abs(y - xf) <= 1.0 * sd + np.abs(y) * 2.0 ** -8 + bf16_sub_ulp + np.abs(xf) * 2.0 ** -3)


def _expand(meta, kind, shape):
    T, H, D = shape
    if kind == "key":
        return np.repeat(meta, 16, axis=0)[:T]
    return np.repeat(meta, 16, axis=2)[..., :D]


@pytest.mark.parametrize("kind", ["key", "value"])
def test_invariants_c2(kind):
    x = c2_tensors(0)["K" if kind == "key" else "V"][:512]
    p = oracle.pack(x, kind, "nvfp4")
    xf = bf16_to_f32(x).astype(np.float64)
    amax = np.abs(xf).max()
    assert p.global_scale[0] == np.float32(2688.0) / np.float32(amax)
    g = np.float64(p.global_scale[0])
    sf = e4m3_value(p.meta0)
    assert p.meta0.max() <= 0x7E
    # the block holding the tensor amax gets the top scale 448
    i = np.unravel_index(np.argmax(np.abs(xf)), xf.shape)
    blk = (i[0] // 16, i[1], i[2]) if kind == "key" else (i[0], i[1], i[2] // 16)
    assert p.meta0[blk] == 0x7E
    c = nibbles(p.codes, x.shape[2])
    assert np.all((c >= 8) == np.signbit(xf))
    s_dec = _expand((sf / g), kind, x.shape)
    y = bf16_to_f32(oracle.unpack(p)).astype(np.float64)
    # |q| <= 6 up to the E4M3 rounding of the block scale; half-gap of E2M1 is at most 1
    q = np.abs(xf) / np.where(s_dec > 0, s_dec, 1)
    half_gap = np.where(q <= 2, 0.25, np.where(q <= 4, 0.5, 1.0))
    over = np.maximum(q - 6.0, 0)  # clamp loss when the rounded scale fell below bamax/6
    # (+ the binary32 rounding of q = x * (1 / s_dec) itself, a few ulps of q)
    bound = (half_gap + over + q * 2.0 ** -21) * s_dec + np.abs(y) * 2.0 ** -8 + 1e-12
    assert np.all(np.abs(y - xf) <= bound)
    # nibble order and axis: a single large entry only changes its own block's scale
    x2 = bf16_bits(np.ones((32, 1, 32)))
    x2[5, 0, 21] = bf16_bits(np.array([100.0]))[0]
    p2 = oracle.pack(x2, kind, "nvfp4")
    big = np.argwhere(p2.meta0 == 0x7E)
    assert big.tolist() == ([[0, 0, 21]] if kind == "key" else [[5, 0, 1]])


def test_nibble_low_first():
    x64 = np.zeros((1, 1, 4))
    x64[0, 0] = [6.0, -0.5, 1.0, -6.0]  # codes 7, 9, 2, 15
    p = oracle.pack(bf16_bits(x64), "value", "nvfp4")
    assert list(p.codes[0, 0]) == [0x97, 0xF2]


def test_error_magnitude_matches_pages_band():
    """Context, not a parity pin: the codec page reports 9.52% synthetic random-KV relative error
    for NVFP4 (shape and grouping not stated); N(0,1) V blocks land in a loose band around it."""
    rng = np.random.default_rng(3)
    x = bf16_bits(rng.standard_normal((512, 8, 128)))
    y = bf16_to_f32(oracle.unpack(oracle.pack(x, "value", "nvfp4"))).astype(np.float64)
    xf = bf16_to_f32(x).astype(np.float64)
    rel = np.linalg.norm(y - xf) / np.linalg.norm(xf)
    assert 0.07 < rel < 0.12, rel


def test_partial_blocks():
    rng = np.random.default_rng(5)
    x = bf16_bits(rng.standard_normal((37, 2, 21)))
    pk = oracle.pack(x, "key", "nvfp4")
    assert pk.meta0.shape == (3, 2, 21)
    pv = oracle.pack(x, "value", "nvfp4")
    assert pv.meta0.shape == (37, 2, 2)
    xf = bf16_to_f32(x).astype(np.float64)
    g = np.float64(pk.global_scale[0])
    # the 5-token last K block's scale follows its own amax
    bam = np.abs(xf[32:]).max(axis=0)
    s = np.minimum(np.float32(g) * (bam.astype(np.float32) / np.float32(6)), 448)
    np.testing.assert_array_equal(pk.meta0[2], oracle.f32_to_e4m3(s.astype(np.float32)))
