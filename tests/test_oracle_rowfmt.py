"""Pins of the oracle's row formats (CPU only): NVFP4 with one FP32 multiplier per (token, head)
row, and FP8 E4M3 with one FP32 scale per row (FreeToken pull request #408: "Summary", the fp8
commit and the nvfp4 codec-port commit).

What pins them:
  * FP8-row against torch's own float8_e4m3fn conversion: the scale is one float32 division,
    the scaled values one float32 division each (numpy), clipped to +-448 and cast by torch;
    the decode is torch's float8 -> float32 widening, one float32 product and torch's bf16
    rounding. Rows cover six decades of magnitude, bf16 subnormals, signed zeros and all-zero
    rows;
  * FP8-row closed form: E4M3 grid values times 2^k with amax 448 * 2^k give scale 2^k and an
    exact round trip;
  * NVFP4-row is, row by row, exactly the (separately pinned) per-tensor NVFP4 encoding of that
    one (token, head) row taken as its own tensor: same codes, same E4M3 block scales, and the
    row multiplier equals that tensor's multiplier;
  * NVFP4-row closed form: a row of E2M1 grid values with amax 6 has multiplier 448, block
    scales 1.0 and an exact round trip; an all-zero row has multiplier 1 and zero codes;
  * both row formats ignore the K/V kind (their groups run along channels for either);
  * error bound: FP8 within half an E4M3 step of the scaled value (the NVFP4 bound carries over
    from the per-tensor format through the row-by-row identity above).
Storage of both formats is pinned in test_oracle_storage.py, residual pairings in
test_oracle_residual.py.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits, bf16_to_f32, normal_kv


def varied_rows(seed, T=40, H=3, D=48):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H, D)) * 10.0 ** rng.uniform(-3, 3, (T, H, 1))
    x[0, 0] = 0.0                      # all-zero row
    x[1, H - 1] = -0.0                 # all negative zeros
    x[2, H - 1, ::3] = -0.0            # signed zeros inside a row
    x[3, 0] *= 2.0 ** -128             # bf16 subnormals (scale subnormal in float32)
    x[4, H - 1, :] = 0.0
    x[4, H - 1, 7] = -3.0e-39          # one tiny nonzero value
    return bf16_bits(x)


def torch_fp8_row(x_bits):
    x = bf16_to_f32(x_bits)
    amax = np.abs(x).max(axis=2)
    s = (amax / np.float32(448.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        q = (x / s[..., None]).astype(np.float32)
    q = np.where(s[..., None] == 0, np.copysign(np.float32(0.0), x), q)
    q = np.clip(q, -448.0, 448.0).astype(np.float32)
    codes = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    dec = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32) * torch.from_numpy(s)[..., None]
    y = dec.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return codes, s, y


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("kind", ["key", "value"])
def test_fp8_row_matches_torch_float8(seed, kind):
    x = varied_rows(seed)
    codes, s, y = torch_fp8_row(x)
    p = oracle.pack(x, kind, "fp8_row", 0)
    np.testing.assert_array_equal(p.meta0, s)
    np.testing.assert_array_equal(p.codes, codes)
    np.testing.assert_array_equal(oracle.unpack(p), y)


def test_fp8_row_strided_view():
    base = varied_rows(5, T=12, H=4, D=64)
    big = np.zeros((12, 3, 4, 64), np.uint16)
    big[:, 1] = base
    view = big[:, 1]
    a, b = oracle.pack(view, "value", "fp8_row", 0), oracle.pack(base, "value", "fp8_row", 0)
    np.testing.assert_array_equal(a.codes, b.codes)
    np.testing.assert_array_equal(a.meta0, b.meta0)


def e4m3_grid():
    vals = sorted({oracle.e4m3_to_f32(b) for b in range(0x7F)})  # non-negative finite codes
    return np.array(vals, np.float64)


@pytest.mark.parametrize("k", [-20, -3, 0, 5, 40])
def test_fp8_row_grid_round_trip(k):
    rng = np.random.default_rng(k + 100)
    grid = e4m3_grid()
    D = 64
    x = rng.choice(grid, (6, 2, D)) * rng.choice([-1.0, 1.0], (6, 2, D))
    x[..., 0] = 448.0  # amax = 448 -> scale 1 before the 2^k shift
    x = x * 2.0 ** k
    xb = bf16_bits(x)
    assert np.array_equal(bf16_to_f32(xb).astype(np.float64), x)  # grid * 2^k is bf16-exact
    p = oracle.pack(xb, "value", "fp8_row", 0)
    assert np.all(p.meta0 == np.float32(2.0 ** k))
    np.testing.assert_array_equal(oracle.unpack(p), xb)


def test_fp8_row_error_bound():
    x = normal_kv(np.random.default_rng(7), 64, 2, 128)
    p = oracle.pack(x, "value", "fp8_row", 0)
    xf = bf16_to_f32(x).astype(np.float64)
    s = p.meta0.astype(np.float64)[..., None]
    q = xf / s
    deq = np.array([oracle.e4m3_to_f32(int(c)) for c in p.codes.ravel()]).reshape(q.shape)
    # an E4M3 step is at most 2^-3 of the value above 2^-6, and 2^-9 below (subnormals)
    step = np.maximum(np.abs(q) * 2.0 ** -3, 2.0 ** -9)
    assert np.all(np.abs(deq - q) <= 0.5 * step + 1e-12)


@pytest.mark.parametrize("kind", ["key", "value"])
@pytest.mark.parametrize("D", [16, 40, 128])
def test_nvfp4_row_is_per_row_tensor_encoding(kind, D):
    x = varied_rows(11, T=9, H=3, D=D)
    p = oracle.pack(x, kind, "nvfp4_row", 16)
    y = oracle.unpack(p)
    for t in range(9):
        for h in range(3):
            one = oracle.pack(np.ascontiguousarray(x[t:t + 1, h:h + 1, :]), "value", "nvfp4", 16)
            np.testing.assert_array_equal(p.codes[t, h], one.codes[0, 0])
            np.testing.assert_array_equal(p.meta0[t, h], one.meta0[0, 0])
            assert p.meta1[t, h] == one.global_scale[0]
            np.testing.assert_array_equal(y[t, h], oracle.unpack(one)[0, 0])


def test_nvfp4_row_closed_forms():
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float64)
    rng = np.random.default_rng(3)
    x = rng.choice(grid, (4, 2, 32)) * rng.choice([-1.0, 1.0], (4, 2, 32))
    x[..., 0] = 6.0
    x[..., 16] = -6.0
    x[3, 1] = 0.0
    xb = bf16_bits(x)
    p = oracle.pack(xb, "value", "nvfp4_row", 16)
    assert np.all(p.meta1[:3] == 448.0) and p.meta1[3, 0] == 448.0 and p.meta1[3, 1] == 1.0
    # block scale: min(448 * 6/6, 448) = 448 -> E4M3 0x7E; s_dec = 448 / 448 = 1
    assert np.all(p.meta0[:3] == 0x7E) and np.all(p.meta0[3, 0] == 0x7E)
    assert np.all(p.meta0[3, 1] == 0) and np.all(p.codes[3, 1] == 0)
    y = oracle.unpack(p)
    np.testing.assert_array_equal(y[:3], xb[:3])  # exact, -0 included (code 0x8 decodes to -0.0)


@pytest.mark.parametrize("fmt,G", [("nvfp4_row", 16), ("fp8_row", 0)])
def test_row_formats_ignore_kind(fmt, G):
    x = varied_rows(21, T=17, H=2, D=32)
    a, b = oracle.pack(x, "key", fmt, G), oracle.pack(x, "value", fmt, G)
    np.testing.assert_array_equal(a.codes, b.codes)
    np.testing.assert_array_equal(a.meta0, b.meta0)
    np.testing.assert_array_equal(oracle.unpack(a), oracle.unpack(b))


def test_row_format_group_sizes_rejected():
    x = normal_kv(np.random.default_rng(0), 4, 1, 32)
    with pytest.raises(ValueError):
        oracle.pack(x, "value", "nvfp4_row", 32)
    with pytest.raises(ValueError):
        oracle.pack(x, "value", "fp8_row", 16)
