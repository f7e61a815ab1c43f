"""Pins of the oracle's operation order and rounding steps (CPU only).

The codec's readings fix each floating-point step as one IEEE binary32 operation rounded to
nearest even, in a stated order. Plausible slips keep every closed form and invariant intact
and move a result only where a value lands on or next to a rounding boundary: a reciprocal
multiply in place of a division, the other order of a product and a quotient, a plain `<` in
place of totalOrder for signed zeros. The tests here put inputs on those boundaries and check
the oracle against results derived in exact rational arithmetic from the definitions:

  * ``round_fraction`` rounds an exact rational to the nearest value of a binary format with
    p significand bits and smallest normal exponent emin, ties to the even significand
    (binary32: p=24, emin=-126; bf16: 8, -126; binary16: 11, -14; E4M3: 4, -6; E2M1: 2, 0).
    It shares nothing with the oracle's own conversions (which scale in double, or scan the
    E2M1 grid).
  * every step of the readings is then one ``rn32`` of the exact result of its operands.

Sources: [PR166] "Purpose" (affine FP32 groups with FP16 minimum and scale; NVFP4 with E4M3
block scales, an FP32 global multiplier and the direct-division fallback) and the first codec
review (the reference oracle had "device-dependent division handling", which is why the
division is pinned here as IEEE on every device); [PR166] "Test Plan" (signed zero, FP8 scale
rounding and nearest-even midpoints as oracle categories); [PR408] nvfp4 codec-port commit
(quantize against the stored, rounded block scale).

Each fixture also carries a self-check: the same exact-rational derivation with the slip put
in (division by reciprocal, other product order, ...) must change at least one output, so a
test that passes here would fail an oracle that made that slip.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
from workloads import bf16_bits, bf16_to_f32

TWO = Fraction(2)


def _floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0, from integer bit lengths."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if TWO ** e > a:
        e -= 1
    elif TWO ** (e + 1) <= a:
        e += 1
    return e


def round_fraction(q: Fraction, p: int, emin: int) -> Fraction:
    """Nearest value of a binary format (p significand bits, smallest normal exponent emin,
    gradual underflow below it), ties to the even significand. No overflow handling: callers
    stay inside the format's range."""
    if q == 0:
        return Fraction(0)
    sign = 1 if q > 0 else -1
    a = abs(q)
    e = max(_floor_log2(a), emin)
    quantum = TWO ** (e - p + 1)
    k = a / quantum
    n = k.numerator // k.denominator
    rem = k - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * quantum


def rn32(q: Fraction) -> Fraction:
    return round_fraction(q, 24, -126)


def rn_bf16(q: Fraction) -> Fraction:
    return round_fraction(q, 8, -126)


def fr(x) -> Fraction:
    return Fraction(float(x))


def f16_bits_of(q: Fraction) -> int:
    """binary16 bit pattern of the binary16 value nearest to q (|q| well inside the range)."""
    v = round_fraction(q, 11, -14)
    return int(np.array(float(v), np.float64).astype(np.float16).view(np.uint16))


def e4m3_byte(v: Fraction) -> int:
    """Byte of a non-negative E4M3 value (exactly representable, at most 448)."""
    if v == 0:
        return 0
    e = _floor_log2(v)
    if e < -6:
        return int(v / TWO ** -9)
    return ((e + 7) << 3) | int((v / TWO ** e - 1) * 8)


def e2m1_code(v: Fraction) -> int:
    """3-bit magnitude code of a non-negative E2M1 value (0, 0.5, 1, 1.5, 2, 3, 4, 6)."""
    if v < 1:
        return int(v * 2)
    e = _floor_log2(v)
    return 2 * (e + 1) + int((v / TWO ** e - 1) * 2)


def e2m1_value(code: int) -> Fraction:
    m = code & 7
    v = Fraction(m, 2) if m < 2 else TWO ** (m // 2 - 1) * (1 + Fraction(m % 2, 2))
    return -v if code & 8 else v


def nibbles(codes: np.ndarray, D: int) -> np.ndarray:
    lo = codes & 0xF
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(*codes.shape[:-1], -1)[..., :D]


# --------------------------------------------------------------------------------------------
# INT4: scale = fl(fl(mx - mn) / 15), code = rne(fl(fl(x - mn) / scale))
# --------------------------------------------------------------------------------------------

def int4_group_exact(members, q_recip=False, scale_recip=False):
    """Codes, f16 minimum bits and f16 scale bits of one INT4 group, in exact rationals.
    The flags put in the slips: the quotient as d * fl(1/scale), the scale as range * fl(1/15)."""
    xs = [fr(v) for v in members]
    mn, mx = min(xs), max(xs)
    rng_ = rn32(mx - mn)
    scale = rn32(rng_ * rn32(Fraction(1, 15))) if scale_recip else rn32(rng_ / 15)
    codes = []
    for x in xs:
        if scale == 0:
            codes.append(0)
            continue
        d = rn32(x - mn)
        q = rn32(d * rn32(1 / scale)) if q_recip else rn32(d / scale)
        n = q.numerator // q.denominator
        rem = q - n
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
            n += 1
        codes.append(min(max(n, 0), 15))
    return codes, f16_bits_of(mn), f16_bits_of(scale)


def near_half_groups(n_groups: int, G: int, seed: int) -> np.ndarray:
    """bf16 groups whose members sit at, and one bf16 step either side of, (2k+1)/30 of the
    group's range above its minimum: their quotients land next to k + 1/2, where the rounding
    of the division decides the code. Column 0 holds the minimum, column 1 the maximum."""
    rng = np.random.default_rng(seed)
    mn = bf16_to_f32(bf16_bits(rng.standard_normal(n_groups) * np.exp(rng.uniform(-4, 4, n_groups))))
    span = np.abs(rng.standard_normal(n_groups)) * 3 + 0.01
    mx = bf16_to_f32(bf16_bits(mn.astype(np.float64) + span * np.abs(mn.astype(np.float64)).clip(0.05)))
    k = rng.integers(0, 15, (n_groups, G - 2))
    target = mn[:, None].astype(np.float64) + (2 * k + 1) / 30.0 * (mx - mn)[:, None].astype(np.float64)
    xb = bf16_bits(target).astype(np.int32)
    step = rng.integers(-1, 2, xb.shape)
    xb = xb + np.where(target >= 0, step, -step)  # one bf16 step towards or away from zero
    x = bf16_to_f32(xb.astype(np.uint16))
    x = np.clip(x, mn[:, None], mx[:, None])  # stay inside [mn, mx]
    return bf16_bits(np.concatenate([mn[:, None], mx[:, None], x], axis=1))


@pytest.mark.parametrize("kind", ["value", "key"])
def test_int4_quotient_is_ieee_division_near_half_steps(kind):
    G, NG = 16, 1200
    groups = near_half_groups(NG, G, seed=21)  # [NG, G] bf16 bits
    x = groups.reshape(NG, 1, G) if kind == "value" else np.ascontiguousarray(groups.T).reshape(G, 1, NG)
    p = oracle.pack(x, kind, "int4", G)
    c = nibbles(p.codes, x.shape[2])
    vals = bf16_to_f32(groups)
    slip_q = slip_s = 0
    for g in range(NG):
        want, m16, s16 = int4_group_exact(vals[g])
        got = c[g, 0, :] if kind == "value" else c[:, 0, g]
        assert list(got) == want, g
        mi = (g, 0, 0) if kind == "value" else (0, 0, g)
        assert int(p.meta0[mi]) == m16 and int(p.meta1[mi]) == s16, g
        slip_q += int4_group_exact(vals[g], q_recip=True)[0] != want
        cs, _, s16s = int4_group_exact(vals[g], scale_recip=True)
        slip_s += (cs != want) or (s16s != s16)
    # the fixture would catch both slips many times over
    assert slip_q >= 20 and slip_s >= 20, (slip_q, slip_s)


# (minimum, maximum) bf16 pairs whose scale fl(range / 15) lies next to a binary16 rounding
# boundary, so that fl(range * fl(1/15)) stores a different f16 scale; each pair's f16 scale
# bits under the IEEE division, derived below in exact rationals.
F16_BOUNDARY_PAIRS = [(0x3C1D, 0x402C, 0x31B6), (0x3C85, 0x4094, 0x34EA), (0xBCC7, 0x40A1, 0x3564),
                      (0xBFA5, 0xBBA5, 0x2D7A), (0xBF8D, 0x3B9F, 0x2CB8), (0xBCAF, 0x40B9, 0x3630)]


def test_int4_f16_scale_at_binary16_boundaries():
    mn_b = np.array([p[0] for p in F16_BOUNDARY_PAIRS], np.uint16)
    mx_b = np.array([p[1] for p in F16_BOUNDARY_PAIRS], np.uint16)
    mid = bf16_bits((bf16_to_f32(mn_b).astype(np.float64) + bf16_to_f32(mx_b)) / 2)
    groups = np.stack([mn_b, mx_b, mid, mid], axis=1)  # VALUE groups of 4 channels
    p = oracle.pack(groups.reshape(-1, 1, 4), "value", "int4", 4)
    for i, (a, b, want16) in enumerate(F16_BOUNDARY_PAIRS):
        _, _, s16 = int4_group_exact(bf16_to_f32(groups[i]))
        assert s16 == want16  # the table agrees with the exact derivation
        assert int4_group_exact(bf16_to_f32(groups[i]), scale_recip=True)[2] != want16  # discriminating
        assert int(p.meta1[i, 0, 0]) == want16


# --------------------------------------------------------------------------------------------
# Signed zeros: group minimum in IEEE totalOrder (-0 < +0), whatever the scan order
# --------------------------------------------------------------------------------------------

@pytest.mark.parametrize("kind", ["value", "key"])
@pytest.mark.parametrize("first", [0.0, -0.0])
def test_int4_minimum_of_mixed_signed_zeros(kind, first):
    # Groups whose minimum is a zero of either sign, with +0 and -0 both present, scanned with
    # either zero first. totalOrder puts -0 below +0, so the stored minimum is -0 (f16 0x8000)
    # in both orders; with a plain `<` the first zero met would win.
    second = -first
    rows = [
        [first, second, 1.0, 2.0],          # minimum -0, maximum 2
        [first, second, 0.0, 0.0],          # all zeros: minimum -0, scale 0
        [2.0, first, 3.0, second],          # zeros after a positive member
    ]
    g = np.array(rows, np.float64)
    bits = bf16_bits(g)
    assert all(0x0000 in r and 0x8000 in r for r in bits.tolist())  # both zeros in every group
    x = bits.reshape(3, 1, 4) if kind == "value" else np.ascontiguousarray(bits.T).reshape(4, 1, 3)
    p = oracle.pack(x, kind, "int4", 4)
    m16 = p.meta0[:, 0, 0] if kind == "value" else p.meta0[0, 0, :]
    assert m16.tolist() == [0x8000, 0x8000, 0x8000]
    s16 = p.meta1[:, 0, 0] if kind == "value" else p.meta1[0, 0, :]
    assert s16[1] == 0  # an all-zero group has scale +0 (+0 - (-0) = +0)
    # a group of negatives with both zeros on top: the minimum is the negative member, and the
    # zeros code to 15 from either sign (-0.5 sits at 7.4999996 steps: fl(1/15 * 1) rounds up)
    neg = bf16_bits(np.array([[first, -1.0, second, -0.5]]))
    pn = oracle.pack(neg.reshape(1, 1, 4), "value", "int4", 4)
    assert nibbles(pn.codes, 4)[0, 0].tolist() == [15, 0, 15, 7] == int4_group_exact(bf16_to_f32(neg[0]))[0]
    assert int(pn.meta0[0, 0, 0]) == 0xBC00  # f16 -1.0


# --------------------------------------------------------------------------------------------
# NVFP4: g = fl(2688 / amax); s = min(fl(g * fl(bamax / 6)), 448); sc8 = e4m3(s);
#        s_dec = fl(sf / g); q = fl(x * fl(1 / s_dec)) (or fl(x / s_dec) when that overflows);
#        code = e2m1(min(|q|, 6)) with the sign of x; decode bf16(fl(v * fl(sf / g)))
# --------------------------------------------------------------------------------------------

SLIPS = ("order", "recip6", "recip_amax", "sdec_recip", "q_div", "dec_order", "sf0_passthrough")


def nvfp4_block_exact(amax, members, slip=None):
    """(block-scale byte, member codes, decoded members) of one NVFP4 block of a tensor whose
    amax is `amax`, in exact rationals, optionally with one slip from SLIPS. `members` are
    float32 values (their sign bits give the code signs, zeros included)."""
    members = np.asarray(members, np.float32)
    signs = np.signbit(members)
    a = fr(amax)
    g = rn32(2688 * rn32(1 / a)) if slip == "recip_amax" else rn32(2688 / a)
    xs = [fr(v) for v in members]
    bamax = max(abs(x) for x in xs)
    if slip == "order":
        s = rn32(rn32(g * bamax) / 6)
    elif slip == "recip6":
        s = rn32(g * rn32(bamax * rn32(Fraction(1, 6))))
    else:
        s = rn32(g * rn32(bamax / 6))
    s = min(s, Fraction(448))
    sf = round_fraction(s, 4, -6)
    byte = e4m3_byte(sf)
    sdec = rn32(sf * rn32(1 / g)) if slip == "sdec_recip" else rn32(sf / g)
    codes, dec = [], []
    for x, neg in zip(xs, signs):
        if sf == 0:
            q = x if slip == "sf0_passthrough" else Fraction(0)
        elif slip == "q_div":
            q = rn32(x / sdec)
        else:
            q = rn32(x * rn32(1 / sdec))  # 1/s_dec stays finite for every sdec here
        m = min(abs(q), Fraction(6))
        c = e2m1_code(round_fraction(m, 2, 0)) | (8 if neg else 0)
        codes.append(c)
        v = e2m1_value(c)
        y = rn32(rn32(v * sf) / g) if slip == "dec_order" else rn32(v * sdec)
        dec.append(rn_bf16(y))
    return byte, codes, dec


def nvfp4_case_tensor(amax_bits: int, members_bits: np.ndarray) -> np.ndarray:
    """VALUE tensor [1, 1, 32]: block 0 = the 16 members, block 1 = the amax element and zeros."""
    x = np.zeros((1, 1, 32), np.uint16)
    x[0, 0, :16] = members_bits
    x[0, 0, 16] = amax_bits
    return x


def midpoint_members(amax: float, bamax: float) -> np.ndarray:
    """bamax, then members at every E2M1 midpoint times the block's decode scale (rounded to
    bf16), one bf16 step above each, and one negative midpoint member: their scaled values land
    on or next to E2M1 rounding ties."""
    a, b = fr(amax), fr(bamax)
    g = rn32(2688 / a)
    sf = round_fraction(min(rn32(g * rn32(b / 6)), Fraction(448)), 4, -6)
    sdec = float(rn32(sf / g)) if sf else 0.0
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]) * sdec
    mb = bf16_bits(mids)
    up = (mb.astype(np.int32) + 1).astype(np.uint16)
    neg = bf16_bits(np.array([-2.5 * sdec]))
    m = np.concatenate([bf16_bits(np.array([bamax])), mb, up, neg])
    v = bf16_to_f32(m)
    m[np.abs(v) > bamax] = bf16_bits(np.array([bamax]))[0]  # never raise the block maximum
    return m


def check_case(amax_bits: int, members_bits: np.ndarray):
    x = nvfp4_case_tensor(amax_bits, members_bits)
    p = oracle.pack(x, "value", "nvfp4")
    amax = bf16_to_f32(np.array([amax_bits], np.uint16))[0]
    mem = bf16_to_f32(members_bits)
    byte, codes, dec = nvfp4_block_exact(amax, mem)
    assert float(p.global_scale[0]) == float(rn32(2688 / fr(amax)))
    assert int(p.meta0[0, 0, 0]) == byte
    assert nibbles(p.codes, 32)[0, 0, :16].tolist() == codes
    y = bf16_to_f32(oracle.unpack(p))[0, 0, :16]
    assert [Fraction(float(v)) for v in y] == dec
    # signs of zero survive the decode as well
    assert [bool(np.signbit(v)) for v in y] == [bool(c & 8) for c in codes]
    return byte, codes, dec


def test_nvfp4_hand_derived_block_scales():
    """Three blocks worked by hand (the bytes below follow from exact arithmetic):

    1. amax 17.5, bamax 0.205078125 (= 105 * 2^-9). g = RN(2688/17.5) = RN(153.6)
       = 10066330 * 2^-16. bamax/6 = 35 * 2^-10 exactly, and g * that = 5.25000008...,
       which rounds to exactly 5.25: the E4M3 midpoint between 5.0 and 5.5, tie to the even
       mantissa -> 5.0 = byte 0x4A. The other order, fl(fl(g * bamax) / 6), gives
       fl(31.5000019) / 6 -> 5.25000048 -> 5.5 = 0x4B.
    2. amax 28 (g = 96 exactly), bamax 0.390625 (= 25 * 2^-6). fl(bamax / 6) = RN(25/384);
       96 * that rounds to exactly 6.25, the midpoint between 6.0 and 6.5 -> 6.0 = 0x4C. With
       bamax * fl(1/6) instead, 6.25000048 -> 6.5 = 0x4D.
    3. amax 5.25 (g = 512 exactly), bamax 2.8125: bamax / 6 = 0.46875 exactly, s = 240 = 0x77,
       s_dec = 0.46875, and fl(1 / s_dec) = RN(32/15) = 8947849 * 2^-22, 5.2e-8 above 32/15.
       The members 1.25, 2.5 and 5 times s_dec (0.5859375, 1.171875, 2.34375) therefore
       scale to just above the E2M1 ties 1.25, 2.5 and 5 and take codes 3 (1.5), 5 (3.0) and
       7 (6.0); divided by s_dec they would be exact ties, rounding down to codes 2, 4 and 6.
    """
    # 1
    m1 = np.full(16, bf16_bits(np.array([0.1]))[0], np.uint16)
    m1[3] = bf16_bits(np.array([0.205078125]))[0]
    byte, _, _ = check_case(int(bf16_bits(np.array([17.5]))[0]), m1)
    assert byte == 0x4A
    assert nvfp4_block_exact(17.5, bf16_to_f32(m1), "order")[0] == 0x4B
    # 2
    m2 = np.zeros(16, np.uint16)
    m2[0] = bf16_bits(np.array([0.390625]))[0]
    byte, _, _ = check_case(int(bf16_bits(np.array([28.0]))[0]), m2)
    assert byte == 0x4C
    assert nvfp4_block_exact(28.0, bf16_to_f32(m2), "recip6")[0] == 0x4D
    # 3
    m3 = np.zeros(16, np.uint16)
    m3[:4] = bf16_bits(np.array([2.8125, 0.5859375, 1.171875, 2.34375]))
    byte, codes, _ = check_case(int(bf16_bits(np.array([5.25]))[0]), m3)
    assert byte == 0x77 and codes[:4] == [7, 3, 5, 7]
    assert nvfp4_block_exact(5.25, bf16_to_f32(m3), "q_div")[1][:4] == [7, 2, 4, 6]


def test_nvfp4_zero_block_scale_gives_signed_zero_codes():
    """A block far below the tensor amax: amax 2^20 gives g = 2688 * 2^-20 = 21 * 2^-13 exactly;
    a block with bamax 1 has s = fl(g * fl(1/6)) ~ 4.3e-4, under half the smallest E4M3
    subnormal (2^-10), so its scale byte is 0 and every member codes to a zero of its own sign
    (0x0 / 0x8) even though the members themselves are far from zero."""
    m = bf16_bits(np.array([1.0, -0.75, 0.5, -1.0, 0.0, -0.0, 0.3, -0.2] * 2))
    byte, codes, dec = check_case(int(bf16_bits(np.array([2.0 ** 20]))[0]), m)
    assert byte == 0
    assert codes == [0, 8, 0, 8, 0, 8, 0, 8] * 2
    assert nvfp4_block_exact(2.0 ** 20, bf16_to_f32(m), "sf0_passthrough")[1] != codes


# (amax, bamax) pairs found by a search over bf16 values, on which a slip changes the block
# scale byte or a decoded value; each row names the slip it discriminates.
NVFP4_BOUNDARY_CASES = [
    (17.5, 0.1220703125, "order"), (1.15625, 0.216796875, "order"), (148.0, 0.43359375, "order"),
    (19.25, 0.365234375, "recip6"), (24.5, 0.1708984375, "recip6"),
    (7.0, 5.25, "recip_amax"), (664.0, 249.0, "recip_amax"), (0.40625, 0.3046875, "recip_amax"),
    (3.828125, 2.421875, "sdec_recip"), (21.875, 4.90625, "sdec_recip"),
    (294.0, 77.0, "dec_order"), (490.0, 234.0, "dec_order"),
]


def test_nvfp4_rounding_boundaries_exact_rational():
    rng = np.random.default_rng(33)
    cases = [(float(a), float(b)) for a, b, _ in NVFP4_BOUNDARY_CASES]
    amax = bf16_to_f32(bf16_bits(np.exp(rng.uniform(-6, 9, 300))))
    bam = bf16_to_f32(bf16_bits(amax.astype(np.float64) * rng.uniform(0.002, 1.0, 300)))
    cases += list(zip(amax.tolist(), bam.tolist()))
    hits = dict.fromkeys(SLIPS, 0)
    for a, b in cases:
        mem = midpoint_members(a, b)
        want = check_case(int(bf16_bits(np.array([a]))[0]), mem)
        for slip in SLIPS:
            hits[slip] += nvfp4_block_exact(a, bf16_to_f32(mem), slip) != want
    for a, b, slip in NVFP4_BOUNDARY_CASES:  # each listed pair discriminates its slip
        mem = midpoint_members(a, b)
        assert nvfp4_block_exact(a, bf16_to_f32(mem), slip) != nvfp4_block_exact(a, bf16_to_f32(mem)), (a, b, slip)
    # every slip but the zero-scale one (pinned above) changes outputs somewhere in the fixture
    assert all(hits[s] >= 2 for s in SLIPS if s != "sf0_passthrough"), hits
