// kvq_device.hpp -- device-side numerics of the KV codec (gfx950).
//
// Roundings come in two forms. The integer formulations (namespace kvq::ref) are written from
// the format definitions; the gfx950 conversion instructions used on the hot path
// (v_cvt_pk_bf16_f32, v_cvt_f16_f32, v_cvt_scalef32_pk_fp4_f32 and v_cvt_scalef32_pk_f32_fp4)
// were checked against them for every binary32 input (tests/probes/cvt_probe.hip) and are only
// used where that check holds. Floating-point steps that the format defines as single binary32
// operations are written as separate __fadd_rn/__fmul_rn/__fsub_rn calls (the library is also
// built with -ffp-contract=off), and divisions use the IEEE-correct '/' (the library is built
// with correctly rounded fp32 division and keeps denormals).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

// ---- bf16 ------------------------------------------------------------------------------------

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

namespace ref {
// binary32 -> bf16, round to nearest even (integer formulation). Valid for every non-NaN
// input; values past the largest finite bf16 (by at least half an ulp) give +-inf.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
}  // namespace ref

// Two binary32 values -> two bf16 (low element first), round to nearest even, one
// v_cvt_pk_bf16_f32 (identical to ref::f32_to_bf16 on every non-NaN input).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// bf16 bits of x (round to nearest even)
__device__ __forceinline__ uint32_t bf16_bits(float x) { return pack_bf16x2(x, x) & 0xFFFFu; }

// bf16(fl(a - b)) for the two halves of packed words: the residual subtraction in the input
// dtype ([PR166] "Purpose", fourth bullet).
__device__ __forceinline__ uint32_t sub_bf16x2(uint32_t a, uint32_t b) {
    return pack_bf16x2(__fsub_rn(bf16lo(a), bf16lo(b)), __fsub_rn(bf16hi(a), bf16hi(b)));
}

// Streaming 16-byte load of data read once (non-temporal hint).
__device__ __forceinline__ u32x4 ld_stream(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Wave-uniform global addresses held in SGPRs (opaque to the optimizer), to which a lane adds a
// 32-bit byte offset inside the memory instruction (the scalar-base form of global loads and
// stores): a per-row address then costs scalar instructions only, instead of a 64-bit vector add
// per lane. `p + off` must be the same on every lane of the wave.
typedef const __attribute__((address_space(1))) uint8_t* wave_cptr;
typedef __attribute__((address_space(1))) uint8_t* wave_ptr;

__device__ __forceinline__ uint64_t wave_uniform_u64(uint64_t v) {
    // readfirstlane returns a signed int: widen through uint32_t, never by sign extension
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    return ((uint64_t)hi << 32) | (uint64_t)lo;
}

__device__ __forceinline__ wave_cptr wave_base(const void* p, int64_t off_bytes) {
    wave_cptr b = (wave_cptr)wave_uniform_u64(reinterpret_cast<uint64_t>(static_cast<const uint8_t*>(p) + off_bytes));
    asm("" : "+s"(b));
    return b;
}

__device__ __forceinline__ wave_ptr wave_base_w(void* p, int64_t off_bytes) {
    wave_ptr b = (wave_ptr)wave_uniform_u64(reinterpret_cast<uint64_t>(static_cast<uint8_t*>(p) + off_bytes));
    asm("" : "+s"(b));
    return b;
}

// Streaming 16-byte load at a wave-uniform base plus a lane's byte offset.
__device__ __forceinline__ u32x4 ld_stream_at(wave_cptr base, uint32_t off) {
    return __builtin_nontemporal_load(reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(base + off));
}

// Store of packed codes: non-temporal when NT. The encoders pass NT for a plain pack, whose
// codes are written once and not read back by the same pass; measured on the bulk shape this
// frees the caches for the input stream (INT4 pack 71 -> 66 us). With a residual's second input
// stream the hint slowed the encode, so residual encodes store normally.
template <bool NT, class T>
__device__ __forceinline__ void st_code(T* p, T w) {
    if constexpr (NT)
        __builtin_nontemporal_store(w, p);
    else
        *p = w;
}

// The same at a wave-uniform base plus a lane's byte offset. (The offset passes through an
// empty asm at each store so that the compiler does not widen it once into a 64-bit register
// pair and add the base in vector registers, which would lose the scalar-base form.)
template <bool NT, class T>
__device__ __forceinline__ void st_code_at(wave_ptr base, uint32_t off, T w) {
    asm("" : "+v"(off));
    auto* p = reinterpret_cast<__attribute__((address_space(1))) T*>(base + off);
    if constexpr (NT)
        __builtin_nontemporal_store(w, p);
    else
        *p = w;
}

// ---- f16 (INT4 metadata) --------------------------------------------------------------------

namespace ref {
// binary32 -> binary16 bits, round to nearest even, gradual underflow, overflow to inf
// (integer formulation).
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
    uint32_t x = __float_as_uint(f);
    uint32_t sign = (x >> 16) & 0x8000u;
    uint32_t ax = x & 0x7FFFFFFFu;
    if (ax >= 0x477FF000u) return sign | 0x7C00u;  // >= 65520: rounds to inf
    if (ax >= 0x38800000u) {                        // >= 2^-14: normal half
        uint32_t r = ax + 0x0FFFu + ((ax >> 13) & 1u);
        return sign | ((r >> 13) - (112u << 10));
    }
    // subnormal half: multiple of 2^-24; scaling by 2^24 is exact, rint is nearest-even
    float a = __uint_as_float(ax) * 16777216.0f;
    return sign | (uint32_t)__builtin_rintf(a);
}
}  // namespace ref

// binary32 -> binary16 bits with v_cvt_f16_f32 (identical to ref::f32_to_f16 on every non-NaN
// input, subnormals and overflow included).
__device__ __forceinline__ uint32_t f32_to_f16(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// binary16 bits -> binary32 (exact; f16 subnormals are kept by the denormal mode).
__device__ __forceinline__ float f16_to_f32(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

// ---- E4M3 (NVFP4 block scales) --------------------------------------------------------------

// Non-negative binary32 s <= 448 -> E4M3fn code, nearest even, with E4M3 subnormals (k * 2^-9).
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
    uint32_t x = __float_as_uint(s);
    if (x >= 0x3C800000u) {  // s >= 2^-6: 3 mantissa bits, rebias exponent 127 -> 7
        uint32_t r = x + 0x7FFFFu + ((x >> 20) & 1u);
        return (r >> 20) - (120u << 3);
    }
    return (uint32_t)__builtin_rintf(s * 512.0f);  // exact scaling, then nearest-even
}

// e4m3_encode(s) for 0 <= s <= 448 in one instruction: v_cvt_pk_fp8_f32, which the device probe
// shows equal to e4m3_encode(|v|) with the sign bit of v for every binary32 |v| <= 448.
__device__ __forceinline__ uint32_t e4m3_encode_hw(float s) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(s, s, 0, false) & 0xFFu;
}

// E4M3fn code (sign bit clear, finite) -> binary32, exact.
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
    uint32_t E = (b >> 3) & 0xFu, M = b & 7u;
    if (E == 0) return (float)M * 0.001953125f;  // M * 2^-9
    return __uint_as_float(((E + 120u) << 23) | (M << 20));
}

// ---- E2M1 (NVFP4 codes) ---------------------------------------------------------------------

namespace ref {
// Magnitude code of |q| on {0, .5, 1, 1.5, 2, 3, 4, 6}, nearest with ties to the even code:
// the half-way points 0.25, 1.25, 2.5, 5 go down, 0.75, 1.75, 3.5 go up; anything above 5
// saturates to 6 (code 7). Written as threshold counts.
__device__ __forceinline__ uint32_t e2m1_mag(float q) {
    float m = __builtin_fabsf(q);
    return (uint32_t)(m > 0.25f) + (uint32_t)(m >= 0.75f) + (uint32_t)(m > 1.25f) + (uint32_t)(m >= 1.75f) +
           (uint32_t)(m > 2.5f) + (uint32_t)(m >= 3.5f) + (uint32_t)(m > 5.0f);
}

// Signed E2M1 code -> binary32 value (exact): exponent bits 2..1 with bias 1, mantissa bit 0,
// subnormal 0.5; bit 3 is the sign.
__device__ __forceinline__ float e2m1_value(uint32_t c) {
    uint32_t e = (c >> 1) & 3u, m = c & 1u;
    uint32_t mag = (e == 0) ? (m ? 0x3F000000u : 0u) : (((e + 126u) << 23) | (m << 22));
    return __uint_as_float(mag | ((c & 8u) << 28));
}
}  // namespace ref

// Two scaled values -> one byte of two E2M1 codes (first value in the low nibble), written into
// byte SEL of `word`: v_cvt_scalef32_pk_fp4_f32 with scale 1, which equals ref::e2m1_mag with
// the sign bit of the value for every finite input (saturating above 5, signed zeros kept).
template <int SEL>
__device__ __forceinline__ uint32_t e2m1_pair(uint32_t word, float q0, float q1) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q0, q1, 1.0f, SEL);
}

// The two E2M1 values of byte SEL of `word` (low nibble first): v_cvt_scalef32_pk_f32_fp4 with
// scale 1, equal to ref::e2m1_value for all 16 codes.
template <int SEL>
__device__ __forceinline__ f32x2 e2m1_values(uint32_t word) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
}

// ---- division by the format constants -----------------------------------------------------

// fl(x / K) for x >= 0 and K in {15, 6}, from one multiply by fl(1/K) and one FMA correction:
// q0 = fl(x * c), r = fma(-K, q0, x) (exact), q = fma(r, c, q0). The result equals the IEEE
// quotient for every non-negative binary32 of at least 2^-100 (tests/probes/cvt_probe.hip checks
// all of them); smaller x take the division.
template <int K>
__device__ __forceinline__ float div_const(float x) {
    constexpr float c = 1.0f / (float)K;
    if (__builtin_expect(x < 7.888609052210118e-31f, 0)) return x / (float)K;  // x < 2^-100
    const float q0 = __fmul_rn(x, c);
    const float r = __builtin_fmaf(-(float)K, q0, x);
    return __builtin_fmaf(r, c, q0);
}

// Approximate reciprocal (v_rcp_f32, within one ulp of fl(1/x) for normal x with a normal
// reciprocal, as the probe checks); used only where a bounded error is allowed.
__device__ __forceinline__ float rcp_approx(float x) { return __builtin_amdgcn_rcpf(x); }

// ---- sortable keys --------------------------------------------------------------------------

// bf16 bit pattern -> int with the order of IEEE totalOrder on finite values (-0 < +0):
// negative patterns have their magnitude bits inverted.
__device__ __forceinline__ int bf16_key(uint32_t b16) {
    int s = (int)(int16_t)(uint16_t)b16;
    return s ^ ((s >> 31) & 0x7FFF);
}
// inverse of bf16_key (an involution on the low 16 bits)
__device__ __forceinline__ float key_to_f32(int k) {
    uint32_t b = (uint32_t)(k ^ ((k >> 31) & 0x7FFF)) & 0xFFFFu;
    return __uint_as_float(b << 16);
}

// Packed 16-bit lanes: two keys per 32-bit word.
typedef short short2_t __attribute__((ext_vector_type(2)));
typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ short2_t as_s2(uint32_t w) { return __builtin_bit_cast(short2_t, w); }
__device__ __forceinline__ uint32_t s2_as_u(short2_t v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ ushort2_t as_us2(uint32_t w) { return __builtin_bit_cast(ushort2_t, w); }
__device__ __forceinline__ uint32_t us2_as_u(ushort2_t v) { return __builtin_bit_cast(uint32_t, v); }

// keys of the two bf16 halves of a word (per-half arithmetic shift, mask, xor)
__device__ __forceinline__ short2_t keys2(uint32_t w) {
    short2_t v = as_s2(w);
    short2_t sgn = v >> (short2_t){15, 15};
    return v ^ (sgn & (short2_t){0x7FFF, 0x7FFF});
}
// The same order as unsigned 16-bit keys (the signed key with its top bit flipped), so that the
// two halves of a word combine with one zero-extending half-word min or max.
__device__ __forceinline__ uint32_t ukeys2(uint32_t w) {
    const uint32_t sgn = s2_as_u(as_s2(w) >> (short2_t){15, 15});  // 0xFFFF in each negative half
    return w ^ (sgn | 0x80008000u);
}
__device__ __forceinline__ float ukey_to_f32(uint32_t k) { return key_to_f32((int)(int16_t)(uint16_t)(k ^ 0x8000u)); }
__device__ __forceinline__ ushort2_t umin2(ushort2_t a, ushort2_t b) { return __builtin_elementwise_min(a, b); }
__device__ __forceinline__ short2_t min2(short2_t a, short2_t b) { return __builtin_elementwise_min(a, b); }
__device__ __forceinline__ short2_t max2(short2_t a, short2_t b) { return __builtin_elementwise_max(a, b); }
__device__ __forceinline__ ushort2_t umax2(ushort2_t a, ushort2_t b) { return __builtin_elementwise_max(a, b); }
// magnitudes |x| of both halves as unsigned 16-bit patterns (order of |x| = unsigned order)
__device__ __forceinline__ ushort2_t mag2(uint32_t w) { return as_us2(w & 0x7FFF7FFFu); }

// ---- cross-lane (DPP) -----------------------------------------------------------------------

// Row-local data-parallel-primitive moves, every lane active: quad_perm [1,0,3,2] = 0xB1
// (xor 1), [2,3,0,1] = 0x4E (xor 2), row_half_mirror = 0x141 (i -> 7-i within 8), row_mirror =
// 0x140 (i -> 15-i within 16), row_ror:n = 0x120 + n (rotation within 16; n = 8 pairs i with
// i xor 8). All read a valid lane of the same row, so the bound value (0) is
// never used; asking for it (old = 0, bound_ctrl) lets the compiler fold the move into the
// instruction that consumes it (v_min_u32_dpp and the like).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    static_assert((CTRL >= 0x00 && CTRL <= 0xFF) || (CTRL >= 0x121 && CTRL <= 0x12F) || CTRL == 0x140 || CTRL == 0x141,
                  "in-row permutations only");
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

// All-reduce over aligned groups of `lanes` lanes (1, 2, 4, 8 or 16; uniform across the wave).
template <typename Op>
__device__ __forceinline__ uint32_t group_allreduce(uint32_t v, int lanes, Op op) {
    if (lanes >= 2) v = op(v, dpp<0xB1>(v));
    if (lanes >= 4) v = op(v, dpp<0x4E>(v));
    if (lanes >= 8) v = op(v, dpp<0x141>(v));
    if (lanes >= 16) v = op(v, dpp<0x140>(v));
    return v;
}

// ---- block order ------------------------------------------------------------------------------

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2). This maps the
// hardware block id to a logical one so that every XCD works on one contiguous range of
// logical blocks (a bijection on [0, n)); neighbouring tasks that share data then share an L2.
__device__ __forceinline__ uint32_t xcd_block(uint32_t b, uint32_t n) {
    const uint32_t x = b & 7u, i = b >> 3, q = n >> 3, r = n & 7u;
    return (x < r) ? x * (q + 1u) + i : r * (q + 1u) + (x - r) * q + i;
}

// ---- integer division by a runtime constant --------------------------------------------------

// n / d for 32-bit n with a precomputed multiplier (round-up method): t = mulhi(n, m),
// q = (t + n) >> s, evaluated in 64 bits. Host side fills it with fastdiv_make().
struct FastDiv {
    uint32_t d, m, s, pad;
};
__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
    uint32_t t = __umulhi(n, f.m);
    return (uint32_t)(((uint64_t)t + n) >> f.s);
}

// ---- INT4 element code ----------------------------------------------------------------------

// The codes need rne(fl(d / scale)) bit for bit, where d = fl(x - mn). fl(d / scale) lands on a
// half-integer (and then rounds to even) far more often than chance, because fl(range / 15)
// is within half an ulp of range / 15, so a quotient is exact only if it is correctly rounded.
// This is done without a division or a branch by Markstein's theorem (P. Markstein, IBM J.
// Res. Dev. 34(1), 1990; also the Handbook of Floating-Point Arithmetic, division chapter): if
// y = RN(1/b) and q is a faithful approximation of a/b, then r = a - b*q is exact under FMA and
// RN(q + r*y) = RN(a/b).
//  * y: one Newton step on v_rcp_f32; that this equals RN(1/scale) for every scale in
//    [2^-100, 2^100] is checked exhaustively on the device.
//  * q: q0 = RN(d*y), one multiply. It is within about two ulps of d/scale, not always one, so
//    the theorem alone does not cover it; the device probe does: for every scale significand at
//    eight exponents from 2^-100 to 2^99, the corrected quotient equals the IEEE d / scale at
//    and next to every half-integer and float midpoint near it (the only places where an ulp
//    can move the code), and on random d. (The same identity with the host's IEEE operations,
//    on a sample of those inputs, is a CPU test: tests/test_quotient_identity.py.)
//  * range: for 2^-100 <= scale <= 2^100 no intermediate underflows for any member whose quotient
//    reaches 0.25 (smaller quotients give code 0 whatever their last bits), and none overflows.
// Other scales: 0 gives y = 0 and every code 0; the rest (subnormal or huge) set `slow` and
// divide.
struct Int4Group {
    float mn, scale, y;
    bool slow;
};

__device__ __forceinline__ float rcp_rn(float s) {
    const float y0 = rcp_approx(s);
    const float e = __builtin_fmaf(-s, y0, 1.0f);
    return __builtin_fmaf(e, y0, y0);
}

// Group constants for a given FP32 scale.
__device__ __forceinline__ Int4Group int4_group_scale(float mn, float scale) {
    Int4Group g;
    g.mn = mn;
    g.scale = scale;
    const bool fast = scale >= 7.888609052210118e-31f && scale <= 1.2676506002282294e30f;  // 2^-100, 2^100
    const float y = rcp_rn(scale);
    g.y = fast ? y : 0.0f;
    g.slow = !fast && scale != 0.0f;
    return g;
}

__device__ __forceinline__ Int4Group int4_group(float mn, float mx) {
    return int4_group_scale(mn, div_const<15>(__fsub_rn(mx, mn)));  // fl(fl(mx - mn) / 15), exactly
}

// fl(d / scale) for a fast group and d >= 0 whose quotient is at least 0.25; below that it
// stays below 0.5 (0 for a zero scale).
__device__ __forceinline__ float int4_quot_raw(float d, const Int4Group& g) {
    const float q0 = __fmul_rn(d, g.y);
    const float r = __builtin_fmaf(-g.scale, q0, d);
    return __builtin_fmaf(r, g.y, q0);
}

// rne(fl(d / scale)) as a float, for a fast group and any d >= 0.
__device__ __forceinline__ float int4_quot(float d, const Int4Group& g) { return __builtin_rintf(int4_quot_raw(d, g)); }

// code = clamp(rne(fl(fl(x - mn) / scale)), 0, 15).
// The clamp never binds for bf16 members: x >= mn gives d >= +0, and d <= fl(mx - mn) with
// scale >= (mx - mn)/15 * (1 - 2^-13) (the worst case is a subnormal scale over the smallest
// nonzero bf16 range 2^-133) keeps q below 15.01, so rne(q) is already in [0, 15].
__device__ __forceinline__ uint32_t int4_code(float x, const Int4Group& g) {
    const float d = __fsub_rn(x, g.mn);
    const float c = __builtin_expect(g.slow, 0) ? __builtin_rintf(d / g.scale) : int4_quot(d, g);
    return (uint32_t)c;
}

// INT4 decode before the final rounding to bf16: fl(fl(c * scale16) + min16). For a code
// c in 0..15 and a scale widened from f16 (at most 11 significant bits, never below 2^-24 unless
// zero) the product c * scale16 has at most 15 significant bits and is exact in FP32, so one
// FMA gives the same result as the multiply and the add (the device probe checks the product
// for every code and every finite f16).
__device__ __forceinline__ float int4_value_f(float c, float s16, float m16) { return __builtin_fmaf(c, s16, m16); }
__device__ __forceinline__ float int4_value(uint32_t c, float s16, float m16) { return int4_value_f((float)c, s16, m16); }

// ---- NVFP4 block constants ------------------------------------------------------------------

// Block scale from the block amax (bf16 magnitude bits) and the tensor multiplier g:
// s = min(fl(g * fl(bamax / 6)), 448); code = e4m3(s); decode scale s_dec = fl(f32(code) / g);
// element multiplier r = fl(1 / s_dec), 0 when the code is 0, with `div` set when the
// reciprocal overflows (then q = fl(x / s_dec)).
struct Fp4Block {
    uint32_t code;
    float s_dec, rcp;
    bool div;
};

// Per-code decode scale and multiplier for one tensor multiplier g: s_dec = fl(f32(c) / g),
// r = fl(1 / s_dec) (+inf when it overflows, 0 for the zero code). Computed with IEEE divisions.
__device__ __forceinline__ f32x2 fp4_code_scales(uint32_t c, float g) {
    const float sf = e4m3_decode(c);
    const float s_dec = sf / g;
    const float r = (sf != 0.0f) ? 1.0f / s_dec : 0.0f;
    return (f32x2){s_dec, r};
}

// The per-code table of one kernel launch, in LDS: entry c holds fp4_code_scales(c, g) for
// the 127 finite positive E4M3 codes (block scales never exceed 448 = code 126).
struct Fp4Table {
    f32x2 e[128];
};

// Fill the table (every thread of the block must call it; ends with a barrier).
__device__ __forceinline__ void fp4_table_fill(Fp4Table& t, float g) {
    for (uint32_t c = threadIdx.x; c < 128u; c += blockDim.x) t.e[c] = fp4_code_scales(c, g);
    __syncthreads();
}

__device__ __forceinline__ Fp4Block fp4_block(uint32_t bamax_bits, float g, const Fp4Table& t) {
    Fp4Block b;
    const float t6 = div_const<6>(bf16_to_f32(bamax_bits));  // fl(bamax / 6), exactly
    float s = __fmul_rn(g, t6);
    s = (s <= 448.0f) ? s : 448.0f;  // also maps +inf to 448
    b.code = e4m3_encode_hw(s);  // s in [0, 448]
    const f32x2 e = t.e[b.code];
    b.s_dec = e[0];
    b.div = __builtin_isinf(e[1]);
    b.rcp = e[1];
    return b;
}

// Scaled element q = fl(x * r), or fl(x / s_dec) when 1/s_dec overflowed; the E2M1 code of q
// carries the sign of x (q has it too: r and s_dec are positive or r is zero).
__device__ __forceinline__ float fp4_scaled(float x, const Fp4Block& b) {
    return b.div ? (x / b.s_dec) : __fmul_rn(x, b.rcp);
}

// Reference single-element code (generic paths).
__device__ __forceinline__ uint32_t fp4_code(float x, const Fp4Block& b) {
    return e2m1_pair<0>(0u, fp4_scaled(x, b), 0.0f) & 0xFu;
}

// 8 NVFP4 codes of one chunk: scaled values, then 4 packed E2M1 conversions. One (rarely
// taken) branch per chunk applies the direct division where a block's 1/s_dec overflowed.
__device__ __forceinline__ uint32_t fp4_word(const u32x4& v, const Fp4Block* fb, int stride) {
    float q[8];
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    bool div = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        q[2 * j] = __fmul_rn(bf16lo(w4[j]), fb[(2 * j) * stride].rcp);
        q[2 * j + 1] = __fmul_rn(bf16hi(w4[j]), fb[(2 * j + 1) * stride].rcp);
        div |= fb[(2 * j) * stride].div | fb[(2 * j + 1) * stride].div;
    }
    if (__builtin_expect(div, 0)) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (fb[k * stride].div) {
                const uint32_t w = w4[k >> 1];
                q[k] = ((k & 1) ? bf16hi(w) : bf16lo(w)) / fb[k * stride].s_dec;
            }
        }
    }
    uint32_t word = e2m1_pair<0>(0u, q[0], q[1]);
    word = e2m1_pair<1>(word, q[2], q[3]);
    word = e2m1_pair<2>(word, q[4], q[5]);
    word = e2m1_pair<3>(word, q[6], q[7]);
    return word;
}

// NVFP4 global multiplier from the tensor amax (bf16 magnitude bits): fl(2688 / amax);
// amax == 0 -> 1; an overflowing quotient -> FLT_MAX.
__device__ __forceinline__ float fp4_global(uint32_t amax_bits) {
    float amax = bf16_to_f32(amax_bits);
    if (amax == 0.0f) return 1.0f;
    float g = 2688.0f / amax;
    return __builtin_isinf(g) ? 3.4028234663852886e38f : g;
}

// ---- NVFP4-row: per-row divisions without the IEEE division sequence -------------------------
//
// The encoder's per-row constants: a row's multiplier g = fl(2688 / amax), a block's decode scale
// s_dec = fl(sf / g) and its reciprocal fl(1 / s_dec), by the Markstein correction of the INT4
// quotient (the unpack decoders keep the plain division, which measured faster there; decode
// attention uses this one for s_dec): y = RN(1/b)
// (rcp_rn), q0 = RN(a y), q = fma(fma(-b, q0, a), y, q0), for divisors b in [2^-100, 2^100];
// other divisors divide. The inputs are finite positive bf16 amax values (2^15 of them) and the
// 126 positive E4M3 scales, so the device probe compares all three with the IEEE quotients
// exhaustively (every amax, every amax x code pair).
struct RcpPair {
    float b, y;
    bool fast;
};

__device__ __forceinline__ RcpPair rcp_pair(float b) {
    RcpPair p;
    p.b = b;
    p.fast = b >= 7.888609052210118e-31f && b <= 1.2676506002282294e30f;  // 2^-100, 2^100
    p.y = rcp_rn(b);
    return p;
}

// fl(a / b) for a >= 0
__device__ __forceinline__ float quot_rn(float a, const RcpPair& p) {
    if (__builtin_expect(!p.fast, 0)) return a / p.b;
    const float q0 = __fmul_rn(a, p.y);
    return __builtin_fmaf(__builtin_fmaf(-p.b, q0, a), p.y, q0);
}

// fp4_global without the IEEE division (same results; probe check [15])
__device__ __forceinline__ float fp4_global_rn(uint32_t amax_bits) {
    const float amax = bf16_to_f32(amax_bits);
    if (amax == 0.0f) return 1.0f;
    const float g = quot_rn(2688.0f, rcp_pair(amax));
    return __builtin_isinf(g) ? 3.4028234663852886e38f : g;
}

// fp4_code_scales(c, g) without IEEE divisions, gp = rcp_pair(g) (probe checks [16], [17])
__device__ __forceinline__ f32x2 fp4_code_scales_rn(uint32_t c, const RcpPair& gp) {
    const float sf = e4m3_decode(c);
    const float s_dec = quot_rn(sf, gp);
    float r = 0.0f;
    if (sf != 0.0f) {
        const bool fast = s_dec >= 7.888609052210118e-31f && s_dec <= 1.2676506002282294e30f;
        r = __builtin_expect(fast, 1) ? rcp_rn(s_dec) : 1.0f / s_dec;
    }
    return (f32x2){s_dec, r};
}

// Block constants for a multiplier that changes from row to row (NVFP4-row): the same values
// as fp4_block, with the decode scale and its reciprocal computed per row (gp = rcp_pair(g))
// instead of looked up in a per-launch table.
__device__ __forceinline__ Fp4Block fp4_block_direct(uint32_t bamax_bits, float g, const RcpPair& gp) {
    Fp4Block b;
    const float t6 = div_const<6>(bf16_to_f32(bamax_bits));
    float s = __fmul_rn(g, t6);
    s = (s <= 448.0f) ? s : 448.0f;
    b.code = e4m3_encode_hw(s);  // s in [0, 448]
    const f32x2 e = fp4_code_scales_rn(b.code, gp);
    b.s_dec = e[0];
    b.rcp = e[1];
    b.div = __builtin_isinf(e[1]);
    return b;
}

// ---- FP8-row ---------------------------------------------------------------------------------

// Row constants: scale = fl(amax / 448) (IEEE division) and, for the branch-free quotient, the
// reciprocal of the INT4 codes' Markstein correction (y = RN(1/scale)). `fast` covers scales in
// [2^-90, 2^100]: there the product, the FMA remainder and the correction neither underflow nor
// overflow for any |x / scale| >= 2^-11, and the corrected quotient is fl(x / scale) exactly
// (tests/probes/cvt_probe.hip sweeps this range at and next to float midpoints); smaller
// quotients stay below 2^-10, where E4M3 rounds to zero either way. A zero scale uses y = 0
// (every quotient is +-0); other scales divide.
struct Fp8Row {
    float s, y;
    bool slow;
};

__device__ __forceinline__ Fp8Row fp8_row_scale(float s) {
    Fp8Row r;
    r.s = s;
    const bool fast = r.s >= 8.077935669463161e-28f && r.s <= 1.2676506002282294e30f;  // 2^-90, 2^100
    const float y = rcp_rn(r.s);
    r.y = fast ? y : 0.0f;
    r.slow = !fast && r.s != 0.0f;
    return r;
}

__device__ __forceinline__ Fp8Row fp8_row(float amax) { return fp8_row_scale(amax / 448.0f); }

// fl(x / s) for a fast row (sign of zero not kept: callers re-attach the sign of x).
__device__ __forceinline__ float fp8_quot(float x, const Fp8Row& r) {
    const float q0 = __fmul_rn(x, r.y);
    const float rem = __builtin_fmaf(-r.s, q0, x);
    return __builtin_fmaf(rem, r.y, q0);
}

// Scaled value to convert: min(|q|, 448) with the sign bit of x.
__device__ __forceinline__ float fp8_clamped(float q, float x) {
    const float m = __builtin_fminf(__builtin_fabsf(q), 448.0f);
    return __uint_as_float(__float_as_uint(m) | (__float_as_uint(x) & 0x80000000u));
}

// Two clamped values -> two E4M3 codes in the low (HI false) or high half of `word`:
// v_cvt_pk_fp8_f32, which the device probe shows equal to e4m3_encode(|v|) with the sign bit of
// v for every binary32 |v| <= 448 (signed zeros included).
template <bool HI>
__device__ __forceinline__ uint32_t fp8_pair(uint32_t word, float v0, float v1) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, (int)word, HI);
}

// The two E4M3 values of the low (HI false) or high half of `word`: v_cvt_pk_f32_fp8, equal to
// the signed e4m3_decode for every finite code (device probe).
template <bool HI>
__device__ __forceinline__ f32x2 fp8_values(uint32_t word) {
    return __builtin_amdgcn_cvt_pk_f32_fp8((int)word, HI);
}

}  // namespace kvq
