// cvt_probe.hip -- exhaustive check of gfx950 conversion instructions against the codec's
// software roundings (test infrastructure; loaded only by tests/test_gpu_cvt_proof.py).
//
// For every binary32 bit pattern (2^32 inputs, NaNs skipped) it compares
//   [0] v_cvt_pk_bf16_f32            with kvq::ref::f32_to_bf16       (round to nearest even)
//   [1] v_cvt_f16_f32                with kvq::ref::f32_to_f16        (nearest even, gradual underflow)
//   [2] v_cvt_scalef32_pk_fp4_f32    with kvq::ref::e2m1_mag + sign   (scale 1.0), all finite inputs
//   [3] the same, restricted to |x| <= 8 (the range the NVFP4 encoder feeds it)
// and, for the 16 E2M1 codes,
//   [4] v_cvt_scalef32_pk_f32_fp4    with kvq::ref::e2m1_value        (scale 1.0)
//   [5] nibble order of both packed instructions (first value in the low nibble), the exact
//       widening of all 65536 binary16 patterns to binary32 (NaNs skipped), and
//       v_cvt_pk_u8_f32 on the integer-valued floats 0..15 (byte placement, other bytes kept)
//   [6] kvq::div_const<15>(x) with the IEEE quotient x / 15, every finite x >= 0
//   [7] kvq::div_const<6>(x)  with the IEEE quotient x / 6,  every finite x >= 0
//   [8] kvq::rcp_approx(x) within one ulp of the IEEE 1 / x, every normal x > 0 whose
//       reciprocal is normal
//   [9] kvq::rcp_rn(x) (v_rcp_f32 plus one Newton step) equal to the IEEE 1 / x, every x in
//       [2^-100, 2^100]
//   [11] v_cvt_pk_fp8_f32 with kvq::e4m3_encode(|x|) plus the sign bit of x, every |x| <= 448
//        (signed zeros included), in both halves of the packed word
//   [12] v_cvt_pk_f32_fp8 with the signed kvq::e4m3_decode, every finite E4M3 code, both halves
//   [14] for every INT4 code c (0..15) and every finite f16 scale s: c * f32(s) is exact in FP32
//        (fma(c, s, -fl(c * s)) == 0), which makes kvq::int4_value_f's single FMA equal to the
//        multiply-then-add; also kvq::int4_value_f(c, s, m) == fl(fl(c * s) + m) for 4 minimums
// and, in a second kernel, the INT4 quotient kvq::int4_quot_raw(d, group(scale)) against the
// IEEE d / scale for every scale significand (2^23) at eight exponents from 2^-100 to 2^99:
//   [10] d = RN(m * scale) and its two neighbours for the 512 points m = h + k * ulp(h) / 2
//        (h = 0.5 ... 15.5, k = -16 ... 15), i.e. quotients at and next to every half-integer
//        and float midpoint near it, plus one pseudo-random d in [scale / 2, 16 scale): the
//        quotient bits must match; for d = RN(scale * 2^-j), j = 3 ... 40, the code (rint) must match;
// and, in a third kernel, the FP8-row quotient kvq::fp8_quot(x, fp8_row_scale(scale)) against
// the IEEE x / scale for every scale significand at eight exponents from 2^-90 to 2^99:
//   [13] signed x = RN(m * scale) and its two neighbours, m a float midpoint in a pseudo-random
//        binade from 2^-12 to 2^9 with a pseudo-random significand: the quotient bits must
//        match; for tiny quotients (scale * 2^-11 ... 2^-48) the E4M3 codes must match;
// and, in a fourth kernel, the NVFP4-row per-row constants without the IEEE division, for
// every finite positive bf16 row amax (0x0001 ... 0x7F7F) and every E4M3 scale code 0 ... 126:
//   [15] kvq::fp4_global_rn(amax) == kvq::fp4_global(amax) (the IEEE 2688 / amax)
//   [16] kvq::fp4_code_scales_rn(c, rcp_pair(g))[0] == fl(e4m3(c) / g), g the row multiplier
//   [17] its reciprocal [1] == fl(1 / s_dec) (+inf where that overflows, 0 for code 0)
//   [18] v_cvt_pk_u8_f32 of every binary32 in [+0, 15.5] (and -0) == its round-to-nearest-even
//        integer in the selected byte, the other bytes kept
// and, in a fifth kernel, the NVFP4-row decode scale for any stored row multiplier (decoders
// read g from memory, so it need not come from a bf16 amax):
//   [19] kvq::quot_rn(e4m3(c), rcp_pair(g)) == the IEEE e4m3(c) / g for every g significand
//        (2^23) at six exponents from 2^-100 to 2^99 and every E4M3 code 0 ... 126
// counting mismatches and recording the smallest mismatching input of each check.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_device.hpp"

using namespace kvq;

namespace {

constexpr int kChecks = 20;

__global__ __launch_bounds__(256) void k_probe(unsigned long long* counts, uint32_t* first) {
    unsigned long long c[kChecks] = {};
    uint32_t f[kChecks];
    for (int i = 0; i < kChecks; ++i) f[i] = 0xFFFFFFFFu;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < (1ull << 32); u += stride) {
        const uint32_t bits = (uint32_t)u;
        const float x = __uint_as_float(bits);
        if (__builtin_isnan(x)) continue;
        typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
        typedef float f2 __attribute__((ext_vector_type(2)));
        const f2 w = {x, x};
        const uint32_t hw_bf = __builtin_bit_cast(uint32_t, __builtin_convertvector(w, bf2)) & 0xFFFFu;
        if (hw_bf != ref::f32_to_bf16(x)) { ++c[0]; f[0] = min(f[0], bits); }
        const uint32_t hw_h = __builtin_bit_cast(uint16_t, (_Float16)x);
        if (hw_h != ref::f32_to_f16(x)) { ++c[1]; f[1] = min(f[1], bits); }
        if (!__builtin_isinf(x)) {
            const uint32_t hw4 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x, x, 1.0f, 0) & 0xFu;
            const uint32_t sw4 = ref::e2m1_mag(x) | ((bits >> 28) & 8u);
            if (hw4 != sw4) {
                ++c[2]; f[2] = min(f[2], bits);
                if (__builtin_fabsf(x) <= 8.0f) { ++c[3]; f[3] = min(f[3], bits); }
            }
        }
        if (!(bits >> 31) && !__builtin_isinf(x)) {
            if (__float_as_uint(div_const<15>(x)) != __float_as_uint(x / 15.0f)) { ++c[6]; f[6] = min(f[6], bits); }
            if (__float_as_uint(div_const<6>(x)) != __float_as_uint(x / 6.0f)) { ++c[7]; f[7] = min(f[7], bits); }
            if (x >= 1.1754943508222875e-38f && x <= 8.507059173023462e37f) {  // x and 1/x normal
                const int32_t e = (int32_t)__float_as_uint(rcp_approx(x)) - (int32_t)__float_as_uint(1.0f / x);
                if (e > 1 || e < -1) { ++c[8]; f[8] = min(f[8], bits); }
            }
            if (x >= 7.888609052210118e-31f && x <= 1.2676506002282294e30f) {  // 2^-100 .. 2^100
                if (__float_as_uint(rcp_rn(x)) != __float_as_uint(1.0f / x)) { ++c[9]; f[9] = min(f[9], bits); }
            }
        }
        if (__builtin_fabsf(x) <= 448.0f) {
            const uint32_t want = e4m3_encode(__builtin_fabsf(x)) | ((bits >> 24) & 0x80u);
            const uint32_t lo = fp8_pair<false>(0xA5A5A5A5u, x, x);  // bytes 0, 1; bytes 2, 3 kept
            const uint32_t hi = fp8_pair<true>(0xA5A5A5A5u, x, x);   // bytes 2, 3; bytes 0, 1 kept
            if (lo != (0xA5A50000u | want | (want << 8)) || hi != (0x0000A5A5u | (want << 16) | (want << 24))) {
                ++c[11];
                f[11] = min(f[11], bits);
            }
        }
        if (bits < 65536u) {
            // binary16 -> binary32 widening, compared with the exact value h * 2^-24 (subnormal)
            // or the rebiased pattern (normal, inf)
            const uint32_t hb = bits;
            const _Float16 hh = __builtin_bit_cast(_Float16, (uint16_t)hb);
            const uint32_t E = (hb >> 10) & 31u, M = hb & 1023u, S = (hb & 0x8000u) << 16;
            if (!(E == 31u && M != 0u)) {
                uint32_t want;
                if (E == 0u)
                    want = S | __float_as_uint((float)M * 5.9604644775390625e-8f);
                else if (E == 31u)
                    want = S | 0x7F800000u;
                else
                    want = S | ((E + 112u) << 23) | (M << 13);
                if (__float_as_uint((float)hh) != want) { ++c[5]; f[5] = min(f[5], bits); }
            }
        }
        if (bits == 0u) {
            // pair order: 1.0 (code 2) and -6.0 (code 15) -> byte 0xF2; byte 0xF2 -> {1.0, -6.0}
            const uint32_t enc = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, 1.0f, -6.0f, 1.0f, 0) & 0xFFu;
            const auto dec = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(0xF2u, 1.0f, 0);
            if (enc != 0xF2u || dec[0] != 1.0f || dec[1] != -6.0f) { ++c[5]; f[5] = min(f[5], 0xF2u); }
            // v_cvt_pk_u8_f32 of the integer-valued floats 0..15 (INT4 code packing)
            for (uint32_t k = 0; k < 16u; ++k) {
                const uint32_t b = __builtin_amdgcn_cvt_pk_u8_f32((float)k, 2, 0xAABBCCDDu);
                if (b != ((0xAABBCCDDu & 0xFF00FFFFu) | (k << 16))) { ++c[5]; f[5] = min(f[5], 0x100u + k); }
            }
        }
        if (bits < (1u << 20)) {  // bits = c << 16 | f16 scale
            const uint32_t cc = bits >> 16, hs = bits & 0xFFFFu;
            if (((hs >> 10) & 31u) != 31u) {
                const float sf = f16_to_f32(hs), cf = (float)cc;
                const float prod = __fmul_rn(cf, sf);
                bool bad = __builtin_fmaf(cf, sf, -prod) != 0.0f;
                const float ms[4] = {0.0f, -0.0f, 1.5f, -3.0517578125e-05f};
                for (int i = 0; i < 4; ++i)
                    bad |= __float_as_uint(int4_value_f(cf, sf, ms[i])) != __float_as_uint(__fadd_rn(prod, ms[i]));
                if (bad) { ++c[14]; f[14] = min(f[14], bits); }
            }
        }
        if (bits < 256u && (bits & 0x7Fu) != 0x7Fu) {
            const float want = __uint_as_float(__float_as_uint(e4m3_decode(bits & 0x7Fu)) | ((bits & 0x80u) << 24));
            const f32x2 lo = fp8_values<false>(bits << 8), hi = fp8_values<true>(bits << 16);
            if (__float_as_uint(lo[1]) != __float_as_uint(want) || __float_as_uint(hi[0]) != __float_as_uint(want)) {
                ++c[12];
                f[12] = min(f[12], bits);
            }
        }
        if (bits <= 0x41780000u || bits == 0x80000000u) {  // every binary32 in [+0, 15.5], and -0
            // v_cvt_pk_u8_f32 of an INT4 quotient rounds it to the nearest integer, ties to even
            const uint32_t want = (uint32_t)__builtin_rintf(x);
            const uint32_t b0 = __builtin_amdgcn_cvt_pk_u8_f32(x, 0, 0xAABBCCDDu);
            const uint32_t b3 = __builtin_amdgcn_cvt_pk_u8_f32(x, 3, 0xAABBCCDDu);
            if (b0 != (0xAABBCC00u | want) || b3 != (0x00BBCCDDu | (want << 24))) { ++c[18]; f[18] = min(f[18], bits); }
        }
        if (bits < 16u) {
            const float hv = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(bits, 1.0f, 0)[0];
            if (__float_as_uint(hv) != __float_as_uint(ref::e2m1_value(bits))) { ++c[4]; f[4] = min(f[4], bits); }
        }
    }
    for (int i = 0; i < kChecks; ++i) {
        if (c[i]) {
            atomicAdd(&counts[i], c[i]);
            atomicMin(&first[i], f[i]);
        }
    }
}

// One scale significand and one of the 512 (h, k) points per thread, for eight exponents.
__global__ __launch_bounds__(256) void k_probe_div(unsigned long long* counts, uint32_t* first) {
    unsigned long long c = 0;
    uint32_t f = 0xFFFFFFFFu;
    const int kExp[8] = {-100, -99, -60, -1, 0, 1, 37, 99};
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < (1ull << 32); u += stride) {
        const uint32_t sig = (uint32_t)u & 0x7FFFFFu, j = (uint32_t)(u >> 23);
        const double h = 0.5 + (double)(j & 15u);
        const int k = (int)((j >> 4) & 31u) - 16;
        const int eh = (h < 1.0) ? -1 : (h < 2.0) ? 0 : (h < 4.0) ? 1 : (h < 8.0) ? 2 : 3;
        const double m = h + (double)k * __builtin_ldexp(1.0, eh - 24);
        for (int ei = 0; ei < 8; ++ei) {
            const float s = __builtin_ldexpf(__uint_as_float(0x3F800000u | sig), kExp[ei]);
            const Int4Group g = int4_group_scale(0.0f, s);
            if (g.slow || g.y == 0.0f) { ++c; f = min(f, (uint32_t)u); continue; }
            const float d0 = (float)(m * (double)s);
            const uint32_t db = __float_as_uint(d0);
            const uint32_t hsh = (uint32_t)(u * 2654435761ull) ^ (uint32_t)ei * 0x9E3779B9u;
            const float dr = __uint_as_float(__float_as_uint(s) - (1u << 23) + hsh % (5u << 23));
            const float ds[4] = {d0, __uint_as_float(db - 1u), __uint_as_float(db + 1u), dr};
            for (int t = 0; t < 4; ++t) {
                if (__float_as_uint(int4_quot_raw(ds[t], g)) != __float_as_uint(ds[t] / s)) {
                    ++c;
                    f = min(f, (uint32_t)u);
                }
            }
            if (j < 38u) {  // tiny quotients: only the code is specified
                const float dt = __builtin_ldexpf(s, -(int)j - 3);
                if (int4_quot(dt, g) != __builtin_rintf(dt / s)) { ++c; f = min(f, (uint32_t)u); }
            }
        }
    }
    if (c) {
        atomicAdd(&counts[10], c);
        atomicMin(&first[10], f);
    }
}

// FP8-row quotient: one scale significand and one (binade, sign) choice per thread, eight
// scale exponents.
__global__ __launch_bounds__(256) void k_probe_fp8div(unsigned long long* counts, uint32_t* first) {
    unsigned long long c = 0;
    uint32_t f = 0xFFFFFFFFu;
    const int kExp[8] = {-90, -89, -50, -1, 0, 1, 60, 99};
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t u = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; u < (1ull << 32); u += stride) {
        const uint32_t sig = (uint32_t)u & 0x7FFFFFu, j = (uint32_t)(u >> 23);
        const uint32_t hsh = (uint32_t)((u * 0x9E3779B97F4A7C15ull) >> 32);
        const int em = (int)(j % 22u) - 12;                     // quotient binade 2^-12 .. 2^9
        const double neg = ((j / 22u) & 1u) ? -1.0 : 1.0;
        const double m0 = __builtin_ldexp(1.0 + (double)(hsh & 0x7FFFFFu) * 0x1p-23, em);
        const double m = neg * (m0 + __builtin_ldexp(1.0, em - 24));  // a float midpoint
        for (int ei = 0; ei < 8; ++ei) {
            const float s = __builtin_ldexpf(__uint_as_float(0x3F800000u | sig), kExp[ei]);
            const Fp8Row r = fp8_row_scale(s);
            if (r.slow || r.y == 0.0f) { ++c; f = min(f, (uint32_t)u); continue; }
            const float x0 = (float)(m * (double)s);
            const uint32_t xb = __float_as_uint(x0);
            const float xs[3] = {x0, __uint_as_float(xb - 1u), __uint_as_float(xb + 1u)};
            for (int t = 0; t < 3; ++t) {
                if (__float_as_uint(fp8_quot(xs[t], r)) != __float_as_uint(xs[t] / s)) {
                    ++c;
                    f = min(f, (uint32_t)u);
                }
            }
            if (j < 38u) {  // tiny quotients: only the E4M3 code is specified
                const float xt = (float)neg * __builtin_ldexpf(s, -(int)j - 11);
                const uint32_t a = e4m3_encode(__builtin_fabsf(fp8_clamped(fp8_quot(xt, r), xt)));
                const uint32_t b = e4m3_encode(__builtin_fabsf(fp8_clamped(xt / s, xt)));
                if (a != b) { ++c; f = min(f, (uint32_t)u); }
            }
        }
    }
    if (c) {
        atomicAdd(&counts[13], c);
        atomicMin(&first[13], f);
    }
}

// NVFP4-row constants: one row amax per thread, all scale codes.
__global__ __launch_bounds__(256) void k_probe_nvfp4row(unsigned long long* counts, uint32_t* first) {
    const uint32_t b = blockIdx.x * blockDim.x + threadIdx.x + 1u;  // bf16 magnitude bits
    if (b > 0x7F7Fu) return;
    unsigned long long c[3] = {0, 0, 0};
    const float g = fp4_global(b);
    const float gr = fp4_global_rn(b);
    if (__float_as_uint(g) != __float_as_uint(gr)) ++c[0];
    const RcpPair gp = rcp_pair(gr);
    for (uint32_t code = 0; code <= 126u; ++code) {
        const f32x2 e = fp4_code_scales(code, g);
        const f32x2 f = fp4_code_scales_rn(code, gp);
        if (__float_as_uint(e[0]) != __float_as_uint(f[0])) ++c[1];
        if (__float_as_uint(e[1]) != __float_as_uint(f[1])) ++c[2];
    }
    for (int k = 0; k < 3; ++k) {
        if (c[k]) {
            atomicAdd(&counts[15 + k], c[k]);
            atomicMin(&first[15 + k], b);
        }
    }
}

// NVFP4-row decode scale for arbitrary multipliers: one g significand per thread.
__global__ __launch_bounds__(256) void k_probe_sdec(unsigned long long* counts, uint32_t* first) {
    const uint32_t sig = blockIdx.x * blockDim.x + threadIdx.x;
    if (sig >= (1u << 23)) return;
    const int kExp[6] = {-100, -99, -40, 0, 63, 99};
    unsigned long long c = 0;
    for (int ei = 0; ei < 6; ++ei) {
        const float g = __builtin_ldexpf(__uint_as_float(0x3F800000u | sig), kExp[ei]);
        const RcpPair gp = rcp_pair(g);
        for (uint32_t code = 0; code <= 126u; ++code) {
            const float sf = e4m3_decode(code);
            if (__float_as_uint(quot_rn(sf, gp)) != __float_as_uint(sf / g)) ++c;
        }
    }
    if (c) {
        atomicAdd(&counts[19], c);
        atomicMin(&first[19], sig);
    }
}

}  // namespace

extern "C" int kvq_probe_cvt(unsigned long long* counts_host, uint32_t* first_host) {
    unsigned long long* counts = nullptr;
    uint32_t* first = nullptr;
    if (hipMalloc(&counts, kChecks * sizeof(unsigned long long)) != hipSuccess) return 1;
    if (hipMalloc(&first, kChecks * sizeof(uint32_t)) != hipSuccess) return 2;
    hipMemset(counts, 0, kChecks * sizeof(unsigned long long));
    hipMemset(first, 0xFF, kChecks * sizeof(uint32_t));
    hipLaunchKernelGGL(k_probe, dim3(4096), dim3(256), 0, 0, counts, first);
    if (hipGetLastError() != hipSuccess) return 3;
    hipLaunchKernelGGL(k_probe_div, dim3(4096), dim3(256), 0, 0, counts, first);
    if (hipGetLastError() != hipSuccess) return 3;
    hipLaunchKernelGGL(k_probe_fp8div, dim3(4096), dim3(256), 0, 0, counts, first);
    if (hipGetLastError() != hipSuccess) return 3;
    hipLaunchKernelGGL(k_probe_nvfp4row, dim3((0x7F7Fu + 255u) / 256u), dim3(256), 0, 0, counts, first);
    if (hipGetLastError() != hipSuccess) return 3;
    hipLaunchKernelGGL(k_probe_sdec, dim3((1u << 23) / 256u), dim3(256), 0, 0, counts, first);
    if (hipGetLastError() != hipSuccess) return 3;
    if (hipDeviceSynchronize() != hipSuccess) return 4;
    hipMemcpy(counts_host, counts, kChecks * sizeof(unsigned long long), hipMemcpyDeviceToHost);
    hipMemcpy(first_host, first, kChecks * sizeof(uint32_t), hipMemcpyDeviceToHost);
    hipFree(counts);
    hipFree(first);
    return 0;
}
