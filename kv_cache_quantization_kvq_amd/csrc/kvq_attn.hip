// kvq_attn.hip -- decode attention that reads the packed KV cache directly: the codec's
// dequantization (and optionally one residual's reconstruction) happens in registers and the
// products run on bf16 MFMA (vllm-rlt PR #166, the reviews' hot-path discussion: dequantize to
// BF16 in registers and keep the BF16 matrix multiply; compare formats after fusing
// dequantization and residual reconstruction into attention).
//
// One query token per query head attends over all T cached tokens; query head hq reads KV head
// hq / rep. The cached K and V are exactly what kvq_unpack (or kvq_decode_residual on top of it)
// would produce, bf16 value for bf16 value; scores and the softmax run in FP32, P is rounded to
// bf16 for the PV product, accumulation is FP32.
//
// Work split (flash decoding): a block owns one KV head and a range of tokens; each of its 4
// waves walks 16-token sub-tiles with its own online softmax; the waves meet in LDS, the block
// writes one partial (max, sum, unnormalized output) per query row, and a second kernel folds the
// partials of all blocks.
//
// MFMA v_mfma_f32_16x16x16_bf16 (lane l, q = l / 16, j = 0..3): A[l % 16][4q + j],
// B[4q + j][l % 16], D[4q + j][l % 16] (checked on the device). Scores are computed transposed,
// S^T = K Q^T: A = K (lane: token l % 16; the reduction axis is permuted so that lane group q
// covers channels 32q .. 32q + 31, one 16-byte load of codes), B = Q^T. The accumulator then
// holds S[row l % 16][token 4q + j], which is exactly the B operand P^T of O^T = V^T P^T; there
// A = V^T (lane: channels 8 (l % 16) + N of the output tile N, tokens 4q + j, one 4-byte load per
// token), and the accumulator holds O[row l % 16][channel 32q + 8j + N].
#include <type_traits>

#include "kvq_launch.hpp"

namespace kvq {

namespace {

constexpr int kD = KVQ_ATTN_D;  // head_dim
constexpr int kWaves = 4;       // waves per block
constexpr int kSub = 16;        // tokens per sub-tile (one MFMA tile)
constexpr int kNone = KVQ_ATTN_NO_RESIDUAL;

typedef short s4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float lane_max(float v) {
    v = __builtin_fmaxf(v, __shfl_xor(v, 16));
    return __builtin_fmaxf(v, __shfl_xor(v, 32));
}

template <bool ON>
using TableT = std::conditional_t<ON, Fp4Table, char>;

// --- K: 32 channels (32q .. 32q + 31) of one token, as 8 MFMA operands (4 channels each) ---

// Decoded bf16 values of the lane's 32 K channels for token t, one float per channel.
template <int FMT>
__device__ __forceinline__ void k_values(const AttnPlanes& p, const Fp4Table* tab, int64_t t, int H, int h, int q,
                                        float (&y)[32]) {
    const size_t row = (size_t)t * H + h;
    const u32x4 cw = *reinterpret_cast<const u32x4*>(p.codes + row * (kD / 2) + 16 * q);
    const uint32_t w[4] = {cw.x, cw.y, cw.z, cw.w};
    if constexpr (FMT == FMT_INT4) {
        const size_t mb = ((size_t)(t / p.G) * H + h) * kD + 32 * q;
        const u32x4* mn = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.meta0) + mb);
        const u32x4* sc = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(p.meta1) + mb);
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // word i: channels 8i .. 8i + 7
            const u32x4 m4 = mn[i], s4 = sc[i];
            const uint32_t mm[4] = {m4.x, m4.y, m4.z, m4.w}, ss[4] = {s4.x, s4.y, s4.z, s4.w};
            const uint32_t lo = w[i] & 0x0F0F0F0Fu, hi = (w[i] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
            for (int b = 0; b < 4; ++b) {  // byte b: channels 8i + 2b, 8i + 2b + 1
                const float c0 = (float)((lo >> (8 * b)) & 0xFFu), c1 = (float)((hi >> (8 * b)) & 0xFFu);
                y[8 * i + 2 * b] = int4_value_f(c0, f16_to_f32(ss[b] & 0xFFFFu), f16_to_f32(mm[b] & 0xFFFFu));
                y[8 * i + 2 * b + 1] = int4_value_f(c1, f16_to_f32(ss[b] >> 16), f16_to_f32(mm[b] >> 16));
            }
        }
    } else {
        const size_t sb = ((size_t)(t / 16) * H + h) * kD + 32 * q;
        const u32x4* s8 = reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(p.meta0) + sb);
        const u32x4 sa = s8[0], sbv = s8[1];
        const uint32_t sw[8] = {sa.x, sa.y, sa.z, sa.w, sbv.x, sbv.y, sbv.z, sbv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const f32x2 e0 = e2m1_values<0>(w[i]), e1 = e2m1_values<1>(w[i]);
            const f32x2 e2 = e2m1_values<2>(w[i]), e3 = e2m1_values<3>(w[i]);
            const float e[8] = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int c = 8 * i + k;
                const uint32_t code = (sw[c >> 2] >> (8 * (c & 3))) & 0x7Fu;
                y[c] = __fmul_rn(e[k], tab->e[code][0]);
            }
        }
    }
}

// --- V: channels 8m .. 8m + 7 of one token ---

template <int FMT>
__device__ __forceinline__ void v_values(const AttnPlanes& p, const Fp4Table* tab, int64_t t, int H, int h, int m,
                                        float (&y)[8]) {
    const size_t row = (size_t)t * H + h;
    const uint32_t w = *reinterpret_cast<const uint32_t*>(p.codes + row * (kD / 2) + 4 * m);
    if constexpr (FMT == FMT_INT4) {
        const size_t mi = row * (size_t)(kD / p.G) + (8 * m) / p.G;
        const float s = f16_to_f32(reinterpret_cast<const uint16_t*>(p.meta1)[mi]);
        const float mn = f16_to_f32(reinterpret_cast<const uint16_t*>(p.meta0)[mi]);
        const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            y[2 * b] = int4_value_f((float)((lo >> (8 * b)) & 0xFFu), s, mn);
            y[2 * b + 1] = int4_value_f((float)((hi >> (8 * b)) & 0xFFu), s, mn);
        }
    } else {
        const uint32_t code = reinterpret_cast<const uint8_t*>(p.meta0)[row * (kD / 16) + (m >> 1)] & 0x7Fu;
        const float s_dec = tab->e[code][0];
        const f32x2 e0 = e2m1_values<0>(w), e1 = e2m1_values<1>(w), e2 = e2m1_values<2>(w), e3 = e2m1_values<3>(w);
        const float e[8] = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = __fmul_rn(e[k], s_dec);
    }
}

// bf16 of a decoded value, or for a residual bf16(bf16(base) + bf16(residual)) (the codec's
// decode_residual, both roundings in the input dtype)
__device__ __forceinline__ uint32_t rebuild2(float b0, float b1, float r0, float r1, bool res) {
    const uint32_t bb = pack_bf16x2(b0, b1);
    if (!res) return bb;
    const uint32_t rb = pack_bf16x2(r0, r1);
    return pack_bf16x2(__fadd_rn(bf16lo(bb), bf16lo(rb)), __fadd_rn(bf16hi(bb), bf16hi(rb)));
}

__device__ __forceinline__ s4_t as_s4(uint32_t lo, uint32_t hi) {
    const u2_t v = {lo, hi};
    return __builtin_bit_cast(s4_t, v);
}

template <int FMT, int RFMT>
__global__ __launch_bounds__(64 * kWaves) void k_attn_split(AttnArgs a) {
    constexpr bool RES = RFMT != kNone;
    __shared__ TableT<FMT == FMT_NVFP4> tk, tv;
    __shared__ TableT<RFMT == FMT_NVFP4> trk, trv;
    __shared__ float s_o[kWaves][16][kD];
    __shared__ float s_m[kWaves][16], s_l[kWaves][16];
    if constexpr (FMT == FMT_NVFP4) {
        fp4_table_fill(tk, *a.k.gscale);
        fp4_table_fill(tv, *a.v.gscale);
    }
    if constexpr (RFMT == FMT_NVFP4) {
        fp4_table_fill(trk, *a.rk.gscale);
        fp4_table_fill(trv, *a.rv.gscale);
    }
    const Fp4Table* ptk = nullptr;
    const Fp4Table* ptv = nullptr;
    const Fp4Table* ptrk = nullptr;
    const Fp4Table* ptrv = nullptr;
    if constexpr (FMT == FMT_NVFP4) { ptk = &tk; ptv = &tv; }
    if constexpr (RFMT == FMT_NVFP4) { ptrk = &trk; ptrv = &trv; }

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int r = lane & 15;  // query row of the group (and the K token / V channel-octet index)
    const int q = lane >> 4;
    const int h = blockIdx.y;
    const int64_t t_begin = (int64_t)blockIdx.x * a.tc;
    const int64_t t_end = min<int64_t>(a.T, t_begin + a.tc);

    // Q^T operand: row r (query head h * rep + r), channels 32q + 4s + j for step s
    uint32_t qw[16];
    if (r < a.rep) {
        const u32x4* qp = reinterpret_cast<const u32x4*>(a.q + ((size_t)h * a.rep + r) * kD + 32 * q);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 v = qp[i];
            qw[4 * i] = v.x; qw[4 * i + 1] = v.y; qw[4 * i + 2] = v.z; qw[4 * i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) qw[i] = 0u;
    }

    float m_run = -__builtin_inff(), l_run = 0.0f;
    f4_t o[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) o[n] = (f4_t){0.0f, 0.0f, 0.0f, 0.0f};

    for (int64_t t0 = t_begin + (int64_t)wave * kSub; t0 < t_end; t0 += kWaves * kSub) {
        // ---- scores S^T = K Q^T for tokens t0 .. t0 + 15 ----
        const int64_t tk_ = min<int64_t>(t0 + r, t_end - 1);
        float kv[32], kr[32];
        k_values<FMT>(a.k, ptk, tk_, a.H, h, q, kv);
        if constexpr (RES) k_values<RFMT>(a.rk, ptrk, tk_, a.H, h, q, kr);
        f4_t sacc = (f4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int c = 4 * s;
            const uint32_t k01 = rebuild2(kv[c], kv[c + 1], RES ? kr[c] : 0.0f, RES ? kr[c + 1] : 0.0f, RES);
            const uint32_t k23 = rebuild2(kv[c + 2], kv[c + 3], RES ? kr[c + 2] : 0.0f, RES ? kr[c + 3] : 0.0f, RES);
            sacc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_s4(k01, k23), as_s4(qw[2 * s], qw[2 * s + 1]), sacc, 0,
                                                             0, 0);
        }
        // ---- online softmax over this sub-tile: lane holds S[row r][token t0 + 4q + j] ----
        float sc[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sc[j] = (t0 + 4 * q + j < t_end) ? sacc[j] * a.qscale : -__builtin_inff();
        const float m_tile = lane_max(__builtin_fmaxf(__builtin_fmaxf(sc[0], sc[1]), __builtin_fmaxf(sc[2], sc[3])));
        const float m_new = __builtin_fmaxf(m_run, m_tile);  // finite: token t0 is in range
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(sc[j] - m_new);
        l_run = l_run * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
        m_run = m_new;
#pragma unroll
        for (int n = 0; n < 8; ++n) o[n] *= alpha;
        const s4_t pb = as_s4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
        // ---- O^T += V^T P^T: lane loads tokens t0 + 4q + j, channels 8r .. 8r + 7 ----
        float vv[4][8], vr[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t tv_ = min<int64_t>(t0 + 4 * q + j, t_end - 1);
            v_values<FMT>(a.v, ptv, tv_, a.H, h, r, vv[j]);
            if constexpr (RES) v_values<RFMT>(a.rv, ptrv, tv_, a.H, h, r, vr[j]);
        }
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const uint32_t v01 = rebuild2(vv[0][n], vv[1][n], RES ? vr[0][n] : 0.0f, RES ? vr[1][n] : 0.0f, RES);
            const uint32_t v23 = rebuild2(vv[2][n], vv[3][n], RES ? vr[2][n] : 0.0f, RES ? vr[3][n] : 0.0f, RES);
            o[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_s4(v01, v23), pb, o[n], 0, 0, 0);
        }
    }

    // ---- fold the block's 4 waves: lane holds O[row r][channel 32q + 8j + n] ----
    float l_row = l_run + __shfl_xor(l_run, 16);  // the row's 4 lanes share m_run
    l_row += __shfl_xor(l_row, 32);
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int j = 0; j < 4; ++j) s_o[wave][r][32 * q + 8 * j + n] = o[n][j];
    if (q == 0) {
        s_m[wave][r] = m_run;  // -inf for a wave without tokens (then l = 0 and O = 0)
        s_l[wave][r] = l_row;
    }
    __syncthreads();
    const size_t pbase = ((size_t)h * a.n_split + blockIdx.x) * a.rep;
    for (int idx = threadIdx.x; idx < a.rep * kD; idx += 64 * kWaves) {
        const int row = idx / kD, c = idx - row * kD;
        float M = s_m[0][row];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = __builtin_fmaxf(M, s_m[w][row]);
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = (s_m[w][row] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(s_m[w][row] - M);
            L += s_l[w][row] * f;
            O += s_o[w][row][c] * f;
        }
        a.part_o[(pbase + row) * kD + c] = O;
        if (c == 0) {
            a.part_ml[(pbase + row) * 2] = M;
            a.part_ml[(pbase + row) * 2 + 1] = L;
        }
    }
}

// out[hq][c] = sum_s O_s e^(m_s - M) / sum_s l_s e^(m_s - M) over the blocks' partials.
__global__ __launch_bounds__(256) void k_attn_combine(AttnArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int Hq = a.H * a.rep;
    if (idx >= (int64_t)Hq * kD) return;
    const int hq = (int)(idx / kD), c = (int)(idx - (int64_t)hq * kD);
    const int h = hq / a.rep, row = hq - h * a.rep;
    float M = -__builtin_inff();
    for (int s = 0; s < a.n_split; ++s)
        M = __builtin_fmaxf(M, a.part_ml[(((size_t)h * a.n_split + s) * a.rep + row) * 2]);
    float L = 0.0f, O = 0.0f;
    for (int s = 0; s < a.n_split; ++s) {
        const size_t pi = ((size_t)h * a.n_split + s) * a.rep + row;
        const float f = __builtin_amdgcn_exp2f(a.part_ml[pi * 2] - M);
        L += a.part_ml[pi * 2 + 1] * f;
        O += a.part_o[pi * kD + c] * f;
    }
    a.out[idx] = O / L;
}

template <int FMT, int RFMT>
hipError_t attn_launch(const AttnArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((k_attn_split<FMT, RFMT>), dim3(a.n_split, a.H), dim3(64 * kWaves), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const uint64_t n = (uint64_t)a.H * a.rep * kD;
    hipLaunchKernelGGL(k_attn_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int FMT>
hipError_t attn_fmt(int rfmt, const AttnArgs& a, hipStream_t s) {
    if (rfmt == kNone) return attn_launch<FMT, kNone>(a, s);
    if (rfmt == FMT_INT4) return attn_launch<FMT, FMT_INT4>(a, s);
    if (rfmt == FMT_NVFP4) return attn_launch<FMT, FMT_NVFP4>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attention(int fmt, int rfmt, const AttnArgs& a, hipStream_t s) {
    if (fmt == FMT_INT4) return attn_fmt<FMT_INT4>(rfmt, a, s);
    if (fmt == FMT_NVFP4) return attn_fmt<FMT_NVFP4>(rfmt, a, s);
    return hipErrorInvalidValue;
}

}  // namespace kvq
