// kvq_rowfmt.hip -- the two row formats, where every (token, KV head) row carries its own FP32
// scale (FreeToken PR #408, "feat(kvcache): add nvfp4 kv quantization": "Summary", the fp8
// commit and the nvfp4 codec-port commit):
//   NVFP4-row  E2M1 nibbles (low first), one E4M3 block scale per 16 channels, and the row
//              multiplier g_row = fl(2688 / row amax) (0 -> 1, overflow -> FLT_MAX); each row is
//              encoded exactly as a one-row NVFP4 tensor. 76 B per head_dim-128 row.
//   FP8-row    one E4M3 code per channel and scale = fl(row amax / 448); code = e4m3(min(|q|,
//              448)) with q = fl(x / scale) and the sign bit of x; decode bf16(e4m3 * scale).
// Because rows are independent, the same kernels serve slot writes (encoded row r lands in
// packed row dst[r]) and slot reads (output row r decodes packed row src[r]).
//
// Vector path (head_dim a power of two from 8 to 512, 16-byte aligned rows): a lane owns 8
// channels of a row, a (token, head) row spans D/8 adjacent lanes, and its amax is an
// all-reduce over them (DPP within 16 lanes, lane shuffles beyond). Generic path: one thread
// per (row, head) for encode, per (row, head, byte) for decode.
#include "kvq_launch.hpp"

namespace kvq {

namespace {

constexpr int kThreads = 256;

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t umax_u(uint32_t x, uint32_t y) { return max(x, y); }

// Max over aligned groups of `lanes` lanes (a power of two up to 64; all lanes active).
__device__ __forceinline__ uint32_t lanes_umax(uint32_t v, int lanes) {
    v = group_allreduce(v, lanes < 16 ? lanes : 16, umax_u);
    if (lanes >= 32) v = max(v, (uint32_t)__shfl_xor((int)v, 16));
    if (lanes >= 64) v = max(v, (uint32_t)__shfl_xor((int)v, 32));
    return v;
}

// bf16 magnitude bits of the largest |x| among a lane's 8 channels
__device__ __forceinline__ uint32_t chunk_amax(const u32x4& v) {
    const ushort2_t m = umax2(umax2(mag2(v.x), mag2(v.y)), umax2(mag2(v.z), mag2(v.w)));
    return max((uint32_t)m.x, (uint32_t)m.y);
}

// bf16 bits of the encoded value of element (t, h, d) (generic path)
template <bool DIFF>
__device__ __forceinline__ uint32_t row_load(const EncArgs& a, int64_t t, int64_t h, int64_t d) {
    uint32_t c = a.cur[row_offset(t, a.cpshift, a.cpst, a.cst) + h * a.csh + d];
    if constexpr (DIFF) {
        uint32_t p = a.prev[t * a.pst + h * a.psh + d];
        return bf16_bits(__fsub_rn(bf16_to_f32(c), bf16_to_f32(p)));
    }
    return c;
}

// RW rows' chunks of one lane, residual applied (same loads as the other vector encoders).
// UNI: r0 is the same on every lane, so a row's address is a scalar base plus the lane's 32-bit
// byte offset (the host keeps a row's span below 2^31 bytes).
template <int RW, bool DIFF, bool GATHER, bool UNI>
__device__ __forceinline__ void row_chunks(const EncArgs& a, int64_t r0, uint32_t h, uint32_t d, u32x4 (&v)[RW]) {
    int64_t t[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const int64_t r = min<int64_t>(r0 + i, a.rows - 1);
        t[i] = GATHER ? (int64_t)a.pos[r] : r;
    }
    if constexpr (UNI) {
        const uint32_t coff = (uint32_t)(((int64_t)h * a.csh + d) * 2);
#pragma unroll
        for (int i = 0; i < RW; ++i)
            v[i] = ld_stream_at(wave_base(a.cur, row_offset(t[i], a.cpshift, a.cpst, a.cst) * 2), coff);
    } else {
#pragma unroll
        for (int i = 0; i < RW; ++i)
            v[i] = ld_stream(a.cur + row_offset(t[i], a.cpshift, a.cpst, a.cst) + (int64_t)h * a.csh + d);
    }
    if constexpr (DIFF) {
        u32x4 p[RW];
        if constexpr (UNI) {
            const uint32_t poff = (uint32_t)(((int64_t)h * a.psh + d) * 2);
#pragma unroll
            for (int i = 0; i < RW; ++i) p[i] = ld_stream_at(wave_base(a.prev, t[i] * a.pst * 2), poff);
        } else {
#pragma unroll
            for (int i = 0; i < RW; ++i) p[i] = ld_stream(a.prev + t[i] * a.pst + (int64_t)h * a.psh + d);
        }
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            v[i].x = sub_bf16x2(v[i].x, p[i].x);
            v[i].y = sub_bf16x2(v[i].y, p[i].y);
            v[i].z = sub_bf16x2(v[i].z, p[i].z);
            v[i].w = sub_bf16x2(v[i].w, p[i].w);
        }
    }
}

// 8 FP8 codes of one chunk (channel d+k in byte k), as two words.
__device__ __forceinline__ uint2 fp8_chunk(const u32x4& v, const Fp8Row& rs) {
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    float c[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float x0 = bf16lo(w4[j]), x1 = bf16hi(w4[j]);
        float q0, q1;
        if (__builtin_expect(rs.slow, 0)) {
            q0 = x0 / rs.s;
            q1 = x1 / rs.s;
        } else {
            q0 = fp8_quot(x0, rs);
            q1 = fp8_quot(x1, rs);
        }
        c[2 * j] = fp8_clamped(q0, x0);
        c[2 * j + 1] = fp8_clamped(q1, x1);
    }
    uint2 o;
    o.x = fp8_pair<true>(fp8_pair<false>(0u, c[0], c[1]), c[2], c[3]);
    o.y = fp8_pair<true>(fp8_pair<false>(0u, c[4], c[5]), c[6], c[7]);
    return o;
}

// One wave task: RW = KVQ_ROW_ENCODE_ROWS rows of a 64-chunk slab.
template <int FMT, bool DIFF, bool GATHER, bool LG, bool WIN>
__global__ __launch_bounds__(kThreads) void k_row_encode_vec(EncArgs a) {
    constexpr int RW = KVQ_ROW_ENCODE_ROWS;
    static_assert(RW % 2 == 0, "NVFP4-row encode splits a task's rows over a lane pair");
    if (WIN && blockIdx.x >= a.win_block0) {  // blocks of the carried row copy
        window_copy_wave(a.win, __builtin_amdgcn_readfirstlane((blockIdx.x - a.win_block0) * 4u + (threadIdx.x >> 6)),
                         threadIdx.x & 63);
        return;
    }
    const int lane = threadIdx.x & 63;
    const uint32_t task = __builtin_amdgcn_readfirstlane(blockIdx.x * 4u + (threadIdx.x >> 6));
    if (task >= a.n_tasks) return;
    uint32_t rtile, c8raw;
    task_lane<LG>(a, task, lane, rtile, c8raw);
    const bool valid = c8raw < (uint32_t)a.C8;
    const uint32_t c8 = valid ? c8raw : (uint32_t)a.C8 - 1u;
    const uint32_t h = fdiv(c8, a.div_D8);
    const uint32_t dc = c8 - h * (uint32_t)a.D8;  // chunk within the (token, head) row
    const uint32_t d = dc * 8u;
    const int64_t r0 = (int64_t)rtile * RW;
    const int nr = (int)min<int64_t>(RW, a.rows - r0);
    const int lpr = a.D8;  // lanes per (token, head) row
    const bool row_leader = valid && dc == 0u;

    u32x4 v[RW];
    // scalar-base row addresses measured faster for FP8-row (more code bytes per row) and slower
    // for NVFP4-row (whose per-row scale work already keeps the scalar unit busy)
    constexpr bool UNI = !LG && FMT == FMT_FP8_ROW;
    row_chunks<RW, DIFF, GATHER, UNI>(a, r0, h, d, v);

    // NVFP4-row: a row pair's multipliers g and this lane's block constants, worked out before
    // the pair's codes. A 16-channel block is a lane pair (l, l ^ 1) whose lanes hold the same row
    // and block maxima, so the even lane works out the even row and the odd lane the odd row, and
    // the two swap the results (one lane per block when D = 8).
    float gq[2];
    Fp4Block fq[2];
    const bool odd = (c8raw & 1u) != 0u;

#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const int64_t r = r0 + i;
        const int64_t wr = a.dst ? (int64_t)a.dst[min<int64_t>(r, a.rows - 1)] : r;
        const bool sbase = UNI && a.dst == nullptr;  // packed row r0 + i, the same on every lane
        const size_t hr = (size_t)wr * (uint32_t)a.H + h;  // (packed row, head) index
        if constexpr (FMT == FMT_FP8_ROW) {
            const uint32_t amax = lanes_umax(chunk_amax(v[i]), lpr);
            const Fp8Row rs = fp8_row(bf16_to_f32(amax));
            const uint2 o = fp8_chunk(v[i], rs);
            if (i < nr) {
                if (valid) {
                    if (sbase)
                        st_code_at<!DIFF>(wave_base_w(a.codes, r * (int64_t)a.H * a.D), (uint32_t)(h * (uint32_t)a.D + d),
                                          (u32x2){o.x, o.y});
                    else
                        st_code<!DIFF>(reinterpret_cast<u32x2*>(a.codes + hr * (uint32_t)a.D + d), (u32x2){o.x, o.y});
                }
                if (row_leader) reinterpret_cast<float*>(a.meta0)[hr] = rs.s;
            }
        } else {
            if ((i & 1) == 0) {
                uint32_t amx[2], bam[2];
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const uint32_t am = chunk_amax(v[i + k]);
                    amx[k] = lanes_umax(am, lpr);
                    bam[k] = (lpr >= 2) ? max(am, dpp<0xB1>(am)) : am;
                }
                if (lpr >= 2) {
                    const float gm = fp4_global_rn(odd ? amx[1] : amx[0]);
                    const Fp4Block bm = fp4_block_direct(odd ? bam[1] : bam[0], gm, rcp_pair(gm));
                    const float go = __uint_as_float(dpp<0xB1>(__float_as_uint(gm)));
                    Fp4Block bo;
                    bo.rcp = __uint_as_float(dpp<0xB1>(__float_as_uint(bm.rcp)));
                    bo.s_dec = __uint_as_float(dpp<0xB1>(__float_as_uint(bm.s_dec)));
                    const uint32_t cd = dpp<0xB1>(bm.code | (bm.div ? 0x100u : 0u));
                    bo.code = cd & 0xFFu;
                    bo.div = (cd >> 8) != 0u;
                    gq[0] = odd ? go : gm;
                    gq[1] = odd ? gm : go;
                    fq[0] = odd ? bo : bm;
                    fq[1] = odd ? bm : bo;
                } else {
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        gq[k] = fp4_global_rn(amx[k]);
                        fq[k] = fp4_block_direct(bam[k], gq[k], rcp_pair(gq[k]));
                    }
                }
            }
            const float g = gq[i & 1];
            const Fp4Block fb = fq[i & 1];
            const uint32_t word = fp4_word(v[i], &fb, 0);
            if (i < nr && valid) {
                if (sbase)
                    st_code_at<!DIFF>(wave_base_w(a.codes, r * (int64_t)a.C8 * 4), c8 * 4u, word);
                else
                    st_code<!DIFF>(reinterpret_cast<uint32_t*>(a.codes) + (size_t)wr * (uint32_t)a.C8 + c8, word);
                const uint32_t nb = ((uint32_t)a.D + 15u) / 16u;
                if ((dc & 1u) == 0u) reinterpret_cast<uint8_t*>(a.meta0)[hr * nb + (dc >> 1)] = (uint8_t)fb.code;
                if (row_leader) reinterpret_cast<float*>(a.meta1)[hr] = g;
            }
        }
        if constexpr (GATHER) {
            if (i < nr && c8raw == 0) a.pos_out[r] = a.pos[r];
        }
    }
}

// Generic encoder: one thread per (row, head).
template <int FMT, bool DIFF, bool GATHER>
__global__ __launch_bounds__(kThreads) void k_row_encode_gen(EncArgs a) {
    const int64_t idx = (int64_t)(a.gen_base + (uint64_t)blockIdx.x * kThreads + threadIdx.x);
    if (idx >= a.rows * a.H) return;
    const int64_t r = idx / a.H;
    const int64_t h = idx - r * a.H;
    const int64_t t = GATHER ? (int64_t)a.pos[r] : r;
    const int64_t wr = a.dst ? (int64_t)a.dst[r] : r;
    const int D = a.D;
    const size_t hr = (size_t)(wr * a.H + h);
    uint32_t amax = 0;
    for (int dd = 0; dd < D; ++dd) amax = max(amax, row_load<DIFF>(a, t, h, dd) & 0x7FFFu);
    if constexpr (FMT == FMT_FP8_ROW) {
        const float s = bf16_to_f32(amax) / 448.0f;
        reinterpret_cast<float*>(a.meta0)[hr] = s;
        uint8_t* crow = a.codes + hr * (size_t)D;
        for (int dd = 0; dd < D; ++dd) {
            const float x = bf16_to_f32(row_load<DIFF>(a, t, h, dd));
            const float q = (s != 0.0f) ? x / s : 0.0f;
            const float m = __builtin_fminf(__builtin_fabsf(q), 448.0f);
            crow[dd] = (uint8_t)(e4m3_encode(m) | ((__float_as_uint(x) >> 24) & 0x80u));
        }
    } else {
        const float g = fp4_global_rn(amax);
        const RcpPair gp = rcp_pair(g);
        reinterpret_cast<float*>(a.meta1)[hr] = g;
        const int nb = (D + 15) / 16, Dp = (D + 1) / 2;
        uint8_t* crow = a.codes + hr * (size_t)Dp;
        uint8_t* srow = reinterpret_cast<uint8_t*>(a.meta0) + hr * (size_t)nb;
        for (int b = 0; b < nb; ++b) {
            const int d0 = b * 16, d1 = min(D, d0 + 16);
            uint32_t bam = 0;
            for (int dd = d0; dd < d1; ++dd) bam = max(bam, row_load<DIFF>(a, t, h, dd) & 0x7FFFu);
            const Fp4Block fb = fp4_block_direct(bam, g, gp);
            srow[b] = (uint8_t)fb.code;
            for (int dd = d0; dd < d1; dd += 2) {
                const uint32_t lo = fp4_code(bf16_to_f32(row_load<DIFF>(a, t, h, dd)), fb);
                const uint32_t hi = (dd + 1 < D) ? fp4_code(bf16_to_f32(row_load<DIFF>(a, t, h, dd + 1)), fb) : 0u;
                crow[dd >> 1] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
    if constexpr (GATHER) {
        if (h == 0) a.pos_out[r] = (int32_t)t;
    }
}

// Output word of two decoded values (bf16 each, or bf16(prev + bf16(y)) for a residual).
template <bool ADD>
__device__ __forceinline__ uint32_t row_finish(float y0, float y1, uint32_t prev_word) {
    const uint32_t yb = pack_bf16x2(y0, y1);
    if constexpr (!ADD) return yb;
    return pack_bf16x2(__fadd_rn(bf16lo(prev_word), bf16lo(yb)), __fadd_rn(bf16hi(prev_word), bf16hi(yb)));
}

template <int FMT, bool ADD, bool SCATTER, bool LG, bool WIN>
__global__ __launch_bounds__(kThreads) void k_row_decode_vec(DecArgs a) {
    constexpr int RW = KVQ_DECODE_ROWS;
    static_assert(RW % 2 == 0, "NVFP4-row decode splits a task's rows over a lane pair");
    if (WIN && blockIdx.x >= a.win_block0) {  // blocks of the carried row copy
        window_copy_wave(a.win, __builtin_amdgcn_readfirstlane((blockIdx.x - a.win_block0) * 4u + (threadIdx.x >> 6)),
                         threadIdx.x & 63);
        return;
    }
    const int lane = threadIdx.x & 63;
    const uint32_t task =
        __builtin_amdgcn_readfirstlane(xcd_block(blockIdx.x, WIN ? a.win_block0 : gridDim.x) * 4u + (threadIdx.x >> 6));
    if (task >= a.n_tasks) return;
    uint32_t rtile, c8raw;
    task_lane<LG>(a, task, lane, rtile, c8raw);
    const bool valid = c8raw < (uint32_t)a.C8;
    const uint32_t c8 = valid ? c8raw : (uint32_t)a.C8 - 1u;
    const uint32_t h = fdiv(c8, a.div_D8);
    const uint32_t dc = c8 - h * (uint32_t)a.D8;
    const uint32_t d = dc * 8u;
    const int64_t r0 = (int64_t)rtile * RW;
    const int nr = (int)min<int64_t>(RW, a.rows - r0);

    int64_t rs[RW], tt[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const int64_t rr = min<int64_t>(r0 + i, a.rows - 1);
        rs[i] = a.src ? (int64_t)a.src[rr] : rr;
        tt[i] = SCATTER ? (int64_t)a.pos[rr] : rr;
    }
    u32x2 cw8[RW];
    uint32_t cw4[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const size_t hr = (size_t)rs[i] * (uint32_t)a.H + h;
        if constexpr (FMT == FMT_FP8_ROW)
            cw8[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(a.codes + hr * (uint32_t)a.D + d));
        else
            cw4[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(a.codes) + (size_t)rs[i] * (uint32_t)a.C8 + c8);
    }
    u32x4 pv[RW];
    if constexpr (ADD) {
#pragma unroll
        for (int i = 0; i < RW; ++i) pv[i] = ld_stream(a.prev + tt[i] * a.pst + (int64_t)h * a.psh + d);
    }
    float sc[RW];
    if constexpr (FMT == FMT_FP8_ROW) {
#pragma unroll
        for (int i = 0; i < RW; ++i) sc[i] = reinterpret_cast<const float*>(a.meta0)[(size_t)rs[i] * (uint32_t)a.H + h];
    } else {
        const uint32_t nb = ((uint32_t)a.D + 15u) / 16u;
        const auto s_dec = [&](int i) {
            const size_t hr = (size_t)rs[i] * (uint32_t)a.H + h;
            const uint32_t code = reinterpret_cast<const uint8_t*>(a.meta0)[hr * nb + (dc >> 1)] & 0x7Fu;
            return fp4_code_scales(code, reinterpret_cast<const float*>(a.meta1)[hr])[0];
        };
        if (a.D8 >= 2) {
            // A 16-channel block is a lane pair (l, l ^ 1): the even lane divides for the even
            // rows, the odd lane for the odd rows, and the two swap their quotients.
            const bool odd = (c8raw & 1u) != 0u;
#pragma unroll
            for (int j = 0; j < RW / 2; ++j) {
                const float mine = s_dec(2 * j + (odd ? 1 : 0));
                const float other = __uint_as_float(dpp<0xB1>(__float_as_uint(mine)));
                sc[2 * j] = odd ? other : mine;
                sc[2 * j + 1] = odd ? mine : other;
            }
        } else {
#pragma unroll
            for (int i = 0; i < RW; ++i) sc[i] = s_dec(i);
        }
    }
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        float y[8];
        if constexpr (FMT == FMT_FP8_ROW) {
            const f32x2 e0 = fp8_values<false>(cw8[i][0]), e1 = fp8_values<true>(cw8[i][0]);
            const f32x2 e2 = fp8_values<false>(cw8[i][1]), e3 = fp8_values<true>(cw8[i][1]);
            const float e[8] = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
#pragma unroll
            for (int k = 0; k < 8; ++k) y[k] = __fmul_rn(e[k], sc[i]);
        } else {
            const f32x2 e0 = e2m1_values<0>(cw4[i]), e1 = e2m1_values<1>(cw4[i]);
            const f32x2 e2 = e2m1_values<2>(cw4[i]), e3 = e2m1_values<3>(cw4[i]);
            const float e[8] = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
#pragma unroll
            for (int k = 0; k < 8; ++k) y[k] = __fmul_rn(e[k], sc[i]);
        }
        u32x4 o;
        o.x = row_finish<ADD>(y[0], y[1], ADD ? pv[i].x : 0u);
        o.y = row_finish<ADD>(y[2], y[3], ADD ? pv[i].y : 0u);
        o.z = row_finish<ADD>(y[4], y[5], ADD ? pv[i].z : 0u);
        o.w = row_finish<ADD>(y[6], y[7], ADD ? pv[i].w : 0u);
        if (i < nr && valid)
            *reinterpret_cast<u32x4*>(a.out + row_offset(tt[i], a.opshift, a.opst, a.ost) + (int64_t)h * a.osh + d) = o;
    }
}

// Generic decoder: one thread per (row, head, channel pair).
template <int FMT, bool ADD, bool SCATTER>
__global__ __launch_bounds__(kThreads) void k_row_decode_gen(DecArgs a) {
    const int D = a.D;
    const int Dp = (D + 1) / 2;
    const int64_t idx = (int64_t)(a.gen_base + (uint64_t)blockIdx.x * kThreads + threadIdx.x);
    if (idx >= a.rows * a.H * Dp) return;
    const int64_t r = idx / ((int64_t)a.H * Dp);
    const int64_t rem = idx - r * a.H * Dp;
    const int64_t h = rem / Dp;
    const int j = (int)(rem - h * Dp);
    const int64_t t = SCATTER ? (int64_t)a.pos[r] : r;
    const int64_t rs = a.src ? (int64_t)a.src[r] : r;
    const size_t hr = (size_t)(rs * a.H + h);
    for (int k = 0; k < 2; ++k) {
        const int dd = 2 * j + k;
        if (dd >= D) break;
        float y;
        if constexpr (FMT == FMT_FP8_ROW) {
            const uint32_t c = a.codes[hr * (size_t)D + dd];
            const float v = __uint_as_float(__float_as_uint(e4m3_decode(c & 0x7Fu)) | ((c & 0x80u) << 24));
            y = __fmul_rn(v, reinterpret_cast<const float*>(a.meta0)[hr]);
        } else {
            const uint32_t c = (a.codes[hr * (size_t)Dp + j] >> (4 * k)) & 0xFu;
            const uint32_t sc8 = reinterpret_cast<const uint8_t*>(a.meta0)[hr * (size_t)((D + 15) / 16) + dd / 16] & 0x7Fu;
            const float s_dec = fp4_code_scales(sc8, reinterpret_cast<const float*>(a.meta1)[hr])[0];
            y = __fmul_rn(e2m1_values<0>(c)[0], s_dec);
        }
        uint32_t outb = bf16_bits(y);
        if constexpr (ADD) {
            const float p = bf16_to_f32(a.prev[t * a.pst + h * a.psh + dd]);
            outb = bf16_bits(__fadd_rn(p, bf16_to_f32(outb)));
        }
        a.out[row_offset(t, a.opshift, a.opst, a.ost) + h * a.osh + dd] = (uint16_t)outb;
    }
}

inline uint32_t ceil_div_u(uint64_t a, uint64_t b) { return (uint32_t)((a + b - 1) / b); }

template <int FMT, bool DIFF, bool GATHER>
void row_encode_launch(const EncArgs& a, bool vec, hipStream_t s) {
    EncArgs b = a;
    const dim3 grid = grid_with_copy(b, ceil_div_u(a.n_tasks, 4), 4u);
    const bool win = !GATHER && a.win_tasks;  // a window never gathers
    if (vec && a.ri_shift > 0) {
        if (win) hipLaunchKernelGGL((k_row_encode_vec<FMT, DIFF, false, true, true>), grid, dim3(kThreads), 0, s, b);
        else hipLaunchKernelGGL((k_row_encode_vec<FMT, DIFF, GATHER, true, false>), grid, dim3(kThreads), 0, s, b);
    } else if (vec) {
        if (win) hipLaunchKernelGGL((k_row_encode_vec<FMT, DIFF, false, false, true>), grid, dim3(kThreads), 0, s, b);
        else hipLaunchKernelGGL((k_row_encode_vec<FMT, DIFF, GATHER, false, false>), grid, dim3(kThreads), 0, s, b);
    } else {
        launch_in_chunks(a, (uint64_t)a.rows * a.H, kThreads, [&](const EncArgs& b, dim3 grid) {
            hipLaunchKernelGGL((k_row_encode_gen<FMT, DIFF, GATHER>), grid, dim3(kThreads), 0, s, b);
        });
    }
}

template <int FMT, bool ADD, bool SCATTER>
void row_decode_launch(const DecArgs& a, bool vec, hipStream_t s) {
    if (vec) {
        DecArgs b = a;
        const dim3 grid = grid_with_copy(b, ceil_div_u(a.n_tasks, 4), 4u);
        const bool win = !SCATTER && a.win_tasks;  // a window never scatters
        if (a.ri_shift > 0) {
            if (win) hipLaunchKernelGGL((k_row_decode_vec<FMT, ADD, false, true, true>), grid, dim3(kThreads), 0, s, b);
            else hipLaunchKernelGGL((k_row_decode_vec<FMT, ADD, SCATTER, true, false>), grid, dim3(kThreads), 0, s, b);
        } else {
            if (win) hipLaunchKernelGGL((k_row_decode_vec<FMT, ADD, false, false, true>), grid, dim3(kThreads), 0, s, b);
            else hipLaunchKernelGGL((k_row_decode_vec<FMT, ADD, SCATTER, false, false>), grid, dim3(kThreads), 0, s, b);
        }
    } else {
        const uint64_t n = (uint64_t)a.rows * a.H * ((a.D + 1) / 2);
        launch_in_chunks(a, n, kThreads, [&](const DecArgs& b, dim3 grid) {
            hipLaunchKernelGGL((k_row_decode_gen<FMT, ADD, SCATTER>), grid, dim3(kThreads), 0, s, b);
        });
    }
}

template <int FMT>
void row_encode_fmt(const EncArgs& a, bool diff, bool gather, bool vec, hipStream_t s) {
    if (diff) {
        if (gather) row_encode_launch<FMT, true, true>(a, vec, s);
        else row_encode_launch<FMT, true, false>(a, vec, s);
    } else {
        if (gather) row_encode_launch<FMT, false, true>(a, vec, s);
        else row_encode_launch<FMT, false, false>(a, vec, s);
    }
}

template <int FMT>
void row_decode_fmt(const DecArgs& a, bool add, bool scatter, bool vec, hipStream_t s) {
    if (add) {
        if (scatter) row_decode_launch<FMT, true, true>(a, vec, s);
        else row_decode_launch<FMT, true, false>(a, vec, s);
    } else {
        if (scatter) row_decode_launch<FMT, false, true>(a, vec, s);
        else row_decode_launch<FMT, false, false>(a, vec, s);
    }
}

}  // namespace

hipError_t launch_row_encode(int fmt, const EncArgs& a, bool diff, bool gather, bool vec, hipStream_t s) {
    if (fmt == FMT_FP8_ROW) row_encode_fmt<FMT_FP8_ROW>(a, diff, gather, vec, s);
    else if (fmt == FMT_NVFP4_ROW) row_encode_fmt<FMT_NVFP4_ROW>(a, diff, gather, vec, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_row_decode(int fmt, const DecArgs& a, bool add, bool scatter, bool vec, hipStream_t s) {
    if (fmt == FMT_FP8_ROW) row_decode_fmt<FMT_FP8_ROW>(a, add, scatter, vec, s);
    else if (fmt == FMT_NVFP4_ROW) row_decode_fmt<FMT_NVFP4_ROW>(a, add, scatter, vec, s);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace kvq
