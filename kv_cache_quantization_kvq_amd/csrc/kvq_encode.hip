// kvq_encode.hip -- encode kernels: pack_kv and encode_residual for INT4 and NVFP4.
//
// Group axes ([PR166] = vllm-rlt PR #166 "INT4 KV packing/unpacking and cross-loop residual
// reconstruction", section "Purpose", third bullet): a KEY group is G consecutive token rows of
// one (head, channel); a VALUE group is G consecutive channels of one (token, head). The last
// group along the axis may be partial.
//
// Vector path (D % 8 == 0, 16-byte aligned rows): one lane owns 8 consecutive channels of a
// row and moves them with one 16-byte load; codes leave as one 32-bit word per lane.
//   VALUE: a group is G/8 adjacent lanes; its min/max (or abs-max) is an all-reduce over those
//          lanes with DPP row moves.
//   KEY:   a group is a column of G rows; each lane keeps its rows in registers and reduces over
//          them itself (no transpose); when a group is split over several waves the partial
//          results meet in LDS once.
// Generic path: any D, G, stride or alignment; one thread per (row, head) for VALUE and per
// (token group, head, channel pair) for KEY, two passes over the members.
#include "kvq_launch.hpp"

namespace kvq {

namespace {

constexpr int kThreads = 256;

// ---- element access ----------------------------------------------------------------------------

template <bool DIFF>
__device__ __forceinline__ uint4 load_row8(const EncArgs& a, int64_t t, uint32_t h, uint32_t d) {
    uint4 v = *reinterpret_cast<const uint4*>(a.cur + t * a.cst + (int64_t)h * a.csh + d);
    if constexpr (DIFF) {
        uint4 p = *reinterpret_cast<const uint4*>(a.prev + t * a.pst + (int64_t)h * a.psh + d);
        v.x = sub_bf16x2(v.x, p.x);
        v.y = sub_bf16x2(v.y, p.y);
        v.z = sub_bf16x2(v.z, p.z);
        v.w = sub_bf16x2(v.w, p.w);
    }
    return v;
}

// bf16 bits of the encoded value of element (t, h, d) (generic path)
template <bool DIFF>
__device__ __forceinline__ uint32_t load_one(const EncArgs& a, int64_t t, int64_t h, int64_t d) {
    uint32_t c = a.cur[t * a.cst + h * a.csh + d];
    if constexpr (DIFF) {
        uint32_t p = a.prev[t * a.pst + h * a.psh + d];
        return f32_to_bf16(__fsub_rn(bf16_to_f32(c), bf16_to_f32(p)));
    }
    return c;
}

__device__ __forceinline__ uint32_t imin_op(uint32_t x, uint32_t y) { return (uint32_t)min((int)x, (int)y); }
__device__ __forceinline__ uint32_t imax_op(uint32_t x, uint32_t y) { return (uint32_t)max((int)x, (int)y); }
__device__ __forceinline__ uint32_t umax_op(uint32_t x, uint32_t y) { return max(x, y); }

template <int FMT, typename GC>
__device__ __forceinline__ uint32_t code_of(float x, const GC& g) {
    if constexpr (FMT == FMT_INT4)
        return int4_code(x, g);
    else
        return fp4_code(x, g);
}

template <int FMT, typename GC>
__device__ __forceinline__ uint32_t codes8(const uint4& v, const GC& g) {
    return code_of<FMT>(bf16lo(v.x), g) | (code_of<FMT>(bf16hi(v.x), g) << 4) | (code_of<FMT>(bf16lo(v.y), g) << 8) |
           (code_of<FMT>(bf16hi(v.y), g) << 12) | (code_of<FMT>(bf16lo(v.z), g) << 16) |
           (code_of<FMT>(bf16hi(v.z), g) << 20) | (code_of<FMT>(bf16lo(v.w), g) << 24) |
           (code_of<FMT>(bf16hi(v.w), g) << 28);
}

// ---- VALUE, vector path ------------------------------------------------------------------------

// A wave task is RW consecutive rows of one 64-chunk column slab.
template <int FMT, bool DIFF, bool GATHER>
__global__ __launch_bounds__(kThreads) void k_encode_v_vec(EncArgs a) {
    constexpr int RW = 4;
    const int lane = threadIdx.x & 63;
    const uint32_t task = __builtin_amdgcn_readfirstlane(blockIdx.x * 4u + (threadIdx.x >> 6));
    if (task >= a.n_tasks) return;
    const uint32_t rtile = fdiv(task, a.div_slabs);
    const uint32_t slab = task - rtile * (uint32_t)a.n_slabs;
    const uint32_t c8 = slab * 64u + lane;
    const bool valid = c8 < (uint32_t)a.C8;
    const uint32_t h = fdiv(c8, a.div_D8);
    const uint32_t d = (c8 - h * (uint32_t)a.D8) * 8u;
    const int64_t r0 = (int64_t)rtile * RW;
    const int nr = (int)min<int64_t>(RW, a.rows - r0);
    const int lpg = a.lpg;

    uint4 v[RW];
    int64_t tt[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        v[i] = make_uint4(0u, 0u, 0u, 0u);
        tt[i] = r0 + i;
        if (i < nr) {
            if constexpr (GATHER) tt[i] = a.pos[r0 + i];
            if (valid) v[i] = load_row8<DIFF>(a, tt[i], h, d);
        }
    }
    float g = 0.0f;
    if constexpr (FMT == FMT_NVFP4) g = *a.gscale;
    const bool leader = valid && ((lane & (lpg - 1)) == 0);

#pragma unroll
    for (int i = 0; i < RW; ++i) {
        if (i >= nr) break;
        const int64_t r = r0 + i;
        uint32_t word;
        const size_t midx = (size_t)r * (uint32_t)a.ngr + (c8 >> a.lpg_shift);
        if constexpr (FMT == FMT_INT4) {
            short2_t k = keys2(v[i].x), mn = k, mx = k;
            k = keys2(v[i].y); mn = min2(mn, k); mx = max2(mx, k);
            k = keys2(v[i].z); mn = min2(mn, k); mx = max2(mx, k);
            k = keys2(v[i].w); mn = min2(mn, k); mx = max2(mx, k);
            uint32_t kmn = (uint32_t)min((int)mn.x, (int)mn.y);
            uint32_t kmx = (uint32_t)max((int)mx.x, (int)mx.y);
            kmn = group_allreduce(kmn, lpg, imin_op);
            kmx = group_allreduce(kmx, lpg, imax_op);
            const Int4Group gp = int4_group(key_to_f32((int)kmn), key_to_f32((int)kmx));
            word = codes8<FMT_INT4>(v[i], gp);
            if (leader) {
                reinterpret_cast<uint16_t*>(a.meta0)[midx] = (uint16_t)f32_to_f16(gp.mn);
                reinterpret_cast<uint16_t*>(a.meta1)[midx] = (uint16_t)f32_to_f16(gp.scale);
            }
        } else {
            ushort2_t m = umax2(umax2(mag2(v[i].x), mag2(v[i].y)), umax2(mag2(v[i].z), mag2(v[i].w)));
            uint32_t bam = max((uint32_t)m.x, (uint32_t)m.y);
            bam = group_allreduce(bam, lpg, umax_op);
            const Fp4Block fb = fp4_block(bam, g);
            word = codes8<FMT_NVFP4>(v[i], fb);
            if (leader) reinterpret_cast<uint8_t*>(a.meta0)[midx] = (uint8_t)fb.code;
        }
        if (valid) reinterpret_cast<uint32_t*>(a.codes)[(size_t)r * (uint32_t)a.C8 + c8] = word;
        if constexpr (GATHER) {
            if (c8 == 0) a.pos_out[r] = (int32_t)tt[i];
        }
    }
}

// ---- KEY, vector path --------------------------------------------------------------------------

// An item is one token group (G rows) of one 64-chunk column slab. WPG waves share an item,
// RPW rows each; a block of 4 waves holds 4/WPG items.
template <int FMT, int G, bool DIFF, bool GATHER>
__global__ __launch_bounds__(kThreads) void k_encode_k_vec(EncArgs a) {
    constexpr int WPG = (G >= 64) ? 4 : G / 16;
    constexpr int RPW = G / WPG;
    constexpr int IPB = 4 / WPG;
    constexpr int NW = (FMT == FMT_INT4) ? 8 : 4;  // exchanged words per lane
    __shared__ uint32_t lds[WPG > 1 ? 4 * NW * 64 : 1];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wsub = wave % WPG;
    const uint32_t item = blockIdx.x * (uint32_t)IPB + (uint32_t)(wave / WPG);
    const bool item_ok = item < a.n_tasks;
    const uint32_t b = fdiv(item, a.div_slabs);
    const uint32_t slab = item - b * (uint32_t)a.n_slabs;
    const uint32_t c8 = slab * 64u + lane;
    const bool valid = item_ok && c8 < (uint32_t)a.C8;
    const uint32_t h = fdiv(c8, a.div_D8);
    const uint32_t d = (c8 - h * (uint32_t)a.D8) * 8u;
    const int64_t r0 = (int64_t)b * G + (int64_t)wsub * RPW;
    const int nr = item_ok ? (int)max<int64_t>(0, min<int64_t>(RPW, a.rows - r0)) : 0;

    uint4 v[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        v[i] = make_uint4(0u, 0u, 0u, 0u);
        if (i < nr && valid) {
            const int64_t t = GATHER ? (int64_t)a.pos[r0 + i] : r0 + i;
            v[i] = load_row8<DIFF>(a, t, h, d);
        }
    }

    // per-channel statistics over this wave's rows: channel 2j in .x, 2j+1 in .y of word j
    uint32_t st[NW];
    if constexpr (FMT == FMT_INT4) {
        short2_t mn[4], mx[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            mn[j] = (short2_t){0x7FFF, 0x7FFF};
            mx[j] = (short2_t){-32768, -32768};
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            if (i < nr) {
                const uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    short2_t k = keys2(w4[j]);
                    mn[j] = min2(mn[j], k);
                    mx[j] = max2(mx[j], k);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            st[j] = s2_as_u(mn[j]);
            st[4 + j] = s2_as_u(mx[j]);
        }
    } else {
        ushort2_t am[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) am[j] = (ushort2_t){0, 0};
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            if (i < nr) {
                am[0] = umax2(am[0], mag2(v[i].x));
                am[1] = umax2(am[1], mag2(v[i].y));
                am[2] = umax2(am[2], mag2(v[i].z));
                am[3] = umax2(am[3], mag2(v[i].w));
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) st[j] = us2_as_u(am[j]);
    }

    if constexpr (WPG > 1) {
#pragma unroll
        for (int k = 0; k < NW; ++k) lds[(wave * NW + k) * 64 + lane] = st[k];
        __syncthreads();
        const int base = (wave / WPG) * WPG;
#pragma unroll
        for (int o = 1; o < WPG; ++o) {
            const int w2 = base + (wsub + o) % WPG;
            if constexpr (FMT == FMT_INT4) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    st[j] = s2_as_u(min2(as_s2(st[j]), as_s2(lds[(w2 * NW + j) * 64 + lane])));
                    st[4 + j] = s2_as_u(max2(as_s2(st[4 + j]), as_s2(lds[(w2 * NW + 4 + j) * 64 + lane])));
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    st[j] = us2_as_u(umax2(as_us2(st[j]), as_us2(lds[(w2 * NW + j) * 64 + lane])));
            }
        }
    }
    if (!item_ok) return;

    const size_t mbase = ((size_t)b * (uint32_t)a.C8 + c8) * 8u;
    if constexpr (FMT == FMT_INT4) {
        Int4Group gp[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const short2_t mn = as_s2(st[j]), mx = as_s2(st[4 + j]);
            gp[2 * j] = int4_group(key_to_f32(mn.x), key_to_f32(mx.x));
            gp[2 * j + 1] = int4_group(key_to_f32(mn.y), key_to_f32(mx.y));
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            if (i < nr && valid) {
                const uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
                uint32_t word = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    word |= int4_code(bf16lo(w4[j]), gp[2 * j]) << (8 * j);
                    word |= int4_code(bf16hi(w4[j]), gp[2 * j + 1]) << (8 * j + 4);
                }
                reinterpret_cast<uint32_t*>(a.codes)[(size_t)(r0 + i) * (uint32_t)a.C8 + c8] = word;
            }
        }
        if (wsub == 0 && valid) {
            uint4 mins, scales;
            mins.x = f32_to_f16(gp[0].mn) | (f32_to_f16(gp[1].mn) << 16);
            mins.y = f32_to_f16(gp[2].mn) | (f32_to_f16(gp[3].mn) << 16);
            mins.z = f32_to_f16(gp[4].mn) | (f32_to_f16(gp[5].mn) << 16);
            mins.w = f32_to_f16(gp[6].mn) | (f32_to_f16(gp[7].mn) << 16);
            scales.x = f32_to_f16(gp[0].scale) | (f32_to_f16(gp[1].scale) << 16);
            scales.y = f32_to_f16(gp[2].scale) | (f32_to_f16(gp[3].scale) << 16);
            scales.z = f32_to_f16(gp[4].scale) | (f32_to_f16(gp[5].scale) << 16);
            scales.w = f32_to_f16(gp[6].scale) | (f32_to_f16(gp[7].scale) << 16);
            *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.meta0) + mbase) = mins;
            *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(a.meta1) + mbase) = scales;
        }
    } else {
        const float g = *a.gscale;
        Fp4Block fb[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const ushort2_t am = as_us2(st[j]);
            fb[2 * j] = fp4_block(am.x, g);
            fb[2 * j + 1] = fp4_block(am.y, g);
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            if (i < nr && valid) {
                const uint32_t w4[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
                uint32_t word = 0;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    word |= fp4_code(bf16lo(w4[j]), fb[2 * j]) << (8 * j);
                    word |= fp4_code(bf16hi(w4[j]), fb[2 * j + 1]) << (8 * j + 4);
                }
                reinterpret_cast<uint32_t*>(a.codes)[(size_t)(r0 + i) * (uint32_t)a.C8 + c8] = word;
            }
        }
        if (wsub == 0 && valid) {
            uint2 sc;
            sc.x = fb[0].code | (fb[1].code << 8) | (fb[2].code << 16) | (fb[3].code << 24);
            sc.y = fb[4].code | (fb[5].code << 8) | (fb[6].code << 16) | (fb[7].code << 24);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(a.meta0) + mbase) = sc;
        }
    }
    if constexpr (GATHER) {
        if (slab == 0 && lane == 0)
            for (int i = 0; i < nr; ++i) a.pos_out[r0 + i] = a.pos[r0 + i];
    }
}

// ---- generic paths -----------------------------------------------------------------------------

// VALUE: one thread per (row, head), groups walked along the row.
template <int FMT, bool DIFF, bool GATHER>
__global__ __launch_bounds__(kThreads) void k_encode_v_gen(EncArgs a) {
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= a.rows * a.H) return;
    const int64_t r = idx / a.H;
    const int64_t h = idx - r * a.H;
    const int64_t t = GATHER ? (int64_t)a.pos[r] : r;
    const int D = a.D, G = a.G;
    const int ngr = (D + G - 1) / G;
    const int Dp = (D + 1) / 2;
    float g = 0.0f;
    if constexpr (FMT == FMT_NVFP4) g = *a.gscale;
    uint8_t* crow = a.codes + (size_t)(r * a.H + h) * Dp;
    uint32_t pending = 0;
    for (int c = 0; c < ngr; ++c) {
        const int d0 = c * G, d1 = min(D, d0 + G);
        const size_t midx = (size_t)(r * a.H + h) * ngr + c;
        if constexpr (FMT == FMT_INT4) {
            int kmn = 0x7FFF, kmx = -32768;
            for (int dd = d0; dd < d1; ++dd) {
                const int k = bf16_key(load_one<DIFF>(a, t, h, dd));
                kmn = min(kmn, k);
                kmx = max(kmx, k);
            }
            const Int4Group gp = int4_group(key_to_f32(kmn), key_to_f32(kmx));
            reinterpret_cast<uint16_t*>(a.meta0)[midx] = (uint16_t)f32_to_f16(gp.mn);
            reinterpret_cast<uint16_t*>(a.meta1)[midx] = (uint16_t)f32_to_f16(gp.scale);
            for (int dd = d0; dd < d1; ++dd) {
                const uint32_t code = int4_code(bf16_to_f32(load_one<DIFF>(a, t, h, dd)), gp);
                if (dd & 1)
                    crow[dd >> 1] = (uint8_t)(pending | (code << 4));
                else
                    pending = code;
            }
        } else {
            uint32_t bam = 0;
            for (int dd = d0; dd < d1; ++dd) bam = max(bam, load_one<DIFF>(a, t, h, dd) & 0x7FFFu);
            const Fp4Block fb = fp4_block(bam, g);
            reinterpret_cast<uint8_t*>(a.meta0)[midx] = (uint8_t)fb.code;
            for (int dd = d0; dd < d1; ++dd) {
                const uint32_t code = fp4_code(bf16_to_f32(load_one<DIFF>(a, t, h, dd)), fb);
                if (dd & 1)
                    crow[dd >> 1] = (uint8_t)(pending | (code << 4));
                else
                    pending = code;
            }
        }
    }
    if (D & 1) crow[D >> 1] = (uint8_t)pending;
    if constexpr (GATHER) {
        if (h == 0) a.pos_out[r] = (int32_t)t;
    }
}

// KEY: one thread per (token group, head, channel pair 2j / 2j+1).
template <int FMT, bool DIFF, bool GATHER>
__global__ __launch_bounds__(kThreads) void k_encode_k_gen(EncArgs a) {
    const int D = a.D, G = a.G;
    const int Dp = (D + 1) / 2;
    const int64_t nb = (a.rows + G - 1) / G;
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= nb * a.H * Dp) return;
    const int64_t b = idx / ((int64_t)a.H * Dp);
    const int64_t rem = idx - b * a.H * Dp;
    const int64_t h = rem / Dp;
    const int j = (int)(rem - h * Dp);
    const int nch = (2 * j + 1 < D) ? 2 : 1;
    const int64_t r_begin = b * G, r_end = min<int64_t>(a.rows, r_begin + G);
    float g = 0.0f;
    if constexpr (FMT == FMT_NVFP4) g = *a.gscale;

    Int4Group gp[2];
    Fp4Block fb[2];
    for (int k = 0; k < nch; ++k) {
        const int dd = 2 * j + k;
        const size_t midx = (size_t)(b * a.H + h) * D + dd;
        if constexpr (FMT == FMT_INT4) {
            int kmn = 0x7FFF, kmx = -32768;
            for (int64_t r = r_begin; r < r_end; ++r) {
                const int64_t t = GATHER ? (int64_t)a.pos[r] : r;
                const int key = bf16_key(load_one<DIFF>(a, t, h, dd));
                kmn = min(kmn, key);
                kmx = max(kmx, key);
            }
            gp[k] = int4_group(key_to_f32(kmn), key_to_f32(kmx));
            reinterpret_cast<uint16_t*>(a.meta0)[midx] = (uint16_t)f32_to_f16(gp[k].mn);
            reinterpret_cast<uint16_t*>(a.meta1)[midx] = (uint16_t)f32_to_f16(gp[k].scale);
        } else {
            uint32_t bam = 0;
            for (int64_t r = r_begin; r < r_end; ++r) {
                const int64_t t = GATHER ? (int64_t)a.pos[r] : r;
                bam = max(bam, load_one<DIFF>(a, t, h, dd) & 0x7FFFu);
            }
            fb[k] = fp4_block(bam, g);
            reinterpret_cast<uint8_t*>(a.meta0)[midx] = (uint8_t)fb[k].code;
        }
    }
    for (int64_t r = r_begin; r < r_end; ++r) {
        const int64_t t = GATHER ? (int64_t)a.pos[r] : r;
        uint32_t byte = 0;
        for (int k = 0; k < nch; ++k) {
            const float x = bf16_to_f32(load_one<DIFF>(a, t, h, 2 * j + k));
            const uint32_t code = (FMT == FMT_INT4) ? int4_code(x, gp[k]) : fp4_code(x, fb[k]);
            byte |= code << (4 * k);
        }
        a.codes[(size_t)(r * a.H + h) * Dp + j] = (uint8_t)byte;
        if constexpr (GATHER) {
            if (h == 0 && j == 0) a.pos_out[r] = (int32_t)t;
        }
    }
}

// ---- NVFP4 tensor amax + global multiplier -----------------------------------------------------

// Grid-stride max of |x| (bf16 magnitude bits) over every encoded element. Each block folds its
// maximum into ws[0]; the last block to finish (counter ws[1]) turns the tensor amax into the
// global multiplier, stores it, and returns the workspace to zero for the next call.
template <bool DIFF, bool GATHER, bool VEC>
__global__ __launch_bounds__(kThreads) void k_amax(EncArgs a, uint64_t total) {
    constexpr int U = 4;
    uint32_t m = 0;
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    for (uint64_t u0 = (uint64_t)blockIdx.x * kThreads + threadIdx.x; u0 < total; u0 += stride * U) {
        if constexpr (VEC) {
            uint4 v[U];
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const uint64_t u = u0 + k * stride;
                v[k] = make_uint4(0u, 0u, 0u, 0u);
                if (u < total) {
                    const uint32_t r = fdiv((uint32_t)u, a.div_C8);
                    const uint32_t c8 = (uint32_t)u - r * (uint32_t)a.C8;
                    const uint32_t h = fdiv(c8, a.div_D8);
                    const uint32_t d = (c8 - h * (uint32_t)a.D8) * 8u;
                    const int64_t t = GATHER ? (int64_t)a.pos[r] : (int64_t)r;
                    v[k] = load_row8<DIFF>(a, t, h, d);
                }
            }
#pragma unroll
            for (int k = 0; k < U; ++k) {
                ushort2_t mm = umax2(umax2(mag2(v[k].x), mag2(v[k].y)), umax2(mag2(v[k].z), mag2(v[k].w)));
                m = max(m, max((uint32_t)mm.x, (uint32_t)mm.y));
            }
        } else {
            const int64_t HD = (int64_t)a.H * a.D;
            for (int k = 0; k < U; ++k) {
                const uint64_t u = u0 + k * stride;
                if (u < total) {
                    const int64_t r = (int64_t)(u / (uint64_t)HD);
                    const int64_t rem = (int64_t)u - r * HD;
                    const int64_t h = rem / a.D;
                    const int64_t d = rem - h * a.D;
                    const int64_t t = GATHER ? (int64_t)a.pos[r] : r;
                    m = max(m, load_one<DIFF>(a, t, h, d) & 0x7FFFu);
                }
            }
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    __shared__ uint32_t sm[kThreads / 64];
    if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = max(max(sm[0], sm[1]), max(sm[2], sm[3]));
        atomicMax(&a.ws[0], m);
        __threadfence();
        const uint32_t ticket = atomicAdd(&a.ws[1], 1u);
        if (ticket == gridDim.x - 1) {
            __threadfence();
            const uint32_t amax = atomicMax(&a.ws[0], 0u);
            *a.gscale = fp4_global(amax);
            atomicExch(&a.ws[0], 0u);
            atomicExch(&a.ws[1], 0u);
        }
    }
}

__global__ void k_set_global(float* gscale, uint32_t bits) { *gscale = __uint_as_float(bits); }

inline uint32_t ceil_div_u(uint64_t a, uint64_t b) { return (uint32_t)((a + b - 1) / b); }

template <int FMT, bool DIFF, bool GATHER>
hipError_t encode_dispatch(int kind, const EncArgs& a, bool vec, hipStream_t s) {
    if (vec) {
        if (kind == KIND_VALUE) {
            hipLaunchKernelGGL((k_encode_v_vec<FMT, DIFF, GATHER>), dim3(ceil_div_u(a.n_tasks, 4)), dim3(kThreads), 0,
                               s, a);
        } else {
            switch (a.G) {
                case 16:
                    hipLaunchKernelGGL((k_encode_k_vec<FMT, 16, DIFF, GATHER>), dim3(ceil_div_u(a.n_tasks, 4)),
                                       dim3(kThreads), 0, s, a);
                    break;
                case 32:
                    if constexpr (FMT == FMT_INT4)
                        hipLaunchKernelGGL((k_encode_k_vec<FMT, 32, DIFF, GATHER>), dim3(ceil_div_u(a.n_tasks, 2)),
                                           dim3(kThreads), 0, s, a);
                    break;
                case 64:
                    if constexpr (FMT == FMT_INT4)
                        hipLaunchKernelGGL((k_encode_k_vec<FMT, 64, DIFF, GATHER>), dim3(a.n_tasks), dim3(kThreads), 0,
                                           s, a);
                    break;
                case 128:
                    if constexpr (FMT == FMT_INT4)
                        hipLaunchKernelGGL((k_encode_k_vec<FMT, 128, DIFF, GATHER>), dim3(a.n_tasks), dim3(kThreads),
                                           0, s, a);
                    break;
                default:
                    return hipErrorInvalidValue;
            }
        }
    } else {
        if (kind == KIND_VALUE) {
            const uint64_t n = (uint64_t)a.rows * a.H;
            hipLaunchKernelGGL((k_encode_v_gen<FMT, DIFF, GATHER>), dim3(ceil_div_u(n, kThreads)), dim3(kThreads), 0,
                               s, a);
        } else {
            const uint64_t nb = (uint64_t)(a.rows + a.G - 1) / a.G;
            const uint64_t n = nb * a.H * ((a.D + 1) / 2);
            hipLaunchKernelGGL((k_encode_k_gen<FMT, DIFF, GATHER>), dim3(ceil_div_u(n, kThreads)), dim3(kThreads), 0,
                               s, a);
        }
    }
    return hipGetLastError();
}

template <int FMT>
hipError_t encode_fmt(int kind, const EncArgs& a, bool diff, bool gather, bool vec, hipStream_t s) {
    if (diff) {
        return gather ? encode_dispatch<FMT, true, true>(kind, a, vec, s)
                      : encode_dispatch<FMT, true, false>(kind, a, vec, s);
    }
    return gather ? encode_dispatch<FMT, false, true>(kind, a, vec, s)
                  : encode_dispatch<FMT, false, false>(kind, a, vec, s);
}

template <bool DIFF, bool GATHER>
hipError_t amax_dispatch(const EncArgs& a, bool vec, hipStream_t s) {
    const uint64_t total = vec ? (uint64_t)a.rows * (uint64_t)a.C8 : (uint64_t)a.rows * a.H * a.D;
    uint64_t blocks = (total + kThreads * 4 - 1) / (kThreads * 4);
    if (blocks > 1024) blocks = 1024;
    if (blocks < 1) blocks = 1;
    if (vec)
        hipLaunchKernelGGL((k_amax<DIFF, GATHER, true>), dim3((uint32_t)blocks), dim3(kThreads), 0, s, a, total);
    else
        hipLaunchKernelGGL((k_amax<DIFF, GATHER, false>), dim3((uint32_t)blocks), dim3(kThreads), 0, s, a, total);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_encode(int fmt, int kind, const EncArgs& a, bool diff, bool gather, bool vec, hipStream_t s) {
    return fmt == FMT_INT4 ? encode_fmt<FMT_INT4>(kind, a, diff, gather, vec, s)
                           : encode_fmt<FMT_NVFP4>(kind, a, diff, gather, vec, s);
}

hipError_t launch_amax(const EncArgs& a, bool diff, bool gather, bool vec, hipStream_t s) {
    if (diff) return gather ? amax_dispatch<true, true>(a, vec, s) : amax_dispatch<true, false>(a, vec, s);
    return gather ? amax_dispatch<false, true>(a, vec, s) : amax_dispatch<false, false>(a, vec, s);
}

hipError_t launch_set_global(float* gscale, uint32_t bits, hipStream_t s) {
    hipLaunchKernelGGL(k_set_global, dim3(1), dim3(1), 0, s, gscale, bits);
    return hipGetLastError();
}

}  // namespace kvq
