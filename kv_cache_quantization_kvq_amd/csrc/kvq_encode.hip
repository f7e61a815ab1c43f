// kvq_encode.hip -- encode kernels: pack_kv and encode_residual for INT4 and NVFP4.
//
// Group axes ([PR166] = vllm-rlt PR #166 "INT4 KV packing/unpacking and cross-loop residual
// reconstruction", section "Purpose", third bullet): a KEY group is G consecutive token rows of
// one (head, channel); a VALUE group is G consecutive channels of one (token, head). The last
// group along the axis may be partial.
//
// Vector path (D % 8 == 0, 16-byte aligned rows): one lane owns 8 consecutive channels of a
// row and moves them with one 16-byte streaming load; codes leave as one 32-bit word per lane.
//   VALUE: a group is G/8 adjacent lanes; its min/max (or abs-max) is an all-reduce over those
//          lanes with DPP row moves.
//   KEY:   a group is a column of G rows; each lane keeps its rows in registers and reduces over
//          them itself (no transpose); when a group is split over several waves the partial
//          results meet in LDS once.
// All loads of a wave task are issued before any arithmetic and without branches: a tail row
// or an idle lane reads an in-bounds duplicate (the last row of the same group, or a valid
// chunk) whose value cannot change a min, max or abs-max, and only the stores are masked.
// Generic path: any D, G, stride or alignment; one thread per (row, head) for VALUE and per
// (token group, head, channel pair) for KEY, two passes over the members.
#include <type_traits>

#include "kvq_launch.hpp"

namespace kvq {

namespace {

constexpr int kThreads = 256;
typedef float f4_t __attribute__((ext_vector_type(4)));
constexpr uint32_t kAmaxMaxBlocks = KVQ_AMAX_MAX_BLOCKS;  // partial maxima held in the workspace

// ---- element access ----------------------------------------------------------------------------

// bf16 bits of the encoded value of element (t, h, d) (generic path)
template <bool DIFF>
__device__ __forceinline__ uint32_t load_one(const EncArgs& a, int64_t t, int64_t h, int64_t d) {
    uint32_t c = a.cur[row_offset(t, a.cpshift, a.cpst, a.cst) + h * a.csh + d];
    if constexpr (DIFF) {
        uint32_t p = a.prev[t * a.pst + h * a.psh + d];
        return bf16_bits(__fsub_rn(bf16_to_f32(c), bf16_to_f32(p)));
    }
    return c;
}

// Loads the RW rows' 8-channel chunks of one lane (all issued before use), residual applied.
// UNI: r0 is the same on every lane, so each row's address is a scalar base plus the lane's
// 32-bit byte offset within the row (the host keeps a row's span below 2^31 bytes).
template <int RW, bool DIFF, bool GATHER, bool UNI>
__device__ __forceinline__ void load_rows8(const EncArgs& a, int64_t r0, uint32_t h, uint32_t d, u32x4 (&v)[RW]) {
    int64_t t[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const int64_t r = min<int64_t>(r0 + i, a.rows - 1);  // tail rows duplicate the last row
        t[i] = GATHER ? (int64_t)a.pos[r] : r;
    }
    if constexpr (UNI) {
        const uint32_t coff = (uint32_t)(((int64_t)h * a.csh + d) * 2);
#pragma unroll
        for (int i = 0; i < RW; ++i)
            v[i] = ld_stream_at(wave_base(a.cur, row_offset(t[i], a.cpshift, a.cpst, a.cst) * 2), coff);
    } else {
#pragma unroll
        for (int i = 0; i < RW; ++i) v[i] = ld_stream(a.cur + row_offset(t[i], a.cpshift, a.cpst, a.cst) + (int64_t)h * a.csh + d);
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

__device__ __forceinline__ uint32_t imin_op(uint32_t x, uint32_t y) { return (uint32_t)min((int)x, (int)y); }
__device__ __forceinline__ uint32_t imax_op(uint32_t x, uint32_t y) { return (uint32_t)max((int)x, (int)y); }
__device__ __forceinline__ uint32_t umax_op(uint32_t x, uint32_t y) { return max(x, y); }

// 8 INT4 codes of one chunk (channel 2j in nibble 2j); group constants gp[k * stride].
// `slow` (a lane's OR of its groups' slow flags) sends the whole chunk through the division.
// The quotients lie in [0, 15.5); v_cvt_pk_u8_f32 rounds each to the nearest integer, ties to
// even (the device probe checks it on every binary32 in that range), which is the code, and
// places the even channels' codes in the bytes of one word and the odd channels' in another;
// one shift-or interleaves them.
__device__ __forceinline__ uint32_t int4_word(const u32x4& v, const Int4Group* gp, int stride, bool slow) {
    const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
    float d[8], c[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        d[2 * j] = __fsub_rn(bf16lo(w4[j]), gp[(2 * j) * stride].mn);
        d[2 * j + 1] = __fsub_rn(bf16hi(w4[j]), gp[(2 * j + 1) * stride].mn);
    }
    if (__builtin_expect(slow, 0)) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const Int4Group& g = gp[k * stride];
            c[k] = g.slow ? d[k] / g.scale : int4_quot_raw(d[k], g);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) c[k] = int4_quot_raw(d[k], gp[k * stride]);
    }
    uint32_t even = 0, odd = 0;
    even = __builtin_amdgcn_cvt_pk_u8_f32(c[0], 0, even);
    odd = __builtin_amdgcn_cvt_pk_u8_f32(c[1], 0, odd);
    even = __builtin_amdgcn_cvt_pk_u8_f32(c[2], 1, even);
    odd = __builtin_amdgcn_cvt_pk_u8_f32(c[3], 1, odd);
    even = __builtin_amdgcn_cvt_pk_u8_f32(c[4], 2, even);
    odd = __builtin_amdgcn_cvt_pk_u8_f32(c[5], 2, odd);
    even = __builtin_amdgcn_cvt_pk_u8_f32(c[6], 3, even);
    odd = __builtin_amdgcn_cvt_pk_u8_f32(c[7], 3, odd);
    return even | (odd << 4);
}


// ---- VALUE, vector path ------------------------------------------------------------------------

// INT4 VALUE groups of 64 channels (8 lanes) over RW = 8, 4 or 2 rows per task: instead of
// all-reducing every row's minimum and maximum over the group's 8 lanes (and then computing the
// same group constants on all 8), the statistics are reduce-scattered so that lane j of the group
// ends with row j's (RW = 8; with RW = 4 lanes j and j ^ 1 both end with row j / 2, with RW = 2
// lanes 0-3 with row 0 and 4-7 with row 1), computes that row's constants alone, and the
// constants reach the other lanes by ds_bpermute. Every lane then holds exactly the constants the
// all-reduce would give it, so the codes and metadata are the same bits. Three butterfly steps
// pair lanes j <-> 7 - j (DPP row_half_mirror), j <-> j ^ 2 and j <-> j ^ 1; at each step a lane
// keeps the half of its rows whose index bit matches its own lane bit and sends the other half
// (once a lane holds a single row, the remaining steps combine the row its partner holds too).
template <int RW, bool DIFF, bool GATHER, bool LG>
__device__ __forceinline__ void int4_value_g64(const EncArgs& a, const u32x4 (&v)[RW], int lane, int64_t r0, int nr,
                                               bool valid, uint32_t c8, uint32_t c8raw) {
    static_assert(RW == 8 || RW == 4 || RW == 2, "G64 VALUE rows per task");
    uint32_t mn8[RW], mx8[RW];  // unsigned keys
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        ushort2_t k = as_us2(ukeys2(v[i].x)), mn = k, mx = k;
        k = as_us2(ukeys2(v[i].y)); mn = umin2(mn, k); mx = umax2(mx, k);
        k = as_us2(ukeys2(v[i].z)); mn = umin2(mn, k); mx = umax2(mx, k);
        k = as_us2(ukeys2(v[i].w)); mn = umin2(mn, k); mx = umax2(mx, k);
        mn8[i] = min((uint32_t)mn.x, (uint32_t)mn.y);
        mx8[i] = max((uint32_t)mx.x, (uint32_t)mx.y);
    }
    const uint32_t j = (uint32_t)lane & 7u;
    const bool b2 = (j & 4u) != 0u, b1 = (j & 2u) != 0u, b0 = (j & 1u) != 0u;
    constexpr int H1 = RW / 2, H2 = RW / 4;
    uint32_t mn4[H1], mx4[H1];  // rows H1 b2 + k
#pragma unroll
    for (int k = 0; k < H1; ++k) {
        mn4[k] = min(b2 ? mn8[k + H1] : mn8[k], dpp<0x141>(b2 ? mn8[k] : mn8[k + H1]));
        mx4[k] = max(b2 ? mx8[k + H1] : mx8[k], dpp<0x141>(b2 ? mx8[k] : mx8[k + H1]));
    }
    uint32_t mn2[H2 > 0 ? H2 : 1], mx2[H2 > 0 ? H2 : 1];  // rows H1 b2 + H2 b1 + k
#pragma unroll
    for (int k = 0; k < H2; ++k) {
        mn2[k] = min(b1 ? mn4[k + H2] : mn4[k], dpp<0x4E>(b1 ? mn4[k] : mn4[k + H2]));
        mx2[k] = max(b1 ? mx4[k + H2] : mx4[k], dpp<0x4E>(b1 ? mx4[k] : mx4[k + H2]));
    }
    uint32_t gmn, gmx;  // row jr of this lane
    if constexpr (RW == 8) {
        gmn = min(b0 ? mn2[1] : mn2[0], dpp<0xB1>(b0 ? mn2[0] : mn2[1]));
        gmx = max(b0 ? mx2[1] : mx2[0], dpp<0xB1>(b0 ? mx2[0] : mx2[1]));
    } else if constexpr (RW == 4) {
        gmn = min(mn2[0], dpp<0xB1>(mn2[0]));
        gmx = max(mx2[0], dpp<0xB1>(mx2[0]));
    } else {  // one row per half of the 8 lanes: all-reduce over each half
        const uint32_t n = min(mn4[0], dpp<0x4E>(mn4[0])), x = max(mx4[0], dpp<0x4E>(mx4[0]));
        gmn = min(n, dpp<0xB1>(n));
        gmx = max(x, dpp<0xB1>(x));
    }
    constexpr uint32_t LPR = 8 / RW;  // lanes per row after the scatter
    const uint32_t jr = j / LPR;
    const Int4Group gj = int4_group(ukey_to_f32(gmn), ukey_to_f32(gmx));
    if ((j % LPR) == 0 && (int)jr < nr && valid) {  // row jr's metadata (a group's 8 lanes are all valid or all idle)
        const int64_t r = r0 + jr;
        const int64_t wr = a.dst ? (int64_t)a.dst[r] : r;
        const size_t midx = (size_t)wr * (uint32_t)a.ngr + (c8 >> 3);
        reinterpret_cast<uint16_t*>(a.meta0)[midx] = (uint16_t)f32_to_f16(gj.mn);
        reinterpret_cast<uint16_t*>(a.meta1)[midx] = (uint16_t)f32_to_f16(gj.scale);
    }
    const uint32_t slowb = (uint32_t)(__ballot(gj.slow) >> (lane & 56)) & 0xFFu;
    const int gbase = lane & ~7;
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        Int4Group g;
        g.mn = __shfl(gj.mn, gbase + (int)LPR * i);
        g.scale = __shfl(gj.scale, gbase + (int)LPR * i);
        g.y = __shfl(gj.y, gbase + (int)LPR * i);
        g.slow = ((slowb >> (LPR * i)) & 1u) != 0u;
        const uint32_t word = int4_word(v[i], &g, 0, g.slow);
        if (i < nr) {
            const int64_t r = r0 + i;
            if (!LG && a.dst == nullptr) {
                if (valid) st_code_at<!DIFF>(wave_base_w(a.codes, r * (int64_t)a.C8 * 4), c8 * 4u, word);
            } else {
                const int64_t wr = a.dst ? (int64_t)a.dst[min<int64_t>(r, a.rows - 1)] : r;
                if (valid) st_code<!DIFF>(reinterpret_cast<uint32_t*>(a.codes) + (size_t)wr * (uint32_t)a.C8 + c8, word);
            }
            if constexpr (GATHER) {
                if (c8raw == 0) a.pos_out[r] = a.pos[r];
            }
        }
    }
}

// A wave task is RW consecutive rows of one 64-chunk column slab.
template <int FMT, bool DIFF, bool GATHER, bool LG, bool WIN>
__global__ __launch_bounds__(kThreads) void k_encode_v_vec(EncArgs a) {
    constexpr int RW = value_encode_rows(FMT == FMT_NVFP4, DIFF);
    if (WIN && blockIdx.x >= a.win_block0) {  // blocks of the carried row copy
        window_copy_wave(a.win, __builtin_amdgcn_readfirstlane((blockIdx.x - a.win_block0) * 4u + (threadIdx.x >> 6)),
                         threadIdx.x & 63);
        return;
    }
    __shared__ std::conditional_t<FMT == FMT_NVFP4, Fp4Table, char> tab;
    float g = 0.0f;
    if constexpr (FMT == FMT_NVFP4) {
        g = *a.gscale;
        fp4_table_fill(tab, g);
    }
    const int lane = threadIdx.x & 63;
    const uint32_t task = __builtin_amdgcn_readfirstlane(blockIdx.x * 4u + (threadIdx.x >> 6));
    if (task >= a.n_tasks) return;
    uint32_t rtile, c8raw;
    task_lane<LG>(a, task, lane, rtile, c8raw);  // with LG a lane group past the last row tile stores nothing
    const bool valid = c8raw < (uint32_t)a.C8;
    const uint32_t c8 = valid ? c8raw : (uint32_t)a.C8 - 1u;  // idle lanes read a valid chunk
    const uint32_t h = fdiv(c8, a.div_D8);
    const uint32_t d = (c8 - h * (uint32_t)a.D8) * 8u;
    const int64_t r0 = (int64_t)rtile * RW;
    const int nr = (int)min<int64_t>(RW, a.rows - r0);
    const int lpg = a.lpg;

    u32x4 v[RW];
    load_rows8<RW, DIFF, GATHER, !LG>(a, r0, h, d, v);
    if constexpr (FMT == FMT_INT4 && (RW == 8 || RW == 4 || RW == 2)) {
        if (lpg == 8) {  // G = 64 (wave-uniform)
            int4_value_g64<RW, DIFF, GATHER, LG>(a, v, lane, r0, nr, valid, c8, c8raw);
            return;
        }
    }
    const bool leader = valid && ((lane & (lpg - 1)) == 0);

#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const int64_t r = r0 + i;
        // packed row written (slot writes map it; tail rows read an in-range entry, never store)
        const int64_t wr = a.dst ? (int64_t)a.dst[min<int64_t>(r, a.rows - 1)] : r;
        const size_t midx = (size_t)wr * (uint32_t)a.ngr + (c8 >> a.lpg_shift);
        uint32_t word;
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
            word = int4_word(v[i], &gp, 0, gp.slow);
            if (i < nr && leader) {
                reinterpret_cast<uint16_t*>(a.meta0)[midx] = (uint16_t)f32_to_f16(gp.mn);
                reinterpret_cast<uint16_t*>(a.meta1)[midx] = (uint16_t)f32_to_f16(gp.scale);
            }
        } else {
            ushort2_t m = umax2(umax2(mag2(v[i].x), mag2(v[i].y)), umax2(mag2(v[i].z), mag2(v[i].w)));
            uint32_t bam = max((uint32_t)m.x, (uint32_t)m.y);
            bam = group_allreduce(bam, lpg, umax_op);
            const Fp4Block fb = fp4_block(bam, g, tab);
            word = fp4_word(v[i], &fb, 0);
            if (i < nr && leader) reinterpret_cast<uint8_t*>(a.meta0)[midx] = (uint8_t)fb.code;
        }
        if (i < nr) {
            if (valid) st_code<!DIFF>(reinterpret_cast<uint32_t*>(a.codes) + (size_t)wr * (uint32_t)a.C8 + c8, word);
            if constexpr (GATHER) {
                if (c8raw == 0) a.pos_out[r] = a.pos[r];
            }
        }
    }
}

// ---- KEY, vector path --------------------------------------------------------------------------

// An item is one token group (G rows) of one 64-chunk column slab. WPG waves share an item,
// RPW rows each; a block of WPB waves holds WPB/WPG items.
template <int FMT, int G, bool DIFF, bool GATHER, bool LG, bool WIN>
__global__ __launch_bounds__(64 * key_waves_per_block(G, DIFF, FMT == FMT_INT4)) void k_encode_k_vec(EncArgs a) {
    constexpr int WPG = key_waves_per_group(G, DIFF, FMT == FMT_INT4);
    constexpr int RPW = key_rows_per_wave(G, DIFF, FMT == FMT_INT4);
    constexpr int WPB = key_waves_per_block(G, DIFF, FMT == FMT_INT4);
    constexpr int IPB = WPB / WPG;
    constexpr int NW = (FMT == FMT_INT4) ? 8 : 4;  // exchanged words per lane
    static_assert(WPB <= 16 && WPB % WPG == 0, "KEY encoder block shape");
    if (WIN && blockIdx.x >= a.win_block0) {  // blocks of the carried row copy
        window_copy_wave(a.win,
                         __builtin_amdgcn_readfirstlane((blockIdx.x - a.win_block0) * (uint32_t)WPB + (threadIdx.x >> 6)),
                         threadIdx.x & 63);
        return;
    }
    __shared__ uint32_t lds[WPG > 1 ? WPB * NW * 64 : 1];
    // INT4 with a group split over waves: each item's 8 channels' constants per lane
    constexpr bool SPLIT = FMT == FMT_INT4 && WPG > 1;
    __shared__ f4_t cst[SPLIT ? IPB * 8 * 64 : 1];
    __shared__ std::conditional_t<FMT == FMT_NVFP4, Fp4Table, char> tab;
    float g = 0.0f;
    if constexpr (FMT == FMT_NVFP4) {
        g = *a.gscale;
        fp4_table_fill(tab, g);
    }

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wsub = wave % WPG;
    const uint32_t item_raw = blockIdx.x * (uint32_t)IPB + (uint32_t)(wave / WPG);
    const bool item_ok = item_raw < a.n_tasks;
    const uint32_t item = item_ok ? item_raw : a.n_tasks - 1u;  // surplus waves mirror the last item
    uint32_t b, c8raw;  // token group and chunk of this lane
    task_lane<LG>(a, item, lane, b, c8raw);
    // with LG a lane group past the last token group loads rows of the last one and stores nothing
    const bool valid = item_ok && c8raw < (uint32_t)a.C8 && (int64_t)b * G < a.rows;
    const uint32_t c8 = (c8raw < (uint32_t)a.C8) ? c8raw : (uint32_t)a.C8 - 1u;
    const uint32_t h = fdiv(c8, a.div_D8);
    const uint32_t d = (c8 - h * (uint32_t)a.D8) * 8u;
    const int64_t r0 = (int64_t)b * G + (int64_t)wsub * RPW;
    // rows of this wave that exist; the others load row rows-1, which lies in this (last) group
    const int nr = item_ok ? (int)max<int64_t>(0, min<int64_t>(RPW, a.rows - r0)) : 0;

    u32x4 v[RPW];
    load_rows8<RPW, DIFF, GATHER, !LG>(a, r0, h, d, v);

    // per-channel statistics over this wave's rows: channel 2j in .x, 2j+1 in .y of word j
    uint32_t st[NW];
    if constexpr (FMT == FMT_INT4) {
        short2_t mn[4], mx[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            mn[j] = keys2(v[0][j]);
            mx[j] = mn[j];
        }
#pragma unroll
        for (int i = 1; i < RPW; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const short2_t k = keys2(v[i][j]);
                mn[j] = min2(mn[j], k);
                mx[j] = max2(mx[j], k);
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
        for (int j = 0; j < 4; ++j) am[j] = mag2(v[0][j]);
#pragma unroll
        for (int i = 1; i < RPW; ++i) {
#pragma unroll
            for (int j = 0; j < 4; ++j) am[j] = umax2(am[j], mag2(v[i][j]));
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) st[j] = us2_as_u(am[j]);
    }

    if constexpr (SPLIT) {
        // The group's waves share the constants' work: wave wsub reduces channels wsub,
        // wsub + WPG, ... of every lane over the group's waves, computes their constants and
        // leaves them in LDS (the slow flag as a negative reciprocal, which only the fast path
        // reads); after a second barrier every wave reads all 8.
#pragma unroll
        for (int k = 0; k < NW; ++k) lds[(wave * NW + k) * 64 + lane] = st[k];
        __syncthreads();
        const int base = (wave / WPG) * WPG;
        const int il = wave / WPG;
        for (int c = wsub; c < 8; c += WPG) {  // wave-uniform
            const int j = c >> 1;
            uint32_t m = lds[(base * NW + j) * 64 + lane], x = lds[(base * NW + 4 + j) * 64 + lane];
#pragma unroll
            for (int o = 1; o < WPG; ++o) {
                m = s2_as_u(min2(as_s2(m), as_s2(lds[((base + o) * NW + j) * 64 + lane])));
                x = s2_as_u(max2(as_s2(x), as_s2(lds[((base + o) * NW + 4 + j) * 64 + lane])));
            }
            const short2_t ms = as_s2(m), xs = as_s2(x);
            const Int4Group gc = int4_group(key_to_f32((c & 1) ? ms.y : ms.x), key_to_f32((c & 1) ? xs.y : xs.x));
            cst[(il * 8 + c) * 64 + lane] = (f4_t){gc.mn, gc.scale, gc.slow ? -1.0f : gc.y, 0.0f};
        }
        __syncthreads();
    } else if constexpr (WPG > 1) {
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
    if constexpr (SPLIT) {
        // Codes channel pair by channel pair: only two channels' constants are held at a time
        // (instead of all eight), and each row's even and odd channels' codes gather in the bytes
        // of two words, interleaved into nibbles at the end.
        const int il = wave / WPG;
        uint32_t ev[RPW], od[RPW];
#pragma unroll
        for (int i = 0; i < RPW; ++i) ev[i] = od[i] = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f4_t t0 = cst[(il * 8 + 2 * j) * 64 + lane], t1 = cst[(il * 8 + 2 * j + 1) * 64 + lane];
            Int4Group g0, g1;
            g0.mn = t0[0]; g0.scale = t0[1]; g0.y = t0[2]; g0.slow = t0[2] < 0.0f;
            g1.mn = t1[0]; g1.scale = t1[1]; g1.y = t1[2]; g1.slow = t1[2] < 0.0f;
            if (__builtin_expect(g0.slow || g1.slow, 0)) {
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    const float d0 = __fsub_rn(bf16lo(v[i][j]), g0.mn), d1 = __fsub_rn(bf16hi(v[i][j]), g1.mn);
                    ev[i] = __builtin_amdgcn_cvt_pk_u8_f32(g0.slow ? d0 / g0.scale : int4_quot_raw(d0, g0), j, ev[i]);
                    od[i] = __builtin_amdgcn_cvt_pk_u8_f32(g1.slow ? d1 / g1.scale : int4_quot_raw(d1, g1), j, od[i]);
                }
            } else {
#pragma unroll
                for (int i = 0; i < RPW; ++i) {
                    const float d0 = __fsub_rn(bf16lo(v[i][j]), g0.mn), d1 = __fsub_rn(bf16hi(v[i][j]), g1.mn);
                    ev[i] = __builtin_amdgcn_cvt_pk_u8_f32(int4_quot_raw(d0, g0), j, ev[i]);
                    od[i] = __builtin_amdgcn_cvt_pk_u8_f32(int4_quot_raw(d1, g1), j, od[i]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const uint32_t word = ev[i] | (od[i] << 4);
            if (i < nr && valid) {
                if constexpr (LG)
                    st_code<!DIFF>(reinterpret_cast<uint32_t*>(a.codes) + (size_t)(r0 + i) * (uint32_t)a.C8 + c8, word);
                else
                    st_code_at<!DIFF>(wave_base_w(a.codes, (r0 + i) * (int64_t)a.C8 * 4), c8 * 4u, word);
            }
        }
        if (wsub == 0 && valid) {
            u32x4 mins, scales;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f4_t t0 = cst[(il * 8 + 2 * j) * 64 + lane], t1 = cst[(il * 8 + 2 * j + 1) * 64 + lane];
                mins[j] = f32_to_f16(t0[0]) | (f32_to_f16(t1[0]) << 16);
                scales[j] = f32_to_f16(t0[1]) | (f32_to_f16(t1[1]) << 16);
            }
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.meta0) + mbase) = mins;
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.meta1) + mbase) = scales;
        }
    } else if constexpr (FMT == FMT_INT4) {  // a group held by one wave
        Int4Group gp[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const short2_t mn = as_s2(st[j]), mx = as_s2(st[4 + j]);
            gp[2 * j] = int4_group(key_to_f32(mn.x), key_to_f32(mx.x));
            gp[2 * j + 1] = int4_group(key_to_f32(mn.y), key_to_f32(mx.y));
        }
        bool slow = false;
#pragma unroll
        for (int k = 0; k < 8; ++k) slow |= gp[k].slow;
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const uint32_t word = int4_word(v[i], gp, 1, slow);
            if (i < nr && valid) {
                if constexpr (LG)
                    st_code<!DIFF>(reinterpret_cast<uint32_t*>(a.codes) + (size_t)(r0 + i) * (uint32_t)a.C8 + c8, word);
                else
                    st_code_at<!DIFF>(wave_base_w(a.codes, (r0 + i) * (int64_t)a.C8 * 4), c8 * 4u, word);
            }
        }
        if (wsub == 0 && valid) {
            u32x4 mins, scales;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                mins[j] = f32_to_f16(gp[2 * j].mn) | (f32_to_f16(gp[2 * j + 1].mn) << 16);
                scales[j] = f32_to_f16(gp[2 * j].scale) | (f32_to_f16(gp[2 * j + 1].scale) << 16);
            }
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.meta0) + mbase) = mins;
            *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.meta1) + mbase) = scales;
        }
    } else {
        Fp4Block fb[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const ushort2_t am = as_us2(st[j]);
            fb[2 * j] = fp4_block(am.x, g, tab);
            fb[2 * j + 1] = fp4_block(am.y, g, tab);
        }
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
            const uint32_t word = fp4_word(v[i], fb, 1);
            if (i < nr && valid) {
                if constexpr (LG)
                    st_code<!DIFF>(reinterpret_cast<uint32_t*>(a.codes) + (size_t)(r0 + i) * (uint32_t)a.C8 + c8, word);
                else
                    st_code_at<!DIFF>(wave_base_w(a.codes, (r0 + i) * (int64_t)a.C8 * 4), c8 * 4u, word);
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
        if (c8raw == 0)  // one lane per token group (per lane group with LG)
            for (int i = 0; i < nr; ++i) a.pos_out[r0 + i] = a.pos[r0 + i];
    }
}

// INT4 G64 KEY pack or dense residual encode over half slabs (an unpaged view whose rows hold a
// multiple of 32 chunks): an item is one 64-token group of 32 chunks (256 channels), its 8 waves
// take 8 rows each, and a lane loads 4 of them: lanes 0-31 the first and lanes 32-63 the second
// row of each of the wave's 4 row pairs. A wave then holds 4 KB of each input in flight, and the
// grid has twice the blocks of the full-slab kernel with 8 rows per wave. Lanes l and l + 32 hold
// the same channels and first merge their statistics (lane swap across the halves); the rest is
// the full-slab kernel's: the LDS exchange over the group's waves, wave w working out every
// lane's channel w constants, and the codes channel pair by channel pair. Same codes and
// metadata, bit for bit. With DIFF the lane loads the same rows of `prev` and codes
// bf16(cur - prev); with WIN, blocks from win_block0 on copy a BF16 window's protected rows.
template <bool DIFF, bool WIN>
__global__ __launch_bounds__(512) void k_encode_k_half(EncArgs a) {
    constexpr int G = 64, WPG = 8, RL = 4;  // RL: rows per lane
    if (WIN && blockIdx.x >= a.win_block0) {
        window_copy_wave(a.win, __builtin_amdgcn_readfirstlane((blockIdx.x - a.win_block0) * 8u + (threadIdx.x >> 6)),
                         threadIdx.x & 63);
        return;
    }
    __shared__ uint32_t lds[WPG * 8 * 64];
    __shared__ f4_t cst[8 * 64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t nhs = (uint32_t)a.C8 >> 5;  // half slabs per row
    const uint32_t b = __builtin_amdgcn_readfirstlane(blockIdx.x / nhs);
    const uint32_t hs = blockIdx.x - b * nhs;
    const uint32_t sub = (uint32_t)lane >> 5;
    const uint32_t c8 = hs * 32u + ((uint32_t)lane & 31u);
    const uint32_t h = fdiv(c8, a.div_D8);
    const uint32_t d = (c8 - h * (uint32_t)a.D8) * 8u;
    const int64_t rw = (int64_t)b * G + (int64_t)wave * (2 * RL);  // the wave's first row
    const bool full = (int64_t)(b + 1) * G <= a.rows;               // wave-uniform

    u32x4 v[RL], p[DIFF ? RL : 1];
    if (full) {  // a row pair's second row lies one token pitch after the first
        const uint32_t off = (uint32_t)(((int64_t)h * a.csh + d) * 2 + (int64_t)sub * a.cst * 2);
#pragma unroll
        for (int i = 0; i < RL; ++i) v[i] = ld_stream_at(wave_base(a.cur, (rw + 2 * i) * a.cst * 2), off);
        if constexpr (DIFF) {
            const uint32_t poff = (uint32_t)(((int64_t)h * a.psh + d) * 2 + (int64_t)sub * a.pst * 2);
#pragma unroll
            for (int i = 0; i < RL; ++i) p[i] = ld_stream_at(wave_base(a.prev, (rw + 2 * i) * a.pst * 2), poff);
        }
    } else {  // the last, partial group: rows past the end read the last row, which lies in it
#pragma unroll
        for (int i = 0; i < RL; ++i) {
            const int64_t r = min<int64_t>(rw + 2 * i + sub, a.rows - 1);
            v[i] = ld_stream(a.cur + r * a.cst + (int64_t)h * a.csh + d);
            if constexpr (DIFF) p[i] = ld_stream(a.prev + r * a.pst + (int64_t)h * a.psh + d);
        }
    }
    if constexpr (DIFF) {  // the residual bf16(cur - prev)
#pragma unroll
        for (int i = 0; i < RL; ++i) {
            v[i].x = sub_bf16x2(v[i].x, p[i].x);
            v[i].y = sub_bf16x2(v[i].y, p[i].y);
            v[i].z = sub_bf16x2(v[i].z, p[i].z);
            v[i].w = sub_bf16x2(v[i].w, p[i].w);
        }
    }

    // per-channel statistics over the lane's rows, then over both halves
    short2_t mn[4], mx[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        mn[j] = keys2(v[0][j]);
        mx[j] = mn[j];
    }
#pragma unroll
    for (int i = 1; i < RL; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const short2_t k = keys2(v[i][j]);
            mn[j] = min2(mn[j], k);
            mx[j] = max2(mx[j], k);
        }
    }
    uint32_t st[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const auto pn = __builtin_amdgcn_permlane32_swap(s2_as_u(mn[j]), s2_as_u(mn[j]), false, false);
        const auto px = __builtin_amdgcn_permlane32_swap(s2_as_u(mx[j]), s2_as_u(mx[j]), false, false);
        st[j] = s2_as_u(min2(as_s2(pn[0]), as_s2(pn[1])));
        st[4 + j] = s2_as_u(max2(as_s2(px[0]), as_s2(px[1])));
    }

    // wave w reduces channel w of every lane over the group's waves and leaves its constants in
    // LDS (the slow flag as a negative reciprocal); after a second barrier every wave reads all 8
#pragma unroll
    for (int k = 0; k < 8; ++k) lds[(wave * 8 + k) * 64 + lane] = st[k];
    __syncthreads();
    {
        const int c = wave, j = c >> 1;
        uint32_t m = lds[j * 64 + lane], x = lds[(4 + j) * 64 + lane];
#pragma unroll
        for (int o = 1; o < WPG; ++o) {
            m = s2_as_u(min2(as_s2(m), as_s2(lds[(o * 8 + j) * 64 + lane])));
            x = s2_as_u(max2(as_s2(x), as_s2(lds[(o * 8 + 4 + j) * 64 + lane])));
        }
        const short2_t ms = as_s2(m), xs = as_s2(x);
        const Int4Group gc = int4_group(key_to_f32((c & 1) ? ms.y : ms.x), key_to_f32((c & 1) ? xs.y : xs.x));
        cst[c * 64 + lane] = (f4_t){gc.mn, gc.scale, gc.slow ? -1.0f : gc.y, 0.0f};
    }
    __syncthreads();

    uint32_t ev[RL], od[RL];
#pragma unroll
    for (int i = 0; i < RL; ++i) ev[i] = od[i] = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f4_t t0 = cst[(2 * j) * 64 + lane], t1 = cst[(2 * j + 1) * 64 + lane];
        Int4Group g0, g1;
        g0.mn = t0[0]; g0.scale = t0[1]; g0.y = t0[2]; g0.slow = t0[2] < 0.0f;
        g1.mn = t1[0]; g1.scale = t1[1]; g1.y = t1[2]; g1.slow = t1[2] < 0.0f;
        if (__builtin_expect(g0.slow || g1.slow, 0)) {
#pragma unroll
            for (int i = 0; i < RL; ++i) {
                const float d0 = __fsub_rn(bf16lo(v[i][j]), g0.mn), d1 = __fsub_rn(bf16hi(v[i][j]), g1.mn);
                ev[i] = __builtin_amdgcn_cvt_pk_u8_f32(g0.slow ? d0 / g0.scale : int4_quot_raw(d0, g0), j, ev[i]);
                od[i] = __builtin_amdgcn_cvt_pk_u8_f32(g1.slow ? d1 / g1.scale : int4_quot_raw(d1, g1), j, od[i]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < RL; ++i) {
                const float d0 = __fsub_rn(bf16lo(v[i][j]), g0.mn), d1 = __fsub_rn(bf16hi(v[i][j]), g1.mn);
                ev[i] = __builtin_amdgcn_cvt_pk_u8_f32(int4_quot_raw(d0, g0), j, ev[i]);
                od[i] = __builtin_amdgcn_cvt_pk_u8_f32(int4_quot_raw(d1, g1), j, od[i]);
            }
        }
    }
    const uint32_t coff = (sub * (uint32_t)a.C8 + c8) * 4u;
#pragma unroll
    for (int i = 0; i < RL; ++i) {
        const uint32_t word = ev[i] | (od[i] << 4);
        if (full || rw + 2 * i + sub < a.rows)
            st_code_at<!DIFF>(wave_base_w(a.codes, (rw + 2 * i) * (int64_t)a.C8 * 4), coff, word);
    }
    if (wave == 0 && sub == 0) {
        const size_t mbase = ((size_t)b * (uint32_t)a.C8 + c8) * 8u;
        u32x4 mins, scales;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f4_t t0 = cst[(2 * j) * 64 + lane], t1 = cst[(2 * j + 1) * 64 + lane];
            mins[j] = f32_to_f16(t0[0]) | (f32_to_f16(t1[0]) << 16);
            scales[j] = f32_to_f16(t0[1]) | (f32_to_f16(t1[1]) << 16);
        }
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.meta0) + mbase) = mins;
        *reinterpret_cast<u32x4*>(reinterpret_cast<uint16_t*>(a.meta1) + mbase) = scales;
    }
}

// ---- generic paths -----------------------------------------------------------------------------

// VALUE: one thread per (row, head), groups walked along the row.
template <int FMT, bool DIFF, bool GATHER>
__global__ __launch_bounds__(kThreads) void k_encode_v_gen(EncArgs a) {
    __shared__ std::conditional_t<FMT == FMT_NVFP4, Fp4Table, char> tab;
    float g = 0.0f;
    if constexpr (FMT == FMT_NVFP4) {
        g = *a.gscale;
        fp4_table_fill(tab, g);
    }
    const int64_t idx = (int64_t)(a.gen_base + (uint64_t)blockIdx.x * kThreads + threadIdx.x);
    if (idx >= a.rows * a.H) return;
    const int64_t r = idx / a.H;
    const int64_t h = idx - r * a.H;
    const int64_t t = GATHER ? (int64_t)a.pos[r] : r;
    const int64_t wr = a.dst ? (int64_t)a.dst[r] : r;  // packed row written
    const int D = a.D, G = a.G;
    const int ngr = (D + G - 1) / G;
    const int Dp = (D + 1) / 2;
    uint8_t* crow = a.codes + (size_t)(wr * a.H + h) * Dp;
    uint32_t pending = 0;
    for (int c = 0; c < ngr; ++c) {
        const int d0 = c * G, d1 = min(D, d0 + G);
        const size_t midx = (size_t)(wr * a.H + h) * ngr + c;
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
            const Fp4Block fb = fp4_block(bam, g, tab);
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
    __shared__ std::conditional_t<FMT == FMT_NVFP4, Fp4Table, char> tab;
    float g = 0.0f;
    if constexpr (FMT == FMT_NVFP4) {
        g = *a.gscale;
        fp4_table_fill(tab, g);
    }
    const int D = a.D, G = a.G;
    const int Dp = (D + 1) / 2;
    const int64_t nb = (a.rows + G - 1) / G;
    const int64_t idx = (int64_t)(a.gen_base + (uint64_t)blockIdx.x * kThreads + threadIdx.x);
    if (idx >= nb * a.H * Dp) return;
    const int64_t b = idx / ((int64_t)a.H * Dp);
    const int64_t rem = idx - b * a.H * Dp;
    const int64_t h = rem / Dp;
    const int j = (int)(rem - h * Dp);
    const int nch = (2 * j + 1 < D) ? 2 : 1;
    const int64_t r_begin = b * G, r_end = min<int64_t>(a.rows, r_begin + G);

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
            fb[k] = fp4_block(bam, g, tab);
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

// max |x| (bf16 magnitude bits) over every encoded element, in two launches without atomics:
// each block of the amax kernel writes its partial maximum to ws[blockIdx.x]; a one-block
// finalize kernel folds the partials into the tensor amax and stores the global multiplier.
// Vector path: a wave task is RW rows of one 64-chunk slab (all loads issued at once); waves
// stride over tasks.
__device__ __forceinline__ uint32_t block_max(uint32_t m) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    __shared__ uint32_t sm[kThreads / 64];
    if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
    __syncthreads();
    return max(max(sm[0], sm[1]), max(sm[2], sm[3]));
}

template <bool DIFF, bool GATHER, bool LG>
__global__ __launch_bounds__(kThreads) void k_amax_vec(EncArgs a) {
    constexpr int RW = DIFF ? 4 : 8;
    const int lane = threadIdx.x & 63;
    uint32_t m = 0;
    const uint32_t nwaves = gridDim.x * 4u;
    for (uint32_t task = __builtin_amdgcn_readfirstlane(blockIdx.x * 4u + (threadIdx.x >> 6)); task < a.n_tasks;
         task += nwaves) {
        uint32_t rtile, c8raw;  // with LG a lane group past the last row tile re-reads the last row
        task_lane<LG>(a, task, lane, rtile, c8raw);
        const uint32_t c8 = (c8raw < (uint32_t)a.C8) ? c8raw : (uint32_t)a.C8 - 1u;
        const uint32_t h = fdiv(c8, a.div_D8);
        const uint32_t d = (c8 - h * (uint32_t)a.D8) * 8u;
        u32x4 v[RW];
        load_rows8<RW, DIFF, GATHER, !LG>(a, (int64_t)rtile * RW, h, d, v);
        ushort2_t mm = (ushort2_t){0, 0};
#pragma unroll
        for (int i = 0; i < RW; ++i)
            mm = umax2(mm, umax2(umax2(mag2(v[i].x), mag2(v[i].y)), umax2(mag2(v[i].z), mag2(v[i].w))));
        m = max(m, max((uint32_t)mm.x, (uint32_t)mm.y));
    }
    m = block_max(m);
    if (threadIdx.x == 0) a.ws[blockIdx.x] = m;
}

// Generic path: grid-stride over elements.
template <bool DIFF, bool GATHER>
__global__ __launch_bounds__(kThreads) void k_amax_gen(EncArgs a, uint64_t total) {
    uint32_t m = 0;
    const uint64_t stride = (uint64_t)gridDim.x * kThreads;
    const int64_t HD = (int64_t)a.H * a.D;
    for (uint64_t u = (uint64_t)blockIdx.x * kThreads + threadIdx.x; u < total; u += stride) {
        const int64_t r = (int64_t)(u / (uint64_t)HD);
        const int64_t rem = (int64_t)u - r * HD;
        const int64_t h = rem / a.D;
        const int64_t d = rem - h * a.D;
        const int64_t t = GATHER ? (int64_t)a.pos[r] : r;
        m = max(m, load_one<DIFF>(a, t, h, d) & 0x7FFFu);
    }
    m = block_max(m);
    if (threadIdx.x == 0) a.ws[blockIdx.x] = m;
}

// One block of 1024 threads folds up to kAmaxMaxBlocks partials (four independent loads per
// thread) and stores the global multiplier.
__global__ __launch_bounds__(1024) void k_amax_finalize(const uint32_t* parts, uint32_t nparts, float* gscale) {
    uint32_t v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t i = threadIdx.x + 1024u * k;
        v[k] = (i < nparts) ? parts[i] : 0u;
    }
    uint32_t m = max(max(v[0], v[1]), max(v[2], v[3]));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
    __shared__ uint32_t sm[16];
    if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t t = 0;
        for (int w = 0; w < 16; ++w) t = max(t, sm[w]);
        *gscale = fp4_global(t);
    }
}

static_assert(KVQ_AMAX_MAX_BLOCKS <= 4096u, "finalize folds at most 4 partials per thread");

__global__ void k_set_global(float* gscale, uint32_t bits) { *gscale = __uint_as_float(bits); }

inline uint32_t ceil_div_u(uint64_t a, uint64_t b) { return (uint32_t)((a + b - 1) / b); }

// One block per WPB / WPG token-group items (and the blocks of a carried row copy).
template <int FMT, int G, bool DIFF, bool GATHER, bool WIN>
void launch_key_vec_w(const EncArgs& a, hipStream_t s) {
    constexpr uint32_t wpb = (uint32_t)key_waves_per_block(G, DIFF, FMT == FMT_INT4);
    constexpr uint32_t ipb = wpb / (uint32_t)key_waves_per_group(G, DIFF, FMT == FMT_INT4);
    EncArgs b = a;
    const dim3 grid = grid_with_copy(b, ceil_div_u(a.n_tasks, ipb), wpb);
    if (a.ri_shift > 0)
        hipLaunchKernelGGL((k_encode_k_vec<FMT, G, DIFF, GATHER, true, WIN>), grid, dim3(64 * wpb), 0, s, b);
    else
        hipLaunchKernelGGL((k_encode_k_vec<FMT, G, DIFF, GATHER, false, WIN>), grid, dim3(64 * wpb), 0, s, b);
}

// A row copy rides only on dense launches (a window never gathers).
template <int FMT, int G, bool DIFF, bool GATHER>
void launch_key_vec(const EncArgs& a, hipStream_t s) {
    if constexpr (FMT == FMT_INT4 && G == 64 && !GATHER) {
        // the half-slab kernel (bulk shape: pack 61.5 -> 59.4 us; dense residual encode 105.5 ->
        // 100.5 us on a clean cache, the same in step): full-width rows, unpaged, token pitches
        // whose odd rows stay within the 32-bit lane offsets
        const bool pitches = a.cst >= 0 && a.cst < ((int64_t)1 << 29) &&
                             (!DIFF || (a.pst >= 0 && a.pst < ((int64_t)1 << 29)));
        if (a.ri_shift == 0 && a.C8 % 32 == 0 && a.cpshift == kNoPaging && pitches) {
            EncArgs b = a;
            const uint32_t items = (uint32_t)((a.rows + G - 1) / G) * (uint32_t)(a.C8 / 32);
            if (a.win_tasks) {
                const dim3 grid = grid_with_copy(b, items, 8u);  // sets b.win_block0 before the launch copies b
                hipLaunchKernelGGL((k_encode_k_half<DIFF, true>), grid, dim3(512), 0, s, b);
            } else {
                hipLaunchKernelGGL((k_encode_k_half<DIFF, false>), dim3(items), dim3(512), 0, s, b);
            }
            return;
        }
    }
    if constexpr (!GATHER) {
        if (a.win_tasks) return launch_key_vec_w<FMT, G, DIFF, GATHER, true>(a, s);
    }
    launch_key_vec_w<FMT, G, DIFF, GATHER, false>(a, s);
}

template <int FMT, bool DIFF, bool GATHER>
hipError_t encode_dispatch(int kind, const EncArgs& a, bool vec, hipStream_t s) {
    if (vec) {
        if (kind == KIND_VALUE) {
            EncArgs b = a;
            const dim3 grid = grid_with_copy(b, ceil_div_u(a.n_tasks, 4), 4u);
            const bool win = !GATHER && a.win_tasks;
            if (a.ri_shift > 0) {
                if (win) hipLaunchKernelGGL((k_encode_v_vec<FMT, DIFF, false, true, true>), grid, dim3(kThreads), 0, s, b);
                else hipLaunchKernelGGL((k_encode_v_vec<FMT, DIFF, GATHER, true, false>), grid, dim3(kThreads), 0, s, b);
            } else {
                if (win) hipLaunchKernelGGL((k_encode_v_vec<FMT, DIFF, false, false, true>), grid, dim3(kThreads), 0, s, b);
                else hipLaunchKernelGGL((k_encode_v_vec<FMT, DIFF, GATHER, false, false>), grid, dim3(kThreads), 0, s, b);
            }
        } else {
            switch (a.G) {
                case 16:
                    launch_key_vec<FMT, 16, DIFF, GATHER>(a, s);
                    break;
                case 32:
                    if constexpr (FMT == FMT_INT4) launch_key_vec<FMT, 32, DIFF, GATHER>(a, s);
                    break;
                case 64:
                    if constexpr (FMT == FMT_INT4) launch_key_vec<FMT, 64, DIFF, GATHER>(a, s);
                    break;
                case 128:
                    if constexpr (FMT == FMT_INT4) launch_key_vec<FMT, 128, DIFF, GATHER>(a, s);
                    break;
                default:
                    return hipErrorInvalidValue;
            }
        }
    } else {
        if (kind == KIND_VALUE) {
            const uint64_t n = (uint64_t)a.rows * a.H;
            launch_in_chunks(a, n, kThreads, [&](const EncArgs& b, dim3 grid) {
                hipLaunchKernelGGL((k_encode_v_gen<FMT, DIFF, GATHER>), grid, dim3(kThreads), 0, s, b);
            });
        } else {
            const uint64_t nb = (uint64_t)(a.rows + a.G - 1) / a.G;
            const uint64_t n = nb * a.H * ((a.D + 1) / 2);
            launch_in_chunks(a, n, kThreads, [&](const EncArgs& b, dim3 grid) {
                hipLaunchKernelGGL((k_encode_k_gen<FMT, DIFF, GATHER>), grid, dim3(kThreads), 0, s, b);
            });
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
    uint32_t blocks;
    if (vec) {
        // amax tiles: 8 rows per wave task (4 for a residual, which loads two tensors)
        const uint32_t rw = DIFF ? 4u : 8u;
        EncArgs b = a;
        const uint64_t tiles = (uint64_t)((a.rows + rw - 1) / rw);
        b.n_tasks = a.ri_shift > 0 ? (uint32_t)((tiles + (1u << a.ri_shift) - 1) >> a.ri_shift)
                                   : (uint32_t)tiles * (uint32_t)a.n_slabs;
        blocks = ceil_div_u(b.n_tasks, 4);
        if (blocks > kAmaxMaxBlocks) blocks = kAmaxMaxBlocks;
        if (a.ri_shift > 0)
            hipLaunchKernelGGL((k_amax_vec<DIFF, GATHER, true>), dim3(blocks), dim3(kThreads), 0, s, b);
        else
            hipLaunchKernelGGL((k_amax_vec<DIFF, GATHER, false>), dim3(blocks), dim3(kThreads), 0, s, b);
    } else {
        const uint64_t total = (uint64_t)a.rows * a.H * a.D;
        const uint64_t want = (total + kThreads * 4 - 1) / (kThreads * 4);
        blocks = (uint32_t)(want > 1024 ? 1024 : (want < 1 ? 1 : want));
        hipLaunchKernelGGL((k_amax_gen<DIFF, GATHER>), dim3(blocks), dim3(kThreads), 0, s, a, total);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_amax_finalize, dim3(1), dim3(1024), 0, s, a.ws, blocks, a.gscale);
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
