// kvq_attn.hip -- decode attention that reads the packed KV cache directly: the codec's
// dequantization (and optionally one residual's reconstruction) happens in registers and the
// products run on bf16 MFMA (vllm-rlt PR #166, the reviews' hot-path discussion: dequantize to
// BF16 in registers and keep the BF16 matrix multiply; compare formats after fusing
// dequantization and residual reconstruction into attention).
//
// One query token per query head attends over all T cached tokens; query head hq reads KV head
// hq / rep. The cached K and V are exactly what kvq_unpack (or kvq_decode_residual on top of it)
// would produce, bf16 value for bf16 value; scores and the softmax run in FP32, P is rounded to
// bf16 for the PV product, accumulation is FP32. Head dimension D is 64, 128 or 256.
//
// Work split (flash decoding): a block owns one KV head, a range of tokens and a tile of up to 16
// of the head's query rows (grid z; more than 16 query heads per KV head take several tiles,
// each reading the same K/V); each of its 4 waves walks 16-token sub-tiles with its own online
// softmax; the waves meet in LDS, the block writes one partial (max, sum, unnormalized output) per
// query row, and a second kernel folds the partials of all blocks.
//
// MFMA (lane l, q = l / 16): v_mfma_f32_16x16x16_bf16 takes A[l % 16][4q + j], B[4q + j][l % 16]
// for j = 0..3 and v_mfma_f32_16x16x32_bf16 A[l % 16][8q + j], B[8q + j][l % 16] for j = 0..7;
// both leave D[4q + j][l % 16], j = 0..3 (checked on the device). Scores are computed transposed,
// S^T = K Q^T, with the 16x16x32 form: A = K (lane: token l % 16; the reduction axis is permuted so
// that lane group q covers channels (D/4) q .. (D/4) q + D/4 - 1, one contiguous load of codes),
// B = Q^T, D/32 steps. The accumulator then holds S[row l % 16][token 4q + j], which is exactly
// the B operand P^T of O^T = V^T P^T in the 16x16x16 form (16 tokens per sub-tile); there
// A = V^T with D/16 output tiles N (lane: channels (D/16)(l % 16) + N of tokens 4q + j, one
// contiguous load per token), and the accumulator of tile N holds
// O[row l % 16][channel (D/16)(4q + j) + N].
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "kvq_launch.hpp"

namespace kvq {

namespace {

constexpr int kWaves = 4;  // waves per block
constexpr int kSub = 16;   // tokens per sub-tile (one MFMA tile)
constexpr int kNone = KVQ_ATTN_NO_RESIDUAL;

typedef short s4_t __attribute__((ext_vector_type(4)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u2_t __attribute__((ext_vector_type(2)));

// max over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four lane groups of one query row), with the
// gfx950 lane-swap moves (VALU) instead of two LDS-routed shuffles: swapping a register with
// itself across halves (rows) leaves each lane's partner value in one of the two results.
__device__ __forceinline__ float lane_max(float v) {
    const auto h = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __builtin_fmaxf(__uint_as_float(h[0]), __uint_as_float(h[1]));
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <bool ON>
using TableT = std::conditional_t<ON, Fp4Table, char>;

// Formats whose K metadata belongs to a group of tokens (it goes through the LDS slots); the
// row formats carry their metadata per (token, KV head) row and load it with the codes.
template <int FMT>
constexpr bool kGroupMeta = FMT == FMT_INT4 || FMT == FMT_NVFP4;

// Per-lane geometry of head dimension D and format FMT.
template <int D, int FMT>
struct Geo {
    static constexpr int QC = D / 4;                             // K channels per lane group
    static constexpr int VC = D / 16;                            // V channels per lane (= output tiles)
    static constexpr int RB = FMT == FMT_FP8_ROW ? D : D / 2;    // code bytes per (token, head) row
    static constexpr int KB = FMT == FMT_FP8_ROW ? QC : QC / 2;  // K code bytes per lane
    static constexpr int VB = FMT == FMT_FP8_ROW ? VC : VC / 2;  // V code bytes per lane and token
    static constexpr int KW = KB / 4;                            // K code words per lane
    static constexpr int VW = VB >= 4 ? VB / 4 : 1;              // V code words per lane and token
    static constexpr int KBLK = QC / 16;                         // NVFP4-row K blocks per lane
};

// A value the optimizer must treat as unknown: it keeps nibble masks from merging into the byte
// extraction (so the four bytes convert with v_cvt_f32_ubyte0..3) and offsets from being widened
// outside a loop.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
    asm("" : "+v"(v));
    return v;
}

// A wave-uniform global address kept in SGPRs and opaque to the optimizer, so that a lane's
// 32-bit byte offset is added by the load itself (the scalar-base form of global loads).
typedef const __attribute__((address_space(1))) uint8_t* gptr;

__device__ __forceinline__ gptr sbase(const void* p, size_t off) {
    const uint64_t v = reinterpret_cast<uint64_t>(static_cast<const uint8_t*>(p) + off);
    // readfirstlane returns a signed int: widen through uint32_t, never by sign extension
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint64_t u = ((uint64_t)hi << 32) | (uint64_t)lo;
    gptr b = (gptr)u;
    asm("" : "+s"(b));
    return b;
}

// (The offset passes through opaque() at the load so that its widening is not hoisted out of
// the loop as a 64-bit register pair, which would cost the scalar-base form.)
template <class T>
__device__ __forceinline__ T ld_at(gptr base, uint32_t off) {
    return *reinterpret_cast<const __attribute__((address_space(1))) T*>(base + opaque(off));
}

template <class T>
__device__ __forceinline__ T ld_nt_at(gptr base, uint32_t off) {
    return __builtin_nontemporal_load(
        reinterpret_cast<const __attribute__((address_space(1))) T*>(base + opaque(off)));
}

// BYTES contiguous code bytes (2 to 64, aligned to their size up to 16) into words, low first.
template <int BYTES, int N>
__device__ __forceinline__ void ld_codes(gptr base, uint32_t off, uint32_t (&w)[N]) {
    if constexpr (BYTES == 2) {
        w[0] = __builtin_nontemporal_load(
            reinterpret_cast<const __attribute__((address_space(1))) uint16_t*>(base + opaque(off)));
    } else if constexpr (BYTES == 4) {
        w[0] = ld_nt_at<uint32_t>(base, off);
    } else if constexpr (BYTES == 8) {
        const u2_t v = ld_nt_at<u2_t>(base, off);
        w[0] = v.x;
        w[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < BYTES / 16; ++i) {
            const u32x4 v = ld_nt_at<u32x4>(base, off + 16 * i);
            w[4 * i] = v.x; w[4 * i + 1] = v.y; w[4 * i + 2] = v.z; w[4 * i + 3] = v.w;
        }
    }
}

// --- K metadata in LDS ---------------------------------------------------------------------
//
// A K group's metadata is shared by all its tokens: each wave keeps the current group's (and,
// loaded one sub-tile ahead, the next group's) metadata of its KV head in two LDS slots of D
// words. INT4: D f16 minimums, then D f16 scales; NVFP4: the D decoded f32 block scales
// e4m3(s) / g of one 16-token block. Lane group q reads its D/4 channels with broadcast reads.

// The lane's share of one group's metadata on its way to LDS.
struct MetaStage {
    uint32_t w[4];
};

template <int D, int FMT>
__device__ __forceinline__ void meta_fetch(const AttnPlanes& p, int64_t t0, int H, int h, int lane, MetaStage& m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) m.w[i] = 0u;
    if constexpr (FMT == FMT_INT4) {
        // lanes 0..31 the minimums, 32..63 the scales: D/64 words (2 D/64 f16) each
        constexpr int NW = D / 64;
        const size_t row = ((size_t)(t0 >> p.gshift) * H + h) * D;  // f16 elements
        const uint16_t* src = reinterpret_cast<const uint16_t*>(lane < 32 ? p.meta0 : p.meta1) + row +
                              2 * NW * (lane & 31);
        if constexpr (NW == 1) {
            m.w[0] = *reinterpret_cast<const uint32_t*>(src);
        } else if constexpr (NW == 2) {
            const u2_t v = *reinterpret_cast<const u2_t*>(src);
            m.w[0] = v.x;
            m.w[1] = v.y;
        } else {
            const u32x4 v = *reinterpret_cast<const u32x4*>(src);
            m.w[0] = v.x; m.w[1] = v.y; m.w[2] = v.z; m.w[3] = v.w;
        }
    } else {
        // the D scale bytes, 4 per lane on lanes 0 .. D/4 - 1
        if (lane < D / 4)
            m.w[0] = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(p.meta0) +
                                                       ((size_t)(t0 >> 4) * H + h) * D)[lane];
    }
}

template <int D, int FMT>
__device__ __forceinline__ void meta_store(uint32_t* slot, const MetaStage& m, int lane, const Fp4Table* tab) {
    if constexpr (FMT == FMT_INT4) {
        constexpr int NW = D / 64;  // lane l: words NW l .. NW l + NW - 1 (minimums, then scales)
#pragma unroll
        for (int i = 0; i < NW; ++i) slot[NW * lane + i] = m.w[i];
    } else if (lane < D / 4) {
        const uint32_t b = m.w[0];  // scale bytes of channels 4 lane .. 4 lane + 3
        const u32x4 f = {__float_as_uint(tab->e[b & 0x7Fu][0]), __float_as_uint(tab->e[(b >> 8) & 0x7Fu][0]),
                         __float_as_uint(tab->e[(b >> 16) & 0x7Fu][0]), __float_as_uint(tab->e[(b >> 24) & 0x7Fu][0])};
        reinterpret_cast<u32x4*>(slot)[lane] = f;
    }
}

// --- raw loads and in-register decoding ---

// Raw data of one sub-tile for this lane.
//   K of token l % 16, channels (D/4) q .. : codes, and for the row formats that row's metadata:
//   NVFP4-row the E4M3 block-scale bytes of these channels and the FP32 row multiplier g,
//   FP8-row the FP32 row scale.
//   V of tokens 4q + j, channels (D/16) r .. : codes and metadata (INT4: f16 scale << 16 | f16
//   minimum; NVFP4, NVFP4-row: the block-scale byte; FP8-row: the row scale's bits), and for
//   NVFP4-row the row multiplier.
template <int D, int FMT>
struct TileRaw {
    uint32_t kc[Geo<D, FMT>::KW];
    uint32_t km;
    float kg;
    uint32_t vc[4][Geo<D, FMT>::VW];
    uint32_t vm[4];
    float vg[4];
};

// Loop-invariant lane byte offsets of one packed tensor, relative to the sub-tile's first row,
// whose addresses are wave-uniform: K codes, K row metadata (block bytes, row FP32), V codes, V
// metadata, V row FP32.
struct LaneOffsets {
    uint32_t kc, km, kg;
    uint32_t vc[4], vm[4], vg[4];
};

template <int D>
constexpr int kLogD = D == 64 ? 6 : D == 128 ? 7 : 8;

template <int D, int FMT>
__device__ __forceinline__ void lane_offsets(const AttnPlanes& pk, const AttnPlanes& pv, int H, int h, int r, int q,
                                             int64_t dt_k, const int64_t (&dt_v)[4], LaneOffsets& o) {
    using G = Geo<D, FMT>;
    const uint64_t krow = (uint64_t)dt_k * H + h;
    o.kc = (uint32_t)(krow * G::RB + G::KB * q);
    o.km = (uint32_t)(krow * (D / 16) + G::KBLK * q);  // NVFP4-row: the lane group's blocks
    o.kg = (uint32_t)(krow * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint64_t row = (uint64_t)dt_v[j] * H + h;
        o.vc[j] = (uint32_t)(row * G::RB + G::VB * r);
        if constexpr (FMT == FMT_INT4)  // f16 entries [row][channel group]
            o.vm[j] = (uint32_t)(2 * ((row << (kLogD<D> - pv.gshift)) + (((uint32_t)G::VC * r) >> pv.gshift)));
        else if constexpr (FMT == FMT_FP8_ROW)  // FP32 [row]
            o.vm[j] = (uint32_t)(row * 4);
        else  // E4M3 bytes [row][16-channel block]
            o.vm[j] = (uint32_t)(row * (D / 16) + ((G::VC * r) >> 4));
        o.vg[j] = (uint32_t)(row * 4);
    }
}

// The sub-tile's K part (codes and row metadata of the lane's token) and V part (codes and
// metadata of its four tokens) load separately, so that each can be issued as soon as the
// previous sub-tile has finished with the registers it fills.
template <int D, int FMT>
__device__ __forceinline__ void tile_load_k(const AttnPlanes& pk, int64_t t0, int H, const LaneOffsets& o,
                                            TileRaw<D, FMT>& x) {
    using G = Geo<D, FMT>;
    const size_t rows = (size_t)t0 * H;  // (token, head) rows before the sub-tile
    ld_codes<G::KB>(sbase(pk.codes, rows * G::RB), o.kc, x.kc);
    if constexpr (FMT == FMT_FP8_ROW) {
        x.kg = __uint_as_float(ld_at<uint32_t>(sbase(pk.meta0, rows * 4), o.kg));
    } else if constexpr (FMT == FMT_NVFP4_ROW) {
        gptr kmb = sbase(pk.meta0, rows * (D / 16));
        if constexpr (G::KBLK == 1) x.km = ld_at<uint8_t>(kmb, o.km);
        else if constexpr (G::KBLK == 2) x.km = ld_at<uint16_t>(kmb, o.km);
        else x.km = ld_at<uint32_t>(kmb, o.km);
        x.kg = __uint_as_float(ld_at<uint32_t>(sbase(pk.meta1, rows * 4), o.kg));
    }
}

template <int D, int FMT>
__device__ __forceinline__ void tile_load_v(const AttnPlanes& pv, int64_t t0, int H, const LaneOffsets& o,
                                            TileRaw<D, FMT>& x) {
    using G = Geo<D, FMT>;
    const size_t rows = (size_t)t0 * H;
    gptr vcb = sbase(pv.codes, rows * G::RB);
#pragma unroll
    for (int j = 0; j < 4; ++j) ld_codes<G::VB>(vcb, o.vc[j], x.vc[j]);
    if constexpr (FMT == FMT_FP8_ROW) {
        gptr vsb = sbase(pv.meta0, rows * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) x.vm[j] = ld_at<uint32_t>(vsb, o.vm[j]);
    } else if constexpr (FMT == FMT_INT4) {
        const size_t g = 2 * (rows << (kLogD<D> - pv.gshift));
        gptr mb = sbase(pv.meta0, g);
        gptr sb = sbase(pv.meta1, g);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            x.vm[j] = (uint32_t)ld_at<uint16_t>(mb, o.vm[j]) | ((uint32_t)ld_at<uint16_t>(sb, o.vm[j]) << 16);
    } else {
        if constexpr (FMT == FMT_NVFP4_ROW) {
            gptr gb = sbase(pv.meta1, rows * 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) x.vg[j] = __uint_as_float(ld_at<uint32_t>(gb, o.vg[j]));
        }
        gptr mb = sbase(pv.meta0, rows * (D / 16));
#pragma unroll
        for (int j = 0; j < 4; ++j) x.vm[j] = ld_at<uint8_t>(mb, o.vm[j]);
    }
}

// NVFP4-row decode scale of one block: fl(e4m3(code) / g), by the Markstein quotient that the
// device probe shows equal to the IEEE division for every g in [2^-100, 2^100] and every code
// (others divide); gp = rcp_pair(g).
__device__ __forceinline__ float nvfp4_row_sdec(uint32_t code, const RcpPair& gp) {
    return quot_rn(e4m3_decode(code & 0x7Fu), gp);
}

// Per-sub-tile K constants of a row format: NVFP4-row the block decode scales of the lane's
// channels, FP8-row the row scale.
template <int D>
struct KPrep {
    float s[D / 64];
};

template <int D, int FMT>
__device__ __forceinline__ void k_prep(const TileRaw<D, FMT>& x, KPrep<D>& k) {
    RcpPair gp;
    if constexpr (FMT == FMT_NVFP4_ROW) gp = rcp_pair(x.kg);  // the lane's token row
#pragma unroll
    for (int b = 0; b < D / 64; ++b) {
        if constexpr (FMT == FMT_NVFP4_ROW)
            k.s[b] = nvfp4_row_sdec((x.km >> (8 * b)) & 0xFFu, gp);
        else if constexpr (FMT == FMT_FP8_ROW)
            k.s[b] = x.kg;
        else
            k.s[b] = 0.0f;
    }
}

// The lane's 8 decoded K values of chunk i (channels (D/4) q + 8i .. + 7): group formats read
// their metadata from the LDS slot, row formats from the sub-tile's own row metadata.
template <int D, int FMT>
__device__ __forceinline__ void k_decode8(const TileRaw<D, FMT>& x, const KPrep<D>& kp, const uint32_t* slot, int q,
                                          int i, float (&y)[8]) {
    constexpr int QC = D / 4;
    if constexpr (FMT == FMT_INT4) {
        const uint32_t w = x.kc[i];
        const u32x4 m4 = reinterpret_cast<const u32x4*>(slot)[(QC / 8) * q + i];
        const u32x4 s4 = reinterpret_cast<const u32x4*>(slot + D / 2)[(QC / 8) * q + i];
        const uint32_t mm[4] = {m4.x, m4.y, m4.z, m4.w}, ss[4] = {s4.x, s4.y, s4.z, s4.w};
        const uint32_t lo = opaque(w & 0x0F0F0F0Fu), hi = opaque((w >> 4) & 0x0F0F0F0Fu);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const float c0 = (float)((lo >> (8 * b)) & 0xFFu), c1 = (float)((hi >> (8 * b)) & 0xFFu);
            y[2 * b] = int4_value_f(c0, f16_to_f32(ss[b] & 0xFFFFu), f16_to_f32(mm[b] & 0xFFFFu));
            y[2 * b + 1] = int4_value_f(c1, f16_to_f32(ss[b] >> 16), f16_to_f32(mm[b] >> 16));
        }
    } else if constexpr (FMT == FMT_FP8_ROW) {
        const uint32_t w0 = x.kc[2 * i], w1 = x.kc[2 * i + 1];
        const f32x2 e0 = fp8_values<false>(w0), e1 = fp8_values<true>(w0);
        const f32x2 e2 = fp8_values<false>(w1), e3 = fp8_values<true>(w1);
        const float e[8] = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
#pragma unroll
        for (int n = 0; n < 8; ++n) y[n] = __fmul_rn(e[n], kp.s[0]);
    } else {
        const uint32_t w = x.kc[i];
        float sd[8];
        if constexpr (FMT == FMT_NVFP4) {
            const u32x4 f0 = reinterpret_cast<const u32x4*>(slot)[(QC / 4) * q + 2 * i];
            const u32x4 f1 = reinterpret_cast<const u32x4*>(slot)[(QC / 4) * q + 2 * i + 1];
            sd[0] = __uint_as_float(f0.x); sd[1] = __uint_as_float(f0.y);
            sd[2] = __uint_as_float(f0.z); sd[3] = __uint_as_float(f0.w);
            sd[4] = __uint_as_float(f1.x); sd[5] = __uint_as_float(f1.y);
            sd[6] = __uint_as_float(f1.z); sd[7] = __uint_as_float(f1.w);
        } else {  // NVFP4-row: chunk i lies in the lane group's block i / 2
#pragma unroll
            for (int n = 0; n < 8; ++n) sd[n] = kp.s[i >> 1];
        }
        const f32x2 e0 = e2m1_values<0>(w), e1 = e2m1_values<1>(w), e2 = e2m1_values<2>(w), e3 = e2m1_values<3>(w);
        const float e[8] = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
#pragma unroll
        for (int n = 0; n < 8; ++n) y[n] = __fmul_rn(e[n], sd[n]);
    }
}

// V of one sub-tile prepared for decoding: the masked nibble words (INT4: low nibbles of each
// token's words, then high), the raw words (NVFP4, NVFP4-row, FP8-row), with each token's scale
// (and INT4 minimum).
template <int D, int FMT>
struct VPrep {
    uint32_t lo[4][Geo<D, FMT>::VW], hi[4][Geo<D, FMT>::VW];
    float s[4], m[4];
};

template <int D, int FMT>
__device__ __forceinline__ void v_prep(const TileRaw<D, FMT>& x, const Fp4Table* tab, VPrep<D, FMT>& v) {
    constexpr int VW = Geo<D, FMT>::VW;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
        for (int w = 0; w < VW; ++w) {
            if constexpr (FMT == FMT_INT4) {
                v.lo[j][w] = opaque(x.vc[j][w] & 0x0F0F0F0Fu);
                v.hi[j][w] = opaque((x.vc[j][w] >> 4) & 0x0F0F0F0Fu);
            } else {
                v.lo[j][w] = x.vc[j][w];
                v.hi[j][w] = 0u;
            }
        }
        if constexpr (FMT == FMT_INT4) {
            v.m[j] = f16_to_f32(x.vm[j] & 0xFFFFu);
            v.s[j] = f16_to_f32(x.vm[j] >> 16);
        } else if constexpr (FMT == FMT_FP8_ROW) {
            v.s[j] = __uint_as_float(x.vm[j]);
            v.m[j] = 0.0f;
        } else if constexpr (FMT == FMT_NVFP4) {
            v.s[j] = tab->e[x.vm[j] & 0x7Fu][0];
            v.m[j] = 0.0f;
        } else {
            v.m[j] = 0.0f;
            if constexpr (D >= 256) v.s[j] = nvfp4_row_sdec(x.vm[j], rcp_pair(x.vg[j]));
        }
    }
    if constexpr (FMT == FMT_NVFP4_ROW && D < 256) {
        // a 16-channel block spans the lane pair (l, l ^ 1), which holds the same tokens: the even
        // lane works out tokens 0 and 2, the odd lane 1 and 3, and the two swap the quotients
        const bool odd = (__lane_id() & 1) != 0;
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const float mine = nvfp4_row_sdec(odd ? x.vm[2 * jj + 1] : x.vm[2 * jj],
                                              rcp_pair(odd ? x.vg[2 * jj + 1] : x.vg[2 * jj]));
            const float other = __uint_as_float(dpp<0xB1>(__float_as_uint(mine)));
            v.s[2 * jj] = odd ? other : mine;
            v.s[2 * jj + 1] = odd ? mine : other;
        }
    }
}

// The decoded V values of channel (D/16) r + n for the four tokens.
template <int D, int FMT>
__device__ __forceinline__ void v_decode_n(const VPrep<D, FMT>& v, int n, float (&y)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if constexpr (FMT == FMT_INT4) {
            // nibble n: word n / 8, byte (n % 8) / 2, low or high half
            const uint32_t w = (n & 1) ? v.hi[j][n >> 3] : v.lo[j][n >> 3];
            y[j] = int4_value_f((float)((w >> (8 * ((n & 7) >> 1))) & 0xFFu), v.s[j], v.m[j]);
        } else if constexpr (FMT == FMT_FP8_ROW) {
            const uint32_t w = v.lo[j][n >> 2];  // byte n of the token's codes
            const f32x2 e = (n & 2) ? fp8_values<true>(w) : fp8_values<false>(w);
            y[j] = __fmul_rn(e[n & 1], v.s[j]);
        } else {
            const uint32_t w = v.lo[j][n >> 3];
            const int sel = (n & 7) >> 1;
            const f32x2 e = sel == 0   ? e2m1_values<0>(w)
                            : sel == 1 ? e2m1_values<1>(w)
                            : sel == 2 ? e2m1_values<2>(w)
                                       : e2m1_values<3>(w);
            y[j] = __fmul_rn(e[n & 1], v.s[j]);
        }
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

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ bf16x8_t as_bf8(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
    const u32x4 v = {w0, w1, w2, w3};
    return __builtin_bit_cast(bf16x8_t, v);
}

template <int RFMT>
constexpr int kResFmt = RFMT == kNone ? FMT_INT4 : RFMT;  // a placeholder type when unused

// Raw data of one 16-token sub-tile (base and, for a residual, the residual planes).
template <int D, int FMT, int RFMT>
struct SubRaw {
    TileRaw<D, FMT> b;
    std::conditional_t<RFMT != kNone, TileRaw<D, kResFmt<RFMT>>, char> r;
};

// Per-wave running state of the online softmax. m is the offset subtracted from the scores
// (log2 units) before exp2; it is raised only when a score passes it by more than kLazy, so
// that the accumulators are rarely rescaled and every p stays below 2^kLazy.
constexpr float kLazy = 8.0f;
template <int D>
struct WaveState {
    float m, l;
    f4_t o[D / 16];
};

// Offsets of every tensor of a call for one sub-tile: `full` sub-tiles use the precomputed
// lane offsets; the last, partial one clamps its tokens to the final row first.
struct CallOffsets {
    LaneOffsets b, r;
};

template <int D, int FMT, int RFMT>
__device__ __forceinline__ void call_offsets(const AttnArgs& a, int h, int r, int q, int64_t t0, int64_t t_end,
                                             CallOffsets& o) {
    const int64_t last = t_end - 1 - t0;  // offset of the final row from t0
    const int64_t dk = min<int64_t>(r, last);
    int64_t dv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) dv[j] = min<int64_t>(4 * q + j, last);
    lane_offsets<D, FMT>(a.k, a.v, a.H, h, r, q, dk, dv, o.b);
    if constexpr (RFMT != kNone) lane_offsets<D, RFMT>(a.rk, a.rv, a.H, h, r, q, dk, dv, o.r);
}

template <int D, int FMT, int RFMT>
__device__ __forceinline__ void sub_load_k(const AttnArgs& a, int64_t t0, const CallOffsets& o,
                                           SubRaw<D, FMT, RFMT>& s) {
    tile_load_k<D, FMT>(a.k, t0, a.H, o.b, s.b);
    if constexpr (RFMT != kNone) tile_load_k<D, RFMT>(a.rk, t0, a.H, o.r, s.r);
}

template <int D, int FMT, int RFMT>
__device__ __forceinline__ void sub_load_v(const AttnArgs& a, int64_t t0, const CallOffsets& o,
                                           SubRaw<D, FMT, RFMT>& s) {
    tile_load_v<D, FMT>(a.v, t0, a.H, o.b, s.b);
    if constexpr (RFMT != kNone) tile_load_v<D, RFMT>(a.rv, t0, a.H, o.r, s.r);
}

// One sub-tile's scores, online softmax and PV product; `after_k` runs once the K codes have
// been consumed (the caller issues the next sub-tile's K loads there).
template <int D, int FMT, int RFMT, bool TAIL, class AfterK>
__device__ __forceinline__ void sub_compute(const AttnArgs& a, int n_valid, int q, const uint32_t (&qw)[D / 8],
                                            const SubRaw<D, FMT, RFMT>& s, const uint32_t* kslot,
                                            const uint32_t* rkslot, const Fp4Table* ptv, const Fp4Table* ptrv,
                                            WaveState<D>& st, AfterK&& after_k) {
    constexpr bool RES = RFMT != kNone;
    constexpr int RF = kResFmt<RFMT>;
    constexpr int NT = D / 16;  // output tiles
    // ---- scores S^T = K Q^T, 8 channels (one 16x16x32 bf16 MFMA step) at a time, in two
    // accumulators so that consecutive products do not wait for each other ----
    f4_t sacc = (f4_t){0.0f, 0.0f, 0.0f, 0.0f}, sacc2 = sacc;
    KPrep<D> kpb, kpr;
    k_prep<D, FMT>(s.b, kpb);
    if constexpr (RES) k_prep<D, RF>(s.r, kpr);
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
        float kv[8], kr[8];
        k_decode8<D, FMT>(s.b, kpb, kslot, q, i, kv);
        if constexpr (RES) k_decode8<D, RF>(s.r, kpr, rkslot, q, i, kr);
        uint32_t kw[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            kw[c] = rebuild2(kv[2 * c], kv[2 * c + 1], RES ? kr[2 * c] : 0.0f, RES ? kr[2 * c + 1] : 0.0f, RES);
        const bf16x8_t ka = as_bf8(kw[0], kw[1], kw[2], kw[3]);
        const bf16x8_t qb = as_bf8(qw[4 * i], qw[4 * i + 1], qw[4 * i + 2], qw[4 * i + 3]);
        if (i & 1)
            sacc2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb, sacc2, 0, 0, 0);
        else
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb, sacc, 0, 0, 0);
    }
    after_k();
    sacc += sacc2;
    // ---- online softmax: lane holds S[row r][token t0 + 4q + j] ----
    float sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sc[j] = (!TAIL || 4 * q + j < n_valid) ? sacc[j] * a.qscale : -__builtin_inff();
    const float m_tile = lane_max(__builtin_fmaxf(__builtin_fmaxf(sc[0], sc[1]), __builtin_fmaxf(sc[2], sc[3])));
    const bool up = m_tile > st.m + kLazy;  // always for the first sub-tile (m = -inf; token 0 is valid)
    if (__any(up)) {
        const float m_new = up ? m_tile : st.m;
        const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);  // 0 from m = -inf
        st.l *= alpha;
#pragma unroll
        for (int n = 0; n < NT; ++n) st.o[n] *= alpha;
        st.m = m_new;
    }
    float p[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(sc[j] - st.m);
    st.l += (p[0] + p[1]) + (p[2] + p[3]);
    const s4_t pb = as_s4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
    // ---- O^T += V^T P^T, one 16-channel output tile (channel (D/16) r + n of each lane) at a time ----
    VPrep<D, FMT> vb;
    VPrep<D, RF> vr;
    v_prep<D, FMT>(s.b, ptv, vb);
    if constexpr (RES) v_prep<D, RF>(s.r, ptrv, vr);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
        float yb[4], yr[4];
        v_decode_n<D, FMT>(vb, n, yb);
        if constexpr (RES) v_decode_n<D, RF>(vr, n, yr);
        const uint32_t v01 = rebuild2(yb[0], yb[1], RES ? yr[0] : 0.0f, RES ? yr[1] : 0.0f, RES);
        const uint32_t v23 = rebuild2(yb[2], yb[3], RES ? yr[2] : 0.0f, RES ? yr[3] : 0.0f, RES);
        st.o[n] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(as_s4(v01, v23), pb, st.o[n], 0, 0, 0);
    }
}

// log2 of the tokens per K metadata group (NVFP4 K blocks are 16 tokens; row formats have no
// K groups)
template <int FMT>
__device__ __forceinline__ int kgroup_shift(const AttnPlanes& p) {
    return FMT == FMT_INT4 ? p.gshift : 4;
}

// LDS metadata slots per wave: two for a group-format base, two more for a group-format residual.
template <int FMT, int RFMT>
constexpr int kSlots = (kGroupMeta<FMT> ? 2 : 0) + (RFMT != kNone && kGroupMeta<kResFmt<RFMT>> ? 2 : 0);

// Waves per SIMD to ask the register allocator for (128 VGPRs for four).
template <int D, int RFMT>
constexpr int kMinWaves = D == 256 ? 2 : (RFMT == kNone ? 4 : 3);

template <int D, int FMT, int RFMT>
__global__ __launch_bounds__(64 * kWaves, (kMinWaves<D, RFMT>)) void k_attn_split(AttnArgs a) {
    constexpr bool RES = RFMT != kNone;
    constexpr int RF = kResFmt<RFMT>;
    constexpr int NT = D / 16;
    __shared__ TableT<FMT == FMT_NVFP4> tk, tv;
    __shared__ TableT<RFMT == FMT_NVFP4> trk, trv;
    // Each wave's region holds its K metadata slots during the token loop and its unnormalized
    // output rows (16 x D floats) afterwards; only that wave touches it until the barrier.
    static_assert(kSlots<FMT, RFMT> <= 16, "metadata slots fit in the output rows");
    __shared__ uint32_t s_wave[kWaves][16 * D];
    __shared__ float s_m[kWaves][16], s_l[kWaves][16];
    constexpr bool SKEW = !RES && FMT == FMT_FP8_ROW;  // next sub-tile's loads during this one
    constexpr bool GK = kGroupMeta<FMT>;        // base K metadata via LDS
    constexpr bool GR = RES && kGroupMeta<RF>;  // residual K metadata via LDS
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
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15;  // query row of the tile (and the K token / V channel-group index)
    const int q = lane >> 4;
    const int h = blockIdx.y;
    const int64_t t_begin = (int64_t)blockIdx.x * a.tc;
    const int64_t t_end = min<int64_t>(a.T, t_begin + a.tc);
    // each wave walks its own contiguous quarter of the block's tokens (a multiple of 16)
    const int64_t w_len = a.tc / kWaves;
    const int64_t w_begin = t_begin + (int64_t)wave * w_len;
    const int64_t w_end = min<int64_t>(t_end, w_begin + w_len);

    // Q^T operand: row r of this block's query tile (query head h * rep + row0 + r), channels
    // (D/4) q + 4s + j for step s; rows past the tile are zero
    const int row0 = 16 * (int)blockIdx.z;
    const int nrows = min(16, a.rep - row0);
    uint32_t qw[D / 8];
    if (r < nrows) {
        const u32x4* qp = reinterpret_cast<const u32x4*>(a.q + ((size_t)h * a.rep + row0 + r) * D + (D / 4) * q);
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
            const u32x4 v = qp[i];
            qw[4 * i] = v.x; qw[4 * i + 1] = v.y; qw[4 * i + 2] = v.z; qw[4 * i + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < D / 8; ++i) qw[i] = 0u;
    }

    WaveState<D> st;
    st.m = -__builtin_inff();
    st.l = 0.0f;
#pragma unroll
    for (int n = 0; n < NT; ++n) st.o[n] = (f4_t){0.0f, 0.0f, 0.0f, 0.0f};

    int ks = 0, rks = 0;
    if constexpr (GK) ks = kgroup_shift<FMT>(a.k);
    if constexpr (GR) rks = kgroup_shift<RF>(a.rk);
    uint32_t* slots = &s_wave[wave][0];
    auto kslot = [&](int64_t t) { return GK ? slots + ((t >> ks) & 1) * D : nullptr; };
    auto rkslot = [&](int64_t t) { return GR ? slots + ((GK ? 2 : 0) + ((t >> rks) & 1)) * D : nullptr; };

    // Full sub-tiles (all 16 tokens in range) run in the main loop with loop-invariant offsets;
    // the block's last sub-tile may be partial and runs after it, its rows clamped to the last.
    CallOffsets full;
    call_offsets<D, FMT, RFMT>(a, h, r, q, 0, kSub, full);
    const int64_t w_full = w_begin + ((w_end - w_begin) & ~(int64_t)(kSub - 1));

    // One full sub-tile at t from `cur`. With SKEW (FP8-row without a residual, the format that
    // moves the most bytes per value decoded) its K and V loads went out during the sub-tile
    // before it: the next full sub-tile's K loads (into `nxt`) are issued as soon as this one's K
    // codes are consumed and its V loads after this one's PV product, so each is in flight over
    // most of a sub-tile while one copy of each part is live. Otherwise the sub-tile loads its
    // own data first, both tensors' K parts before their V parts. Where the next sub-tile opens a
    // new K group, that group's metadata is fetched first and goes to its LDS slot (the one the
    // current group does not use) afterwards.
    auto step = [&](int64_t t, SubRaw<D, FMT, RFMT>& cur, SubRaw<D, FMT, RFMT>& nxt) {
        const int64_t tn = t + kSub;
        const bool more = tn < w_end;
        const bool pf = SKEW && tn < w_full;
        if constexpr (!SKEW) {
            sub_load_k<D, FMT, RFMT>(a, t, full, cur);
            sub_load_v<D, FMT, RFMT>(a, t, full, cur);
        }
        const bool nk = GK && more && (tn >> ks) != (t >> ks);
        const bool nr = GR && more && (tn >> rks) != (t >> rks);
        MetaStage mk, mr;
        if constexpr (GK) {
            if (nk) meta_fetch<D, FMT>(a.k, tn, a.H, h, lane, mk);
        }
        if constexpr (GR) {
            if (nr) meta_fetch<D, RF>(a.rk, tn, a.H, h, lane, mr);
        }
        __builtin_amdgcn_wave_barrier();
        sub_compute<D, FMT, RFMT, false>(a, kSub, q, qw, cur, kslot(t), rkslot(t), ptv, ptrv, st, [&] {
            if (pf) sub_load_k<D, FMT, RFMT>(a, tn, full, nxt);
        });
        if (pf) sub_load_v<D, FMT, RFMT>(a, tn, full, nxt);
        if constexpr (GK) {
            if (nk) meta_store<D, FMT>(kslot(tn), mk, lane, ptk);
        }
        if constexpr (GR) {
            if (nr) meta_store<D, RF>(rkslot(tn), mr, lane, ptrk);
        }
        __builtin_amdgcn_wave_barrier();
    };

    int64_t t0 = w_begin;
    SubRaw<D, FMT, RFMT> A, B;
    if (t0 < w_end) {
        MetaStage m;
        if constexpr (GK) {
            meta_fetch<D, FMT>(a.k, t0, a.H, h, lane, m);
            meta_store<D, FMT>(kslot(t0), m, lane, ptk);
        }
        if constexpr (GR) {
            meta_fetch<D, RF>(a.rk, t0, a.H, h, lane, m);
            meta_store<D, RF>(rkslot(t0), m, lane, ptrk);
        }
    }
    if (SKEW && t0 < w_full) {
        sub_load_k<D, FMT, RFMT>(a, t0, full, A);
        sub_load_v<D, FMT, RFMT>(a, t0, full, A);
    }
    while (t0 < w_full) {  // unrolled twice so that the two raw buffers swap roles for free
        step(t0, A, B);
        t0 += kSub;
        if (t0 >= w_full) break;
        step(t0, B, A);
        t0 += kSub;
    }
    if (t0 < w_end) {  // the partial sub-tile (its group's metadata is already in place)
        CallOffsets tail;
        call_offsets<D, FMT, RFMT>(a, h, r, q, t0, w_end, tail);
        sub_load_k<D, FMT, RFMT>(a, t0, tail, A);
        sub_load_v<D, FMT, RFMT>(a, t0, tail, A);
        __builtin_amdgcn_wave_barrier();
        sub_compute<D, FMT, RFMT, true>(a, (int)(w_end - t0), q, qw, A, kslot(t0), rkslot(t0), ptv, ptrv, st,
                                        [] {});
    }

    // ---- fold the block's 4 waves: lane holds O[row r][channel (D/16)(4q + j) + n] ----
    float l_row = st.l + __shfl_xor(st.l, 16);  // the row's 4 lanes share m
    l_row += __shfl_xor(l_row, 32);
    __builtin_amdgcn_wave_barrier();  // the wave's metadata reads are done: its region holds rows now
    float* s_o = reinterpret_cast<float*>(&s_wave[wave][0]);  // [16][D]
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int j = 0; j < 4; ++j) s_o[r * D + NT * (4 * q + j) + n] = st.o[n][j];
    if (q == 0) {
        s_m[wave][r] = st.m;  // -inf for a wave without tokens (then l = 0 and O = 0)
        s_l[wave][r] = l_row;
    }
    __syncthreads();
    const size_t pbase = ((size_t)h * a.n_split + blockIdx.x) * a.rep + row0;
    for (int idx = threadIdx.x; idx < nrows * D; idx += 64 * kWaves) {
        const int row = idx / D, c = idx - row * D;
        float M = s_m[0][row];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = __builtin_fmaxf(M, s_m[w][row]);
        float L = 0.0f, O = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = (s_m[w][row] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(s_m[w][row] - M);
            L += s_l[w][row] * f;
            O += reinterpret_cast<const float*>(&s_wave[w][0])[row * D + c] * f;
        }
        a.part_o[(pbase + row) * D + c] = O;
        if (c == 0) {
            a.part_ml[(pbase + row) * 2] = M;
            a.part_ml[(pbase + row) * 2 + 1] = L;
        }
    }
}

// out[hq][c] = sum_s O_s 2^(m_s - M) / sum_s l_s 2^(m_s - M) over the blocks' partials (M the
// largest m_s). One wave per (query head, 32 channels): lane 8 g + c holds channels 4 c .. 4 c + 3
// of the chunk and takes splits g, g + 8, g + 16, ... in batches of kBatch, all of a batch's loads
// issued before any arithmetic; three butterfly steps then merge the eight split groups.
typedef float f4v __attribute__((ext_vector_type(4)));

constexpr int kBatch = 16;

struct Fold {
    float m, l;
    f4v o;
};

// (m, l, o) of two disjoint sets of splits -> that of their union (a side with m = -inf is empty)
__device__ __forceinline__ Fold fold_merge(const Fold& x, const Fold& y) {
    const float m = __builtin_fmaxf(x.m, y.m);
    const float fa = (x.m == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(x.m - m);
    const float fb = (y.m == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(y.m - m);
    return {m, x.l * fa + y.l * fb, x.o * fa + y.o * fb};
}

template <int D>
__global__ __launch_bounds__(64) void k_attn_combine(AttnArgs a) {
    constexpr int CH = D / 32;  // 32-channel chunks per output row
    const int hq = blockIdx.x / CH, ch = blockIdx.x - hq * CH;
    const int h = hq / a.rep, row = hq - h * a.rep;
    const int lane = threadIdx.x;
    const int c4 = lane & 7, g = lane >> 3;
    const size_t base = (size_t)h * a.n_split * a.rep + row;  // partial index of split 0
    const size_t step = (size_t)a.rep;                       // partial index step per split
    const float* ml = a.part_ml + base * 2;
    const f4v* po = reinterpret_cast<const f4v*>(a.part_o + base * D + 32 * ch) + c4;
    Fold f = {-__builtin_inff(), 0.0f, {0.0f, 0.0f, 0.0f, 0.0f}};
    for (int s0 = g; s0 < a.n_split; s0 += 8 * kBatch) {
        float mb[kBatch], lb[kBatch];
        f4v ob[kBatch];
        // every load is issued (splits past the end re-read the last one, then count as empty), so
        // that no branch separates them
#pragma unroll
        for (int i = 0; i < kBatch; ++i) {
            const int s = min(s0 + 8 * i, a.n_split - 1);
            mb[i] = ml[(size_t)s * step * 2];
            lb[i] = ml[(size_t)s * step * 2 + 1];
            ob[i] = po[(size_t)s * step * (D / 4)];
        }
#pragma unroll
        for (int i = 0; i < kBatch; ++i)
            if (s0 + 8 * i >= a.n_split) mb[i] = -__builtin_inff();
        Fold b = {mb[0], 0.0f, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
        for (int i = 1; i < kBatch; ++i) b.m = __builtin_fmaxf(b.m, mb[i]);
        if (b.m != -__builtin_inff()) {
#pragma unroll
            for (int i = 0; i < kBatch; ++i) {
                const float w = (mb[i] == -__builtin_inff()) ? 0.0f : __builtin_amdgcn_exp2f(mb[i] - b.m);
                b.l += lb[i] * w;
                b.o += ob[i] * w;
            }
        }
        f = fold_merge(f, b);
    }
#pragma unroll
    for (int x = 8; x < 64; x <<= 1) {
        Fold y;
        y.m = __shfl_xor(f.m, x);
        y.l = __shfl_xor(f.l, x);
        y.o = (f4v){__shfl_xor(f.o.x, x), __shfl_xor(f.o.y, x), __shfl_xor(f.o.z, x), __shfl_xor(f.o.w, x)};
        f = fold_merge(f, y);
    }
    if (g == 0) reinterpret_cast<f4v*>(a.out + (size_t)hq * D + 32 * ch)[c4] = f.o / f.l;
}

// Resident blocks of a kernel on the current device (compute units x blocks per unit), cached
// per device for each kernel.
template <int D, int FMT, int RFMT>
int resident_blocks() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, k_attn_split<D, FMT, RFMT>, 64 * kWaves, 0) != hipSuccess)
        return 0;
    // residual kernels at head dim 64 or 128 (three resident per unit by registers) split as if
    // four were: measured faster with the extra splits (T = 131072, INT4 pair: 125-135 -> 114 us)
    if (RFMT != kNone && D <= 128 && per < 4) per = 4;
    n = cus * per;
    if (n > 0) cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// The split of one call: as many blocks per KV head and query tile as fill the device once
// (within the bound the workspace was sized for), each a multiple of 64 tokens.
template <int D, int FMT, int RFMT>
hipError_t attn_launch(AttnArgs a, hipStream_t s) {
    const int32_t bound = a.n_split;
    if (bound < 1 || bound > KVQ_ATTN_MAX_SPLIT) return hipErrorInvalidValue;  // the bound the workspace was sized for
    const int n_qt = (a.rep + 15) / 16;  // 16-row query tiles per KV head (grid z)
    const int resident = resident_blocks<D, FMT, RFMT>();
    const int64_t want = resident > 0 ? std::max<int64_t>(1, resident / ((int64_t)a.H * n_qt)) : bound;
    const int64_t splits = std::min<int64_t>(want, bound);
    const int64_t per = (a.T + 64 * splits - 1) / (64 * splits);
    a.tc = 64 * per;
    a.n_split = (int32_t)((a.T + a.tc - 1) / a.tc);  // <= splits
    a.part_ml = a.part_o + (size_t)a.H * a.n_split * a.rep * D;
    hipLaunchKernelGGL((k_attn_split<D, FMT, RFMT>), dim3(a.n_split, a.H, n_qt), dim3(64 * kWaves), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_attn_combine<D>, dim3((unsigned)(a.H * a.rep * (D / 32))), dim3(64), 0, s, a);
    return hipGetLastError();
}

template <int D, int FMT>
hipError_t attn_fmt(int rfmt, const AttnArgs& a, hipStream_t s) {
    if (rfmt == kNone) return attn_launch<D, FMT, kNone>(a, s);
    if (rfmt == FMT_INT4) return attn_launch<D, FMT, FMT_INT4>(a, s);
    if (rfmt == FMT_NVFP4) return attn_launch<D, FMT, FMT_NVFP4>(a, s);
    if (rfmt == FMT_NVFP4_ROW) return attn_launch<D, FMT, FMT_NVFP4_ROW>(a, s);
    if (rfmt == FMT_FP8_ROW) return attn_launch<D, FMT, FMT_FP8_ROW>(a, s);
    return hipErrorInvalidValue;
}

template <int D>
hipError_t attn_dim(int fmt, int rfmt, const AttnArgs& a, hipStream_t s) {
    if (fmt == FMT_INT4) return attn_fmt<D, FMT_INT4>(rfmt, a, s);
    if (fmt == FMT_NVFP4) return attn_fmt<D, FMT_NVFP4>(rfmt, a, s);
    if (fmt == FMT_NVFP4_ROW) return attn_fmt<D, FMT_NVFP4_ROW>(rfmt, a, s);
    if (fmt == FMT_FP8_ROW) return attn_fmt<D, FMT_FP8_ROW>(rfmt, a, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attention(int fmt, int rfmt, const AttnArgs& a, hipStream_t s) {
    if (a.D == 64) return attn_dim<64>(fmt, rfmt, a, s);
    if (a.D == 128) return attn_dim<128>(fmt, rfmt, a, s);
    if (a.D == 256) return attn_dim<256>(fmt, rfmt, a, s);
    return hipErrorInvalidValue;
}

}  // namespace kvq
