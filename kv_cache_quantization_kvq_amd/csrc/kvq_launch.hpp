// kvq_launch.hpp -- argument blocks and launchers shared by the C ABI and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_device.hpp"

namespace kvq {

enum : int { FMT_INT4 = 0, FMT_NVFP4 = 1, FMT_NVFP4_ROW = 2, FMT_FP8_ROW = 3 };

// Row offset of row t in a (possibly paged) view: rows come in pages of 2^pshift rows,
// consecutive rows of a page `st` apart and pages `pst` apart. An unpaged view uses pshift 62
// (every row in page 0), so the offset is t * st.
__host__ __device__ __forceinline__ int64_t row_offset(int64_t t, int32_t pshift, int64_t pst, int64_t st) {
    return (t >> pshift) * pst + (t & (((int64_t)1 << pshift) - 1)) * st;
}
constexpr int32_t kNoPaging = 62;

// The NVFP4 amax pass writes one partial maximum per block into the workspace.
#define KVQ_AMAX_MAX_BLOCKS 4096u

// Rows per wave task of the vector encoders and decoder, shared by the host code that sizes the
// grids and the kernels. All measured on the bulk shape ([131072, 8, 128]) against eight rows:
//  * decoder: four rows (a KEY decode needs G % KVQ_DECODE_ROWS == 0 so that a task's rows share
//    one token group), 6-7% faster on residual decodes and plain unpacks; two rows were slower.
//  * VALUE encoder: four rows for a residual encode, eight for a plain NVFP4 pack (four were
//    2 us slower there) and two for the other plain packs. Residual encodes gained most: INT4
//    98.5 -> 96 us and NVFP4 198 -> 192 us in step, 3-4 us on a clean cache. The INT4 G64 pack
//    went 62 -> 61 us at four rows and to 59 us at two (60.5 -> 59.5 us on a clean cache).
//  * row-format encoders (NVFP4-row, FP8-row; an even count for NVFP4-row's lane pairs): four,
//    packs 2-4 us and residual encodes 4-5 us faster, in step and on a clean cache; two rows
//    made the packs 1-3 us slower again.
//  * KEY encoder: min(G, 8) rows per wave for a pack, min(G, 4) for a residual encode (a power
//    of two), but at least G / 16 so that the G / rows waves sharing a token group fit one block
//    of at most 1024 threads. Four rows: INT4 G64 residual encode 100.5 -> 97.5 us and NVFP4
//    199 -> 195.5 us in step (within 1 us on a clean cache); the INT4 pack was 1 us slower.
//    The INT4 G16 pack (page-local groups of 16-token pages) takes four rows as well: 63.8 ->
//    62 us in step, 66 -> 63 us on a clean cache; the NVFP4 G16 pack keeps eight (four made
//    its head-shard pack 9% slower).
//    The INT4 G64 pack and dense residual encode of full-width unpaged rows instead run the
//    half-slab kernel (k_encode_k_half: 8 rows per wave over 256 channels, 4 per lane): pack
//    61.5 -> 59 us, residual encode 105.5 -> 100.5 us on a clean cache.
#ifndef KVQ_DECODE_ROWS
#define KVQ_DECODE_ROWS 4
#endif
#ifndef KVQ_ROW_ENCODE_ROWS
#define KVQ_ROW_ENCODE_ROWS 4
#endif
constexpr int value_encode_rows(bool nvfp4, bool residual) { return residual ? 4 : nvfp4 ? 8 : 2; }
constexpr int key_rows_per_wave(int G, bool residual, bool int4) {
    const int cap = residual || (int4 && G == 16) ? 4 : 8;
    const int r = G < cap ? G : cap;
    return r < G / 16 ? G / 16 : r;
}
constexpr int key_waves_per_group(int G, bool residual, bool int4) {
    return G / key_rows_per_wave(G, residual, int4);
}
constexpr int key_waves_per_block(int G, bool residual, bool int4) {
    return key_waves_per_group(G, residual, int4) > 4 ? key_waves_per_group(G, residual, int4) : 4;
}
enum : int { KIND_KEY = 0, KIND_VALUE = 1 };

// Row copy: row r of src to row r of dst, except that rows r >= split are read src_jump
// elements further on and written dst_jump elements further on (two row ranges in one launch;
// jumps of 0 for a plain copy).
struct CopyArgs {
    const uint16_t* src;
    int64_t sst, ssh;
    uint16_t* dst;
    int64_t dst_t, dsh;
    int64_t T;
    int64_t split, src_jump, dst_jump;
    int32_t H, D, C8;
    FastDiv div_C8, div_D8;
    uint64_t gen_base;  // first work item of this launch (launch_in_chunks)
};

// A generic kernel (one work item per thread) over n items runs as launches of at most
// kGenChunk items, each told its first item in `gen_base`, so that no dispatch reaches the
// 32-bit limit on work items (tensors of up to 2^36 elements take the generic kernels when
// their layout does not suit the vector ones).
constexpr uint64_t kGenChunk = (uint64_t)1 << 31;
template <class Args, class F>
inline void launch_in_chunks(Args a, uint64_t n, uint32_t threads, F&& launch_one) {
    for (uint64_t b0 = 0; b0 < n; b0 += kGenChunk) {
        a.gen_base = b0;
        const uint64_t m = n - b0 < kGenChunk ? n - b0 : kGenChunk;
        launch_one(a, dim3((uint32_t)((m + threads - 1) / threads)));
    }
}

// A launch of the vector encoder or decoder can carry a row copy (a BF16 window's protected
// rows): the launcher appends blocks from win_block0 on, and their waves copy kWinChunks
// 16-byte chunks each (win_tasks such waves; 0: no copy).
constexpr uint32_t kWinChunks = 256;

// Rows being encoded: row r is source row t = pos ? pos[r] : r; the element value is
// cur[t, h, d], or bf16(cur[t, h, d] - prev[t, h, d]) for a residual.
struct EncArgs {
    const uint16_t* cur;
    int64_t cst, csh;
    int32_t cpshift;       // paging of `cur` (kNoPaging when unpaged)
    int64_t cpst;
    const uint16_t* prev;  // residual only
    int64_t pst, psh;
    const int32_t* pos;    // sparse residual only
    int32_t* pos_out;      // owned copy of pos
    const int32_t* dst;    // slot writes: encoded row r lands in packed row dst[r] (NULL: row r)
    int64_t rows;
    int32_t H, D, G;
    // vector-path geometry: C8 = H*D/8 chunks of 8 channels per row; a VALUE group spans
    // lpg = G/8 = 1 << lpg_shift lanes, ngr = C8 / lpg groups per row
    int32_t C8, D8, n_slabs, lpg, lpg_shift, ngr;
    int32_t ri_shift, c8_shift;  // lane groups of short rows (see task_lane); 0 when unused
    uint32_t n_tasks;
    FastDiv div_D8, div_slabs, div_C8;
    uint8_t* codes;
    void* meta0;
    void* meta1;
    float* gscale;
    uint32_t* ws;  // NVFP4: per-block partial maxima of the amax pass
    CopyArgs win;
    uint32_t win_tasks, win_block0;
    uint64_t gen_base;  // generic kernels: first work item of this launch
};

// Rows being decoded: output row r reads packed row src ? src[r] : r and goes to output row
// t = pos ? pos[r] : r; with `prev` the output is bf16(prev[t] + bf16(decoded)).
struct DecArgs {
    const uint8_t* codes;
    const void* meta0;
    const void* meta1;
    const float* gscale;
    const int32_t* pos;
    const int32_t* src;    // slot reads (NULL: identity)
    const uint16_t* prev;
    int64_t pst, psh;
    uint16_t* out;
    int64_t ost, osh;
    int32_t opshift;       // paging of `out` (kNoPaging when unpaged)
    int64_t opst;
    int64_t rows;
    int32_t H, D, G;
    int32_t C8, D8, n_slabs, lpg, lpg_shift, ngr;
    int32_t ri_shift, c8_shift;  // lane groups of short rows (see task_lane); 0 when unused
    uint32_t n_tasks;
    FastDiv div_D8, div_slabs;
    CopyArgs win;
    uint32_t win_tasks, win_block0;
    uint64_t gen_base;  // generic kernels: first work item of this launch
};

// Lanes of a vector-path task. Rows of 64 or more 8-channel chunks (or a count that does not
// divide 64): the wave's 64 lanes take 64 consecutive chunks (a slab) of one row tile, and a
// task is (row tile, slab). Shorter rows (LG): C8 = 1 << c8_shift chunks per row, and the lanes
// form 1 << ri_shift groups of C8, group k taking row tile (task << ri_shift) + k, so every lane
// has work (a head-sharded [T, 1, 128] tensor has 16 chunks per row).
template <bool LG, class Args>
__device__ __forceinline__ void task_lane(const Args& a, uint32_t task, int lane, uint32_t& rtile, uint32_t& c8raw) {
    if constexpr (LG) {
        rtile = (task << a.ri_shift) + ((uint32_t)lane >> a.c8_shift);
        c8raw = (uint32_t)lane & ((1u << a.c8_shift) - 1u);
    } else {
        rtile = fdiv(task, a.div_slabs);
        c8raw = (task - rtile * (uint32_t)a.n_slabs) * 64u + (uint32_t)lane;
    }
}

// Decode attention over packed K/V (head_dim 64, 128 or 256; KVQ_ATTN_NO_RESIDUAL: no residual).
#define KVQ_ATTN_NO_RESIDUAL (-1)
#define KVQ_ATTN_MAX_SPLIT 2048  // token blocks per KV head at most
#define KVQ_ATTN_STATIC_SCRATCH_BYTES (32u << 20)  // kvq_decode_attention_noalloc's scratch
struct AttnPlanes {
    const uint8_t* codes;
    const void* meta0;
    const void* meta1;
    const float* gscale;
    int32_t gshift;  // log2 of the group size (INT4; NVFP4 blocks are 16)
};
struct AttnArgs {
    const uint16_t* q;  // [H * rep, D] bf16
    AttnPlanes k, v, rk, rv;
    int64_t T;
    int32_t H, rep, D;
    int32_t n_split;    // token blocks per KV head (on entry to the launcher: the bound)
    int64_t tc;         // tokens per block (a multiple of 64), set by the launcher
    float qscale;       // softmax scale * log2(e)
    float* part_o;      // [H, n_split, rep, D]
    float* part_ml;     // [H, n_split, rep, 2]
    float* out;         // [H * rep, D] fp32
};

// One wave of a carried row copy: chunks [task * kWinChunks, (task + 1) * kWinChunks) of the
// copy's rows * C8, all loads before the stores (the host keeps rows * C8 below 2^31). A chunk
// moves as two 64-bit words (merged into 16-byte accesses): accessed as a vector of 32-bit
// words, the copy's stores would be taken to alias the codec blocks' wave-uniform int and float
// loads (row maps, the NVFP4 multiplier), which would then lose their scalar form.
__device__ __forceinline__ void window_copy_wave(const CopyArgs& c, uint32_t task, int lane) {
    constexpr int K = (int)(kWinChunks / 64);
    const uint32_t total = (uint32_t)c.T * (uint32_t)c.C8;
    const uint32_t D8 = (uint32_t)c.D / 8u;
    uint64_t v[K][2];
    int64_t dofs[K];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const uint32_t u = min(task * kWinChunks + (uint32_t)(k * 64 + lane), total - 1u);
        const uint32_t r = fdiv(u, c.div_C8);
        const uint32_t c8 = u - r * (uint32_t)c.C8;
        const uint32_t h = fdiv(c8, c.div_D8);
        const uint32_t d = (c8 - h * D8) * 8u;
        const bool far = (int64_t)r >= c.split;
        const uint64_t* sp = reinterpret_cast<const uint64_t*>(c.src + (far ? c.src_jump : 0) + (int64_t)r * c.sst +
                                                               (int64_t)h * c.ssh + d);
        v[k][0] = sp[0];
        v[k][1] = sp[1];
        dofs[k] = (far ? c.dst_jump : 0) + (int64_t)r * c.dst_t + (int64_t)h * c.dsh + d;
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
        if (task * kWinChunks + (uint32_t)(k * 64 + lane) < total) {
            uint64_t* dp = reinterpret_cast<uint64_t*>(c.dst + dofs[k]);
            dp[0] = v[k][0];
            dp[1] = v[k][1];
        }
    }
}

// Grid of a vector launch: `main` blocks of `wpb` waves, then the blocks of the row copy the
// arguments carry (sets win_block0).
template <class Args>
inline dim3 grid_with_copy(Args& b, uint32_t main, uint32_t wpb) {
    b.win_block0 = main;
    return dim3(main + (b.win_tasks + wpb - 1u) / wpb);
}

// ---- launchers (return hipGetLastError() of the launch) ----
// vec: the 8-channel vector path is legal for these arguments (alignment, strides, G).

hipError_t launch_amax(const EncArgs& a, bool diff, bool gather, bool vec, hipStream_t s);
hipError_t launch_set_global(float* gscale, uint32_t value_bits, hipStream_t s);
hipError_t launch_encode(int fmt, int kind, const EncArgs& a, bool diff, bool gather, bool vec, hipStream_t s);
hipError_t launch_decode(int fmt, int kind, const DecArgs& a, bool add, bool scatter, bool vec, hipStream_t s);
hipError_t launch_copy_rows(const CopyArgs& a, bool vec, hipStream_t s);
// Row formats (NVFP4-row, FP8-row): encode / decode of rows that each carry their own scale.
hipError_t launch_row_encode(int fmt, const EncArgs& a, bool diff, bool gather, bool vec, hipStream_t s);
hipError_t launch_row_decode(int fmt, const DecArgs& a, bool add, bool scatter, bool vec, hipStream_t s);
// Decode attention: base format of K and V, residual format (or KVQ_ATTN_NO_RESIDUAL).
hipError_t launch_attention(int fmt, int rfmt, const AttnArgs& a, hipStream_t s);
hipError_t launch_copy_i32(int32_t* dst, const int32_t* src, int64_t n, hipStream_t s);
hipError_t launch_validate_positions(const int32_t* pos, int64_t M, int64_t T, uint32_t* scratch, int32_t* status,
                                     hipStream_t s);

}  // namespace kvq
