// kvq_decode.hip -- decode kernels: unpack_kv and decode_residual for INT4 and NVFP4, plus the
// row copy used by an out-of-place sparse decode and the opt-in position-map check.
//
// Decoding ([PR166] = vllm-rlt PR #166 "INT4 KV packing/unpacking and cross-loop residual
// reconstruction", section "Purpose"):
//   INT4  y = bf16(fl(fl(code * f32(scale16)) + f32(min16)))
//   NVFP4 y = bf16(fl(e2m1(code) * fl(f32(e4m3 block scale) / g)))
//   residual: out = bf16(fl(prev + y)) (y already rounded to bf16: both steps in the input
//   dtype); a sparse residual writes only the rows named in its position map.
//
// Vector path (D % 8 == 0, aligned rows): a lane turns one 32-bit code word into 8 channels and
// writes them with one 16-byte store. A wave task is RW consecutive rows of one 64-chunk slab;
// for KEY those rows share their token group (G % RW == 0), so the lane loads its 8 channels'
// metadata once per task.
#include <type_traits>

#include "kvq_launch.hpp"

namespace kvq {

namespace {

constexpr int kThreads = 256;

// Output word of two decoded values: bf16 of each, or for a residual the bf16 of prev plus the
// bf16-rounded decoded value (both steps in the input dtype).
template <bool ADD>
__device__ __forceinline__ uint32_t finish_pair(float y0, float y1, uint32_t prev_word) {
    const uint32_t yb = pack_bf16x2(y0, y1);
    if constexpr (!ADD) return yb;
    return pack_bf16x2(__fadd_rn(bf16lo(prev_word), bf16lo(yb)), __fadd_rn(bf16hi(prev_word), bf16hi(yb)));
}

template <int FMT, int KIND, bool ADD, bool SCATTER, bool LG, bool WIN>
__global__ __launch_bounds__(kThreads) void k_decode_vec(DecArgs a) {
    constexpr int RW = KVQ_DECODE_ROWS;
    if (WIN && blockIdx.x >= a.win_block0) {  // blocks of the carried row copy
        window_copy_wave(a.win, __builtin_amdgcn_readfirstlane((blockIdx.x - a.win_block0) * 4u + (threadIdx.x >> 6)),
                         threadIdx.x & 63);
        return;
    }
    __shared__ std::conditional_t<FMT == FMT_NVFP4, Fp4Table, char> tab;
    if constexpr (FMT == FMT_NVFP4) fp4_table_fill(tab, *a.gscale);
    const int lane = threadIdx.x & 63;
    const uint32_t task =
        __builtin_amdgcn_readfirstlane(xcd_block(blockIdx.x, WIN ? a.win_block0 : gridDim.x) * 4u + (threadIdx.x >> 6));
    if (task >= a.n_tasks) return;
    uint32_t rtile, c8raw;
    task_lane<LG>(a, task, lane, rtile, c8raw);  // with LG a lane group past the last row tile stores nothing
    const bool valid = c8raw < (uint32_t)a.C8;
    const uint32_t c8 = valid ? c8raw : (uint32_t)a.C8 - 1u;  // idle lanes read a valid chunk
    const uint32_t h = fdiv(c8, a.div_D8);
    const uint32_t d = (c8 - h * (uint32_t)a.D8) * 8u;
    const int64_t r0 = (int64_t)rtile * RW;
    const int nr = (int)min<int64_t>(RW, a.rows - r0);

    // all loads first (tail rows re-read the last row; only stores are masked). Output row i
    // reads packed row rs[i] (slot reads; KEY only without a source map) and writes row tt[i].
    int64_t rs[RW], tt[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i) {
        const int64_t rr = min<int64_t>(r0 + i, a.rows - 1);
        rs[i] = a.src ? (int64_t)a.src[rr] : rr;
        tt[i] = SCATTER ? (int64_t)a.pos[rr] : rr;
    }
    uint32_t cw[RW];
#pragma unroll
    for (int i = 0; i < RW; ++i)
        cw[i] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(a.codes) + (size_t)rs[i] * (uint32_t)a.C8 + c8);
    u32x4 pv[RW];
    if constexpr (ADD) {
#pragma unroll
        for (int i = 0; i < RW; ++i) pv[i] = ld_stream(a.prev + tt[i] * a.pst + (int64_t)h * a.psh + d);
    }
    // per-row metadata (VALUE): one group per lane and row
    float vs[RW], vm[RW];
    uint32_t vc[RW];
    if constexpr (KIND == KIND_VALUE) {
#pragma unroll
        for (int i = 0; i < RW; ++i) {
            const size_t midx = (size_t)rs[i] * (uint32_t)a.ngr + (c8 >> a.lpg_shift);
            if constexpr (FMT == FMT_INT4) {
                vs[i] = f16_to_f32(reinterpret_cast<const uint16_t*>(a.meta1)[midx]);
                vm[i] = f16_to_f32(reinterpret_cast<const uint16_t*>(a.meta0)[midx]);
            } else {
                vc[i] = reinterpret_cast<const uint8_t*>(a.meta0)[midx] & 0x7Fu;  // scaled below
                vm[i] = 0.0f;
            }
        }
    }

    // KEY: per-channel metadata of this task's token group (G % RW == 0), loaded once
    float ks[8], km[8];
    if constexpr (KIND == KIND_KEY) {
        // (a lane group past the last row tile, which stores nothing, reads the last group's).
        // Rows stay below 2^31, so the wave-uniform group index is a 32-bit shift for a
        // power-of-two G and a 32-bit division otherwise.
        const uint32_t rm = (uint32_t)min<int64_t>(r0, a.rows - 1), gsz = (uint32_t)a.G;
        const uint32_t gi = (gsz & (gsz - 1u)) == 0u ? rm >> __builtin_ctz(gsz) : rm / gsz;
        const size_t mbase = ((size_t)gi * (uint32_t)a.C8 + c8) * 8u;
        if constexpr (FMT == FMT_INT4) {
            const u32x4 mins = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.meta0) + mbase);
            const u32x4 scs = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.meta1) + mbase);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                km[2 * j] = f16_to_f32(mins[j] & 0xFFFFu);
                km[2 * j + 1] = f16_to_f32(mins[j] >> 16);
                ks[2 * j] = f16_to_f32(scs[j] & 0xFFFFu);
                ks[2 * j + 1] = f16_to_f32(scs[j] >> 16);
            }
        } else {
            const uint2 sc = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(a.meta0) + mbase);
            const uint32_t sw[2] = {sc.x, sc.y};
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                ks[k] = tab.e[(sw[k >> 2] >> (8 * (k & 3))) & 0x7Fu][0];  // sign bit of a stored scale is 0
                km[k] = 0.0f;
            }
        }
    } else if constexpr (FMT == FMT_NVFP4) {
#pragma unroll
        for (int i = 0; i < RW; ++i) vs[i] = tab.e[vc[i]][0];
    }

#pragma unroll
    for (int i = 0; i < RW; ++i) {
        float y[8];
        if constexpr (FMT == FMT_INT4) {
            // nibbles 2j / 2j+1 sit in the low / high half of byte j
            const uint32_t lo = cw[i] & 0x0F0F0F0Fu, hi = (cw[i] >> 4) & 0x0F0F0F0Fu;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float c0 = (float)((lo >> (8 * j)) & 0xFFu), c1 = (float)((hi >> (8 * j)) & 0xFFu);
                if constexpr (KIND == KIND_KEY) {
                    y[2 * j] = int4_value_f(c0, ks[2 * j], km[2 * j]);
                    y[2 * j + 1] = int4_value_f(c1, ks[2 * j + 1], km[2 * j + 1]);
                } else {
                    y[2 * j] = int4_value_f(c0, vs[i], vm[i]);
                    y[2 * j + 1] = int4_value_f(c1, vs[i], vm[i]);
                }
            }
        } else {
            const f32x2 e0 = e2m1_values<0>(cw[i]), e1 = e2m1_values<1>(cw[i]);
            const f32x2 e2 = e2m1_values<2>(cw[i]), e3 = e2m1_values<3>(cw[i]);
            const float e[8] = {e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
#pragma unroll
            for (int k = 0; k < 8; ++k) y[k] = __fmul_rn(e[k], (KIND == KIND_KEY) ? ks[k] : vs[i]);
        }
        u32x4 o;
        o.x = finish_pair<ADD>(y[0], y[1], ADD ? pv[i].x : 0u);
        o.y = finish_pair<ADD>(y[2], y[3], ADD ? pv[i].y : 0u);
        o.z = finish_pair<ADD>(y[4], y[5], ADD ? pv[i].z : 0u);
        o.w = finish_pair<ADD>(y[6], y[7], ADD ? pv[i].w : 0u);
        if (i < nr && valid)
            *reinterpret_cast<u32x4*>(a.out + row_offset(tt[i], a.opshift, a.opst, a.ost) + (int64_t)h * a.osh + d) = o;
    }
}

// Generic path: one thread per (row, head, channel pair).
template <int FMT, int KIND, bool ADD, bool SCATTER>
__global__ __launch_bounds__(kThreads) void k_decode_gen(DecArgs a) {
    __shared__ std::conditional_t<FMT == FMT_NVFP4, Fp4Table, char> tab;
    if constexpr (FMT == FMT_NVFP4) fp4_table_fill(tab, *a.gscale);
    const int D = a.D, G = a.G;
    const int Dp = (D + 1) / 2;
    const int64_t idx = (int64_t)(a.gen_base + (uint64_t)blockIdx.x * kThreads + threadIdx.x);
    if (idx >= a.rows * a.H * Dp) return;
    const int64_t r = idx / ((int64_t)a.H * Dp);
    const int64_t rem = idx - r * a.H * Dp;
    const int64_t h = rem / Dp;
    const int j = (int)(rem - h * Dp);
    const int64_t t = SCATTER ? (int64_t)a.pos[r] : r;
    const int64_t rs = a.src ? (int64_t)a.src[r] : r;  // packed row read
    const uint32_t byte = a.codes[(size_t)(rs * a.H + h) * Dp + j];
    for (int k = 0; k < 2; ++k) {
        const int dd = 2 * j + k;
        if (dd >= D) break;
        const size_t midx = (KIND == KIND_KEY) ? (size_t)((rs / G) * a.H + h) * D + dd
                                               : (size_t)(rs * a.H + h) * ((D + G - 1) / G) + dd / G;
        const uint32_t c = (byte >> (4 * k)) & 0xFu;
        float y;
        if constexpr (FMT == FMT_INT4) {
            y = int4_value(c, f16_to_f32(reinterpret_cast<const uint16_t*>(a.meta1)[midx]),
                           f16_to_f32(reinterpret_cast<const uint16_t*>(a.meta0)[midx]));
        } else {
            y = __fmul_rn(e2m1_values<0>(c)[0], tab.e[reinterpret_cast<const uint8_t*>(a.meta0)[midx] & 0x7Fu][0]);
        }
        uint32_t outb = bf16_bits(y);
        if constexpr (ADD) {
            const float p = bf16_to_f32(a.prev[t * a.pst + h * a.psh + dd]);
            outb = bf16_bits(__fadd_rn(p, bf16_to_f32(outb)));
        }
        a.out[row_offset(t, a.opshift, a.opst, a.ost) + h * a.osh + dd] = (uint16_t)outb;
    }
}

// Row copy (out-of-place sparse decode: absent rows inherit prev bit for bit; the protected rows
// of a BF16 window, front and back ranges in one launch).
template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_copy_rows(CopyArgs a) {
    if constexpr (VEC) {
        const uint64_t total = (uint64_t)a.T * (uint32_t)a.C8;
        const uint64_t u = a.gen_base + (uint64_t)blockIdx.x * kThreads + threadIdx.x;
        if (u >= total) return;
        const uint32_t r = fdiv((uint32_t)u, a.div_C8);
        const uint32_t c8 = (uint32_t)u - r * (uint32_t)a.C8;
        const uint32_t h = fdiv(c8, a.div_D8);
        const uint32_t d = (c8 - h * (uint32_t)(a.D / 8)) * 8u;
        const bool far = (int64_t)r >= a.split;
        *reinterpret_cast<uint4*>(a.dst + (far ? a.dst_jump : 0) + (int64_t)r * a.dst_t + (int64_t)h * a.dsh + d) =
            *reinterpret_cast<const uint4*>(a.src + (far ? a.src_jump : 0) + (int64_t)r * a.sst + (int64_t)h * a.ssh + d);
    } else {
        const uint64_t total = (uint64_t)a.T * a.H * a.D;
        const uint64_t u = a.gen_base + (uint64_t)blockIdx.x * kThreads + threadIdx.x;
        if (u >= total) return;
        const int64_t HD = (int64_t)a.H * a.D;
        const int64_t r = (int64_t)(u / (uint64_t)HD);
        const int64_t rem = (int64_t)u - r * HD;
        const int64_t h = rem / a.D;
        const int64_t d = rem - h * a.D;
        const bool far = r >= a.split;
        a.dst[(far ? a.dst_jump : 0) + r * a.dst_t + h * a.dsh + d] = a.src[(far ? a.src_jump : 0) + r * a.sst + h * a.ssh + d];
    }
}

__global__ __launch_bounds__(kThreads) void k_copy_i32(int32_t* dst, const int32_t* src, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n) dst[i] = src[i];
}

// Position-map check: clear the bitmap and the status word, then mark every position.
__global__ __launch_bounds__(kThreads) void k_validate_clear(uint32_t* scratch, int64_t words, int32_t* status) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < words) scratch[i] = 0u;
    if (i == 0) *status = 0;
}

__global__ __launch_bounds__(kThreads) void k_validate_mark(const int32_t* pos, int64_t M, int64_t T,
                                                            uint32_t* scratch, int32_t* status) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i >= M) return;
    const int64_t p = pos[i];
    if (p < 0 || p >= T) {
        atomicOr(reinterpret_cast<unsigned int*>(status), 1u);
        return;
    }
    const uint32_t bit = 1u << (p & 31);
    const uint32_t old = atomicOr(&scratch[p >> 5], bit);
    if (old & bit) atomicOr(reinterpret_cast<unsigned int*>(status), 2u);
}

inline uint32_t ceil_div_u(uint64_t a, uint64_t b) { return (uint32_t)((a + b - 1) / b); }

template <int FMT, int KIND, bool ADD, bool SCATTER>
hipError_t decode_launch(const DecArgs& a, bool vec, hipStream_t s) {
    if (vec) {
        DecArgs b = a;
        const dim3 grid = grid_with_copy(b, ceil_div_u(a.n_tasks, 4), 4u);
        const bool win = !SCATTER && a.win_tasks;  // a window never scatters
        if (a.ri_shift > 0) {
            if (win) hipLaunchKernelGGL((k_decode_vec<FMT, KIND, ADD, false, true, true>), grid, dim3(kThreads), 0, s, b);
            else hipLaunchKernelGGL((k_decode_vec<FMT, KIND, ADD, SCATTER, true, false>), grid, dim3(kThreads), 0, s, b);
        } else {
            if (win) hipLaunchKernelGGL((k_decode_vec<FMT, KIND, ADD, false, false, true>), grid, dim3(kThreads), 0, s, b);
            else hipLaunchKernelGGL((k_decode_vec<FMT, KIND, ADD, SCATTER, false, false>), grid, dim3(kThreads), 0, s, b);
        }
    } else {
        const uint64_t n = (uint64_t)a.rows * a.H * ((a.D + 1) / 2);
        launch_in_chunks(a, n, kThreads, [&](const DecArgs& b, dim3 grid) {
            hipLaunchKernelGGL((k_decode_gen<FMT, KIND, ADD, SCATTER>), grid, dim3(kThreads), 0, s, b);
        });
    }
    return hipGetLastError();
}

template <int FMT, int KIND>
hipError_t decode_modes(const DecArgs& a, bool add, bool scatter, bool vec, hipStream_t s) {
    if (add)
        return scatter ? decode_launch<FMT, KIND, true, true>(a, vec, s)
                       : decode_launch<FMT, KIND, true, false>(a, vec, s);
    return scatter ? decode_launch<FMT, KIND, false, true>(a, vec, s) : decode_launch<FMT, KIND, false, false>(a, vec, s);
}

}  // namespace

hipError_t launch_decode(int fmt, int kind, const DecArgs& a, bool add, bool scatter, bool vec, hipStream_t s) {
    if (fmt == FMT_INT4)
        return kind == KIND_KEY ? decode_modes<FMT_INT4, KIND_KEY>(a, add, scatter, vec, s)
                                : decode_modes<FMT_INT4, KIND_VALUE>(a, add, scatter, vec, s);
    return kind == KIND_KEY ? decode_modes<FMT_NVFP4, KIND_KEY>(a, add, scatter, vec, s)
                            : decode_modes<FMT_NVFP4, KIND_VALUE>(a, add, scatter, vec, s);
}

hipError_t launch_copy_rows(const CopyArgs& a, bool vec, hipStream_t s) {
    const uint64_t n = vec ? (uint64_t)a.T * (uint32_t)a.C8 : (uint64_t)a.T * a.H * a.D;
    if (n == 0) return hipSuccess;
    launch_in_chunks(a, n, kThreads, [&](const CopyArgs& b, dim3 grid) {
        if (vec)
            hipLaunchKernelGGL(k_copy_rows<true>, grid, dim3(kThreads), 0, s, b);
        else
            hipLaunchKernelGGL(k_copy_rows<false>, grid, dim3(kThreads), 0, s, b);
    });
    return hipGetLastError();
}

hipError_t launch_copy_i32(int32_t* dst, const int32_t* src, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_copy_i32, dim3(ceil_div_u((uint64_t)n, kThreads)), dim3(kThreads), 0, s, dst, src, n);
    return hipGetLastError();
}

hipError_t launch_validate_positions(const int32_t* pos, int64_t M, int64_t T, uint32_t* scratch, int32_t* status,
                                     hipStream_t s) {
    const int64_t words = (T + 31) / 32;
    const uint64_t n1 = words > 0 ? (uint64_t)words : 1;
    hipLaunchKernelGGL(k_validate_clear, dim3(ceil_div_u(n1, kThreads)), dim3(kThreads), 0, s, scratch, words, status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || M == 0) return e;
    hipLaunchKernelGGL(k_validate_mark, dim3(ceil_div_u((uint64_t)M, kThreads)), dim3(kThreads), 0, s, pos, M, T,
                       scratch, status);
    return hipGetLastError();
}

}  // namespace kvq
