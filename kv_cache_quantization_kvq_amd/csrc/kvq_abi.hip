// kvq_abi.hip -- the C ABI: argument checks, plane sizes, and kernel dispatch on the caller's
// stream. Nothing here allocates, frees or synchronizes.
#include <string.h>

#include <algorithm>
#include <mutex>

#include "kvq.h"
#include "kvq_launch.hpp"

using namespace kvq;

// Scratch memory of kvq_decode_attention_noalloc: the per-block partials (unnormalized outputs,
// maxima and sums) that kvq_decode_attention keeps in a caller workspace live here instead.
// Every GPU the library runs on holds its own copy until the process ends. In host code this
// name is only a stand-in for the symbol: the device address comes from hipGetSymbolAddress.
static __device__ __align__(256) float scratch[KVQ_ATTN_STATIC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr int64_t kMaxElems = (int64_t)1 << 36;
constexpr size_t kWorkspaceBytes = KVQ_AMAX_MAX_BLOCKS * sizeof(uint32_t);

// Device address of `scratch` on each device, looked up once per device (with that device
// current) on the first kvq_decode_attention_noalloc call there.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

kvq_status scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVQ_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return KVQ_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool dims_ok(int64_t rows, int64_t H, int64_t D) {
    if (rows < 0 || H < 0 || D < 0) return false;
    if (rows >= kMaxDim || H >= kMaxDim || D >= kMaxDim) return false;
    return (unsigned __int128)rows * (unsigned __int128)H * (unsigned __int128)D < (unsigned __int128)kMaxElems;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
int log2i(int64_t v) {
    int s = 0;
    while (((int64_t)1 << s) < v) ++s;
    return s;
}
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

FastDiv fastdiv_make(uint32_t d) {
    FastDiv f;
    f.d = d;
    uint32_t l = 0;
    while (((uint64_t)1 << l) < d) ++l;
    f.m = (uint32_t)(((((uint64_t)1 << l) - d) << 32) / d + 1);
    f.s = l;
    f.pad = 0;
    return f;
}

bool row_format(int format) { return format == KVQ_NVFP4_ROW || format == KVQ_FP8_ROW; }

kvq_status check_kind_format(int kind, int format) {
    if (kind != KVQ_KEY && kind != KVQ_VALUE) return KVQ_ERR_FORMAT;
    if (format != KVQ_INT4 && format != KVQ_NVFP4 && !row_format(format)) return KVQ_ERR_FORMAT;
    return KVQ_OK;
}

// group_size 0 selects the default: INT4 64, NVFP4 and NVFP4-row 16, FP8-row 0 (its only value).
int32_t resolve_group(int format, int32_t G) {
    if (G == 0) return format == KVQ_INT4 ? 64 : (format == KVQ_FP8_ROW ? 0 : 16);
    return G;
}

kvq_status check_group(int format, int32_t G) {
    if (format == KVQ_FP8_ROW) return G == 0 ? KVQ_OK : KVQ_ERR_GROUP;
    if (G < 1) return KVQ_ERR_GROUP;
    if ((format == KVQ_NVFP4 || format == KVQ_NVFP4_ROW) && G != 16) return KVQ_ERR_GROUP;
    return KVQ_OK;
}

kvq_status plane_sizes(int format, int kind, int32_t G, int64_t rows, int64_t H, int64_t D, int sparse,
                       uint64_t s[KVQ_NUM_PLANES]) {
    kvq_status st = check_kind_format(kind, format);
    if (st) return st;
    G = resolve_group(format, G);
    if ((st = check_group(format, G))) return st;
    if (!dims_ok(rows, H, D)) return KVQ_ERR_SHAPE;
    const uint64_t rh = (uint64_t)rows * H;
    s[KVQ_PLANE_CODES] = (format == KVQ_FP8_ROW) ? rh * D : rh * cdiv(D, 2);
    s[KVQ_PLANE_META1] = 0;
    s[KVQ_PLANE_GLOBAL] = 0;
    if (format == KVQ_NVFP4_ROW) {
        s[KVQ_PLANE_META0] = rh * cdiv(D, 16);
        s[KVQ_PLANE_META1] = 4 * rh;
    } else if (format == KVQ_FP8_ROW) {
        s[KVQ_PLANE_META0] = 4 * rh;
    } else {
        const uint64_t ng = (kind == KVQ_KEY) ? (uint64_t)cdiv(rows, G) * H * D : rh * cdiv(D, G);
        s[KVQ_PLANE_META0] = (format == KVQ_INT4) ? 2 * ng : ng;
        s[KVQ_PLANE_META1] = (format == KVQ_INT4) ? 2 * ng : 0;
        s[KVQ_PLANE_GLOBAL] = (format == KVQ_NVFP4) ? 4 : 0;
    }
    s[KVQ_PLANE_POSITIONS] = sparse ? 4 * (uint64_t)rows : 0;
    return KVQ_OK;
}

kvq_status check_tensor(const kvq_tensor* x) {
    if (!x) return KVQ_ERR_NULL;
    if (x->dtype != KVQ_BF16) return KVQ_ERR_DTYPE;
    if (!dims_ok(x->T, x->H, x->D)) return KVQ_ERR_SHAPE;
    if (x->stride_t < 0 || x->stride_h < 0) return KVQ_ERR_LAYOUT;
    if (x->T * x->H * x->D > 0 && !x->data) return KVQ_ERR_NULL;
    return KVQ_OK;
}

// A strided view reaches [data, data + span) bytes.
void view_span(const kvq_tensor* x, uintptr_t* lo, uintptr_t* hi) {
    *lo = (uintptr_t)x->data;
    if (x->T * x->H * x->D == 0) {
        *hi = *lo;
        return;
    }
    const int64_t last = (x->T - 1) * x->stride_t + (x->H - 1) * x->stride_h + (x->D - 1);
    *hi = *lo + (uintptr_t)(last + 1) * 2u;
}

bool view_vec_ok(const void* data, int64_t st, int64_t sh) {
    return aligned(data, 16) && (st % 8) == 0 && (sh % 8) == 0;
}

// A bf16 [T, H, D] view as the kernels address it: row t at
// row_offset(t, pshift, pst, st) (pages of 2^pshift rows pst apart, or unpaged).
struct View {
    void* data;
    int64_t T, H, D;
    int64_t st, sh;
    int32_t pshift;
    int64_t pst;
};

View view_of(const kvq_tensor* x) { return View{x->data, x->T, x->H, x->D, x->stride_t, x->stride_h, kNoPaging, 0}; }

bool view_vec_ok(const View& v) {
    return view_vec_ok(v.data, v.st, v.sh) && (v.pshift == kNoPaging || v.pst % 8 == 0);
}

// Checks a paged view and turns it into a View in page-major token order.
kvq_status view_of_paged(const kvq_paged* x, View* v) {
    if (!x) return KVQ_ERR_NULL;
    if (x->dtype != KVQ_BF16) return KVQ_ERR_DTYPE;
    if (x->pages < 0 || x->page_size < 0 || x->pages >= kMaxDim || x->page_size >= kMaxDim) return KVQ_ERR_SHAPE;
    const int64_t T = x->pages * x->page_size;
    if (!dims_ok(T, x->H, x->D)) return KVQ_ERR_SHAPE;
    if (x->stride_page < 0 || x->stride_slot < 0 || x->stride_h < 0) return KVQ_ERR_LAYOUT;
    if (T * x->H * x->D > 0 && !x->data) return KVQ_ERR_NULL;
    *v = View{x->data, T, x->H, x->D, x->stride_slot, x->stride_h, kNoPaging, 0};
    if (x->pages > 1 && x->stride_page != x->page_size * x->stride_slot) {
        if (!is_pow2(x->page_size)) return KVQ_ERR_LAYOUT;
        v->pshift = log2i(x->page_size);
        v->pst = x->stride_page;
    }
    return KVQ_OK;
}

// Vector path of the row formats: head_dim a power of two from 8 to 512 (a (token, head) row
// spans D/8 lanes of one wave).
bool row_vec_dims(int64_t D) { return D % 8 == 0 && is_pow2(D / 8) && D / 8 <= 64; }

// Geometry of the 8-channel vector path. Rows shorter than 64 chunks whose chunk count divides
// 64 use lane groups (several row tiles per task, task_lane); with VALUE groups (lane_groups
// of lpg lanes) the groups must also tile a row's lanes.
template <typename Args>
void fill_vec_geometry(Args& a, int64_t rows, int64_t H, int64_t D, int32_t G, int rows_per_task,
                       bool lane_groups_in_rows = true) {
    a.D8 = (int32_t)(D / 8);
    a.C8 = (int32_t)(H * (D / 8));
    a.n_slabs = (int32_t)cdiv(a.C8, 64);
    a.lpg = (G % 8 == 0) ? G / 8 : 1;
    a.lpg_shift = log2i(a.lpg);
    a.ngr = a.C8 / a.lpg;
    a.div_D8 = fastdiv_make((uint32_t)a.D8);
    a.div_slabs = fastdiv_make((uint32_t)a.n_slabs);
    a.n_tasks = (uint32_t)(cdiv(rows, rows_per_task) * a.n_slabs);
    a.ri_shift = a.c8_shift = 0;
    if (a.C8 < 64 && is_pow2(a.C8) && (!lane_groups_in_rows || a.C8 % a.lpg == 0)) {
        a.c8_shift = log2i(a.C8);
        a.ri_shift = 6 - a.c8_shift;
        a.n_tasks = (uint32_t)cdiv(cdiv(rows, rows_per_task), (int64_t)1 << a.ri_shift);
    }
}

kvq_status hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

// A row copy with the path it can take: the 16-byte vector copy (D % 8 == 0, aligned views,
// rows * H * D / 8 below 2^31) or one element per thread.
struct RowCopy {
    CopyArgs c;
    bool vec;
};

// Rows of a [rows, H, D] bf16 view copied into another; rows r >= split are read src_jump and
// written dst_jump elements further on (both multiples of the row pitches).
RowCopy make_row_copy(const void* src, int64_t sst, int64_t ssh, void* dst, int64_t dst_t, int64_t dsh, int64_t rows,
                      int64_t H, int64_t D, int64_t split, int64_t src_jump, int64_t dst_jump) {
    RowCopy r;
    CopyArgs& c = r.c;
    memset(&c, 0, sizeof c);
    c.split = split;
    c.src_jump = src_jump;
    c.dst_jump = dst_jump;
    c.src = static_cast<const uint16_t*>(src);
    c.sst = sst;
    c.ssh = ssh;
    c.dst = static_cast<uint16_t*>(dst);
    c.dst_t = dst_t;
    c.dsh = dsh;
    c.T = rows;
    c.H = (int32_t)H;
    c.D = (int32_t)D;
    r.vec = rows * H * D > 0 && (D % 8 == 0) && view_vec_ok(src, sst, ssh) && view_vec_ok(dst, dst_t, dsh) &&
            (uint64_t)rows * (uint64_t)(H * D / 8) < ((uint64_t)1 << 31);
    if (r.vec) {
        c.C8 = (int32_t)(H * D / 8);
        c.div_C8 = fastdiv_make((uint32_t)c.C8);
        c.div_D8 = fastdiv_make((uint32_t)(D / 8));
    }
    return r;
}

hipError_t launch_row_copy(const RowCopy& r, hipStream_t stream) { return launch_copy_rows(r.c, r.vec, stream); }

// Hands a vector row copy to a dense vector encode or decode launch, which runs it in blocks
// appended to its grid (one launch instead of two). False when either side takes another path
// or the launch gathers or scatters rows; the caller then launches the copy on its own.
template <class Args>
bool carry_copy(const RowCopy* win, bool vec, Args& a) {
    if (!win || !win->vec || !vec || win->c.T == 0 || a.pos) return false;
    a.win = win->c;
    a.win_tasks = (uint32_t)cdiv(win->c.T * (int64_t)win->c.C8, (int64_t)kWinChunks);
    return true;
}

// Fill the encoder arguments for `rows` encoded rows of `cur` (optionally minus prev, gathered
// by positions, written to packed rows dst[r]) into the planes of `planes`, and launch. With
// amax_only, only the NVFP4 tensor-amax pass runs, storing the multiplier in
// planes->global_scale.
kvq_status encode_run(const View& cur, const kvq_tensor* prev, const int32_t* positions, int64_t rows, int kind,
                      int format, int32_t G, const kvq_packed* planes, void* workspace, const int32_t* dst,
                      hipStream_t stream, bool amax_only = false, const RowCopy* win = nullptr) {
    const int64_t H = cur.H, D = cur.D;
    const bool sparse = positions != nullptr;
    EncArgs a;
    memset(&a, 0, sizeof a);
    a.cur = static_cast<const uint16_t*>(cur.data);
    a.cst = cur.st;
    a.csh = cur.sh;
    a.cpshift = cur.pshift;
    a.cpst = cur.pst;
    if (prev) {
        a.prev = static_cast<const uint16_t*>(prev->data);
        a.pst = prev->stride_t;
        a.psh = prev->stride_h;
    }
    a.pos = positions;
    a.pos_out = sparse ? planes->positions : nullptr;
    a.dst = dst;
    a.rows = rows;
    a.H = (int32_t)H;
    a.D = (int32_t)D;
    a.G = G;
    a.codes = planes->codes;
    a.meta0 = planes->meta0;
    a.meta1 = planes->meta1;
    a.gscale = planes->global_scale;
    a.ws = static_cast<uint32_t*>(workspace);

    // vector path eligibility
    bool vec = (D % 8 == 0) && view_vec_ok(cur) && aligned(planes->codes, 4) &&
               (uint64_t)rows * (uint64_t)(H * D / 8) < ((uint64_t)1 << 31);
    if (prev) vec = vec && view_vec_ok(prev->data, prev->stride_t, prev->stride_h);
    // the vector encoders address a row's elements by a 32-bit byte offset from the row start
    const auto span_ok = [&](int64_t sh) { return sh >= 0 && (H - 1) * sh + D <= ((int64_t)1 << 30); };
    vec = vec && span_ok(cur.sh) && (!prev || span_ok(prev->stride_h));
    if (row_format(format)) {
        vec = vec && row_vec_dims(D) &&
              (format == KVQ_FP8_ROW ? aligned(planes->codes, 8) && aligned(planes->meta0, 4) : aligned(planes->meta1, 4));
    } else if (kind == KVQ_VALUE) {
        vec = vec && (G % 8 == 0) && (D % G == 0) && is_pow2(G / 8) && (G / 8) <= 16;
    } else if (format == KVQ_INT4) {
        vec = vec && (G == 16 || G == 32 || G == 64 || G == 128) && aligned(planes->meta0, 16) &&
              aligned(planes->meta1, 16);
    } else {
        vec = vec && aligned(planes->meta0, 8);
    }
    if (vec) {
        if (row_format(format) || kind == KVQ_VALUE) {
            fill_vec_geometry(a, rows, H, D, row_format(format) ? 8 : G,
                              row_format(format) ? KVQ_ROW_ENCODE_ROWS
                                                 : value_encode_rows(format == KVQ_NVFP4, prev != nullptr));
        } else {
            fill_vec_geometry(a, rows, H, D, G, G, false);  // KEY groups run over tokens
        }
        a.div_C8 = fastdiv_make((uint32_t)a.C8);
    }

    if (amax_only) return hip_status(launch_amax(a, prev != nullptr, sparse, vec, stream));
    const bool carry = carry_copy(win, vec, a);
    hipError_t e = hipSuccess;
    if (row_format(format)) {
        e = launch_row_encode(format, a, prev != nullptr, sparse, vec, stream);
    } else {
        if (format == KVQ_NVFP4) e = launch_amax(a, prev != nullptr, sparse, vec, stream);
        if (e == hipSuccess) e = launch_encode(format, kind, a, prev != nullptr, sparse, vec, stream);
    }
    if (e == hipSuccess && win && !carry) e = launch_row_copy(*win, stream);
    return hip_status(e);
}

kvq_status encode_common(const View& cur, const kvq_tensor* prev, const int32_t* positions, int64_t M, int kind,
                         int format, int32_t G, kvq_packed* out, void* workspace, hipStream_t stream,
                         const RowCopy* win = nullptr) {
    kvq_status st = check_kind_format(kind, format);
    if (st) return st;
    G = resolve_group(format, G);
    if ((st = check_group(format, G))) return st;
    if (prev) {
        if ((st = check_tensor(prev))) return st;
        if (prev->T != cur.T || prev->H != cur.H || prev->D != cur.D) return KVQ_ERR_SHAPE;
    }
    const bool sparse = positions != nullptr;
    if (M < 0 || (sparse && M > cur.T)) return KVQ_ERR_SHAPE;
    if (!sparse && M != 0) return KVQ_ERR_SHAPE;
    const int64_t rows = sparse ? M : cur.T;
    const int64_t H = cur.H, D = cur.D;
    if (!out) return KVQ_ERR_NULL;
    uint64_t sz[KVQ_NUM_PLANES];
    if ((st = plane_sizes(format, kind, G, rows, H, D, sparse ? 1 : 0, sz))) return st;
    if (sz[KVQ_PLANE_CODES] && !out->codes) return KVQ_ERR_NULL;
    if (sz[KVQ_PLANE_META0] && !out->meta0) return KVQ_ERR_NULL;
    if (sz[KVQ_PLANE_META1] && !out->meta1) return KVQ_ERR_NULL;
    if (sz[KVQ_PLANE_GLOBAL] && !out->global_scale) return KVQ_ERR_NULL;
    // a sparse residual always owns a position plane, also with M == 0: a NULL plane would
    // make the descriptor read as dense
    if (sparse && !out->positions) return KVQ_ERR_NULL;
    if (format == KVQ_NVFP4 && !workspace) return KVQ_ERR_WORKSPACE;

    out->format = format;
    out->kind = kind;
    out->group_size = G;
    out->dtype = KVQ_BF16;
    out->rows = rows;
    out->H = H;
    out->D = D;
    out->full_T = cur.T;
    if (!sparse) out->positions = nullptr;

    const int64_t n = rows * H * D;
    if (n == 0) {
        hipError_t e = hipSuccess;
        if (format == KVQ_NVFP4) e = launch_set_global(out->global_scale, 0x3F800000u, stream);  // g = 1
        if (e == hipSuccess && sparse && M > 0) e = launch_copy_i32(out->positions, positions, M, stream);
        if (e == hipSuccess && win) e = launch_row_copy(*win, stream);
        return hip_status(e);
    }
    return encode_run(cur, prev, positions, rows, kind, format, G, out, workspace, nullptr, stream, false, win);
}

kvq_status check_packed(const kvq_packed* p) {
    if (!p) return KVQ_ERR_NULL;
    kvq_status st = check_kind_format(p->kind, p->format);
    if (st) return st;
    if ((st = check_group(p->format, p->group_size))) return st;
    if (p->dtype != KVQ_BF16) return KVQ_ERR_DTYPE;
    if (!dims_ok(p->rows, p->H, p->D)) return KVQ_ERR_SHAPE;
    uint64_t sz[KVQ_NUM_PLANES];
    if ((st = plane_sizes(p->format, p->kind, p->group_size, p->rows, p->H, p->D, 0, sz))) return st;
    if (sz[KVQ_PLANE_CODES] && !p->codes) return KVQ_ERR_NULL;
    if (sz[KVQ_PLANE_META0] && !p->meta0) return KVQ_ERR_NULL;
    if (sz[KVQ_PLANE_META1] && !p->meta1) return KVQ_ERR_NULL;
    if (p->format == KVQ_NVFP4 && !p->global_scale) return KVQ_ERR_NULL;
    return KVQ_OK;
}

// Decode `rows` rows of p into `out` (optionally adding prev): output row r reads packed row
// src ? src[r] : r and lands in row positions ? positions[r] : r.
kvq_status decode_run(const kvq_packed* p, int64_t rows, const kvq_tensor* prev, const View& out,
                      const int32_t* positions, const int32_t* src, hipStream_t stream, const RowCopy* win = nullptr) {
    const int64_t H = p->H, D = p->D;
    if (rows * H * D == 0) return win ? hip_status(launch_row_copy(*win, stream)) : KVQ_OK;
    DecArgs a;
    memset(&a, 0, sizeof a);
    a.codes = p->codes;
    a.meta0 = p->meta0;
    a.meta1 = p->meta1;
    a.gscale = p->global_scale;
    a.pos = positions;
    a.src = src;
    if (prev) {
        a.prev = static_cast<const uint16_t*>(prev->data);
        a.pst = prev->stride_t;
        a.psh = prev->stride_h;
    }
    a.out = static_cast<uint16_t*>(out.data);
    a.ost = out.st;
    a.osh = out.sh;
    a.opshift = out.pshift;
    a.opst = out.pst;
    a.rows = rows;
    a.H = (int32_t)H;
    a.D = (int32_t)D;
    a.G = p->group_size;
    const int32_t G = p->group_size;
    bool vec = (D % 8 == 0) && view_vec_ok(out) && aligned(p->codes, 4) &&
               (uint64_t)rows * (uint64_t)(H * D / 8) < ((uint64_t)1 << 31);
    if (prev) vec = vec && view_vec_ok(prev->data, prev->stride_t, prev->stride_h);
    hipError_t e;
    bool carry;
    if (row_format(p->format)) {
        vec = vec && row_vec_dims(D) && (p->format != KVQ_FP8_ROW || aligned(p->codes, 8));
        if (vec) fill_vec_geometry(a, rows, H, D, 8, KVQ_DECODE_ROWS);
        carry = carry_copy(win, vec, a);
        e = launch_row_decode(p->format, a, prev != nullptr, positions != nullptr, vec, stream);
    } else {
        if (p->kind == KVQ_VALUE) {
            vec = vec && (G % 8 == 0) && (D % G == 0) && is_pow2(G / 8);
        } else {
            // a KEY task loads its token group's metadata once, so slot reads take the generic path
            vec = vec && !src && (G % 8 == 0) && (G % KVQ_DECODE_ROWS == 0) &&
                  (p->format == KVQ_INT4 ? (aligned(p->meta0, 16) && aligned(p->meta1, 16)) : aligned(p->meta0, 8));
        }
        if (vec) fill_vec_geometry(a, rows, H, D, G, KVQ_DECODE_ROWS, p->kind == KVQ_VALUE);
        carry = carry_copy(win, vec, a);
        e = launch_decode(p->format, p->kind, a, prev != nullptr, positions != nullptr, vec, stream);
    }
    if (e == hipSuccess && win && !carry) e = launch_row_copy(*win, stream);
    return hip_status(e);
}

// Rows kept by a BF16 window over T tokens: min(sink, T) in front, then up to `recent` at the end.
void window_split(int64_t T, int64_t sink, int64_t recent, int64_t* ns, int64_t* nr) {
    *ns = sink < T ? sink : T;
    *nr = recent < T - *ns ? recent : T - *ns;
}

// Rows [r0, r0 + n) of a view, as a view.
kvq_tensor row_slice(const kvq_tensor* x, int64_t r0, int64_t n) {
    kvq_tensor v = *x;
    v.data = static_cast<uint16_t*>(x->data) + r0 * x->stride_t;
    v.T = n;
    return v;
}

// Token blocks of decode attention per KV head, at most: blocks of at least 64 tokens, never
// more than KVQ_ATTN_MAX_SPLIT per head (the combine kernel's bound). The launcher picks the
// split it runs (one round of resident blocks on the device) within this bound, which sizes the
// workspace.
int32_t attn_split_bound(int64_t T, int64_t H) {
    const int64_t per_head = KVQ_ATTN_MAX_SPLIT / (H > 0 ? H : 1);
    const int64_t n = std::min<int64_t>(per_head > 0 ? per_head : 1, cdiv(T > 0 ? T : 1, 64));
    return (int32_t)n;
}

size_t attn_workspace(int64_t T, int64_t H, int64_t rep, int64_t D) {
    return (size_t)H * attn_split_bound(T, H) * rep * (D + 2) * sizeof(float);
}

bool attn_head_dim(int64_t D) { return D == 64 || D == 128 || D == 256; }

// One packed tensor of an attention call: dense, the expected kind, head_dim 64, 128 or 256, any
// of the four formats, and for INT4 a group size the kernel's tiling takes (a power of two, K at
// least 16 tokens, V from D/16 (at least 8) to D channels).
kvq_status attn_operand(const kvq_packed* p, int kind, int64_t T, int64_t H, AttnPlanes* out) {
    kvq_status st = check_packed(p);
    if (st) return st;
    if (p->kind != kind || p->positions) return KVQ_ERR_MISMATCH;
    if (!attn_head_dim(p->D)) return KVQ_ERR_SHAPE;
    if (p->rows != T || p->H != H) return KVQ_ERR_MISMATCH;
    const int32_t G = p->group_size;
    int32_t gshift = 0;
    switch (p->format) {
        case KVQ_INT4:
            // powers of two: a K group holds whole 16-token sub-tiles, a V group whole 8-channel lanes
            if (!is_pow2(G) || (kind == KVQ_KEY ? G < 16 : (G < 8 || G < p->D / 16 || G > p->D)))
                return KVQ_ERR_GROUP;
            if (!aligned(p->meta0, 16) || !aligned(p->meta1, 16)) return KVQ_ERR_LAYOUT;
            gshift = log2i(G);
            break;
        case KVQ_NVFP4:
            if (!aligned(p->meta0, 16)) return KVQ_ERR_LAYOUT;
            gshift = 4;
            break;
        case KVQ_NVFP4_ROW:  // block-scale bytes read in pairs, FP32 row multipliers
            if (!aligned(p->meta0, 2) || !aligned(p->meta1, 4)) return KVQ_ERR_LAYOUT;
            break;
        case KVQ_FP8_ROW:  // FP32 row scales
            if (!aligned(p->meta0, 4)) return KVQ_ERR_LAYOUT;
            break;
        default:
            return KVQ_ERR_FORMAT;
    }
    if (!aligned(p->codes, 16)) return KVQ_ERR_LAYOUT;
    *out = AttnPlanes{p->codes, p->meta0, p->meta1, p->global_scale, gshift};
    return KVQ_OK;
}

}  // namespace

extern "C" {

const char* kvq_version(void) { return "kvq 0.1.0 gfx950"; }

const char* kvq_status_string(kvq_status s) {
    switch (s) {
        case KVQ_OK: return "ok";
        case KVQ_ERR_NULL: return "null pointer";
        case KVQ_ERR_SHAPE: return "bad shape";
        case KVQ_ERR_LAYOUT: return "bad layout";
        case KVQ_ERR_FORMAT: return "bad format or kind";
        case KVQ_ERR_GROUP: return "bad group size";
        case KVQ_ERR_DTYPE: return "unsupported dtype";
        case KVQ_ERR_MISMATCH: return "descriptor does not match tensor";
        case KVQ_ERR_HIP: return "HIP launch failed";
        case KVQ_ERR_WORKSPACE: return "missing workspace";
        case KVQ_ERR_SCRATCH: return "needs more scratch than the static buffer holds";
    }
    return "unknown status";
}

kvq_status kvq_storage_bytes(kvq_format format, kvq_kind kind, int32_t group_size, int64_t rows, int64_t H, int64_t D,
                             int32_t sparse, uint64_t* bytes) {
    if (!bytes) return KVQ_ERR_NULL;
    uint64_t s[KVQ_NUM_PLANES];
    kvq_status st = plane_sizes(format, kind, group_size, rows, H, D, sparse, s);
    if (st) return st;
    *bytes = s[0] + s[1] + s[2] + s[3] + s[4];
    return KVQ_OK;
}

kvq_status kvq_plane_bytes(kvq_format format, kvq_kind kind, int32_t group_size, int64_t rows, int64_t H, int64_t D,
                           int32_t sparse, uint64_t sizes[KVQ_NUM_PLANES]) {
    if (!sizes) return KVQ_ERR_NULL;
    return plane_sizes(format, kind, group_size, rows, H, D, sparse, sizes);
}

size_t kvq_workspace_bytes(void) { return kWorkspaceBytes; }

kvq_status kvq_pack(const kvq_tensor* x, kvq_kind kind, kvq_format format, int32_t group_size, kvq_packed* out,
                    void* workspace, hipStream_t stream) {
    kvq_status st = check_tensor(x);
    if (st) return st;
    return encode_common(view_of(x), nullptr, nullptr, 0, kind, format, group_size, out, workspace, stream);
}

kvq_status kvq_encode_residual(const kvq_tensor* cur, const kvq_tensor* prev, const int32_t* positions, int64_t M,
                               kvq_kind kind, kvq_format format, int32_t group_size, kvq_packed* out,
                               void* workspace, hipStream_t stream) {
    if (!prev) return KVQ_ERR_NULL;
    if (!positions && M != 0) return KVQ_ERR_SHAPE;
    kvq_status st = check_tensor(cur);
    if (st) return st;
    return encode_common(view_of(cur), prev, positions, M, kind, format, group_size, out, workspace, stream);
}

kvq_status kvq_unpack(const kvq_packed* p, const kvq_tensor* out, hipStream_t stream) {
    kvq_status st = check_packed(p);
    if (st) return st;
    if ((st = check_tensor(out))) return st;
    if (out->T != p->rows || out->H != p->H || out->D != p->D) return KVQ_ERR_MISMATCH;
    return decode_run(p, p->rows, nullptr, view_of(out), nullptr, nullptr, stream);
}

kvq_status kvq_decode_residual(const kvq_packed* r, const kvq_tensor* prev, const kvq_tensor* out,
                               hipStream_t stream) {
    kvq_status st = check_packed(r);
    if (st) return st;
    if ((st = check_tensor(prev))) return st;
    if ((st = check_tensor(out))) return st;
    if (prev->H != r->H || prev->D != r->D || prev->T != r->full_T) return KVQ_ERR_MISMATCH;
    if (out->T != prev->T || out->H != prev->H || out->D != prev->D) return KVQ_ERR_SHAPE;
    const bool sparse = r->positions != nullptr;
    if (!sparse && r->rows != r->full_T) return KVQ_ERR_MISMATCH;
    if (sparse && r->rows > r->full_T) return KVQ_ERR_MISMATCH;

    const bool same = out->data == prev->data && out->stride_t == prev->stride_t && out->stride_h == prev->stride_h;
    if (!same) {
        uintptr_t plo, phi, olo, ohi;
        view_span(prev, &plo, &phi);
        view_span(out, &olo, &ohi);
        if (plo < ohi && olo < phi) return KVQ_ERR_LAYOUT;  // partial overlap
    }
    if (sparse && !same && prev->T * prev->H * prev->D > 0) {
        // absent rows inherit prev: copy it whole, then decode the named rows over it
        const RowCopy c = make_row_copy(prev->data, prev->stride_t, prev->stride_h, out->data, out->stride_t,
                                        out->stride_h, prev->T, prev->H, prev->D, 0, 0, 0);
        if (launch_row_copy(c, stream) != hipSuccess) return KVQ_ERR_HIP;
    }
    return decode_run(r, r->rows, prev, view_of(out), r->positions, nullptr, stream);
}

kvq_status kvq_pack_paged(const kvq_paged* x, kvq_kind kind, kvq_format format, int32_t group_size,
                          int32_t page_local, kvq_packed* out, void* workspace, hipStream_t stream) {
    View v;
    kvq_status st = view_of_paged(x, &v);
    if (st) return st;
    if ((st = check_kind_format(kind, format))) return st;
    int32_t G = resolve_group(format, group_size);
    if ((st = check_group(format, G))) return st;
    if (page_local && kind == KVQ_KEY && x->page_size > 0) {
        // keep every KEY group inside one page: groups of min(G, page_size) tokens that tile it
        const int64_t S = x->page_size;
        if (format == KVQ_INT4) {
            if (G % S != 0 && S % G != 0) return KVQ_ERR_GROUP;
            if (S < G) G = (int32_t)S;
        } else if (format == KVQ_NVFP4) {
            if (S % 16 != 0) return KVQ_ERR_GROUP;
        }
    }
    return encode_common(v, nullptr, nullptr, 0, kind, format, G, out, workspace, stream);
}

kvq_status kvq_unpack_paged(const kvq_packed* p, const kvq_paged* out, hipStream_t stream) {
    kvq_status st = check_packed(p);
    if (st) return st;
    View v;
    if ((st = view_of_paged(out, &v))) return st;
    if (v.T != p->rows || v.H != p->H || v.D != p->D) return KVQ_ERR_MISMATCH;
    return decode_run(p, p->rows, nullptr, v, nullptr, nullptr, stream);
}

kvq_status kvq_store_rows(const kvq_tensor* rows, const int32_t* slots, kvq_packed* cache, hipStream_t stream) {
    kvq_status st = check_tensor(rows);
    if (st) return st;
    if ((st = check_packed(cache))) return st;
    if (!((cache->format == KVQ_INT4 && cache->kind == KVQ_VALUE) || row_format(cache->format))) return KVQ_ERR_FORMAT;
    if (cache->positions) return KVQ_ERR_MISMATCH;  // a sparse residual is not a slot cache
    if (rows->H != cache->H || rows->D != cache->D) return KVQ_ERR_MISMATCH;
    const int64_t N = rows->T;
    if (N > cache->rows) return KVQ_ERR_SHAPE;  // slots are distinct
    if (N * rows->H * rows->D == 0) return KVQ_OK;
    if (!slots) return KVQ_ERR_NULL;
    return encode_run(view_of(rows), nullptr, nullptr, N, cache->kind, cache->format, cache->group_size, cache,
                      nullptr, slots, stream);
}

kvq_status kvq_load_rows(const kvq_packed* cache, const int32_t* slots, const kvq_tensor* out, hipStream_t stream) {
    kvq_status st = check_packed(cache);
    if (st) return st;
    if ((st = check_tensor(out))) return st;
    if (out->H != cache->H || out->D != cache->D) return KVQ_ERR_MISMATCH;
    const int64_t N = out->T;
    if (N * out->H * out->D == 0) return KVQ_OK;
    if (!slots) return KVQ_ERR_NULL;
    if (cache->rows == 0) return KVQ_ERR_SHAPE;  // no slot to read
    return decode_run(cache, N, nullptr, view_of(out), nullptr, slots, stream);
}

kvq_status kvq_encode_window(const kvq_tensor* cur, const kvq_tensor* prev, int64_t sink, int64_t recent,
                             kvq_kind kind, kvq_format format, int32_t group_size, kvq_packed* out, void* window,
                             void* workspace, hipStream_t stream) {
    kvq_status st = check_tensor(cur);
    if (st) return st;
    if (sink < 0 || recent < 0) return KVQ_ERR_SHAPE;
    if (prev) {
        if ((st = check_tensor(prev))) return st;
        if (prev->T != cur->T || prev->H != cur->H || prev->D != cur->D) return KVQ_ERR_SHAPE;
    }
    int64_t ns, nr;
    window_split(cur->T, sink, recent, &ns, &nr);
    const int64_t T = cur->T, H = cur->H, D = cur->D, mid = T - ns - nr;
    if ((ns + nr) * H * D > 0 && !window) return KVQ_ERR_NULL;
    const kvq_tensor cm = row_slice(cur, ns, mid);
    kvq_tensor pm;
    if (prev) pm = row_slice(prev, ns, mid);
    // window rows [0, ns) <- cur rows [0, ns); window rows [ns, ns + nr) <- cur rows [T - nr, T)
    const RowCopy wc = make_row_copy(cur->data, cur->stride_t, cur->stride_h, window, H * D, D, ns + nr, H, D, ns,
                                     mid * cur->stride_t, 0);
    if ((st = encode_common(view_of(&cm), prev ? &pm : nullptr, nullptr, 0, kind, format, group_size, out, workspace,
                            stream, (ns + nr) * H * D > 0 ? &wc : nullptr)))
        return st;
    out->full_T = T;
    return KVQ_OK;
}

kvq_status kvq_decode_window(const kvq_packed* p, const void* window, int64_t sink, int64_t recent,
                             const kvq_tensor* prev, const kvq_tensor* out, hipStream_t stream) {
    kvq_status st = check_packed(p);
    if (st) return st;
    if ((st = check_tensor(out))) return st;
    if (sink < 0 || recent < 0) return KVQ_ERR_SHAPE;
    int64_t ns, nr;
    window_split(out->T, sink, recent, &ns, &nr);
    const int64_t T = out->T, H = out->H, D = out->D, mid = T - ns - nr;
    if (p->positions || p->rows != mid || p->full_T != T || p->H != H || p->D != D) return KVQ_ERR_MISMATCH;
    if ((ns + nr) * H * D > 0 && !window) return KVQ_ERR_NULL;
    if (prev) {
        if ((st = check_tensor(prev))) return st;
        if (prev->T != T || prev->H != H || prev->D != D) return KVQ_ERR_SHAPE;
        const bool same = out->data == prev->data && out->stride_t == prev->stride_t && out->stride_h == prev->stride_h;
        if (!same) {
            uintptr_t plo, phi, olo, ohi;
            view_span(prev, &plo, &phi);
            view_span(out, &olo, &ohi);
            if (plo < ohi && olo < phi) return KVQ_ERR_LAYOUT;  // partial overlap
        }
    }
    const kvq_tensor om = row_slice(out, ns, mid);
    kvq_tensor pm;
    if (prev) pm = row_slice(prev, ns, mid);
    // out rows [0, ns) <- window rows [0, ns); out rows [T - nr, T) <- window rows [ns, ns + nr)
    const RowCopy wc = make_row_copy(window, H * D, D, out->data, out->stride_t, out->stride_h, ns + nr, H, D, ns, 0,
                                     mid * out->stride_t);
    return decode_run(p, mid, prev ? &pm : nullptr, view_of(&om), nullptr, nullptr, stream,
                      (ns + nr) * H * D > 0 ? &wc : nullptr);
}

size_t kvq_attention_workspace_bytes(int64_t T, int64_t H, int64_t Hq, int64_t D) {
    if (T < 1 || H < 1 || Hq < H || Hq % H != 0 || T >= kMaxDim || H >= kMaxDim || Hq >= kMaxDim ||
        !attn_head_dim(D))
        return 0;
    return attn_workspace(T, H, Hq / H, D);
}

kvq_status kvq_decode_attention(const void* q, int64_t Hq, const kvq_packed* k, const kvq_packed* v,
                                const kvq_packed* k_res, const kvq_packed* v_res, float softmax_scale, float* out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!q || !out || !k || !v || !workspace) return KVQ_ERR_NULL;
    if ((k_res == nullptr) != (v_res == nullptr)) return KVQ_ERR_NULL;
    const int64_t T = k->rows, H = k->H;
    if (T < 1 || H < 1 || Hq < 1 || Hq % H != 0 || Hq >= kMaxDim || Hq / H > 16 * 65535) return KVQ_ERR_SHAPE;
    AttnArgs a;
    memset(&a, 0, sizeof a);
    kvq_status st = attn_operand(k, KVQ_KEY, T, H, &a.k);
    if (!st) st = attn_operand(v, KVQ_VALUE, T, H, &a.v);
    if (st) return st;
    if (k->format != v->format) return KVQ_ERR_FORMAT;
    if (v->D != k->D) return KVQ_ERR_MISMATCH;
    int rfmt = KVQ_ATTN_NO_RESIDUAL;
    if (k_res) {
        if ((st = attn_operand(k_res, KVQ_KEY, T, H, &a.rk))) return st;
        if ((st = attn_operand(v_res, KVQ_VALUE, T, H, &a.rv))) return st;
        if (k_res->format != v_res->format) return KVQ_ERR_FORMAT;
        if (k_res->D != k->D || v_res->D != k->D) return KVQ_ERR_MISMATCH;
        rfmt = k_res->format;
    }
    if (!aligned(q, 16) || !aligned(out, 4) || !aligned(workspace, 4)) return KVQ_ERR_LAYOUT;
    const int64_t rep = Hq / H;
    if (workspace_bytes < attn_workspace(T, H, rep, k->D)) return KVQ_ERR_WORKSPACE;
    a.q = static_cast<const uint16_t*>(q);
    a.T = T;
    a.H = (int32_t)H;
    a.rep = (int32_t)rep;
    a.D = (int32_t)k->D;
    a.n_split = attn_split_bound(T, H);  // the launcher chooses the split within this bound
    a.qscale = softmax_scale * 1.4426950408889634f;  // scores in log2 units: exp(x) = exp2(x log2 e)
    a.part_o = static_cast<float*>(workspace);      // the launcher places part_ml after its split
    a.out = out;
    return hip_status(launch_attention(k->format, rfmt, a, stream));
}

kvq_status kvq_nvfp4_global_scale(const kvq_tensor* cur, const kvq_tensor* prev, const int32_t* positions, int64_t M,
                                  float* global_scale, void* workspace, hipStream_t stream) {
    kvq_status st = check_tensor(cur);
    if (st) return st;
    const View v = view_of(cur);
    if (prev) {
        if ((st = check_tensor(prev))) return st;
        if (prev->T != v.T || prev->H != v.H || prev->D != v.D) return KVQ_ERR_SHAPE;
    }
    const bool sparse = positions != nullptr;
    if (M < 0 || (sparse && M > v.T) || (!sparse && M != 0)) return KVQ_ERR_SHAPE;
    if (!global_scale) return KVQ_ERR_NULL;
    if (!workspace) return KVQ_ERR_WORKSPACE;
    const int64_t rows = sparse ? M : v.T;
    if (rows * v.H * v.D == 0) return hip_status(launch_set_global(global_scale, 0x3F800000u, stream));  // g = 1
    kvq_packed planes;
    memset(&planes, 0, sizeof planes);
    planes.global_scale = global_scale;
    return encode_run(v, prev, positions, rows, KVQ_VALUE, KVQ_NVFP4, 16, &planes, workspace, nullptr, stream, true);
}

kvq_status kvq_decode_attention_noalloc(const void* q, int64_t Hq, const kvq_packed* k, const kvq_packed* v,
                                        const kvq_packed* k_res, const kvq_packed* v_res, float softmax_scale,
                                        float* out, hipStream_t stream) {
    if (!q || !out || !k || !v) return KVQ_ERR_NULL;
    // sizes the regular entry point rejects give 0 here and are rejected there, before any launch
    if (kvq_attention_workspace_bytes(k->rows, k->H, Hq, k->D) > KVQ_ATTN_STATIC_SCRATCH_BYTES)
        return KVQ_ERR_SCRATCH;
    void* ws = nullptr;
    kvq_status st = scratch_address(&ws);
    if (st) return st;
    return kvq_decode_attention(q, Hq, k, v, k_res, v_res, softmax_scale, out, ws, KVQ_ATTN_STATIC_SCRATCH_BYTES,
                                stream);
}

kvq_status kvq_validate_positions(const int32_t* positions, int64_t M, int64_t T, uint32_t* seen, int32_t* status,
                                  hipStream_t stream) {
    if (M < 0 || T < 0 || T >= kMaxDim || M >= kMaxDim) return KVQ_ERR_SHAPE;
    if (!status || (M > 0 && !positions) || (T > 0 && !seen)) return KVQ_ERR_NULL;
    return hip_status(launch_validate_positions(positions, M, T, seen, status, stream));
}

}  // extern "C"
