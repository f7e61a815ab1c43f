/*
 * kvq.h -- C ABI of the KV-cache quantization codec for AMD Instinct MI355X (gfx950).
 *
 * The library packs and unpacks one request/layer's logical [token, KV head, channel] K or V
 * tensor, and encodes/decodes cross-loop residuals against a reconstructed predecessor, in two
 * 4-bit per-tensor formats and two row formats (one FP32 scale per token and head). Paged
 * views [pages, page_size, H, D] are packed and unpacked directly, and row formats can be
 * written into, and read from, cache slots named by a device index array. All compute runs in
 * HIP kernels on the caller's stream.
 *
 * Sources (by page title and section):
 *   [PR166] vllm-rlt pull request #166, "INT4 KV packing/unpacking and cross-loop residual
 *           reconstruction": "Purpose" (API, formats, group axes, residual semantics), the
 *           first codec review (FP32 codes before FP16 metadata; 4.5 bits per element), the
 *           interface review (payload-only storage accounting; no device sync in validation).
 *   [PR408] FreeToken pull request #408, "feat(kvcache): add nvfp4 kv quantization":
 *           "Summary" (76 B per D=128 row; graph-safe writes with device-resident ids), the fp8
 *           commit (E4M3 codes with one FP32 scale per token and KV head; one fused
 *           quantize-and-scatter launch whose slot ids are a device tensor) and the nvfp4
 *           codec-port commit (low-nibble-first packing; quantize against the stored, rounded
 *           block scale; one FP32 row scale).
 *
 * Conventions shared by every entry point:
 *   - Tensors are bf16, logical [T, H, D] (token, KV head, channel), with channel stride 1 and
 *     arbitrary non-negative token/head strides in elements (e.g. K as a view into a fused QKV
 *     buffer). All data pointers are device pointers.
 *   - The library never allocates, frees or synchronizes. The caller allocates every buffer;
 *     kvq_plane_bytes gives the size of each packed plane.
 *   - Every call is asynchronous on `stream` and only enqueues kernels (no memset/memcpy
 *     nodes), so it may be captured into a HIP graph.
 *   - Host-detectable errors return a status before anything is enqueued. A failed launch
 *     returns KVQ_ERR_HIP. Data preconditions that only the device can see (finite inputs,
 *     positions in range and distinct) are not checked on the hot path; see
 *     kvq_validate_positions.
 *   - Sizes: rows, H, D < 2^31 and rows*H*D < 2^36 elements.
 */
#ifndef KVQ_H_
#define KVQ_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvq_status {
    KVQ_OK = 0,
    KVQ_ERR_NULL = 1,      /* a required pointer is NULL */
    KVQ_ERR_SHAPE = 2,     /* negative or too large size, or shapes that disagree */
    KVQ_ERR_LAYOUT = 3,    /* negative stride, or out/prev partially overlapping */
    KVQ_ERR_FORMAT = 4,    /* unknown format or kind, or a format the call does not take */
    KVQ_ERR_GROUP = 5,     /* group size invalid for the format (NVFP4 and NVFP4-row require
                              16, FP8-row 0) or for the page size */
    KVQ_ERR_DTYPE = 6,     /* tensor dtype other than bf16 */
    KVQ_ERR_MISMATCH = 7,  /* packed descriptor disagrees with the tensors it is used with */
    KVQ_ERR_HIP = 8,       /* a kernel launch failed */
    KVQ_ERR_WORKSPACE = 9, /* NVFP4 encode without a workspace, or a workspace too small */
    KVQ_ERR_SCRATCH = 10   /* the call needs more than the library's static scratch holds */
} kvq_status;

/* Group axis follows the kind ([PR166] "Purpose", third bullet): KEY groups run over token rows
 * for each (head, channel); VALUE groups run over channels for each (token, head). */
typedef enum kvq_kind { KVQ_KEY = 0, KVQ_VALUE = 1 } kvq_kind;

/* KVQ_INT4: affine groups, FP32 math, FP16 minimum and scale, default group size 64.
 * KVQ_NVFP4: E2M1 codes (nearest-even), one E4M3 scale per 16 values, one FP32 global
 * multiplier per encoded tensor; group size 16 only. ([PR166] "Purpose", second bullet.)
 * KVQ_NVFP4_ROW: as NVFP4, but the FP32 multiplier belongs to each (token, head) row
 * (g_row = 2688 / row amax) and the 16-value blocks run along channels for K and V alike, so
 * every row is encoded exactly like a one-row NVFP4 tensor: 76 B per D=128 row ([PR408]
 * "Summary", codec-port commit). Group size 16 only.
 * KVQ_FP8_ROW: one E4M3 code per element and one FP32 scale per (token, head) row,
 * scale = row amax / 448, code = e4m3(min(|x / scale|, 448)) with the sign of x, decoded as
 * code * scale ([PR408] fp8 commit). Group size 0 only (no sub-row groups).
 * The kind does not change the layout of the two row formats. */
typedef enum kvq_format { KVQ_INT4 = 0, KVQ_NVFP4 = 1, KVQ_NVFP4_ROW = 2, KVQ_FP8_ROW = 3 } kvq_format;

typedef enum kvq_dtype { KVQ_BF16 = 0 } kvq_dtype;

/* A strided bf16 view: element (t, h, d) is at data + t*stride_t + h*stride_h + d (elements). */
typedef struct kvq_tensor {
    void* data;
    int32_t dtype; /* kvq_dtype */
    int32_t reserved;
    int64_t T, H, D;
    int64_t stride_t, stride_h;
} kvq_tensor;

/* A paged bf16 view [pages, page_size, H, D] ([PR166] interface review, item 3): element
 * (p, s, h, d) is at data + p*stride_page + s*stride_slot + h*stride_h + d (elements). Its
 * logical token order is page-major: token p*page_size + s. When stride_page is not
 * page_size*stride_slot (pages padded, or K and V interleaved per page) page_size must be a
 * power of two. */
typedef struct kvq_paged {
    void* data;
    int32_t dtype; /* kvq_dtype */
    int32_t reserved;
    int64_t pages, page_size, H, D;
    int64_t stride_page, stride_slot, stride_h;
} kvq_paged;

/* One encoded tensor ([PR166] "Purpose", first bullet: packed objects carry format, axis and
 * group size). The caller owns every plane; the library fills the scalar fields on encode.
 *   codes        [rows, H, ceil(D/2)] u8: channel 2j in the low nibble, 2j+1 in the high
 *                nibble ([PR408] codec-port commit: low first); an odd D leaves the last
 *                high nibble 0. FP8-row: [rows, H, D], one E4M3 byte per element.
 *   meta0        INT4: f16 group minimums; NVFP4: E4M3 block scales (u8), shape KEY
 *                [ceil(rows/G), H, D], VALUE [rows, H, ceil(D/G)]; NVFP4-row: E4M3 block
 *                scales [rows, H, ceil(D/16)] (u8); FP8-row: FP32 row scales [rows, H].
 *   meta1        INT4: f16 group scales (shape as meta0); NVFP4-row: FP32 row multipliers
 *                g_row [rows, H]; NVFP4 and FP8-row: unused (NULL).
 *   global_scale NVFP4: one float, the encoding multiplier g (decode scale = block/g); the
 *                other formats: unused (NULL).
 *   positions    sparse residual: the owned int32 copy of the position map, [rows]. A non-NULL
 *                pointer is what marks a residual sparse; with rows == 0 it is not read.
 *   rows         T for a dense tensor, M for a sparse residual; full_T is the row count of the
 *                tensor it reconstructs (== rows when dense). */
typedef struct kvq_packed {
    int32_t format;     /* kvq_format */
    int32_t kind;       /* kvq_kind */
    int32_t group_size;
    int32_t dtype;      /* dtype of the tensor it decodes to (kvq_dtype) */
    int64_t rows, H, D;
    int64_t full_T;
    uint8_t* codes;
    void* meta0;
    void* meta1;
    float* global_scale;
    int32_t* positions;
} kvq_packed;

/* Plane indices for kvq_plane_bytes. */
enum { KVQ_PLANE_CODES = 0, KVQ_PLANE_META0 = 1, KVQ_PLANE_META1 = 2, KVQ_PLANE_GLOBAL = 3,
       KVQ_PLANE_POSITIONS = 4, KVQ_NUM_PLANES = 5 };

/* Library version string (static storage). */
const char* kvq_version(void);

/* Human-readable name of a status code (static storage). */
const char* kvq_status_string(kvq_status status);

/* Exact payload bytes of one encoded tensor ([PR166] interface review: payload only, no
 * allocator slack, no decode scratch): rows*H*ceil(D/2) code bytes (rows*H*D for FP8-row)
 * + 4 B per INT4 group, or 1 B per NVFP4 / NVFP4-row block, + 4 B global scale (NVFP4) or 4 B
 * per (row, head) (NVFP4-row, FP8-row) + 4 B per row of an owned position map (sparse != 0).
 * group_size 0 selects the format default. Host-only; writes *bytes.
 * Errors: KVQ_ERR_NULL, KVQ_ERR_SHAPE, KVQ_ERR_FORMAT, KVQ_ERR_GROUP. */
kvq_status kvq_storage_bytes(kvq_format format, kvq_kind kind, int32_t group_size, int64_t rows, int64_t H,
                             int64_t D, int32_t sparse, uint64_t* bytes);

/* Per-plane byte sizes (sizes[KVQ_NUM_PLANES], indexed by KVQ_PLANE_*); they sum to
 * kvq_storage_bytes. Host-only. Same errors as kvq_storage_bytes. */
kvq_status kvq_plane_bytes(kvq_format format, kvq_kind kind, int32_t group_size, int64_t rows, int64_t H,
                           int64_t D, int32_t sparse, uint64_t sizes[KVQ_NUM_PLANES]);

/* Bytes of device workspace an NVFP4 encode needs (per-block partial maxima of the tensor-amax
 * pass). No initialization is needed; every call overwrites what it reads. Calls that may run
 * concurrently need distinct workspaces. */
size_t kvq_workspace_bytes(void);

/* pack_kv ([PR166] "Purpose" usage example, first line): encode x into *out.
 * The caller sets out->codes, out->meta0, out->meta1 (INT4), out->global_scale (NVFP4); the
 * library sets the scalar fields and out->positions = NULL. group_size 0 = format default
 * (INT4 64, NVFP4 16). NVFP4 needs `workspace` (kvq_workspace_bytes); INT4 ignores it.
 * The NVFP4 global multiplier is recomputed on every call ([PR166] "Purpose", paragraph after
 * the example). Errors: NULL, SHAPE, LAYOUT, FORMAT, GROUP, DTYPE, WORKSPACE, HIP. */
kvq_status kvq_pack(const kvq_tensor* x, kvq_kind kind, kvq_format format, int32_t group_size, kvq_packed* out,
                    void* workspace, hipStream_t stream);

/* unpack_kv ([PR166] "Purpose" usage example, second line): decode *p into the bf16 view
 * `out` of shape [p->rows, p->H, p->D]. Errors: NULL, SHAPE, LAYOUT, FORMAT, GROUP, DTYPE,
 * MISMATCH, HIP. */
kvq_status kvq_unpack(const kvq_packed* p, const kvq_tensor* out, hipStream_t stream);

/* encode_residual ([PR166] "Purpose", fourth bullet and usage example, third line): encode
 * cur - prev, subtracted in the input dtype (one binary32 subtraction rounded to bf16), where
 * prev is the reconstructed predecessor. Dense when positions == NULL (rows = T); sparse when
 * positions is non-NULL: a device array of M distinct row indices in [0, T) (not read when
 * M == 0, but still non-NULL, as is out->positions). Compact row i is
 * cur[positions[i]] - prev[positions[i]], KEY groups follow compact row order, and the
 * residual keeps its own copy of the map in out->positions (caller-allocated, M int32).
 * The residual's format/kind/group size are independent of how prev was produced (mixed-format
 * chains). Same workspace rule and errors as kvq_pack. */
kvq_status kvq_encode_residual(const kvq_tensor* cur, const kvq_tensor* prev, const int32_t* positions, int64_t M,
                               kvq_kind kind, kvq_format format, int32_t group_size, kvq_packed* out,
                               void* workspace, hipStream_t stream);

/* decode_residual ([PR166] "Purpose", fourth bullet and usage example, fourth line):
 * out = prev + unpack(r), both in the input dtype (the decoded residual is rounded to bf16,
 * then the binary32 sum is rounded to bf16). Sparse: rows not in r->positions are copied from
 * prev bit for bit (absent rows inherit the predecessor). prev and out are [r->full_T, H, D];
 * out may be exactly prev (same data and strides: in place, only kept rows are written), but
 * must not partially overlap it. Errors: NULL, SHAPE, LAYOUT, FORMAT, GROUP, DTYPE, MISMATCH,
 * HIP. */
kvq_status kvq_decode_residual(const kvq_packed* r, const kvq_tensor* prev, const kvq_tensor* out,
                               hipStream_t stream);

/* pack_paged ([PR166] interface review, item 3, and the stacked-PR follow-up): encode the
 * paged view x in its page-major token order into *out (rows = pages*page_size, as kvq_pack
 * would for that token sequence). page_local != 0 keeps every KEY group of INT4 and NVFP4
 * inside one page ([PR166] first review, "Group ownership vs 16-token pages"): INT4 then uses
 * groups of min(G, page_size) tokens, which needs G and page_size to divide one another, and
 * records that size in out->group_size; NVFP4 needs page_size % 16 == 0. VALUE groups and the
 * row formats are page-local already. The NVFP4 multiplier is one per call (all pages).
 * Workspace and errors as kvq_pack; KVQ_ERR_GROUP for sizes page-local grouping cannot take,
 * KVQ_ERR_LAYOUT for a padded page stride with a non-power-of-two page size. */
kvq_status kvq_pack_paged(const kvq_paged* x, kvq_kind kind, kvq_format format, int32_t group_size,
                          int32_t page_local, kvq_packed* out, void* workspace, hipStream_t stream);

/* unpack_paged: decode *p (rows = pages*page_size) into the paged bf16 view `out`.
 * Errors as kvq_unpack. */
kvq_status kvq_unpack_paged(const kvq_packed* p, const kvq_paged* out, hipStream_t stream);

/* Quantize-and-scatter into cache slots ([PR408] fp8 commit: one launch, slot ids in device
 * memory, so it can sit inside a captured graph). Row i of `rows` ([N, H, D], N = rows->T) is
 * encoded exactly as kvq_pack would encode it among those N rows, and its codes and row
 * metadata are written into packed row slots[i] of `cache` (a packed tensor of cache->rows
 * slots whose format, kind and group size are taken from the descriptor). Every other slot is
 * left untouched. Only formats whose rows are encoded on their own qualify: INT4 VALUE,
 * NVFP4-row and FP8-row (KVQ_ERR_FORMAT otherwise). `slots`: device int32 [N], distinct and in
 * [0, cache->rows) (precondition, not checked; kvq_validate_positions can check it with
 * T = cache->rows). Errors: NULL, SHAPE, LAYOUT, FORMAT, GROUP, DTYPE, MISMATCH, HIP. */
kvq_status kvq_store_rows(const kvq_tensor* rows, const int32_t* slots, kvq_packed* cache, hipStream_t stream);

/* Gather-and-decode: output row i ([N, H, D] view `out`, N = out->T) is the decoded packed row
 * slots[i] of `cache`, for every format (a KEY row of INT4 or NVFP4 decodes with the metadata
 * of its token group, slots[i] / G). `slots`: device int32 [N] in [0, cache->rows)
 * (precondition, not checked). Errors: NULL, SHAPE, LAYOUT, FORMAT, GROUP, DTYPE, MISMATCH,
 * HIP. */
kvq_status kvq_load_rows(const kvq_packed* cache, const int32_t* slots, const kvq_tensor* out, hipStream_t stream);

/* Encode with a BF16 protected window ([PR166] "Real Ouro numerical comparison": the first 4
 * and latest 16 tokens kept in BF16, protected rows left out of the quantized payload and
 * passed through bitwise). Of cur's T rows, n_sink = min(sink, T) front rows and
 * n_recent = min(recent, T - n_sink) end rows are copied raw into `window` (device bf16,
 * contiguous [n_sink + n_recent, H, D], front rows first); the middle rows are encoded into
 * *out as a tensor of their own (out->rows = T - n_sink - n_recent, out->full_T = T): packed
 * when prev == NULL, as the residual bf16(cur - prev) otherwise (the window still holds cur,
 * so protected rows reconstruct exactly). The middle encode is the same as kvq_encode_residual
 * with positions = [n_sink, T - n_recent). The row copy runs in the encode launch, so `window`
 * must not overlap cur, prev or the planes. Workspace rule and errors as kvq_pack /
 * kvq_encode_residual; KVQ_ERR_SHAPE for a negative window. */
kvq_status kvq_encode_window(const kvq_tensor* cur, const kvq_tensor* prev, int64_t sink, int64_t recent,
                             kvq_kind kind, kvq_format format, int32_t group_size, kvq_packed* out, void* window,
                             void* workspace, hipStream_t stream);

/* Decode a windowed tensor into `out` ([T, H, D], T = p->full_T): the middle rows are decoded
 * (prev == NULL) or added to prev in the input dtype (residual), the protected rows are copied
 * bit for bit from `window` in the same launch (window must not overlap out or prev). out may be
 * exactly prev. Errors as kvq_unpack / kvq_decode_residual. */
kvq_status kvq_decode_window(const kvq_packed* p, const void* window, int64_t sink, int64_t recent,
                             const kvq_tensor* prev, const kvq_tensor* out, hipStream_t stream);

/* The NVFP4 global encoding multiplier alone ([PR166] "Purpose", second bullet: one FP32
 * multiplier per encoded tensor, recomputed on every encoding call): g = fl(2688 / amax), with
 * amax = max |x| over exactly the rows an NVFP4 kvq_pack (prev == NULL) or kvq_encode_residual
 * of the same arguments would encode -- the plain tensor, the residual rows bf16(cur - prev), or
 * the M rows gathered by `positions` -- and g = 1 when amax is 0 or there are no rows, FLT_MAX
 * if the quotient overflows. Writes the same bits that encode stores in its global_scale plane.
 * Useful on its own to combine the multipliers of several shards (a max over their amaxes).
 *   cur, prev     as in kvq_encode_residual (prev may be NULL: plain tensor)
 *   positions, M  as in kvq_encode_residual (NULL and 0 for dense)
 *   global_scale  device float, written
 *   workspace     kvq_workspace_bytes() of device memory (per-block partial maxima)
 * Errors: NULL, SHAPE, LAYOUT, DTYPE, WORKSPACE, HIP. */
kvq_status kvq_nvfp4_global_scale(const kvq_tensor* cur, const kvq_tensor* prev, const int32_t* positions, int64_t M,
                                  float* global_scale, void* workspace, hipStream_t stream);

/* Bytes of device workspace kvq_decode_attention needs for T cached tokens, H KV heads, Hq
 * query heads and head_dim D (per-block partial maxima, sums and unnormalized outputs); 0 for
 * invalid sizes. No initialization is needed. Calls that may run concurrently need distinct
 * workspaces. */
size_t kvq_attention_workspace_bytes(int64_t T, int64_t H, int64_t Hq, int64_t D);

/* Decode attention that reads the packed cache directly ([PR166] reviews of the codec: the
 * hot-path option of dequantizing to BF16 in registers and keeping a BF16 matrix multiply, and
 * the comparison after fusing dequantization and residual reconstruction into attention). One
 * query token per query head: out[hq, :] = softmax(scale * q[hq] . K[:, hk]^T) V[:, hk] over
 * all T = k->rows cached tokens, with KV head hk = hq / (Hq / H). K and V are reconstructed in
 * registers exactly as kvq_unpack decodes them, or, with k_res and v_res, as kvq_decode_residual
 * of those dense residuals on top (both or neither). Scores and softmax run in FP32, the
 * probabilities are rounded to bf16 for the PV product (bf16 MFMA, FP32 accumulation), so the
 * output matches float64 attention over the decoded cache to within about 2^-9 of max |V|.
 *   q        device bf16 [Hq, D], contiguous, 16-byte aligned
 *   k, v     packed KEY / VALUE tensors of one layer: rows = T >= 1, the same H, the same
 *            head_dim D of 64, 128 or 256, dense, the same format (any of the four); INT4 groups
 *            a power of two, at least 16 tokens for K and from max(8, D/16) to D channels for V;
 *            code planes 16-byte aligned, metadata planes aligned to their element size (INT4
 *            and NVFP4: 16 bytes)
 *   k_res, v_res  optional dense residuals of the same shape (formats may differ from k, v)
 *   Hq       a multiple of H (query heads per KV head beyond 16 run as several 16-row tiles, each
 *            reading the KV head's cache)
 *   out      device float [Hq, D]
 *   workspace  device memory of at least kvq_attention_workspace_bytes(T, H, Hq, D) bytes
 * Errors: NULL, SHAPE, LAYOUT, FORMAT, GROUP, MISMATCH, WORKSPACE, HIP. */
kvq_status kvq_decode_attention(const void* q, int64_t Hq, const kvq_packed* k, const kvq_packed* v,
                                const kvq_packed* k_res, const kvq_packed* v_res, float softmax_scale, float* out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* kvq_decode_attention without a workspace argument and without any allocation, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc. Same arguments, results (bit for bit: the same kernels and
 * split), layouts and errors as kvq_decode_attention; the per-block partials go to a static
 * device buffer of 32 MiB (KVQ_ATTN_STATIC_SCRATCH_BYTES) that the library holds on every GPU it
 * runs on until the process ends. A call whose kvq_attention_workspace_bytes(T, H, Hq, D)
 * exceeds 32 MiB returns KVQ_ERR_SCRATCH before launching anything (head_dim 64 or 128 with
 * Hq / H <= 16, and head_dim 256 with Hq / H <= 8, always fit). The buffer needs no
 * initialization. All calls on one GPU share it: calls that overlap in time on the same GPU
 * (concurrent streams, or several threads) race and must be serialized by the caller.
 * Errors: as kvq_decode_attention, plus SCRATCH; HIP also if the buffer's address cannot be
 * obtained on the current device. */
kvq_status kvq_decode_attention_noalloc(const void* q, int64_t Hq, const kvq_packed* k, const kvq_packed* v,
                                        const kvq_packed* k_res, const kvq_packed* v_res, float softmax_scale,
                                        float* out, hipStream_t stream);

/* Opt-in device-side check of a position map (the codec page's interface review asks that
 * validation never force a host sync). Writes *status (device int32): 0 = valid, bit 0 = some
 * position outside [0, T), bit 1 = some position repeated. `seen` is a device buffer of
 * ceil(T/32) uint32 words, overwritten. Nothing is read back on the host.
 * Errors: NULL, SHAPE, HIP. */
kvq_status kvq_validate_positions(const int32_t* positions, int64_t M, int64_t T, uint32_t* seen,
                                  int32_t* status, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H_ */
