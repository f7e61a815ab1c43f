/*
 * kvq_oracle.c -- plain CPU oracle of the KV-cache quantization codec.
 *
 * TEST INFRASTRUCTURE. This file is the slow, scalar, obviously-correct statement of what the
 * codec computes. Only the test suite, the smoke check and the CPU-baseline leg of the bench may
 * load it. The product path (the HIP library) never links, loads or calls it, and the two share
 * no code, headers, tables or helpers.
 *
 * Sources (cited by page title and section):
 *   [PR166]  vllm-rlt pull request #166, "INT4 KV packing/unpacking and cross-loop residual
 *            reconstruction" (codec page). Sections used: "Purpose" (bullets 1-4 and the
 *            four-line usage example), "Test Plan" (the scalar-oracle category list),
 *            "Unfused codec timing" (group counts), the first codec review by 0z5a (storage
 *            bits per element, FP32-before-FP16 metadata rule), and the second review
 *            ("Sharing one KV-quantization interface": storage_bytes counts payload only).
 *   [PR408]  FreeToken pull request #408, "feat(kvcache): add nvfp4 kv quantization".
 *            Sections used: "Summary" (76 B per D=128 row; packed E2M1, one E4M3 scale per 16
 *            values, one FP32 row scale per token and KV head), the fp8 commit message (one
 *            FP32 symmetric scale per (token, KV head) row; fused quantize + scatter with slot
 *            ids) and the nvfp4 codec-port commit message (nibbles low first, quantize against
 *            the stored block scale, 64 + 8 + 4 = 76 B).
 *
 * Numerics. Every floating-point step is one IEEE-754 binary32 operation rounded to nearest
 * even; build with -O2 -ffp-contract=off (no fused multiply-add) and without -ffast-math.
 * Conversions to bf16, f16 and E4M3 are written from their definition (nearest representable
 * value of the target format, ties to the even significand, gradual underflow) using exact
 * double arithmetic, not with bit tricks.
 *
 * Readings taken where the pages are silent are marked READING below.
 *
 * Threads. Built plainly, this is single-threaded C. Built with -fopenmp (a second library),
 * the loops over independent groups and rows run on all threads; every group is still
 * computed by the same statements, and the tensor amax is a max of per-thread maxima (exact
 * and order-independent), so both builds give the same bits.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define KVQO_KEY 0
#define KVQO_VALUE 1
#define KVQO_INT4 0
#define KVQO_NVFP4 1
#define KVQO_NVFP4_ROW 2
#define KVQO_FP8_ROW 3

/* Threads the loops below run on: 1 for the plain build. */
int kvq_oracle_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* status codes (mirrors nothing; the oracle has its own) */
#define KVQO_OK 0
#define KVQO_BAD_ARG 1
#define KVQO_NOMEM 2

/* ------------------------------------------------------------------------------------------ */
/* Scalar conversions, from the definitions of the formats.                                   */
/* ------------------------------------------------------------------------------------------ */

float kvq_oracle_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16; /* bf16 is the upper half of a binary32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static uint32_t f32_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

/* Nearest value of a binary format with `p` significand bits (leading one included) and
 * smallest normal exponent `emin`, with gradual underflow below 2^emin and ties to the even
 * significand. The input is a finite binary32 widened to double; the scaling by a power of two
 * is exact in double, and nearbyint rounds half to even in the default rounding mode.
 * Overflow is left to the caller (the result may exceed the format's largest finite value). */
static double round_to_binary_format(double x, int p, int emin) {
    if (x == 0.0) return x;
    int e;
    (void)frexp(fabs(x), &e); /* |x| = m * 2^e with m in [0.5, 1): leading bit has weight 2^(e-1) */
    int lead = e - 1;
    if (lead < emin) lead = emin; /* below the normal range the quantum stays 2^(emin-p+1) */
    double quantum = ldexp(1.0, lead - (p - 1));
    double k = nearbyint(x / quantum);
    return k * quantum;
}

/* binary32 -> bfloat16 (8 significand bits, emin -126, largest finite (2-2^-7)*2^127). */
uint16_t kvq_oracle_f32_to_bf16(float x) {
    double r = round_to_binary_format((double)x, 8, -126);
    const double max_bf16 = ldexp(2.0 - ldexp(1.0, -7), 127);
    float rf;
    if (fabs(r) > max_bf16)
        rf = (r > 0) ? INFINITY : -INFINITY;
    else
        rf = (float)r; /* exact: r is a bf16 value */
    if (x == 0.0f) rf = x; /* keep the sign of zero */
    if (r == 0.0 && signbit(x)) rf = -0.0f;
    return (uint16_t)(f32_bits(rf) >> 16);
}

/* binary32 -> binary16 (11 significand bits, emin -14, largest finite 65504, overflow to inf). */
uint16_t kvq_oracle_f32_to_f16(float x) {
    double r = round_to_binary_format((double)x, 11, -14);
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(r);
    if (a > 65504.0) return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);
    int lead = e - 1;
    if (lead < -14) { /* subnormal: value = M * 2^-24 */
        uint16_t m = (uint16_t)(a / ldexp(1.0, -24));
        return (uint16_t)(sign | m);
    }
    uint16_t E = (uint16_t)(lead + 15);
    uint16_t M = (uint16_t)((a / ldexp(1.0, lead) - 1.0) * 1024.0);
    return (uint16_t)(sign | (E << 10) | M);
}

float kvq_oracle_f16_to_f32(uint16_t h) {
    int sign = (h >> 15) & 1;
    int E = (h >> 10) & 0x1F;
    int M = h & 0x3FF;
    double v;
    if (E == 0)
        v = M * ldexp(1.0, -24);
    else if (E == 31)
        v = (M == 0) ? INFINITY : NAN;
    else
        v = (1.0 + M / 1024.0) * ldexp(1.0, E - 15);
    return (float)(sign ? -v : v);
}

/* binary32 -> E4M3 "fn" (4 significand bits, bias 7 so emin -6, subnormals M*2^-9, no
 * infinity, largest finite 448 = 1.75*2^8). Callers only pass values in [0, 448], so the
 * rounded result never exceeds 448 (the next candidate above 448 would be 480). */
uint8_t kvq_oracle_f32_to_e4m3(float x) {
    double r = round_to_binary_format((double)x, 4, -6);
    uint8_t sign = signbit(x) ? 0x80u : 0u;
    double a = fabs(r);
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);
    int lead = e - 1;
    if (lead < -6) return (uint8_t)(sign | (uint8_t)(a / ldexp(1.0, -9)));
    uint8_t E = (uint8_t)(lead + 7);
    uint8_t M = (uint8_t)((a / ldexp(1.0, lead) - 1.0) * 8.0);
    return (uint8_t)(sign | (E << 3) | M);
}

float kvq_oracle_e4m3_to_f32(uint8_t b) {
    int sign = (b >> 7) & 1;
    int E = (b >> 3) & 0xF;
    int M = b & 7;
    double v;
    if (E == 15 && M == 7)
        v = NAN; /* the only non-finite pattern of E4M3fn */
    else if (E == 0)
        v = M * ldexp(1.0, -9);
    else
        v = (1.0 + M / 8.0) * ldexp(1.0, E - 7);
    return (float)(sign ? -v : v);
}

/* The eight non-negative E2M1 magnitudes, by 3-bit code (exponent bits 2..1, mantissa bit 0,
 * bias 1, subnormal 0.5). */
static const float E2M1_GRID[8] = {0.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f, 4.0f, 6.0f};

float kvq_oracle_e2m1_to_f32(uint8_t code) {
    float v = E2M1_GRID[code & 7];
    return (code & 8) ? -v : v;
}

/* Magnitude code of the E2M1 value nearest to m (0 <= m <= 6), ties to the even code, found by
 * scanning the grid. [PR166] "Purpose": E2M1 codes are nearest-even. */
static uint8_t e2m1_nearest_code(float m) {
    int best = 0;
    double best_d = fabs((double)m - (double)E2M1_GRID[0]);
    for (int i = 1; i < 8; ++i) {
        double d = fabs((double)m - (double)E2M1_GRID[i]);
        if (d < best_d || (d == best_d && (i % 2) == 0 && (best % 2) != 0)) {
            best = i;
            best_d = d;
        }
    }
    return (uint8_t)best;
}

/* Full E2M1 encoding of a scaled value q whose sign is taken from the unscaled element x:
 * clamp |q| to the largest magnitude 6, round to nearest (ties even), sign bit = signbit(x).
 * READING: signed zero keeps its sign (IEEE conversion semantics): -0.0 -> code 0x8. */
uint8_t kvq_oracle_e2m1_encode(float q, float x_for_sign) {
    float m = fabsf(q);
    if (m > 6.0f) m = 6.0f;
    uint8_t c = e2m1_nearest_code(m);
    return (uint8_t)(c | (signbit(x_for_sign) ? 8u : 0u));
}

/* IEEE totalOrder restricted to finite values: -0 sorts below +0. READING: the pages do not say
 * how a group whose extreme is a signed zero picks that zero; with totalOrder the result does
 * not depend on scan order. */
static int total_less(float a, float b) {
    if (a < b) return 1;
    if (a == b && signbit(a) && !signbit(b)) return 1;
    return 0;
}

/* ------------------------------------------------------------------------------------------ */
/* Shapes and storage                                                                          */
/* ------------------------------------------------------------------------------------------ */

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* Number of metadata groups. [PR166] "Purpose", third bullet: K is grouped over token rows per
 * (head, channel) and V over channels per (token, head); the last group may be partial. */
static int64_t n_groups(int kind, int32_t G, int64_t rows, int64_t H, int64_t D) {
    if (kind == KVQO_KEY) return ceil_div(rows, G) * H * D;
    return rows * H * ceil_div(D, G);
}

/* Exact payload bytes. [PR166] second review: storage counts payload only (codes, metadata,
 * the FP32 tensor scale and an owned position map), no allocator slack and no decode scratch.
 * INT4 metadata is an FP16 minimum and an FP16 scale per group ([PR166] "Purpose", second
 * bullet); NVFP4 metadata is one E4M3 byte per 16 values plus one FP32 scale per tensor.
 * The row formats ([PR408]) carry one FP32 scale per (token, head) row: NVFP4-row adds one
 * E4M3 byte per 16 channels, FP8-row stores one E4M3 byte per element. */
int64_t kvq_oracle_storage_bytes(int format, int kind, int32_t G, int64_t rows, int64_t H, int64_t D,
                                 int sparse) {
    if (rows < 0 || H < 0 || D < 0) return -1;
    int64_t pos = sparse ? 4 * rows : 0;
    switch (format) {
        case KVQO_INT4:
            if (G < 1) return -1;
            return rows * H * ceil_div(D, 2) + 4 * n_groups(kind, G, rows, H, D) + pos;
        case KVQO_NVFP4:
            if (G != 16) return -1;
            return rows * H * ceil_div(D, 2) + n_groups(kind, 16, rows, H, D) + 4 + pos;
        case KVQO_NVFP4_ROW:
            if (G != 16) return -1;
            return rows * H * (ceil_div(D, 2) + ceil_div(D, 16) + 4) + pos;
        case KVQO_FP8_ROW:
            if (G != 0) return -1;
            return rows * H * (D + 4) + pos;
        default:
            return -1;
    }
}

/* ------------------------------------------------------------------------------------------ */
/* Input materialization: the rows that are encoded, as float32 holding bf16 values.          */
/* ------------------------------------------------------------------------------------------ */

/* Element (t, h, d) of a strided bf16 view: channel stride 1, token stride st, head stride sh. */
static float load_bf16(const uint16_t* base, int64_t st, int64_t sh, int64_t t, int64_t h, int64_t d) {
    return kvq_oracle_bf16_to_f32(base[t * st + h * sh + d]);
}

/* Rows to encode. Plain pack: X itself. Residual ([PR166] "Purpose", fourth bullet): the
 * difference current - previous taken in the input dtype, i.e. one binary32 subtraction
 * rounded to bf16, where previous is the reconstructed predecessor. Sparse residual: compact
 * row i is source row positions[i] (READING: the given order is the compact row order). */
static void materialize(const uint16_t* cur, int64_t cst, int64_t csh, const uint16_t* prev, int64_t pst,
                        int64_t psh, const int32_t* positions, int64_t rows, int64_t H, int64_t D,
                        float* dense) {
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        int64_t t = positions ? (int64_t)positions[i] : i;
        for (int64_t h = 0; h < H; ++h)
            for (int64_t d = 0; d < D; ++d) {
                float c = load_bf16(cur, cst, csh, t, h, d);
                float v = c;
                if (prev) {
                    float p = load_bf16(prev, pst, psh, t, h, d);
                    float diff = c - p;
                    v = kvq_oracle_bf16_to_f32(kvq_oracle_f32_to_bf16(diff));
                }
                dense[(i * H + h) * D + d] = v;
            }
    }
}

/* Pack per-element 4-bit codes into bytes: byte j of row (t, h) holds channel 2j in the low
 * nibble and channel 2j+1 in the high nibble; an odd last channel leaves the high nibble 0.
 * READING: [PR166] only names the upstream nibble order; [PR408]'s codec-port commit states
 * "low first", which is taken for both formats. */
static void pack_nibbles(const uint8_t* c, int64_t rows, int64_t H, int64_t D, uint8_t* codes) {
    int64_t Dp = ceil_div(D, 2);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < rows; ++t)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t j = 0; j < Dp; ++j) {
                int64_t d0 = 2 * j, d1 = 2 * j + 1;
                uint8_t lo = c[(t * H + h) * D + d0] & 0xF;
                uint8_t hi = (d1 < D) ? (c[(t * H + h) * D + d1] & 0xF) : 0;
                codes[(t * H + h) * Dp + j] = (uint8_t)(lo | (hi << 4));
            }
}

static uint8_t nibble_at(const uint8_t* codes, int64_t H, int64_t D, int64_t t, int64_t h, int64_t d) {
    int64_t Dp = ceil_div(D, 2);
    uint8_t byte = codes[(t * H + h) * Dp + d / 2];
    return (d % 2 == 0) ? (byte & 0xF) : (byte >> 4);
}

/* Visit every group: calls f(ctx, member count, member flat indices). Member indices are into
 * the dense [rows, H, D] array; `gid` is the flat index into the metadata plane, whose shape is
 * [ceil(rows/G), H, D] for K and [rows, H, ceil(D/G)] for V. */
typedef void (*group_fn)(void* ctx, int64_t gid, int64_t n, const int64_t* idx);

static void for_each_group(int kind, int32_t G, int64_t rows, int64_t H, int64_t D, group_fn f, void* ctx) {
    int64_t ngroups = n_groups(kind, G, rows, H, D);
    int64_t nc = ceil_div(D, G);
#pragma omp parallel
    {
        int64_t* idx = (int64_t*)malloc(sizeof(int64_t) * (size_t)G);
#pragma omp for schedule(static)
        for (int64_t gid = 0; gid < ngroups; ++gid) {
            int64_t n = 0;
            if (kind == KVQO_KEY) { /* gid = (b * H + h) * D + d: tokens [bG, min(rows, (b+1)G)) */
                int64_t b = gid / (H * D), h = (gid / D) % H, d = gid % D;
                for (int64_t t = b * G; t < rows && t < (b + 1) * G; ++t) idx[n++] = (t * H + h) * D + d;
            } else { /* gid = (t * H + h) * nc + c: channels [cG, min(D, (c+1)G)) */
                int64_t t = gid / (H * nc), h = (gid / nc) % H, c = gid % nc;
                for (int64_t d = c * G; d < D && d < (c + 1) * G; ++d) idx[n++] = (t * H + h) * D + d;
            }
            f(ctx, gid, n, idx);
        }
        free(idx);
    }
}

/* ------------------------------------------------------------------------------------------ */
/* INT4 affine groups                                                                         */
/* ------------------------------------------------------------------------------------------ */

typedef struct {
    const float* x;
    uint8_t* c;
    uint16_t* min16;
    uint16_t* scale16;
} int4_ctx;

/* One INT4 group. [PR166] "Purpose", second bullet: affine quantization in FP32 with an FP16
 * minimum and scale; first review: the codes are computed in FP32 before the metadata is
 * rounded to FP16.
 *   mn, mx  = min, max of the members (totalOrder)
 *   scale   = fl(fl(mx - mn) / 15)                 READING: 4-bit unsigned codes 0..15 span [mn, mx]
 *   code    = clamp(rne(fl(fl(x - mn) / scale)), 0, 15), or 0 when scale == 0   READING (0/0)
 *   stored  = f16(mn), f16(scale)
 * Division is IEEE correctly rounded (one semantics on every device). */
static void int4_group(void* vctx, int64_t gid, int64_t n, const int64_t* idx) {
    int4_ctx* ctx = (int4_ctx*)vctx;
    float mn = ctx->x[idx[0]], mx = ctx->x[idx[0]];
    for (int64_t k = 1; k < n; ++k) {
        float v = ctx->x[idx[k]];
        if (total_less(v, mn)) mn = v;
        if (total_less(mx, v)) mx = v;
    }
    float range = mx - mn;
    float scale = range / 15.0f;
    for (int64_t k = 0; k < n; ++k) {
        float v = ctx->x[idx[k]];
        int code = 0;
        if (scale != 0.0f) {
            float d = v - mn;
            float q = d / scale;
            float r = nearbyintf(q); /* ties to even ([PR166] review praise list: ties-to-even) */
            if (r < 0.0f) r = 0.0f;
            if (r > 15.0f) r = 15.0f;
            code = (int)r;
        }
        ctx->c[idx[k]] = (uint8_t)code;
    }
    ctx->min16[gid] = kvq_oracle_f32_to_f16(mn);
    ctx->scale16[gid] = kvq_oracle_f32_to_f16(scale);
}

static int int4_encode(const float* dense, int kind, int32_t G, int64_t rows, int64_t H, int64_t D,
                       uint8_t* codes, uint16_t* min16, uint16_t* scale16) {
    uint8_t* c = (uint8_t*)calloc((size_t)(rows * H * D) + 1, 1);
    if (!c) return KVQO_NOMEM;
    int4_ctx ctx = {dense, c, min16, scale16};
    for_each_group(kind, G, rows, H, D, int4_group, &ctx);
    pack_nibbles(c, rows, H, D, codes);
    free(c);
    return KVQO_OK;
}

/* INT4 decode: y = bf16(fl(fl(code * f32(scale16)) + f32(min16))).
 * READING: FP32 arithmetic, multiply then add as two rounded operations, one rounding to the
 * input dtype at the end. */
static float int4_decode_one(uint8_t code, uint16_t min16, uint16_t scale16) {
    float s = kvq_oracle_f16_to_f32(scale16);
    float m = kvq_oracle_f16_to_f32(min16);
    float prod = (float)code * s;
    float y = prod + m;
    return kvq_oracle_bf16_to_f32(kvq_oracle_f32_to_bf16(y));
}

/* ------------------------------------------------------------------------------------------ */
/* NVFP4                                                                                      */
/* ------------------------------------------------------------------------------------------ */

/* Global encoding multiplier of one encoded tensor. [PR166] "Purpose", second bullet (a scalar
 * FP32 global encoding multiplier) and the paragraph after the usage example (one per encoded
 * tensor, recomputed on every encoding call).
 * READING: g = fl(2688 / amax), 2688 = 448 (largest E4M3) * 6 (largest E2M1), so the largest
 * block lands on the top E4M3 scale. amax == 0 (all-zero or empty tensor) -> g = 1.
 * An overflowing quotient -> g = FLT_MAX. */
float kvq_oracle_nvfp4_global(float amax) {
    if (amax == 0.0f) return 1.0f;
    float g = 2688.0f / amax;
    if (isinf(g)) g = FLT_MAX;
    return g;
}

typedef struct {
    const float* x;
    uint8_t* c;
    uint8_t* sc8;
    float g;
} nvfp4_ctx;

/* One 16-member NVFP4 block.
 *   bamax = max |x| over the members
 *   s     = min(fl(g * fl(bamax / 6)), 448)           READING: order of operations
 *   sc8   = e4m3(s) (nearest, ties even)              [PR166] "Purpose": E4M3 block scales
 *   s_dec = fl(f32(sc8) / g)                          the stored, rounded scale ([PR408] port commit)
 *   q     = fl(x * fl(1 / s_dec)), or fl(x / s_dec) when that reciprocal overflows
 *           ([PR166] "Purpose": direct-division fallback for tiny scales)
 *   code  = e2m1(min(|q|, 6)) with sign bit signbit(x); sf == 0 -> every q = +-0 READING */
static void nvfp4_group(void* vctx, int64_t gid, int64_t n, const int64_t* idx) {
    nvfp4_ctx* ctx = (nvfp4_ctx*)vctx;
    float bamax = 0.0f;
    for (int64_t k = 0; k < n; ++k) {
        float a = fabsf(ctx->x[idx[k]]);
        if (a > bamax) bamax = a;
    }
    float t6 = bamax / 6.0f;
    float s = ctx->g * t6;
    if (!(s <= 448.0f)) s = 448.0f; /* also catches +inf */
    uint8_t code8 = kvq_oracle_f32_to_e4m3(s);
    float sf = kvq_oracle_e4m3_to_f32(code8);
    ctx->sc8[gid] = code8;
    for (int64_t k = 0; k < n; ++k) {
        float v = ctx->x[idx[k]];
        float q;
        if (sf == 0.0f) {
            q = 0.0f;
        } else {
            float s_dec = sf / ctx->g;
            float r = 1.0f / s_dec;
            if (isinf(r))
                q = v / s_dec;
            else
                q = v * r;
        }
        ctx->c[idx[k]] = kvq_oracle_e2m1_encode(q, v);
    }
}

/* Tensor amax over every encoded element ([PR166] "Purpose": one scale per encoded tensor). */
static float dense_amax(const float* dense, int64_t n) {
    float amax = 0.0f;
#pragma omp parallel for schedule(static) reduction(max : amax)
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(dense[i]);
        if (a > amax) amax = a;
    }
    return amax;
}

/* NVFP4 encode of dense rows. g_given < 0 means "the tensor's own multiplier" (the normal
 * case); a non-negative g_given is the multiplier of a larger tensor these rows belong to,
 * which lets a test check a slice of a tensor too large to encode here in full. */
static int nvfp4_encode(const float* dense, int kind, int64_t rows, int64_t H, int64_t D, uint8_t* codes,
                        uint8_t* sc8, float* gscale, float g_given) {
    float g = (g_given >= 0.0f) ? g_given : kvq_oracle_nvfp4_global(dense_amax(dense, rows * H * D));
    uint8_t* c = (uint8_t*)calloc((size_t)(rows * H * D) + 1, 1);
    if (!c) return KVQO_NOMEM;
    nvfp4_ctx ctx = {dense, c, sc8, g};
    for_each_group(kind, 16, rows, H, D, nvfp4_group, &ctx);
    pack_nibbles(c, rows, H, D, codes);
    free(c);
    *gscale = g;
    return KVQO_OK;
}

/* NVFP4 decode: y = bf16(fl(e2m1(code) * s_dec)), s_dec = fl(f32(sc8) / g). */
static float nvfp4_decode_one(uint8_t code, uint8_t sc8, float g) {
    float sf = kvq_oracle_e4m3_to_f32(sc8);
    float s_dec = sf / g;
    float y = kvq_oracle_e2m1_to_f32(code) * s_dec;
    return kvq_oracle_bf16_to_f32(kvq_oracle_f32_to_bf16(y));
}

/* ------------------------------------------------------------------------------------------ */
/* Row formats: every (token, head) row is quantized on its own ([PR408])                     */
/* ------------------------------------------------------------------------------------------ */

/* NVFP4 with one FP32 multiplier per (token, head) row. [PR408] "Summary": packed E2M1 values,
 * one E4M3 scale per 16 values, one FP32 row scale per token and KV head; nvfp4 port commit:
 * nibbles low first, quantization against the stored block scale, 76 B per D=128 row.
 * READING: the row scale is the tensor format's multiplier computed over the row alone
 * (g_row = 2688 / row amax, with the same zero and overflow rules), and the 16-value blocks
 * run along channels for K and V alike, so each row is encoded exactly as a one-row tensor. */
static int nvfp4_row_encode(const float* dense, int64_t rows, int64_t H, int64_t D, uint8_t* codes, uint8_t* sc8,
                            float* grow) {
    int64_t nb = ceil_div(D, 16);
    uint8_t* c = (uint8_t*)calloc((size_t)(rows * H * D) + 1, 1);
    if (!c) return KVQO_NOMEM;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows * H; ++r) {
        float g = kvq_oracle_nvfp4_global(dense_amax(dense + r * D, D));
        grow[r] = g;
        nvfp4_ctx ctx = {dense + r * D, c + r * D, sc8 + r * nb, g};
        for_each_group(KVQO_VALUE, 16, 1, 1, D, nvfp4_group, &ctx);
    }
    pack_nibbles(c, rows, H, D, codes);
    free(c);
    return KVQO_OK;
}

/* FP8 E4M3 with one FP32 symmetric scale per (token, head) row. [PR408] fp8 commit: a row of
 * head_dim E4M3 codes plus ONE FP32 scale; attention multiplies scores by the row scale, so the
 * stored scale is the decode multiplier.
 * READING: scale = fl(amax_row / 448); q = fl(x / scale) (IEEE division); code =
 * e4m3(min(|q|, 448)) with sign bit signbit(x). A zero scale (an all-zero row, or an amax so
 * small that amax / 448 underflows to 0) gives q = +-0. */
static int fp8_row_encode(const float* dense, int64_t rows, int64_t H, int64_t D, uint8_t* codes, float* srow) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows * H; ++r) {
        const float* x = dense + r * D;
        float s = dense_amax(x, D) / 448.0f;
        srow[r] = s;
        for (int64_t d = 0; d < D; ++d) {
            float v = x[d];
            float m = 0.0f;
            if (s != 0.0f) {
                m = fabsf(v / s);
                if (!(m <= 448.0f)) m = 448.0f;
            }
            codes[r * D + d] = kvq_oracle_f32_to_e4m3(signbit(v) ? -m : m);
        }
    }
    return KVQO_OK;
}

/* FP8-row decode: y = bf16(fl(e4m3(code) * scale)) (the code's sign included). */
static float fp8_row_decode_one(uint8_t code, float s) {
    float y = kvq_oracle_e4m3_to_f32(code) * s;
    return kvq_oracle_bf16_to_f32(kvq_oracle_f32_to_bf16(y));
}

/* ------------------------------------------------------------------------------------------ */
/* Public oracle entry points                                                                 */
/* ------------------------------------------------------------------------------------------ */

/* Group sizes: INT4 any G >= 1; NVFP4 and NVFP4-row 16; FP8-row 0 (one scale per row). */
static int check_common(int kind, int format, int32_t G, int64_t rows, int64_t H, int64_t D) {
    if (kind != KVQO_KEY && kind != KVQO_VALUE) return KVQO_BAD_ARG;
    switch (format) {
        case KVQO_INT4: if (G < 1) return KVQO_BAD_ARG; break;
        case KVQO_NVFP4:
        case KVQO_NVFP4_ROW: if (G != 16) return KVQO_BAD_ARG; break;
        case KVQO_FP8_ROW: if (G != 0) return KVQO_BAD_ARG; break;
        default: return KVQO_BAD_ARG;
    }
    if (rows < 0 || H < 0 || D < 0) return KVQO_BAD_ARG;
    return KVQO_OK;
}

/* Metadata layouts: INT4 meta0 = f16 minimums, meta1 = f16 scales (K [ceil(rows/G), H, D],
 * V [rows, H, ceil(D/G)]); NVFP4 meta0 = E4M3 block scales (same shapes with G = 16), one FP32
 * multiplier in gscale; NVFP4-row meta0 = E4M3 block scales [rows, H, ceil(D/16)], meta1 = FP32
 * row multipliers [rows, H]; FP8-row meta0 = FP32 row scales [rows, H]. Codes are nibbles
 * [rows, H, ceil(D/2)] except FP8-row, one byte per element [rows, H, D]. */
static int encode_dense(const float* dense, int kind, int format, int32_t G, int64_t rows, int64_t H, int64_t D,
                        uint8_t* codes, void* meta0, void* meta1, float* gscale, float g_given) {
    switch (format) {
        case KVQO_INT4: return int4_encode(dense, kind, G, rows, H, D, codes, (uint16_t*)meta0, (uint16_t*)meta1);
        case KVQO_NVFP4: return nvfp4_encode(dense, kind, rows, H, D, codes, (uint8_t*)meta0, gscale, g_given);
        case KVQO_NVFP4_ROW: return nvfp4_row_encode(dense, rows, H, D, codes, (uint8_t*)meta0, (float*)meta1);
        default: return fp8_row_encode(dense, rows, H, D, codes, (float*)meta0);
    }
}

/* pack_kv: encode the strided bf16 view x[T, H, D] (token stride st, head stride sh, channel
 * stride 1) into codes [T, H, ceil(D/2)], metadata planes and (NVFP4) the global scale.
 * Metadata: INT4 meta0 = f16 minimums, meta1 = f16 scales; NVFP4 meta0 = E4M3 block scales,
 * meta1 unused. Plane shapes: K [ceil(T/G), H, D], V [T, H, ceil(D/G)]. */
int kvq_oracle_pack(const uint16_t* x, int64_t T, int64_t H, int64_t D, int64_t st, int64_t sh, int kind, int format,
                    int32_t G, uint8_t* codes, void* meta0, void* meta1, float* gscale, float g_given) {
    int rc = check_common(kind, format, G, T, H, D);
    if (rc) return rc;
    float* dense = (float*)malloc(sizeof(float) * (size_t)(T * H * D) + 4);
    if (!dense) return KVQO_NOMEM;
    materialize(x, st, sh, NULL, 0, 0, NULL, T, H, D, dense);
    rc = encode_dense(dense, kind, format, G, T, H, D, codes, meta0, meta1, gscale, g_given);
    free(dense);
    return rc;
}

/* Decoded value of element (t, h, d) of a packed tensor, as float32 holding a bf16 value. */
static float decode_at(int kind, int format, int32_t G, int64_t H, int64_t D, const uint8_t* codes, const void* meta0,
                       const void* meta1, float g, int64_t t, int64_t h, int64_t d) {
    if (format == KVQO_FP8_ROW) return fp8_row_decode_one(codes[(t * H + h) * D + d], ((const float*)meta0)[t * H + h]);
    uint8_t c = nibble_at(codes, H, D, t, h, d);
    if (format == KVQO_NVFP4_ROW)
        return nvfp4_decode_one(c, ((const uint8_t*)meta0)[(t * H + h) * ceil_div(D, 16) + d / 16],
                                ((const float*)meta1)[t * H + h]);
    int64_t gid = (kind == KVQO_KEY) ? ((t / G) * H + h) * D + d : (t * H + h) * ceil_div(D, G) + d / G;
    if (format == KVQO_INT4)
        return int4_decode_one(c, ((const uint16_t*)meta0)[gid], ((const uint16_t*)meta1)[gid]);
    return nvfp4_decode_one(c, ((const uint8_t*)meta0)[gid], g);
}

/* unpack_kv: write the decoded rows [rows, H, D] as bf16 bits into y (strided: st, sh). */
int kvq_oracle_unpack(int kind, int format, int32_t G, int64_t rows, int64_t H, int64_t D, const uint8_t* codes,
                      const void* meta0, const void* meta1, const float* gscale, uint16_t* y, int64_t st, int64_t sh) {
    int rc = check_common(kind, format, G, rows, H, D);
    if (rc) return rc;
    float g = (format == KVQO_NVFP4) ? *gscale : 0.0f;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < rows; ++t)
        for (int64_t h = 0; h < H; ++h)
            for (int64_t d = 0; d < D; ++d) {
                float v = decode_at(kind, format, G, H, D, codes, meta0, meta1, g, t, h, d);
                y[t * st + h * sh + d] = (uint16_t)(f32_bits(v) >> 16);
            }
    return KVQO_OK;
}

/* encode_residual: dense (positions == NULL, rows = T) or sparse (rows = M compact rows taken
 * at positions[0..M)). The residual is packed with its own kind, format and group size,
 * independent of how `prev` was produced ([PR166] test plan: mixed-format reconstruction).
 * The sparse residual owns a copy of the position map ([PR166] "Purpose", fourth bullet). */
int kvq_oracle_encode_residual(const uint16_t* cur, int64_t cst, int64_t csh, const uint16_t* prev, int64_t pst,
                               int64_t psh, int64_t T, int64_t H, int64_t D, const int32_t* positions, int64_t M,
                               int kind, int format, int32_t G, uint8_t* codes, void* meta0, void* meta1,
                               float* gscale, int32_t* positions_out, float g_given) {
    int64_t rows = positions ? M : T;
    int rc = check_common(kind, format, G, rows, H, D);
    if (rc) return rc;
    if (positions) {
        for (int64_t i = 0; i < M; ++i)
            if (positions[i] < 0 || positions[i] >= T) return KVQO_BAD_ARG;
    }
    float* dense = (float*)malloc(sizeof(float) * (size_t)(rows * H * D) + 4);
    if (!dense) return KVQO_NOMEM;
    materialize(cur, cst, csh, prev, pst, psh, positions, rows, H, D, dense);
    rc = encode_dense(dense, kind, format, G, rows, H, D, codes, meta0, meta1, gscale, g_given);
    free(dense);
    if (positions && positions_out)
        for (int64_t i = 0; i < M; ++i) positions_out[i] = positions[i];
    return rc;
}

/* decode_residual: out = bf16(fl(prev + bf16(unpack(R)))), both in the input dtype (two
 * roundings, READING of "in the input dtype"). Sparse: every row not in the position map is a
 * bitwise copy of prev ([PR166] "Purpose": absent rows inherit the predecessor). `out` and
 * `prev` are full [T, H, D] strided views; out may equal prev. */
int kvq_oracle_decode_residual(int kind, int format, int32_t G, int64_t rows, int64_t H, int64_t D,
                               const uint8_t* codes, const void* meta0, const void* meta1, const float* gscale,
                               const int32_t* positions, const uint16_t* prev, int64_t pst, int64_t psh, int64_t T,
                               uint16_t* out, int64_t ost, int64_t osh) {
    int rc = check_common(kind, format, G, rows, H, D);
    if (rc) return rc;
    if (!positions && rows != T) return KVQO_BAD_ARG;
    float g = (format == KVQO_NVFP4) ? *gscale : 0.0f;
    if (positions) {
        for (int64_t i = 0; i < rows; ++i)
            if (positions[i] < 0 || positions[i] >= T) return KVQO_BAD_ARG;
        if (out != prev || ost != pst || osh != psh) {
#pragma omp parallel for schedule(static)
            for (int64_t t = 0; t < T; ++t)
                for (int64_t h = 0; h < H; ++h)
                    for (int64_t d = 0; d < D; ++d) out[t * ost + h * osh + d] = prev[t * pst + h * psh + d];
        }
    }
    /* kept rows are distinct (precondition), so the rows below never share an output element */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < rows; ++i) {
        int64_t t = positions ? (int64_t)positions[i] : i;
        for (int64_t h = 0; h < H; ++h)
            for (int64_t d = 0; d < D; ++d) {
                float delta = decode_at(kind, format, G, H, D, codes, meta0, meta1, g, i, h, d);
                float p = kvq_oracle_bf16_to_f32(prev[t * pst + h * psh + d]);
                float sum = p + delta;
                out[t * ost + h * osh + d] = kvq_oracle_f32_to_bf16(sum);
            }
    }
    return KVQO_OK;
}

/* Tensor amax of the rows an encode would see (plain tensor, or the residual rows when prev is
 * given, gathered by positions when given), as a float. */
float kvq_oracle_tensor_amax(const uint16_t* cur, int64_t cst, int64_t csh, const uint16_t* prev, int64_t pst,
                             int64_t psh, int64_t T, int64_t H, int64_t D, const int32_t* positions, int64_t M) {
    int64_t rows = positions ? M : T;
    float amax = 0.0f;
#pragma omp parallel reduction(max : amax)
    {
        float* row = (float*)malloc(sizeof(float) * (size_t)(H * D) + 4);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < rows; ++i) {
            const int32_t* p = positions ? positions + i : NULL;
            if (p) {
                materialize(cur, cst, csh, prev, pst, psh, p, 1, H, D, row);
            } else {
                materialize(cur + i * cst, cst, csh, prev ? prev + i * pst : NULL, pst, psh, NULL, 1, H, D, row);
            }
            float a = dense_amax(row, H * D);
            if (a > amax) amax = a;
        }
        free(row);
    }
    return amax;
}

/* Element-wise helpers exposed for the pin tests (vectorized over n values). */
void kvq_oracle_f32_to_bf16_n(const float* x, uint16_t* y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = kvq_oracle_f32_to_bf16(x[i]);
}
void kvq_oracle_f32_to_f16_n(const float* x, uint16_t* y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = kvq_oracle_f32_to_f16(x[i]);
}
void kvq_oracle_f32_to_e4m3_n(const float* x, uint8_t* y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = kvq_oracle_f32_to_e4m3(x[i]);
}
void kvq_oracle_e2m1_encode_n(const float* q, uint8_t* y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = kvq_oracle_e2m1_encode(q[i], q[i]);
}

/* ------------------------------------------------------------------------------------------ */
/* Paged views and slot writes                                                                */
/* ------------------------------------------------------------------------------------------ */

/* Bytes of one row's codes, and of one row's entry in each row-indexed metadata plane. */
static int64_t code_row_bytes(int format, int64_t H, int64_t D) {
    return (format == KVQO_FP8_ROW) ? H * D : H * ceil_div(D, 2);
}

/* Whether a format groups K over tokens (its metadata rows are not the token rows). */
static int token_grouped(int kind, int format) {
    return kind == KVQO_KEY && (format == KVQO_INT4 || format == KVQO_NVFP4);
}

/* Rows of a paged bf16 view x[P, S, H, D] (page stride sp, slot stride ss, head stride sh,
 * channel stride 1) in page-major order: logical token p*S + s is slot s of page p. */
static void materialize_paged(const uint16_t* x, int64_t P, int64_t S, int64_t H, int64_t D, int64_t sp, int64_t ss,
                              int64_t sh, float* dense) {
    for (int64_t p = 0; p < P; ++p)
        for (int64_t s = 0; s < S; ++s)
            for (int64_t h = 0; h < H; ++h)
                for (int64_t d = 0; d < D; ++d)
                    dense[((p * S + s) * H + h) * D + d] = kvq_oracle_bf16_to_f32(x[p * sp + s * ss + h * sh + d]);
}

/* pack_paged over [pages, page_size, heads, dim] ([PR166] interface review, item 3, and the
 * stacked-PR follow-up that adds pack_paged / unpack_paged). Flat grouping packs exactly what
 * pack() packs for the page-major token sequence (a 64-token KEY group then spans four 16-token
 * pages). Page-local grouping ([PR166] first review, "Group ownership vs 16-token pages") keeps
 * every KEY group inside one page: page p is encoded as its own S-token range with KEY groups
 * over slots [b*G, min(S, (b+1)*G)), metadata [P, ceil(S/G), H, D]; the NVFP4 multiplier stays
 * one per call, over all pages. VALUE groups and the row formats are page-local by
 * construction; for them the flag changes nothing. */
int kvq_oracle_pack_paged(const uint16_t* x, int64_t P, int64_t S, int64_t H, int64_t D, int64_t sp, int64_t ss,
                          int64_t sh, int kind, int format, int32_t G, int page_local, uint8_t* codes, void* meta0,
                          void* meta1, float* gscale) {
    if (P < 0 || S < 0) return KVQO_BAD_ARG;
    int rc = check_common(kind, format, G, P * S, H, D);
    if (rc) return rc;
    int64_t rows = P * S;
    float* dense = (float*)malloc(sizeof(float) * (size_t)(rows * H * D) + 4);
    if (!dense) return KVQO_NOMEM;
    materialize_paged(x, P, S, H, D, sp, ss, sh, dense);
    if (page_local && token_grouped(kind, format)) {
        float g = (format == KVQO_NVFP4) ? kvq_oracle_nvfp4_global(dense_amax(dense, rows * H * D)) : -1.0f;
        int64_t mrows = ceil_div(S, G) * H * D; /* metadata entries per page */
        for (int64_t p = 0; p < P && rc == KVQO_OK; ++p) {
            float gp = 0.0f;
            void* m0 = (format == KVQO_INT4) ? (void*)((uint16_t*)meta0 + p * mrows) : (void*)((uint8_t*)meta0 + p * mrows);
            void* m1 = (format == KVQO_INT4) ? (void*)((uint16_t*)meta1 + p * mrows) : NULL;
            rc = encode_dense(dense + p * S * H * D, kind, format, G, S, H, D, codes + p * S * code_row_bytes(format, H, D),
                              m0, m1, &gp, g);
        }
        if (format == KVQO_NVFP4) *gscale = g;
    } else {
        rc = encode_dense(dense, kind, format, G, rows, H, D, codes, meta0, meta1, gscale, -1.0f);
    }
    free(dense);
    return rc;
}

/* unpack_paged: the decoded bf16 rows written back into a paged view y[P, S, H, D]. */
int kvq_oracle_unpack_paged(int kind, int format, int32_t G, int page_local, int64_t P, int64_t S, int64_t H, int64_t D,
                            const uint8_t* codes, const void* meta0, const void* meta1, const float* gscale, uint16_t* y,
                            int64_t sp, int64_t ss, int64_t sh) {
    if (P < 0 || S < 0) return KVQO_BAD_ARG;
    int rc = check_common(kind, format, G, P * S, H, D);
    if (rc) return rc;
    float g = (format == KVQO_NVFP4) ? *gscale : 0.0f;
    int local = page_local && token_grouped(kind, format);
    int64_t mrows = local ? ceil_div(S, G) * H * D : 0;
    for (int64_t p = 0; p < P; ++p) {
        const uint8_t* cp = local ? codes + p * S * code_row_bytes(format, H, D) : codes;
        const void* m0 = meta0;
        const void* m1 = meta1;
        if (local) {
            m0 = (format == KVQO_INT4) ? (const void*)((const uint16_t*)meta0 + p * mrows)
                                       : (const void*)((const uint8_t*)meta0 + p * mrows);
            m1 = (format == KVQO_INT4) ? (const void*)((const uint16_t*)meta1 + p * mrows) : NULL;
        }
        for (int64_t s = 0; s < S; ++s) {
            int64_t t = local ? s : p * S + s;
            for (int64_t h = 0; h < H; ++h)
                for (int64_t d = 0; d < D; ++d) {
                    float v = decode_at(kind, format, G, H, D, cp, m0, m1, g, t, h, d);
                    y[p * sp + s * ss + h * sh + d] = (uint16_t)(f32_bits(v) >> 16);
                }
        }
    }
    return KVQO_OK;
}

/* Slot ids: every id in [0, n_slots) and no id twice. */
static int check_slots(const int32_t* slots, int64_t N, int64_t n_slots) {
    if (N == 0) return KVQO_OK;
    uint8_t* seen = (uint8_t*)calloc((size_t)n_slots + 1, 1);
    if (!seen) return KVQO_NOMEM;
    int rc = KVQO_OK;
    for (int64_t i = 0; i < N && rc == KVQO_OK; ++i) {
        if (slots[i] < 0 || slots[i] >= n_slots || seen[slots[i]]) rc = KVQO_BAD_ARG;
        else seen[slots[i]] = 1;
    }
    free(seen);
    return rc;
}

/* Quantize N new rows src[N, H, D] and write row i into cache row slots[i] ([PR408] fp8
 * commit: fused quantize + scatter, slot ids given as a tensor). Only formats whose rows are
 * encoded independently qualify: INT4 VALUE (channel groups), NVFP4-row and FP8-row. The rows
 * are encoded as one N-row tensor, then each row's codes and row metadata move to its slot;
 * every other cache row is left as it was. */
int kvq_oracle_store_rows(const uint16_t* src, int64_t N, int64_t H, int64_t D, int64_t st, int64_t sh,
                          const int32_t* slots, int kind, int format, int32_t G, int64_t n_slots, uint8_t* codes,
                          void* meta0, void* meta1) {
    int rc = check_common(kind, format, G, N, H, D);
    if (rc) return rc;
    if (!((format == KVQO_INT4 && kind == KVQO_VALUE) || format == KVQO_NVFP4_ROW || format == KVQO_FP8_ROW))
        return KVQO_BAD_ARG;
    rc = check_slots(slots, N, n_slots);
    if (rc) return rc;
    int64_t cb = code_row_bytes(format, H, D);
    /* bytes of one row in meta0 / meta1 */
    int64_t m0b = 0, m1b = 0;
    if (format == KVQO_INT4) m0b = m1b = 2 * H * ceil_div(D, G);
    if (format == KVQO_NVFP4_ROW) { m0b = H * ceil_div(D, 16); m1b = 4 * H; }
    if (format == KVQO_FP8_ROW) m0b = 4 * H;
    float* dense = (float*)malloc(sizeof(float) * (size_t)(N * H * D) + 4);
    uint8_t* c = (uint8_t*)malloc((size_t)(N * cb) + 1);
    uint8_t* t0 = (uint8_t*)malloc((size_t)(N * m0b) + 1);
    uint8_t* t1 = (uint8_t*)malloc((size_t)(N * m1b) + 1);
    if (!dense || !c || !t0 || !t1) rc = KVQO_NOMEM;
    if (rc == KVQO_OK) {
        materialize(src, st, sh, NULL, 0, 0, NULL, N, H, D, dense);
        rc = encode_dense(dense, kind, format, G, N, H, D, c, t0, t1, NULL, -1.0f);
    }
    if (rc == KVQO_OK)
        for (int64_t i = 0; i < N; ++i) {
            int64_t r = slots[i];
            memcpy(codes + r * cb, c + i * cb, (size_t)cb);
            memcpy((uint8_t*)meta0 + r * m0b, t0 + i * m0b, (size_t)m0b);
            if (m1b) memcpy((uint8_t*)meta1 + r * m1b, t1 + i * m1b, (size_t)m1b);
        }
    free(dense);
    free(c);
    free(t0);
    free(t1);
    return rc;
}

/* Gather-and-decode: y row i = decoded cache row slots[i], for any format (a KEY row of a
 * token-grouped format uses the metadata of its group, row slots[i] / G). */
int kvq_oracle_load_rows(int kind, int format, int32_t G, int64_t n_slots, int64_t H, int64_t D, const uint8_t* codes,
                         const void* meta0, const void* meta1, const float* gscale, const int32_t* slots, int64_t N,
                         uint16_t* y, int64_t st, int64_t sh) {
    int rc = check_common(kind, format, G, n_slots, H, D);
    if (rc) return rc;
    float g = (format == KVQO_NVFP4) ? *gscale : 0.0f;
    for (int64_t i = 0; i < N; ++i) {
        int64_t t = slots[i];
        if (t < 0 || t >= n_slots) return KVQO_BAD_ARG;
        for (int64_t h = 0; h < H; ++h)
            for (int64_t d = 0; d < D; ++d) {
                float v = decode_at(kind, format, G, H, D, codes, meta0, meta1, g, t, h, d);
                y[i * st + h * sh + d] = (uint16_t)(f32_bits(v) >> 16);
            }
    }
    return KVQO_OK;
}

/* ------------------------------------------------------------------------------------------ */
/* BF16 protected window                                                                      */
/* ------------------------------------------------------------------------------------------ */

/* Rows kept in BF16 by a window of the first `sink` and the latest `recent` tokens of T:
 * n_sink = min(sink, T) rows at the front and n_recent = min(recent, T - n_sink) at the end;
 * the rest, [n_sink, T - n_recent), is quantized. */
static void window_split(int64_t T, int64_t sink, int64_t recent, int64_t* n_sink, int64_t* n_recent) {
    *n_sink = sink < T ? sink : T;
    *n_recent = recent < T - *n_sink ? recent : T - *n_sink;
}

/* Encode with a BF16 window ([PR166] "Real Ouro numerical comparison": the first 4 and the
 * latest 16 tokens kept in BF16; protected rows are left out of the quantized payload, and a
 * passthrough row reconstructs bitwise). READING: the quantized rows [n_sink, T - n_recent) are
 * encoded as one tensor of their own (KEY groups start at the first quantized row, the NVFP4
 * multiplier covers only them) -- exactly the sparse residual whose positions are that range;
 * the protected rows of `cur` are stored raw in `window` ([n_sink + n_recent, H, D] bf16,
 * front rows first). With prev == NULL the quantized rows are cur itself (pack); otherwise they
 * are bf16(cur - prev) (residual), while the window still stores cur, so the protected rows of
 * a reconstruction equal cur exactly. */
int kvq_oracle_encode_window(const uint16_t* cur, int64_t cst, int64_t csh, const uint16_t* prev, int64_t pst,
                             int64_t psh, int64_t T, int64_t H, int64_t D, int64_t sink, int64_t recent, int kind,
                             int format, int32_t G, uint8_t* codes, void* meta0, void* meta1, float* gscale,
                             uint16_t* window) {
    if (sink < 0 || recent < 0) return KVQO_BAD_ARG;
    int64_t ns, nr;
    window_split(T, sink, recent, &ns, &nr);
    int64_t rows = T - ns - nr;
    int rc = check_common(kind, format, G, rows, H, D);
    if (rc) return rc;
    float* dense = (float*)malloc(sizeof(float) * (size_t)(rows * H * D) + 4);
    if (!dense) return KVQO_NOMEM;
    materialize(cur + ns * cst, cst, csh, prev ? prev + ns * pst : NULL, pst, psh, NULL, rows, H, D, dense);
    rc = encode_dense(dense, kind, format, G, rows, H, D, codes, meta0, meta1, gscale, -1.0f);
    free(dense);
    for (int64_t i = 0; i < ns + nr; ++i) {
        int64_t t = (i < ns) ? i : T - nr + (i - ns);
        for (int64_t h = 0; h < H; ++h)
            for (int64_t d = 0; d < D; ++d) window[(i * H + h) * D + d] = cur[t * cst + h * csh + d];
    }
    return rc;
}

/* Decode with a BF16 window: quantized rows decoded (prev == NULL) or added to prev in the
 * input dtype (residual), protected rows copied bit for bit from `window`. out is [T, H, D]. */
int kvq_oracle_decode_window(int kind, int format, int32_t G, int64_t T, int64_t H, int64_t D, int64_t sink,
                             int64_t recent, const uint8_t* codes, const void* meta0, const void* meta1,
                             const float* gscale, const uint16_t* window, const uint16_t* prev, int64_t pst,
                             int64_t psh, uint16_t* out, int64_t ost, int64_t osh) {
    if (sink < 0 || recent < 0) return KVQO_BAD_ARG;
    int64_t ns, nr;
    window_split(T, sink, recent, &ns, &nr);
    int64_t rows = T - ns - nr;
    int rc = check_common(kind, format, G, rows, H, D);
    if (rc) return rc;
    float g = (format == KVQO_NVFP4) ? *gscale : 0.0f;
    for (int64_t i = 0; i < rows; ++i) {
        int64_t t = ns + i;
        for (int64_t h = 0; h < H; ++h)
            for (int64_t d = 0; d < D; ++d) {
                float v = decode_at(kind, format, G, H, D, codes, meta0, meta1, g, i, h, d);
                if (prev) {
                    float p = kvq_oracle_bf16_to_f32(prev[t * pst + h * psh + d]);
                    float sum = p + v;
                    out[t * ost + h * osh + d] = kvq_oracle_f32_to_bf16(sum);
                } else {
                    out[t * ost + h * osh + d] = (uint16_t)(f32_bits(v) >> 16);
                }
            }
    }
    for (int64_t i = 0; i < ns + nr; ++i) {
        int64_t t = (i < ns) ? i : T - nr + (i - ns);
        for (int64_t h = 0; h < H; ++h)
            for (int64_t d = 0; d < D; ++d) out[t * ost + h * osh + d] = window[(i * H + h) * D + d];
    }
    return KVQO_OK;
}
