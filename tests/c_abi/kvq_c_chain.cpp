// A plain C++ program that drives libkvq through include/kvq.h alone, with the HIP runtime for
// device memory and a stream: pack an INT4 G64 KEY tensor, unpack it, encode a sparse NVFP4
// VALUE residual of a second tensor against that reconstruction, and decode the residual out of
// place. Every plane is sized with kvq_plane_bytes and allocated here (the library allocates
// nothing). Inputs and outputs are written as raw little-endian files into the directory given
// on the command line, for tests/test_gpu_c_abi.py to compare with the CPU oracle.
//
// usage: kvq_c_chain OUT_DIR T H D
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "kvq.h"

#define HIP_OK(x)                                                                       \
    do {                                                                                \
        const hipError_t e_ = (x);                                                      \
        if (e_ != hipSuccess) {                                                         \
            std::fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, hipGetErrorString(e_)); \
            return 2;                                                                   \
        }                                                                               \
    } while (0)
#define KVQ_OK_(x)                                                                        \
    do {                                                                                  \
        const kvq_status s_ = (x);                                                        \
        if (s_ != KVQ_OK) {                                                               \
            std::fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, kvq_status_string(s_)); \
            return 3;                                                                     \
        }                                                                                 \
    } while (0)

namespace {

// float -> bf16 bits, round to nearest even (finite inputs)
uint16_t to_bf16(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// A small xorshift32 generator for the inputs, mapped to roughly N(0, 1) by a sum
// of uniforms; the values only need to be finite and varied.
struct Gen {
    uint32_t s;
    float uniform() {
        s ^= s << 13;
        s ^= s >> 17;
        s ^= s << 5;
        return (float)(s >> 8) * (1.0f / 16777216.0f);
    }
    float normalish() { return uniform() + uniform() + uniform() + uniform() - 2.0f; }
};

bool write_file(const std::string& path, const void* data, size_t bytes) {
    FILE* f = std::fopen(path.c_str(), "wb");
    if (!f) return false;
    const bool ok = std::fwrite(data, 1, bytes, f) == bytes;
    return std::fclose(f) == 0 && ok;
}

// A packed tensor whose planes live in device memory sized by kvq_plane_bytes.
struct Planes {
    uint64_t size[KVQ_NUM_PLANES] = {};
    void* dev[KVQ_NUM_PLANES] = {};
};

int alloc_planes(kvq_format fmt, kvq_kind kind, int32_t G, int64_t rows, int64_t H, int64_t D, int sparse,
                 Planes& p, kvq_packed& out) {
    KVQ_OK_(kvq_plane_bytes(fmt, kind, G, rows, H, D, sparse, p.size));
    for (int i = 0; i < KVQ_NUM_PLANES; ++i)
        if (p.size[i]) HIP_OK(hipMalloc(&p.dev[i], p.size[i]));
    std::memset(&out, 0, sizeof out);
    out.codes = (uint8_t*)p.dev[KVQ_PLANE_CODES];
    out.meta0 = p.dev[KVQ_PLANE_META0];
    out.meta1 = p.dev[KVQ_PLANE_META1];
    out.global_scale = (float*)p.dev[KVQ_PLANE_GLOBAL];
    out.positions = (int32_t*)p.dev[KVQ_PLANE_POSITIONS];
    return 0;
}

int save_planes(const std::string& dir, const std::string& name, const Planes& p) {
    static const char* kNames[KVQ_NUM_PLANES] = {"codes", "meta0", "meta1", "global", "positions"};
    for (int i = 0; i < KVQ_NUM_PLANES; ++i) {
        if (!p.size[i]) continue;
        std::vector<uint8_t> host(p.size[i]);
        HIP_OK(hipMemcpy(host.data(), p.dev[i], p.size[i], hipMemcpyDeviceToHost));
        if (!write_file(dir + "/" + name + "_" + kNames[i] + ".bin", host.data(), host.size())) return 4;
    }
    return 0;
}

kvq_tensor view(void* data, int64_t T, int64_t H, int64_t D) {
    kvq_tensor t;
    std::memset(&t, 0, sizeof t);
    t.data = data;
    t.dtype = KVQ_BF16;
    t.T = T;
    t.H = H;
    t.D = D;
    t.stride_t = H * D;
    t.stride_h = D;
    return t;
}

}  // namespace

int main(int argc, char** argv) {
    if (argc != 5) {
        std::fprintf(stderr, "usage: %s OUT_DIR T H D\n", argv[0]);
        return 1;
    }
    const std::string dir = argv[1];
    const int64_t T = std::atoll(argv[2]), H = std::atoll(argv[3]), D = std::atoll(argv[4]);
    const size_t n = (size_t)(T * H * D);
    std::printf("%s: T=%lld H=%lld D=%lld\n", kvq_version(), (long long)T, (long long)H, (long long)D);

    // inputs: x0, and x1 = x0 + 0.1 noise (both bf16); sparse rows: every third token
    Gen g{12345u};
    std::vector<uint16_t> x0(n), x1(n);
    for (size_t i = 0; i < n; ++i) {
        const float a = g.normalish() * (1.0f + 4.0f * (float)((i / (size_t)D) % 3));
        uint32_t b = (uint32_t)to_bf16(a) << 16;
        float ab;
        std::memcpy(&ab, &b, 4);
        x0[i] = to_bf16(a);
        x1[i] = to_bf16(ab + 0.1f * g.normalish());
    }
    std::vector<int32_t> pos;
    for (int64_t t = 0; t < T; t += 3) pos.push_back((int32_t)t);
    const int64_t M = (int64_t)pos.size();
    if (!write_file(dir + "/x0.bin", x0.data(), n * 2) || !write_file(dir + "/x1.bin", x1.data(), n * 2) ||
        !write_file(dir + "/positions.bin", pos.data(), pos.size() * 4))
        return 4;

    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    void *dx0, *dx1, *dr0, *dr1, *dpos, *ws;
    HIP_OK(hipMalloc(&dx0, n * 2));
    HIP_OK(hipMalloc(&dx1, n * 2));
    HIP_OK(hipMalloc(&dr0, n * 2));
    HIP_OK(hipMalloc(&dr1, n * 2));
    HIP_OK(hipMalloc(&dpos, (size_t)(M > 0 ? M : 1) * 4));
    HIP_OK(hipMalloc(&ws, kvq_workspace_bytes()));
    HIP_OK(hipMemcpy(dx0, x0.data(), n * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dx1, x1.data(), n * 2, hipMemcpyHostToDevice));
    if (M > 0) HIP_OK(hipMemcpy(dpos, pos.data(), (size_t)M * 4, hipMemcpyHostToDevice));

    const kvq_tensor vx0 = view(dx0, T, H, D), vx1 = view(dx1, T, H, D);
    const kvq_tensor vr0 = view(dr0, T, H, D), vr1 = view(dr1, T, H, D);

    // pack_kv / unpack_kv: INT4, KEY, G = 64
    Planes pp;
    kvq_packed p;
    if (int rc = alloc_planes(KVQ_INT4, KVQ_KEY, 64, T, H, D, 0, pp, p)) return rc;
    KVQ_OK_(kvq_pack(&vx0, KVQ_KEY, KVQ_INT4, 64, &p, ws, s));
    KVQ_OK_(kvq_unpack(&p, &vr0, s));

    // encode_residual / decode_residual: sparse NVFP4 VALUE residual of x1 against r0
    Planes rp;
    kvq_packed r;
    if (int rc = alloc_planes(KVQ_NVFP4, KVQ_VALUE, 16, M, H, D, 1, rp, r)) return rc;
    if (!r.positions) {  // a non-NULL map marks the residual sparse, also when M = 0
        HIP_OK(hipMalloc(&rp.dev[KVQ_PLANE_POSITIONS], 4));
        r.positions = (int32_t*)rp.dev[KVQ_PLANE_POSITIONS];
    }
    KVQ_OK_(kvq_encode_residual(&vx1, &vr0, (const int32_t*)dpos, M, KVQ_VALUE, KVQ_NVFP4, 16, &r, ws, s));
    KVQ_OK_(kvq_decode_residual(&r, &vr0, &vr1, s));
    HIP_OK(hipStreamSynchronize(s));

    std::vector<uint16_t> host(n);
    HIP_OK(hipMemcpy(host.data(), dr0, n * 2, hipMemcpyDeviceToHost));
    if (!write_file(dir + "/r0.bin", host.data(), n * 2)) return 4;
    HIP_OK(hipMemcpy(host.data(), dr1, n * 2, hipMemcpyDeviceToHost));
    if (!write_file(dir + "/r1.bin", host.data(), n * 2)) return 4;
    if (int rc = save_planes(dir, "pack", pp)) return rc;
    if (int rc = save_planes(dir, "residual", rp)) return rc;
    std::printf("pack: rows=%lld group=%d; residual: rows=%lld full_T=%lld\n", (long long)p.rows, p.group_size,
                (long long)r.rows, (long long)r.full_T);

    for (void* q : pp.dev) HIP_OK(hipFree(q));
    for (void* q : rp.dev) HIP_OK(hipFree(q));
    for (void* q : {dx0, dx1, dr0, dr1, dpos, ws}) HIP_OK(hipFree(q));
    HIP_OK(hipStreamDestroy(s));
    return 0;
}
