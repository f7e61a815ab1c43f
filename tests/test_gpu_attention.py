"""GPU parity of decode attention over the packed cache (kvq_decode_attention) against the
float64 oracle (oracle/attention.py) over the codec's own decode of the same packed planes.

Tolerance, from the arithmetic: K and V are reconstructed exactly (bf16 for bf16); the scores'
products are exact in FP32 and their D-term FP32 sums (D = 64 .. 256) err by well under 2^-16 relative; the
probabilities are rounded to bf16 (relative error <= 2^-9) before the PV product, which bounds
the output error by 2^-9 * sum_t p_t |v_t| <= 2^-9 * max |V|, plus FP32 accumulation. The tests
use 2^-8 * max |V| per element, and a mean error well below that. Two structural cases are tight:
q = 0 (equal scores: the output is the plain mean of V, accurate to FP32 accumulation) and one
dominant key (the output is that token's V row).
"""

import numpy as np
import pytest
import torch

import kv_cache_quantization_kvq_amd as kvq
import oracle
from gpu_util import dev, to_dev
from oracle.attention import decode_attention, reconstruct
from workloads import bf16_bits, c4_tensors, normal_kv

pytestmark = pytest.mark.gpu

D = 128
FORMS = [("int4", 64, 64), ("int4", 16, 32), ("int4", 128, 8), ("nvfp4", 16, 16), ("nvfp4_row", 16, 16), ("fp8_row", 0, 0)]


def packed_pair(k_bits, v_bits, fmt, gk, gv):
    kd, vd = to_dev(k_bits), to_dev(v_bits)
    gk_, gv_ = kvq.pack(kd, "key", fmt, gk), kvq.pack(vd, "value", fmt, gv)
    ok, ov = oracle.pack(k_bits, "key", fmt, gk), oracle.pack(v_bits, "value", fmt, gv)
    return gk_, gv_, ok, ov


def check(got, want, vmax, what):
    err = np.abs(got.astype(np.float64) - want)
    tol = 2.0 ** -8 * vmax + 1e-6
    assert err.max() <= tol, f"{what}: max err {err.max():.3e} > {tol:.3e}"
    assert err.mean() <= 2.0 ** -12 * vmax + 1e-7, f"{what}: mean err {err.mean():.3e}"


@pytest.mark.parametrize("fmt,gk,gv", FORMS)
@pytest.mark.parametrize("T,H,Hq", [(1, 1, 1), (15, 2, 8), (17, 1, 16), (64, 2, 2), (1000, 2, 16), (4099, 4, 8)])
def test_random_vs_oracle(fmt, gk, gv, T, H, Hq):
    rng = np.random.default_rng(T * 7 + Hq)
    k, v = normal_kv(rng, T, H, D), normal_kv(rng, T, H, D)
    q = bf16_bits(rng.standard_normal((Hq, D)))
    gk_, gv_, ok, ov = packed_pair(k, v, fmt, gk, gv)
    out = kvq.decode_attention(to_dev(q), gk_, gv_).cpu().numpy()
    kr, vr = reconstruct(ok), reconstruct(ov)
    want = decode_attention(q, kr, vr, 1.0 / np.sqrt(D))
    check(out, want, np.abs(oracle.bf16_to_f32(vr)).max(), f"{fmt} T={T}")


@pytest.mark.parametrize("fmt,gk,gv", [("int4", 64, 64), ("nvfp4", 16, 16), ("fp8_row", 0, 0)])
@pytest.mark.parametrize("T,H,Hq", [(500, 1, 40), (300, 2, 64), (77, 1, 128), (1000, 4, 68)])
def test_many_query_heads_per_kv_head(fmt, gk, gv, T, H, Hq):
    """More than 16 query heads per KV head (multi-query models): 16-row query tiles."""
    rng = np.random.default_rng(T + Hq)
    k, v = normal_kv(rng, T, H, D), normal_kv(rng, T, H, D)
    q = bf16_bits(rng.standard_normal((Hq, D)))
    gk_, gv_, ok, ov = packed_pair(k, v, fmt, gk, gv)
    out = kvq.decode_attention(to_dev(q), gk_, gv_).cpu().numpy()
    kr, vr = reconstruct(ok), reconstruct(ov)
    want = decode_attention(q, kr, vr, 1.0 / np.sqrt(D))
    check(out, want, np.abs(oracle.bf16_to_f32(vr)).max(), f"{fmt} T={T} H={H} Hq={Hq}")


@pytest.mark.parametrize("fmt,gk,gv", [("int4", 64, 64), ("nvfp4", 16, 16), ("fp8_row", 0, 0)])
def test_many_token_blocks_per_head(fmt, gk, gv):
    """One KV head over 20 000 tokens splits into 313 token blocks of 64 (one round of resident
    blocks is far more), so the combine folds each query row's partials in three batches of 128."""
    rng = np.random.default_rng(20000)
    T, H, Hq = 20000, 1, 4
    k, v = normal_kv(rng, T, H, D), normal_kv(rng, T, H, D)
    q = bf16_bits(rng.standard_normal((Hq, D)))
    gk_, gv_, ok, ov = packed_pair(k, v, fmt, gk, gv)
    out = kvq.decode_attention(to_dev(q), gk_, gv_).cpu().numpy()
    kr, vr = reconstruct(ok), reconstruct(ov)
    want = decode_attention(q, kr, vr, 1.0 / np.sqrt(D))
    check(out, want, np.abs(oracle.bf16_to_f32(vr)).max(), f"{fmt} T={T} H={H}")
    out0 = kvq.decode_attention(torch.zeros((Hq, D), dtype=torch.bfloat16, device=dev()), gk_, gv_).cpu().numpy()
    vf = oracle.bf16_to_f32(vr).astype(np.float64)
    np.testing.assert_allclose(out0, np.repeat(vf.mean(axis=0), Hq, axis=0), rtol=0, atol=2e-6 * np.abs(vf).max())


@pytest.mark.parametrize("fmt,gk,gv", FORMS)
@pytest.mark.parametrize("T", [16, 333, 5000])
def test_zero_query_is_mean_of_v(fmt, gk, gv, T):
    rng = np.random.default_rng(T)
    H, Hq = 2, 8
    k, v = normal_kv(rng, T, H, D), normal_kv(rng, T, H, D)
    gk_, gv_, ok, ov = packed_pair(k, v, fmt, gk, gv)
    out = kvq.decode_attention(torch.zeros((Hq, D), dtype=torch.bfloat16, device=dev()), gk_, gv_).cpu().numpy()
    vr = oracle.bf16_to_f32(reconstruct(ov)).astype(np.float64)
    want = np.repeat(vr.mean(axis=0), Hq // H, axis=0)
    np.testing.assert_allclose(out, want, rtol=0, atol=2e-6 * np.abs(vr).max())


@pytest.mark.parametrize("fmt,gk,gv", FORMS)
def test_one_dominant_key_selects_its_value(fmt, gk, gv):
    rng = np.random.default_rng(5)
    T, H, Hq = 700, 2, 4
    k = normal_kv(rng, T, H, D) * 0  # zero keys ...
    kf = np.zeros((T, H, D))
    for h in range(H):
        kf[123 + 200 * h, h, 5 + h] = 8.0  # ... except one token per head, on one channel
    k = bf16_bits(kf)
    v = normal_kv(rng, T, H, D)
    q = np.zeros((Hq, D))
    for hq in range(Hq):
        q[hq, 5 + hq // 2] = 60.0  # scores 60 * 8 / sqrt(128) ~ 42 above the rest
    gk_, gv_, ok, ov = packed_pair(k, v, fmt, gk, gv)
    out = kvq.decode_attention(to_dev(bf16_bits(q)), gk_, gv_).cpu().numpy()
    kr = oracle.bf16_to_f32(reconstruct(ok)).astype(np.float64)
    vr = oracle.bf16_to_f32(reconstruct(ov)).astype(np.float64)
    for hq in range(Hq):
        h = hq // 2
        t = int(np.argmax(kr[:, h, 5 + h]))
        assert t == 123 + 200 * h
        np.testing.assert_allclose(out[hq], vr[t, h], rtol=0, atol=1e-5 * np.abs(vr).max())


@pytest.mark.parametrize("bfmt,rfmt", [("int4", "int4"), ("nvfp4", "int4"), ("int4", "nvfp4"), ("fp8_row", "int4"),
                                       ("int4", "fp8_row"), ("nvfp4_row", "nvfp4_row"), ("fp8_row", "nvfp4"),
                                       ("nvfp4", "nvfp4_row")])
def test_fused_residual_reconstruction(bfmt, rfmt):
    rng = np.random.default_rng(9)
    T, H, Hq = 900, 2, 16
    g = {"int4": (64, 64), "nvfp4": (16, 16), "nvfp4_row": (16, 16), "fp8_row": (0, 0)}
    k0, v0 = normal_kv(rng, T, H, D), normal_kv(rng, T, H, D)
    k1 = bf16_bits(oracle.bf16_to_f32(k0).astype(np.float64) + 0.1 * rng.standard_normal(k0.shape))
    v1 = bf16_bits(oracle.bf16_to_f32(v0).astype(np.float64) + 0.1 * rng.standard_normal(v0.shape))
    gk0, gv0, ok0, ov0 = packed_pair(k0, v0, bfmt, *g[bfmt])
    rk0, rv0 = kvq.unpack(gk0), kvq.unpack(gv0)
    grk = kvq.encode_residual(to_dev(k1), rk0, "key", rfmt, g[rfmt][0])
    grv = kvq.encode_residual(to_dev(v1), rv0, "value", rfmt, g[rfmt][1])
    ork = oracle.encode_residual(k1, oracle.unpack(ok0), "key", rfmt, g[rfmt][0])
    orv = oracle.encode_residual(v1, oracle.unpack(ov0), "value", rfmt, g[rfmt][1])
    q = bf16_bits(rng.standard_normal((Hq, D)))
    out = kvq.decode_attention(to_dev(q), gk0, gv0, grk, grv).cpu().numpy()
    kr, vr = reconstruct(ok0, ork), reconstruct(ov0, orv)
    want = decode_attention(q, kr, vr, 1.0 / np.sqrt(D))
    check(out, want, np.abs(oracle.bf16_to_f32(vr)).max(), f"{bfmt}+{rfmt}")


@pytest.mark.parametrize("fmt,gk,gv", [("int4", 64, 64), ("nvfp4", 16, 16), ("nvfp4_row", 16, 16), ("fp8_row", 0, 0)])
def test_bulk_shape(fmt, gk, gv):
    """The bench's shape: T = 131072 tokens, 8 KV heads, 64 query heads (heavy-tailed data)."""
    T, H, Hq = 131072, 8, 64
    d = c4_tensors(0, T=T)
    k, v = d["K"], d["V"]
    rng = np.random.default_rng(1)
    q = bf16_bits(rng.standard_normal((Hq, D)))
    gk_, gv_, ok, ov = packed_pair(k, v, fmt, gk, gv)
    out = kvq.decode_attention(to_dev(q), gk_, gv_).cpu().numpy()
    # the packed planes are the oracle's (checked elsewhere at this size); the reference reads them
    kr, vr = reconstruct(ok), reconstruct(ov)
    want = decode_attention(q, kr, vr, 1.0 / np.sqrt(D))
    check(out, want, np.abs(oracle.bf16_to_f32(vr)).max(), f"bulk {fmt}")


def forms_for(d):
    """Formats at head dim d: an INT4 VALUE group spans d/16 to d channels."""
    if d == 64:
        return [("int4", 64, 64), ("int4", 16, 8), ("int4", 128, 32), ("nvfp4", 16, 16), ("nvfp4_row", 16, 16),
                ("fp8_row", 0, 0)]
    return [("int4", 64, 64), ("int4", 16, 16), ("int4", 128, 256), ("nvfp4", 16, 16), ("nvfp4_row", 16, 16),
            ("fp8_row", 0, 0)]


HEAD_DIM_CASES = [(d, *f) for d in (64, 256) for f in forms_for(d)]


@pytest.mark.parametrize("d,fmt,gk,gv", HEAD_DIM_CASES)
@pytest.mark.parametrize("T,H,Hq", [(1, 1, 1), (17, 1, 16), (333, 2, 8), (4099, 4, 8), (600, 1, 40)])
def test_head_dims_vs_oracle(d, fmt, gk, gv, T, H, Hq):
    """Head dims 64 and 256: the same kernels at their own per-lane geometry (the K lane group
    covers d/4 channels, each V lane d/16)."""
    rng = np.random.default_rng(T * 3 + Hq + d)
    k, v = normal_kv(rng, T, H, d), normal_kv(rng, T, H, d)
    q = bf16_bits(rng.standard_normal((Hq, d)))
    gk_, gv_, ok, ov = packed_pair(k, v, fmt, gk, gv)
    out = kvq.decode_attention(to_dev(q), gk_, gv_).cpu().numpy()
    assert out.shape == (Hq, d)
    kr, vr = reconstruct(ok), reconstruct(ov)
    want = decode_attention(q, kr, vr, 1.0 / np.sqrt(d))
    check(out, want, np.abs(oracle.bf16_to_f32(vr)).max(), f"D={d} {fmt} T={T} Hq={Hq}")


@pytest.mark.parametrize("d,fmt,gk,gv", HEAD_DIM_CASES)
def test_head_dims_zero_query_is_mean_of_v(d, fmt, gk, gv):
    rng = np.random.default_rng(d)
    T, H, Hq = 1000, 2, 8
    k, v = normal_kv(rng, T, H, d), normal_kv(rng, T, H, d)
    gk_, gv_, ok, ov = packed_pair(k, v, fmt, gk, gv)
    out = kvq.decode_attention(torch.zeros((Hq, d), dtype=torch.bfloat16, device=dev()), gk_, gv_).cpu().numpy()
    vr = oracle.bf16_to_f32(reconstruct(ov)).astype(np.float64)
    want = np.repeat(vr.mean(axis=0), Hq // H, axis=0)
    np.testing.assert_allclose(out, want, rtol=0, atol=2e-6 * np.abs(vr).max())


@pytest.mark.parametrize("d", [64, 256])
@pytest.mark.parametrize("bfmt,rfmt", [("int4", "int4"), ("nvfp4", "nvfp4_row"), ("fp8_row", "int4"),
                                       ("nvfp4_row", "fp8_row")])
def test_head_dims_fused_residual(d, bfmt, rfmt):
    rng = np.random.default_rng(d + 1)
    T, H, Hq = 700, 2, 16
    g = {"int4": (64, 64), "nvfp4": (16, 16), "nvfp4_row": (16, 16), "fp8_row": (0, 0)}
    k0, v0 = normal_kv(rng, T, H, d), normal_kv(rng, T, H, d)
    k1 = bf16_bits(oracle.bf16_to_f32(k0).astype(np.float64) + 0.1 * rng.standard_normal(k0.shape))
    v1 = bf16_bits(oracle.bf16_to_f32(v0).astype(np.float64) + 0.1 * rng.standard_normal(v0.shape))
    gk0, gv0, ok0, ov0 = packed_pair(k0, v0, bfmt, *g[bfmt])
    grk = kvq.encode_residual(to_dev(k1), kvq.unpack(gk0), "key", rfmt, g[rfmt][0])
    grv = kvq.encode_residual(to_dev(v1), kvq.unpack(gv0), "value", rfmt, g[rfmt][1])
    ork = oracle.encode_residual(k1, oracle.unpack(ok0), "key", rfmt, g[rfmt][0])
    orv = oracle.encode_residual(v1, oracle.unpack(ov0), "value", rfmt, g[rfmt][1])
    q = bf16_bits(rng.standard_normal((Hq, d)))
    out = kvq.decode_attention(to_dev(q), gk0, gv0, grk, grv).cpu().numpy()
    kr, vr = reconstruct(ok0, ork), reconstruct(ov0, orv)
    want = decode_attention(q, kr, vr, 1.0 / np.sqrt(d))
    check(out, want, np.abs(oracle.bf16_to_f32(vr)).max(), f"D={d} {bfmt}+{rfmt}")


@pytest.mark.parametrize("fmt,gk,gv", [("int4", 64, 64), ("nvfp4", 16, 16)])
def test_head_dim_256_large(fmt, gk, gv):
    """Head dim 256 at a long context: T = 32768 tokens, 4 KV heads, 32 query heads (many token
    blocks per KV head, 8 query heads per KV head)."""
    T, H, Hq, d = 32768, 4, 32, 256
    rng = np.random.default_rng(256)
    k, v = normal_kv(rng, T, H, d), normal_kv(rng, T, H, d)
    q = bf16_bits(rng.standard_normal((Hq, d)))
    gk_, gv_, ok, ov = packed_pair(k, v, fmt, gk, gv)
    out = kvq.decode_attention(to_dev(q), gk_, gv_).cpu().numpy()
    kr, vr = reconstruct(ok), reconstruct(ov)
    want = decode_attention(q, kr, vr, 1.0 / np.sqrt(d))
    check(out, want, np.abs(oracle.bf16_to_f32(vr)).max(), f"D=256 large {fmt}")


N_RANDOM = 48


def draw_attention_case(i):
    """A seeded draw over everything the kernels take: format, K and V group sizes within the
    kernel's constraints, head dim, tokens (ragged against 16-token sub-tiles and 64-token
    blocks), KV heads, query heads per KV head (including tiles past 16 rows), and an optional
    residual of any format."""
    rng = np.random.default_rng(7000 + i)
    d = int(rng.choice([64, 128, 256]))
    fmts = ["int4", "nvfp4", "nvfp4_row", "fp8_row"]

    def groups(fmt):
        if fmt == "int4":
            vg = [g for g in (8, 16, 32, 64, 128, 256) if max(8, d // 16) <= g <= d]
            return int(rng.choice([16, 32, 64, 128])), int(rng.choice(vg))
        return (16, 16) if fmt in ("nvfp4", "nvfp4_row") else (0, 0)

    fmt = fmts[i % 4]
    gk, gv = groups(fmt)
    res = None
    if rng.integers(0, 3) == 0:
        rfmt = fmts[int(rng.integers(0, 4))]
        res = (rfmt, *groups(rfmt))
    H = int(rng.integers(1, 5))
    rep = int(rng.choice([1, 2, 4, 8, 16, 20]))
    T = int(rng.integers(1, 3000))
    return dict(seed=7000 + i, d=d, fmt=fmt, gk=gk, gv=gv, res=res, H=H, Hq=H * rep, T=T)


@pytest.mark.parametrize("i", range(N_RANDOM))
def test_random_attention_vs_oracle(i):
    c = draw_attention_case(i)
    rng = np.random.default_rng(c["seed"])
    d, T, H, Hq, fmt, gk, gv = c["d"], c["T"], c["H"], c["Hq"], c["fmt"], c["gk"], c["gv"]
    k0, v0 = normal_kv(rng, T, H, d), normal_kv(rng, T, H, d)
    q = bf16_bits(rng.standard_normal((Hq, d)))
    gk0, gv0, ok0, ov0 = packed_pair(k0, v0, fmt, gk, gv)
    if c["res"] is None:
        out = kvq.decode_attention(to_dev(q), gk0, gv0).cpu().numpy()
        kr, vr = reconstruct(ok0), reconstruct(ov0)
    else:
        rfmt, rgk, rgv = c["res"]
        k1 = bf16_bits(oracle.bf16_to_f32(k0).astype(np.float64) + 0.1 * rng.standard_normal(k0.shape))
        v1 = bf16_bits(oracle.bf16_to_f32(v0).astype(np.float64) + 0.1 * rng.standard_normal(v0.shape))
        grk = kvq.encode_residual(to_dev(k1), kvq.unpack(gk0), "key", rfmt, rgk)
        grv = kvq.encode_residual(to_dev(v1), kvq.unpack(gv0), "value", rfmt, rgv)
        ork = oracle.encode_residual(k1, oracle.unpack(ok0), "key", rfmt, rgk)
        orv = oracle.encode_residual(v1, oracle.unpack(ov0), "value", rfmt, rgv)
        out = kvq.decode_attention(to_dev(q), gk0, gv0, grk, grv).cpu().numpy()
        kr, vr = reconstruct(ok0, ork), reconstruct(ov0, orv)
    want = decode_attention(q, kr, vr, 1.0 / np.sqrt(d))
    check(out, want, np.abs(oracle.bf16_to_f32(vr)).max(), f"case {i} {c}")
