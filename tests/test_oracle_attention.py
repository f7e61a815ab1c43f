"""Pins of the decode-attention oracle (CPU only).

What pins it:
  * torch's own scaled_dot_product_attention in float64 on the CPU (a library routine, with
    grouped-query heads expanded by repeat_interleave) gives the same output;
  * closed forms: equal scores give the plain mean of V over the tokens; one score far above
    the others selects that token's V row; a single token returns its V row;
  * the grouped-query map: query head hq uses KV head hq // (Hq / H) (changing KV head 1 moves
    exactly the query heads of group 1);
  * reconstruct() is the codec's own decode (unpack, or decode_residual on top of it).
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import decode_attention, reconstruct
from workloads import bf16_bits, normal_kv


@pytest.mark.parametrize("T,H,Hq,D", [(1, 1, 1, 8), (37, 2, 8, 16), (200, 4, 16, 64), (64, 1, 4, 128)])
def test_matches_torch_sdpa_float64(T, H, Hq, D):
    rng = np.random.default_rng(T + Hq)
    q = bf16_bits(rng.standard_normal((Hq, D)))
    k = normal_kv(rng, T, H, D)
    v = normal_kv(rng, T, H, D)
    scale = 1.0 / np.sqrt(D)
    got = decode_attention(q, k, v, scale)
    qt = torch.from_numpy(oracle.bf16_to_f32(q).astype(np.float64))[:, None, :]       # [Hq, 1, D]
    kt = torch.from_numpy(oracle.bf16_to_f32(k).astype(np.float64)).permute(1, 0, 2)  # [H, T, D]
    vt = torch.from_numpy(oracle.bf16_to_f32(v).astype(np.float64)).permute(1, 0, 2)
    rep = Hq // H
    kt = kt.repeat_interleave(rep, dim=0)
    vt = vt.repeat_interleave(rep, dim=0)
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)[:, 0, :].numpy()
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(1)
    T, D = 50, 16
    v = normal_kv(rng, T, 1, D)
    vf = oracle.bf16_to_f32(v).astype(np.float64)[:, 0]
    # zero query: equal scores -> mean of V
    q0 = np.zeros((1, D), np.uint16)
    k = normal_kv(rng, T, 1, D)
    np.testing.assert_allclose(decode_attention(q0, k, v, 1.0)[0], vf.mean(0), rtol=1e-13, atol=1e-15)
    # one key aligned with a huge query dominates: output = that token's V row
    kk = np.zeros((T, 1, D), np.float64)
    kk[17, 0, 3] = 1.0
    qq = np.zeros((1, D))
    qq[0, 3] = 1000.0
    out = decode_attention(bf16_bits(qq), bf16_bits(kk), v, 1.0)
    np.testing.assert_allclose(out[0], vf[17], rtol=0, atol=1e-12)
    # a single token
    np.testing.assert_allclose(decode_attention(bf16_bits(qq), bf16_bits(kk[:1]), v[:1], 0.3)[0], vf[0], atol=0)


def test_grouped_query_heads():
    rng = np.random.default_rng(2)
    T, H, Hq, D = 30, 3, 6, 8
    q = bf16_bits(rng.standard_normal((Hq, D)))
    k = normal_kv(rng, T, H, D)
    v = normal_kv(rng, T, H, D)
    a = decode_attention(q, k, v, 0.5)
    v2 = v.copy()
    v2[:, 1] = normal_kv(rng, T, 1, D)[:, 0]
    b = decode_attention(q, k, v2, 0.5)
    moved = np.any(a != b, axis=1)
    assert list(moved) == [False, False, True, True, False, False]


@pytest.mark.parametrize("fmt,G", [("int4", 64), ("nvfp4", 16)])
def test_reconstruct_is_codec_decode(fmt, G):
    rng = np.random.default_rng(3)
    x0 = normal_kv(rng, 70, 2, 32)
    x1 = bf16_bits(oracle.bf16_to_f32(x0).astype(np.float64) + 0.1 * rng.standard_normal(x0.shape))
    base = oracle.pack(x0, "key", fmt, G)
    r0 = oracle.unpack(base)
    res = oracle.encode_residual(x1, r0, "key", fmt, G)
    np.testing.assert_array_equal(reconstruct(base), r0)
    np.testing.assert_array_equal(reconstruct(base, res), oracle.decode_residual(res, r0))
