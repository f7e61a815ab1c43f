"""GPU parity for short rows: tensors whose (token, head) rows hold fewer than 64 chunks of 8
channels (H * D / 8 in {1, 2, 4, 8, 16, 32}), where the vector kernels split a wave's lanes into
groups that each take their own row tile (or, for KEY encodes, their own token group). This is
the per-GPU shape of head sharding ([T, 1, 128] for one KV head) and of models with few KV
heads. Everything is compared with the oracle bit for bit: packed planes, decoded values, dense
and sparse residuals (unsorted positions), paged views, and slot writes and reads; ragged token
counts leave lane groups past the last tile, which must store nothing.
"""

import numpy as np
import pytest
import torch

import kv_cache_quantization_kvq_amd as kvq
import oracle
from gpu_util import assert_bits_equal, assert_same_packed, dev, planes, to_dev, to_host
from workloads import normal_kv

pytestmark = pytest.mark.gpu

KINDS = ["key", "value"]

SHORT = [
    (1000, 1, 128, "int4", 64),   # one KV head of a D=128 model: 16 chunks, 4 lane groups
    (77, 1, 128, "int4", 16),     # ragged, K G16
    (8, 1, 128, "int4", 16),      # fewer rows than lane groups can take
    (333, 1, 64, "int4", 32),     # 8 chunks, 8 lane groups
    (129, 2, 128, "int4", 128),   # 32 chunks, 2 lane groups, G128
    (65, 1, 8, "int4", 8),        # one chunk per row: 64 lane groups
    (130, 4, 8, "int4", 8),       # 4 chunks per row
    (1000, 1, 128, "nvfp4", 16),
    (50, 2, 64, "nvfp4", 16),
    (3, 1, 16, "nvfp4", 16),
    (1000, 1, 128, "nvfp4_row", 16),
    (77, 2, 64, "nvfp4_row", 16),
    (1000, 1, 128, "fp8_row", 0),
    (9, 1, 32, "fp8_row", 0),
]


@pytest.mark.parametrize("T,H,D,fmt,G", SHORT)
@pytest.mark.parametrize("kind", KINDS)
def test_short_rows(T, H, D, fmt, G, kind):
    rng = np.random.default_rng(T * 7 + H * 131 + D)
    x = normal_kv(rng, T, H, D)
    x[rng.random(x.shape) < 0.02] = 0x8000
    gp = kvq.pack(to_dev(x), kind, fmt, G)
    op = oracle.pack(x, kind, fmt, G)
    assert_same_packed(gp, op, f"{(T, H, D, fmt, G, kind)}")
    assert_bits_equal(to_host(kvq.unpack(gp)), oracle.unpack(op), "decoded")
    p = normal_kv(rng, T, H, D)
    gr = kvq.encode_residual(to_dev(x), to_dev(p), kind, fmt, G)
    orr = oracle.encode_residual(x, p, kind, fmt, G)
    assert_same_packed(gr, orr, "residual")
    assert_bits_equal(to_host(kvq.decode_residual(gr, to_dev(p))), oracle.decode_residual(orr, p), "decode")
    pos = rng.permutation(T)[: max(1, T // 3)].astype(np.int32)
    gs = kvq.encode_residual(to_dev(x), to_dev(p), kind, fmt, G, positions=torch.from_numpy(pos).to(dev()))
    osr = oracle.encode_residual(x, p, kind, fmt, G, positions=pos)
    assert_same_packed(gs, osr, "sparse residual")
    assert_bits_equal(to_host(kvq.decode_residual(gs, to_dev(p))), oracle.decode_residual(osr, p), "sparse decode")


@pytest.mark.parametrize("fmt,kind,G,local", [("int4", "key", 16, True), ("int4", "key", 64, False),
                                              ("int4", "value", 64, False), ("nvfp4", "key", 16, True),
                                              ("fp8_row", "value", 0, False)])
def test_short_rows_paged(fmt, kind, G, local):
    P, S, H, D = 9, 16, 1, 128
    rng = np.random.default_rng(11)
    x4 = normal_kv(rng, P * S, H, D).reshape(P, S, H, D)
    gp = kvq.pack_paged(to_dev(x4), kind, fmt, G, page_local=local)
    op = oracle.pack_paged(x4, kind, fmt, G, page_local=local)
    g, o = planes(gp), planes(op)
    for k in o:
        assert_bits_equal(g[k].reshape(-1), o[k].reshape(-1), f"paged {k}")
    assert_bits_equal(to_host(kvq.unpack_paged(gp, page_size=S)), oracle.unpack_paged(op, P, S), "unpack_paged")


@pytest.mark.parametrize("fmt,kind,G", [("int4", "value", 64), ("nvfp4_row", "key", 16), ("fp8_row", "value", 0)])
def test_short_rows_slots(fmt, kind, G):
    rng = np.random.default_rng(3)
    n_slots, H, D, N = 300, 1, 128, 37
    base = normal_kv(rng, n_slots, H, D)
    cache = kvq.pack(to_dev(base), kind, fmt, G)
    ocache = oracle.pack(base, kind, fmt, G)
    new = normal_kv(rng, N, H, D)
    slots = rng.choice(n_slots, N, replace=False).astype(np.int32)
    kvq.store_rows(cache, to_dev(new), torch.from_numpy(slots).to(dev()))
    oracle.store_rows(ocache, new, slots)
    g, o = planes(cache), planes(ocache)
    for k in o:
        assert_bits_equal(g[k], o[k], f"store_rows {k}")
    rd = rng.choice(n_slots, 61, replace=True).astype(np.int32)
    got = to_host(kvq.load_rows(cache, torch.from_numpy(rd).to(dev())))
    assert_bits_equal(got, oracle.load_rows(ocache, rd), "load_rows")
