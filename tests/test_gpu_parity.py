"""GPU parity: the HIP library through its C ABI against the CPU oracle, bit for bit.

Every plane (codes, metadata, global multiplier, owned positions) and every decoded or
reconstructed bf16 output must equal the oracle's exactly. Inputs are the seeded workloads of
``workloads``; the oracle sees the same host arrays the device sees, and no expected value is
computed from a device result.
"""

import numpy as np
import pytest
import torch

import kv_cache_quantization_kvq_amd as kvq
import oracle
from gpu_util import assert_bits_equal, assert_same_packed, planes, rel_l2, to_dev, to_host
from workloads import (bf16_bits, c1_tensors, c2_tensors, c3_chain_inputs, c5_residual_targets, c5_tensors,
                       normal_kv, tiny_tensor)

pytestmark = pytest.mark.gpu

KINDS = ["key", "value"]


def roundtrip(x_bits, kind, fmt, G, xdev=None):
    """pack + unpack on both sides; returns (gpu packed, oracle packed, gpu decoded, oracle decoded)."""
    xd = to_dev(x_bits) if xdev is None else xdev
    gp = kvq.pack(xd, kind, fmt, G)
    op = oracle.pack(x_bits, kind, fmt, G)
    gy = to_host(kvq.unpack(gp))
    oy = oracle.unpack(op)
    return gp, op, gy, oy


@pytest.mark.parametrize("kind", KINDS)
def test_c1_int4_g64(kind):
    x = c1_tensors(0)["K" if kind == "key" else "V"]
    gp, op, gy, oy = roundtrip(x, kind, "int4", 64)
    assert_same_packed(gp, op, f"c1 {kind}")
    assert_bits_equal(gy, oy, f"c1 {kind} decoded")
    assert gp.nbytes() == 9216 == oracle.storage_bytes("int4", kind, 64, 128, 2, 64)


@pytest.mark.parametrize("kind", KINDS)
def test_c2_nvfp4_g16(kind):
    x = c2_tensors(0)["K" if kind == "key" else "V"]
    gp, op, gy, oy = roundtrip(x, kind, "nvfp4", 16)
    assert_same_packed(gp, op, f"c2 {kind}")
    assert_bits_equal(gy, oy, f"c2 {kind} decoded")
    assert gp.nbytes() == 2359300  # 72 B per (token, head) row + one 4 B tensor scale
    assert kvq.storage_bytes("nvfp4", "value", 16, 1, 1, 128) == 76


@pytest.mark.parametrize("kind", KINDS)
def test_c3_int4_chain_with_sparse_last_loop(kind):
    ch = c3_chain_inputs(0)
    X = ch["XK"] if kind == "key" else ch["XV"]
    pos = ch["positions"]
    # loop 0: base
    gp, op, R0g, R0o = roundtrip(X[0], kind, "int4", 64)
    assert_same_packed(gp, op, "c3 base")
    assert_bits_equal(R0g, R0o, "c3 R0")
    Rg_dev = to_dev(R0g)
    Ro = R0o
    for k in (1, 2, 3):
        sparse = k == 3
        pos_dev = torch.from_numpy(pos).to(Rg_dev.device) if sparse else None
        xk_dev = to_dev(X[k])
        gr = kvq.encode_residual(xk_dev, Rg_dev, kind, "int4", 64, positions=pos_dev)
        orr = oracle.encode_residual(X[k], Ro, kind, "int4", 64, positions=pos if sparse else None)
        assert_same_packed(gr, orr, f"c3 loop {k}")
        if sparse:
            assert gr.nbytes() == 1187840 == oracle.storage_bytes("int4", kind, 64, 2048, 8, 128, sparse=True)
        Rg_dev = kvq.decode_residual(gr, Rg_dev)
        Ro = oracle.decode_residual(orr, Ro)
        assert_bits_equal(to_host(Rg_dev), Ro, f"c3 R{k}")
    # residual chain keeps the error at the single-step level
    assert rel_l2(Ro, X[3]) < 0.2


@pytest.mark.parametrize("kind", KINDS)
def test_c5_mixed_chain_strided(kind):
    c = c5_tensors(0)
    T, H, D = c["V"].shape
    if kind == "key":
        qkv_dev = to_dev(c["QKV"])
        xdev = qkv_dev[:, H * D:2 * H * D].view(T, H, D)  # strided view, row pitch 3*H*D
        assert xdev.stride() == (3 * H * D, D, 1)
        xh = c["K"]
    else:
        xdev = to_dev(c["V"])
        xh = c["V"]
    gp, op, R0g, R0o = roundtrip(xh, kind, "nvfp4", 16, xdev=xdev)
    assert_same_packed(gp, op, f"c5 base {kind}")
    assert_bits_equal(R0g, R0o, f"c5 R0 {kind}")
    # the residual targets are built from the oracle's R0 (equal to the device's, just checked)
    tg = c5_residual_targets(R0o if kind == "key" else np.zeros_like(R0o), R0o if kind == "value" else np.zeros_like(R0o))
    X1 = tg["XK1"] if kind == "key" else tg["XV1"]
    gr = kvq.encode_residual(to_dev(X1), to_dev(R0g), kind, "int4", 32)
    orr = oracle.encode_residual(X1, R0o, kind, "int4", 32)
    assert_same_packed(gr, orr, f"c5 residual {kind}")
    # the INT4 G32 residual has zero-scale groups and f16-subnormal / underflowing scales
    s16 = planes(orr)["meta1"]
    assert np.any(s16 == 0) and np.any((s16 > 0) & (s16 < 0x0400))
    R1g = to_host(kvq.decode_residual(gr, to_dev(R0g)))
    R1o = oracle.decode_residual(orr, R0o)
    assert_bits_equal(R1g, R1o, f"c5 R1 {kind}")


@pytest.mark.parametrize("kind", KINDS)
def test_tiny_tensor_direct_division_path(kind):
    x = tiny_tensor()
    gp, op, gy, oy = roundtrip(x, kind, "nvfp4", 16)
    assert_same_packed(gp, op, f"tiny {kind}")
    assert_bits_equal(gy, oy, f"tiny {kind} decoded")


# ---- generic (non-vector) paths and ragged shapes ------------------------------------------------

SHAPES = [
    (37, 3, 40, "int4", 8),     # C8 = 15 (not a multiple of 64), partial token groups, V G8
    (100, 2, 24, "int4", 24),   # G = 24: generic V and K
    (19, 2, 7, "int4", 3),      # odd D, tiny odd G
    (50, 1, 33, "nvfp4", 16),   # odd D, partial channel blocks
    (41, 5, 64, "int4", 64),    # 41 rows: partial K group in every slab
    (70, 2, 128, "int4", 256),  # V group larger than D (one partial group per row)
    (17, 2, 16, "int4", 1),     # G = 1: every scale 0
    (130, 4, 8, "int4", 128),   # K G128 vector path with 2 partial groups
    (33, 3, 48, "int4", 16),    # V G16 with D % G == 0, C8 = 18
]


@pytest.mark.parametrize("T,H,D,fmt,G", SHAPES)
@pytest.mark.parametrize("kind", KINDS)
def test_ragged_shapes(T, H, D, fmt, G, kind):
    rng = np.random.default_rng(T * 131 + D)
    x = normal_kv(rng, T, H, D)
    x[rng.random(x.shape) < 0.02] = 0x8000
    gp, op, gy, oy = roundtrip(x, kind, fmt, G)
    assert_same_packed(gp, op, f"{(T, H, D, fmt, G, kind)}")
    assert_bits_equal(gy, oy, "decoded")
    # residual against a second tensor, dense and sparse (unsorted positions)
    p = normal_kv(rng, T, H, D)
    gr = kvq.encode_residual(to_dev(x), to_dev(p), kind, fmt, G)
    orr = oracle.encode_residual(x, p, kind, fmt, G)
    assert_same_packed(gr, orr, "residual")
    assert_bits_equal(to_host(kvq.decode_residual(gr, to_dev(p))), oracle.decode_residual(orr, p), "decode")
    pos = rng.permutation(T)[: max(1, T // 3)].astype(np.int32)
    gs = kvq.encode_residual(to_dev(x), to_dev(p), kind, fmt, G, positions=torch.from_numpy(pos).cuda())
    osr = oracle.encode_residual(x, p, kind, fmt, G, positions=pos)
    assert_same_packed(gs, osr, "sparse residual")
    assert_bits_equal(to_host(kvq.decode_residual(gs, to_dev(p))), oracle.decode_residual(osr, p), "sparse decode")


@pytest.mark.parametrize("fmt,G", [("int4", 64), ("nvfp4", 16), ("int4", 16)])
@pytest.mark.parametrize("kind", KINDS)
def test_unaligned_strides_take_generic_path(fmt, G, kind):
    # a token pitch that is not a multiple of 8 elements rules out 16-byte row loads
    rng = np.random.default_rng(11)
    T, H, D = 64, 2, 32
    buf = normal_kv(rng, T, 1, H * D + 3)[:, 0, :]
    x = buf[:, : H * D].reshape(T, H, D)
    xdev = to_dev(buf)[:, : H * D].view(T, H, D)
    assert xdev.stride(0) == H * D + 3
    gp, op, gy, oy = roundtrip(x, kind, fmt, G, xdev=xdev)
    assert_same_packed(gp, op, "unaligned")
    assert_bits_equal(gy, oy, "decoded")


@pytest.mark.parametrize("fmt,G", [("int4", 64), ("nvfp4", 16), ("fp8_row", 0)])
@pytest.mark.parametrize("kind", KINDS)
def test_head_stride_beyond_32bit_row_offsets(fmt, G, kind):
    # 16-byte aligned, but a row spans more than 2^30 elements (heads 2^30 elements apart): the
    # vector kernels address a row's elements by a 32-bit byte offset from the row start, so
    # this view must take the generic path and still match the oracle
    rng = np.random.default_rng(12)
    T, H, D = 32, 2, 64
    sh = (1 << 30) + 64
    x = normal_kv(rng, T, H, D)
    x1 = normal_kv(rng, T, H, D)
    base = torch.zeros((T - 1) * D + (H - 1) * sh + D, dtype=torch.bfloat16, device="cuda")
    view = torch.as_strided(base, (T, H, D), (D, sh, 1))
    view.copy_(to_dev(x))
    gp, op, gy, oy = roundtrip(x, kind, fmt, G, xdev=view)
    assert_same_packed(gp, op, "huge head stride")
    assert_bits_equal(gy, oy, "decoded")
    r0 = to_dev(oy)
    view.copy_(to_dev(x1))
    gr = kvq.encode_residual(view, r0, kind, fmt, G)
    orr = oracle.encode_residual(x1, oy, kind, fmt, G)
    assert_same_packed(gr, orr, "huge head stride residual")
    del base, view


@pytest.mark.parametrize("fmt,G", [("int4", 64), ("nvfp4", 16)])
@pytest.mark.parametrize("kind", KINDS)
def test_empty_tensors(fmt, G, kind):
    for shape in ((0, 8, 128), (16, 0, 128), (16, 8, 0)):
        x = np.zeros(shape, np.uint16)
        gp = kvq.pack(to_dev(x), kind, fmt, G)
        op = oracle.pack(x, kind, fmt, G)
        assert_same_packed(gp, op, f"empty {shape}")
        assert to_host(kvq.unpack(gp)).shape == shape
    # sparse residual with M = 0: decode leaves prev untouched
    p = normal_kv(np.random.default_rng(1), 32, 2, 16)
    gs = kvq.encode_residual(to_dev(p), to_dev(p), kind, fmt, G, positions=torch.zeros(0, dtype=torch.int32).cuda())
    assert gs.rows == 0
    assert_bits_equal(to_host(kvq.decode_residual(gs, to_dev(p))), p, "M=0 decode")


@pytest.mark.parametrize("kind", KINDS)
def test_ties_zeros_and_constants(kind):
    # ramp groups hit exact half-integer quotients (the exact-division fallback of INT4 codes)
    T, H, D = 128, 2, 64
    t = np.arange(T)[:, None, None]
    d = np.arange(D)[None, None, :]
    lvl = (t % 31) if kind == "key" else (d % 31)
    x = bf16_bits(np.broadcast_to(-2.0 + lvl * 0.25, (T, H, D)).copy())
    for fmt, G in (("int4", 64), ("int4", 16), ("nvfp4", 16)):
        gp, op, gy, oy = roundtrip(x, kind, fmt, G)
        assert_same_packed(gp, op, f"ramp {fmt}")
        assert_bits_equal(gy, oy, f"ramp {fmt} decoded")
    # coarse values: many members exactly between two levels
    rng = np.random.default_rng(5)
    q = bf16_bits(rng.integers(-40, 41, (T, H, D)) * 0.1)
    for fmt, G in (("int4", 64), ("int4", 32), ("nvfp4", 16)):
        gp, op, gy, oy = roundtrip(q, kind, fmt, G)
        assert_same_packed(gp, op, f"coarse {fmt}")
        assert_bits_equal(gy, oy, f"coarse {fmt} decoded")
    # zeros (signed) and constants
    z = np.zeros((T, H, D), np.uint16)
    z[::3] = 0x8000
    for fmt, G in (("int4", 64), ("nvfp4", 16)):
        gp, op, gy, oy = roundtrip(z, kind, fmt, G)
        assert_same_packed(gp, op, f"zeros {fmt}")
        assert_bits_equal(gy, oy, f"zeros {fmt} decoded")


def test_key_half_slab_degenerate_groups():
    """The INT4 G64 KEY half-slab kernel (rows of a multiple of 32 chunks, at least 64) on groups
    that take its division path: channels constant over a group (scale 0) and ranges of 2^-120
    (scales below 2^-100; larger scales than 2^100 would overflow the f16 metadata, outside the
    codec's domain), with half-integer ramps, signed zeros, coarse values with many ties, and a
    partial last group (T = 150), for the pack and a dense residual against the reconstruction."""
    T, H, D = 150, 4, 128
    rng = np.random.default_rng(77)
    x = rng.standard_normal((T, H, D))
    t = np.arange(T)[:, None]
    x[:, 0, 0:8] = 3.5                                      # constant channels
    x[:, 0, 8:16] = np.where(t % 2 == 0, 0.0, 2.0 ** -120)  # tiny ranges
    x[:, 1, :32] = -2.0 + (t % 31) * 0.25                   # ramps through half-integer quotients
    x[:, 2, :16] = np.where(t % 2 == 0, 0.0, -0.0)          # signed zeros only
    x[:, 3, 64:] = rng.integers(-40, 41, (T, 64)) * 0.1     # coarse values, many ties
    xb = bf16_bits(x)
    gp, op, gy, oy = roundtrip(xb, "key", "int4", 64)
    assert_same_packed(gp, op, "half-slab pack")
    assert_bits_equal(gy, oy, "half-slab unpack")
    x1 = bf16_bits(oracle.bf16_to_f32(xb).astype(np.float64) + 0.01 * rng.standard_normal((T, H, D)))
    x1[:, 0, 0:8] = xb[:, 0, 0:8]  # residual channels that are exactly zero
    gr = kvq.encode_residual(to_dev(x1), to_dev(gy), "key", "int4", 64)
    orr = oracle.encode_residual(x1, oy, "key", "int4", 64)
    assert_same_packed(gr, orr, "half-slab residual")
    assert_bits_equal(to_host(kvq.decode_residual(gr, to_dev(oy))), oracle.decode_residual(orr, oy),
                      "half-slab residual decode")


def test_workspace_reuse_across_calls():
    rng = np.random.default_rng(9)
    a = normal_kv(rng, 256, 8, 128)
    b = bf16_bits(oracle.bf16_to_f32(normal_kv(rng, 256, 8, 128)) * 1e-3)
    for x in (a, b, a):  # the smaller amax after the larger one must not see a stale maximum
        gp = kvq.pack(to_dev(x), "value", "nvfp4")
        op = oracle.pack(x, "value", "nvfp4")
        assert_same_packed(gp, op, "workspace reuse")


def test_in_place_sparse_decode_and_validation():
    rng = np.random.default_rng(3)
    T, H, D = 96, 4, 64
    C = normal_kv(rng, T, H, D)
    P = normal_kv(rng, T, H, D)
    pos = np.array([5, 90, 1, 33, 34, 60, 7], np.int32)
    gr = kvq.encode_residual(to_dev(C), to_dev(P), "key", "int4", 16, positions=torch.from_numpy(pos).cuda())
    orr = oracle.encode_residual(C, P, "key", "int4", 16, positions=pos)
    assert_same_packed(gr, orr, "sparse")
    pd = to_dev(P)
    out = kvq.decode_residual(gr, pd, out=pd)
    assert out.data_ptr() == pd.data_ptr()
    assert_bits_equal(to_host(pd), oracle.decode_residual(orr, P), "in place")
    st = kvq.validate_positions(torch.from_numpy(pos).cuda(), T)
    assert int(st.item()) == 0
    st = kvq.validate_positions(torch.tensor([1, 2, 96], dtype=torch.int32).cuda(), T)
    assert int(st.item()) == 1
    st = kvq.validate_positions(torch.tensor([4, 2, 4], dtype=torch.int32).cuda(), T)
    assert int(st.item()) == 2


def test_host_errors_before_launch():
    x = to_dev(normal_kv(np.random.default_rng(0), 16, 2, 16))
    with pytest.raises(kvq.KvqError) as e:
        kvq.pack(x, "key", "nvfp4", 32)
    assert e.value.status == 5
    p = kvq.pack(x, "key", "int4", 16)
    with pytest.raises(kvq.KvqError) as e:
        kvq.unpack(p, out=torch.empty((15, 2, 16), dtype=torch.bfloat16, device=x.device))
    assert e.value.status == 7
