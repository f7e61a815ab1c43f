"""GPU parity of the row formats, the paged adapter and slot writes/reads: the HIP library
through its C ABI against the CPU oracle, bit for bit.

Row formats (NVFP4 and FP8 with one FP32 scale per (token, head) row) cover the vector path
(head_dim 8 ... 512, a power of two) and the generic path (other head_dims), magnitude decades,
zero and signed-zero rows, bf16 subnormals, and rows whose FP8 scale falls outside the
branch-free quotient's range (tiny and huge rows divide). Paged views cover flat and page-local
KEY grouping, contiguous and padded page strides; slot writes and reads cover every format that
takes them, on both kernel paths.
"""

import numpy as np
import pytest
import torch

import kv_cache_quantization_kvq_amd as kvq
import oracle
from gpu_util import assert_bits_equal, assert_same_packed, dev, planes, to_dev, to_host
from workloads import bf16_bits, normal_kv

pytestmark = pytest.mark.gpu

ROWF = [("nvfp4_row", 16), ("fp8_row", 0)]


def varied_rows(seed, T, H, D):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H, D)) * 10.0 ** rng.uniform(-3, 3, (T, H, 1))
    x[0, 0] = 0.0
    if T > 1:
        x[1, H - 1] = -0.0
    if T > 2:
        x[2, H - 1, ::3] = -0.0
    if T > 3:
        x[3, 0] *= 2.0 ** -128  # bf16 subnormals
    if T > 4:
        x[4, H - 1] *= 2.0 ** -100  # FP8 scale below 2^-90: the division path
    if T > 5:
        x[5, 0] *= 2.0 ** 110  # FP8 scale above 2^100: the division path
    if T > 6:
        x[6, H - 1, :] = 0.0
        x[6, H - 1, D // 2] = -3.0e-39
    return bf16_bits(x)


SHAPES = [(200, 4, 128), (37, 3, 64), (50, 2, 256), (20, 1, 512), (33, 5, 8), (9, 2, 16),  # vector path
          (40, 3, 40), (25, 2, 96), (16, 2, 7), (11, 1, 1024)]                              # generic path


@pytest.mark.parametrize("fmt,G", ROWF)
@pytest.mark.parametrize("kind", ["key", "value"])
@pytest.mark.parametrize("shape", SHAPES)
def test_row_format_roundtrip(fmt, G, kind, shape):
    x = varied_rows(sum(shape), *shape)
    gp = kvq.pack(to_dev(x), kind, fmt, G)
    op = oracle.pack(x, kind, fmt, G)
    assert_same_packed(gp, op, f"{fmt} {kind} {shape}")
    assert_bits_equal(to_host(kvq.unpack(gp)), oracle.unpack(op), f"{fmt} {kind} {shape} decoded")
    assert gp.nbytes() == kvq.storage_bytes(fmt, kind, G, *shape) == oracle.storage_bytes(fmt, kind, G, *shape)


@pytest.mark.parametrize("fmt,G", ROWF)
def test_row_format_strided_view(fmt, G):
    T, H, D = 64, 4, 128
    qkv = normal_kv(np.random.default_rng(3), T, 3 * H, D).reshape(T, 3, H, D)
    view = qkv[:, 1]  # K of a fused QKV buffer
    qd = to_dev(qkv)
    gp = kvq.pack(qd[:, 1], "key", fmt, G)
    op = oracle.pack(view, "key", fmt, G)
    assert_same_packed(gp, op, f"{fmt} strided")


@pytest.mark.parametrize("fmt,G", ROWF)
@pytest.mark.parametrize("base", [("int4", 64), ("nvfp4", 16), ("fp8_row", 0)])
@pytest.mark.parametrize("shape", [(96, 4, 128), (30, 3, 40)])
def test_row_format_residual_chain(fmt, G, base, shape):
    rng = np.random.default_rng(11)
    X0 = normal_kv(rng, *shape)
    X1 = bf16_bits(oracle.bf16_to_f32(X0).astype(np.float64) + 0.1 * rng.standard_normal(shape))
    R0d = kvq.unpack(kvq.pack(to_dev(X0), "value", *base))
    R0o = oracle.unpack(oracle.pack(X0, "value", *base))
    assert_bits_equal(to_host(R0d), R0o, "base")
    X1d = to_dev(X1)
    # dense
    gr = kvq.encode_residual(X1d, R0d, "key", fmt, G)
    orr = oracle.encode_residual(X1, R0o, "key", fmt, G)
    assert_same_packed(gr, orr, "dense residual")
    assert_bits_equal(to_host(kvq.decode_residual(gr, R0d)), oracle.decode_residual(orr, R0o), "dense decode")
    # sparse, unsorted positions
    pos = rng.choice(shape[0], shape[0] // 3, replace=False).astype(np.int32)
    gs = kvq.encode_residual(X1d, R0d, "value", fmt, G, positions=torch.from_numpy(pos).to(dev()))
    os_ = oracle.encode_residual(X1, R0o, "value", fmt, G, positions=pos)
    assert_same_packed(gs, os_, "sparse residual")
    assert_bits_equal(to_host(kvq.decode_residual(gs, R0d)), oracle.decode_residual(os_, R0o), "sparse decode")


def paged_input(seed, P, S, H, D, pad):
    """Pages of S slots inside a buffer of S + pad slots per page (pad > 0: padded page stride)."""
    buf = normal_kv(np.random.default_rng(seed), P * (S + pad), H, D).reshape(P, S + pad, H, D)
    return buf


PAGED = [("int4", "key", 64, 16, True), ("int4", "key", 64, 16, False), ("int4", "key", 16, 32, True),
         ("int4", "key", 32, 128, True), ("int4", "value", 64, 16, True), ("nvfp4", "key", 16, 16, True),
         ("nvfp4", "key", 16, 32, False), ("nvfp4", "value", 16, 16, False), ("nvfp4_row", "key", 16, 16, True),
         ("fp8_row", "value", 0, 16, False)]


@pytest.mark.parametrize("fmt,kind,G,S,local", PAGED)
@pytest.mark.parametrize("pad", [0, 4])
def test_pack_paged(fmt, kind, G, S, local, pad):
    P, H, D = 12, 2, 128
    buf = paged_input(P * S + pad, P, S, H, D, pad)
    bd = to_dev(buf)
    x4d, x4 = bd[:, :S], buf[:, :S]
    gp = kvq.pack_paged(x4d, kind, fmt, G, page_local=local)
    op = oracle.pack_paged(x4, kind, fmt, G, page_local=local)
    g, o = planes(gp), planes(op)
    for k in o:
        assert_bits_equal(g[k].reshape(-1), o[k].reshape(-1), f"paged {k}")
    assert gp.rows == P * S
    if local and kind == "key" and fmt == "int4":
        assert gp.group_size == min(G, S)
    # unpack into the same padded layout: padding keeps its contents
    out = torch.full((P, S + pad, H, D), -7.0, dtype=torch.bfloat16, device=dev())
    kvq.unpack_paged(gp, out[:, :S])
    got = to_host(out)
    want = oracle.unpack_paged(op, P, S)
    assert_bits_equal(got[:, :S], want, "unpack_paged")
    if pad:
        assert np.all(got[:, S:] == bf16_bits(np.array(-7.0)))


SLOT_FORMS = [("int4", "value", 64), ("int4", "value", 16), ("nvfp4_row", "key", 16), ("fp8_row", "value", 0)]


@pytest.mark.parametrize("fmt,kind,G", SLOT_FORMS)
@pytest.mark.parametrize("D,N", [(128, 300), (128, 5), (64, 40), (40, 17)])
def test_store_and_load_rows(fmt, kind, G, D, N):
    if fmt == "int4" and D % G:
        G = 8
    rng = np.random.default_rng(D + N)
    n_slots, H = 512, 4
    base = normal_kv(rng, n_slots, H, D)
    cache = kvq.pack(to_dev(base), kind, fmt, G)
    ocache = oracle.pack(base, kind, fmt, G)
    new = varied_rows(N, N, H, D)
    slots = rng.choice(n_slots, N, replace=False).astype(np.int32)
    sd = torch.from_numpy(slots).to(dev())
    kvq.store_rows(cache, to_dev(new), sd)
    oracle.store_rows(ocache, new, slots)
    g, o = planes(cache), planes(ocache)
    for k in o:
        assert_bits_equal(g[k], o[k], f"store_rows {k}")
    rd = rng.choice(n_slots, 97, replace=True).astype(np.int32)  # reads may repeat
    got = to_host(kvq.load_rows(cache, torch.from_numpy(rd).to(dev())))
    assert_bits_equal(got, oracle.load_rows(ocache, rd), "load_rows")


@pytest.mark.parametrize("fmt,kind,G", [("int4", "key", 64), ("nvfp4", "key", 16), ("nvfp4", "value", 16),
                                        ("int4", "key", 128)])
def test_load_rows_token_grouped_and_tensor_formats(fmt, kind, G):
    rng = np.random.default_rng(5)
    x = normal_kv(rng, 400, 4, 128)
    cache = kvq.pack(to_dev(x), kind, fmt, G)
    ocache = oracle.pack(x, kind, fmt, G)
    rd = rng.choice(400, 150, replace=False).astype(np.int32)
    got = to_host(kvq.load_rows(cache, torch.from_numpy(rd).to(dev())))
    assert_bits_equal(got, oracle.load_rows(ocache, rd), "load_rows")


def test_store_rows_into_slots_of_a_paged_pool_round_trip():
    # a page-major pool of fp8 rows: write one new token per sequence into its page slot, then
    # read the whole pool back as pages
    P, S, H, D = 16, 16, 8, 128
    rng = np.random.default_rng(9)
    pool = normal_kv(rng, P * S, H, D)
    cache = kvq.pack(to_dev(pool), "key", "fp8_row", 0)
    ocache = oracle.pack(pool, "key", "fp8_row", 0)
    new = normal_kv(rng, P, H, D)
    slots = (np.arange(P) * S + rng.integers(0, S, P)).astype(np.int32)
    kvq.store_rows(cache, to_dev(new), torch.from_numpy(slots).to(dev()))
    oracle.store_rows(ocache, new, slots)
    assert_bits_equal(to_host(kvq.unpack_paged(cache, page_size=S)), oracle.unpack_paged(ocache, P, S), "pool")


WIN_FORMS = [("int4", 64), ("int4", 16), ("nvfp4", 16), ("nvfp4_row", 16), ("fp8_row", 0)]


@pytest.mark.parametrize("fmt,G", WIN_FORMS)
@pytest.mark.parametrize("kind", ["key", "value"])
@pytest.mark.parametrize("T,sink,recent", [(300, 4, 16), (97, 4, 16), (20, 4, 16), (7, 4, 16), (64, 0, 0)])
def test_window_pack_and_residual(fmt, G, kind, T, sink, recent):
    rng = np.random.default_rng(T + 3)
    H, D = 4, 128
    x0 = normal_kv(rng, T, H, D)
    x1 = bf16_bits(oracle.bf16_to_f32(x0).astype(np.float64) + 0.1 * rng.standard_normal((T, H, D)))
    x0d, x1d = to_dev(x0), to_dev(x1)
    # plain pack with a window
    gw = kvq.encode_window(x0d, kind, fmt, G, sink, recent)
    ow = oracle.encode_window(x0, kind, fmt, G, sink, recent)
    assert_same_packed(gw.packed, ow.packed, "window payload")
    assert_bits_equal(to_host(gw.window), ow.window, "window rows")
    R0d = kvq.decode_window(gw)
    R0o = oracle.decode_window(ow)
    assert_bits_equal(to_host(R0d), R0o, "window decode")
    # residual with a window, decoded in place into a copy of prev
    gr = kvq.encode_window(x1d, kind, fmt, G, sink, recent, previous=R0d)
    orr = oracle.encode_window(x1, kind, fmt, G, sink, recent, prev=R0o)
    assert_same_packed(gr.packed, orr.packed, "window residual payload")
    assert_bits_equal(to_host(gr.window), orr.window, "window residual rows")
    buf = R0d.clone()
    kvq.decode_window(gr, previous=buf, out=buf)
    assert_bits_equal(to_host(buf), oracle.decode_window(orr, prev=R0o), "window residual decode")


# The protected-row copy runs inside the encode / decode launch when both take the vector path
# (blocks appended to the grid, 256 chunks of 8 channels per wave), and as a launch of its own
# otherwise (INT4 G=5 takes the generic encoder; an all-window tensor has no encode).
@pytest.mark.parametrize("fmt,G,kind", [("int4", 64, "key"), ("int4", 64, "value"), ("nvfp4", 16, "key"),
                                        ("nvfp4", 16, "value"), ("nvfp4_row", 16, "key"), ("fp8_row", 0, "value"),
                                        ("int4", 5, "key")])
@pytest.mark.parametrize("T,sink,recent,H,D", [(2100, 5, 999, 8, 128), (1040, 1, 1, 8, 128), (700, 4, 16, 1, 128),
                                               (700, 4, 16, 2, 64), (300, 3, 40, 2, 256)])
def test_window_copy_in_launch(fmt, G, kind, T, sink, recent, H, D):
    # H = 1, D = 128 and H = 2, D = 64 (16 chunks per row) run the short-row (lane group) kernels
    # with the copy appended
    rng = np.random.default_rng(T + sink)
    x0 = normal_kv(rng, T, H, D)
    x1 = bf16_bits(oracle.bf16_to_f32(x0).astype(np.float64) + 0.1 * rng.standard_normal((T, H, D)))
    # current as the middle third of a fused [T, 3, H, D] buffer (token pitch 3HD)
    fused = torch.zeros((T, 3, H, D), dtype=torch.bfloat16, device=dev())
    fused[:, 1] = to_dev(x1)
    x1d = fused[:, 1]
    x0d = to_dev(x0)
    gw = kvq.encode_window(x0d, kind, fmt, G, sink, recent)
    ow = oracle.encode_window(x0, kind, fmt, G, sink, recent)
    assert_same_packed(gw.packed, ow.packed, "window payload")
    assert_bits_equal(to_host(gw.window), ow.window, "window rows")
    R0d = kvq.decode_window(gw)
    R0o = oracle.decode_window(ow)
    assert_bits_equal(to_host(R0d), R0o, "window decode")
    gr = kvq.encode_window(x1d, kind, fmt, G, sink, recent, previous=R0d)
    orr = oracle.encode_window(x1, kind, fmt, G, sink, recent, prev=R0o)
    assert_same_packed(gr.packed, orr.packed, "window residual payload")
    assert_bits_equal(to_host(gr.window), orr.window, "window residual rows")
    # out of place into a strided view (token pitch 2HD), and in place
    wide = torch.full((T, 2, H, D), float("nan"), dtype=torch.bfloat16, device=dev())
    kvq.decode_window(gr, previous=R0d, out=wide[:, 0])
    want = oracle.decode_window(orr, prev=R0o)
    assert_bits_equal(to_host(wide[:, 0].contiguous()), want, "window residual decode, strided out")
    assert torch.isnan(wide[:, 1].float()).all()
    buf = R0d.clone()
    kvq.decode_window(gr, previous=buf, out=buf)
    assert_bits_equal(to_host(buf), want, "window residual decode, in place")
