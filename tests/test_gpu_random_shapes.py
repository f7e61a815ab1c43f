"""GPU parity over a seeded sweep of odd shapes and layouts, bit for bit against the oracle.

Each case draws a format, kind and group size, a token count, head count and head dimension
(including head dimensions that are not multiples of 8 and group sizes that leave partial
groups), and a layout for the input views (contiguous, a padded token pitch that keeps 16-byte
rows, a pitch that breaks that alignment, or a padded head stride). It then runs the whole chain
on both sides: pack, unpack, a dense or sparse residual encode against the reconstruction, and
the residual decode, in place or out of place. The layouts steer the library between its vector
and generic kernels and between its long-row and short-row (lane group) tilings, so the sweep
checks that every path reproduces the oracle's bits, not only the bulk shapes.
"""

import numpy as np
import pytest
import torch

import kv_cache_quantization_kvq_amd as kvq
import oracle
from gpu_util import assert_bits_equal, assert_same_packed, dev, planes, to_dev, to_host
from workloads import bf16_bits

pytestmark = pytest.mark.gpu

N_CASES = 160
HEAD_DIMS = [8, 12, 16, 24, 40, 64, 72, 100, 128, 136, 256]
INT4_GROUPS = [5, 8, 16, 24, 32, 64, 128]


def draw_case(i):
    rng = np.random.default_rng(1000 + i)
    fmt = ["int4", "int4", "nvfp4", "nvfp4_row", "fp8_row"][i % 5]
    kind = ["key", "value"][(i // 5) % 2]
    G = {"int4": int(rng.choice(INT4_GROUPS)), "nvfp4": 16, "nvfp4_row": 16, "fp8_row": 0}[fmt]
    T = int(rng.integers(1, 700))
    H = int(rng.integers(1, 6))
    D = int(rng.choice(HEAD_DIMS))
    layout = ["contiguous", "pitch16", "pitch_odd", "head_pad"][int(rng.integers(0, 4))]
    sparse = bool(rng.integers(0, 2))
    in_place = bool(rng.integers(0, 2))
    return dict(seed=1000 + i, fmt=fmt, kind=kind, G=G, T=T, H=H, D=D, layout=layout, sparse=sparse,
                in_place=in_place)


def values(rng, T, H, D):
    """Normal values over a few decades per (token, head) row, with exact and signed zeros."""
    x = rng.standard_normal((T, H, D)) * 10.0 ** rng.uniform(-2, 2, (T, H, 1))
    x[rng.random((T, H, D)) < 0.01] = 0.0
    x[rng.random((T, H, D)) < 0.01] = -0.0
    return bf16_bits(x)


def device_view(bits, layout):
    """The bf16 [T, H, D] bits as a device view in the given layout."""
    T, H, D = bits.shape
    if layout == "contiguous":
        return to_dev(bits)
    if layout == "head_pad":
        buf = torch.zeros((T, H, D + 8), dtype=torch.bfloat16, device=dev())
        buf[:, :, :D] = to_dev(bits)
        return buf[:, :, :D]
    pad = 8 if layout == "pitch16" else 3
    buf = torch.zeros((T, H * D + pad), dtype=torch.bfloat16, device=dev())
    buf[:, :H * D] = to_dev(bits).reshape(T, H * D)
    return buf[:, :H * D].unflatten(1, (H, D))


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape_chain(i):
    c = draw_case(i)
    rng = np.random.default_rng(c["seed"])
    T, H, D, fmt, kind, G = c["T"], c["H"], c["D"], c["fmt"], c["kind"], c["G"]
    what = f"case {i} {c}"
    x0 = values(rng, T, H, D)
    x1 = bf16_bits(oracle.bf16_to_f32(x0).astype(np.float64) + 0.05 * rng.standard_normal((T, H, D)))

    gp = kvq.pack(device_view(x0, c["layout"]), kind, fmt, G)
    op = oracle.pack(x0, kind, fmt, G)
    assert_same_packed(gp, op, what + " pack")
    R0g = kvq.unpack(gp)
    R0o = oracle.unpack(op)
    assert_bits_equal(to_host(R0g), R0o, what + " unpack")

    pos = None
    if c["sparse"]:
        M = int(rng.integers(0, T + 1))
        pos = rng.permutation(T)[:M].astype(np.int32)
        if rng.integers(0, 2):
            pos = np.sort(pos)
    gr = kvq.encode_residual(device_view(x1, c["layout"]), R0g, kind, fmt, G,
                             positions=None if pos is None else torch.from_numpy(pos).to(dev()))
    orr = oracle.encode_residual(x1, R0o, kind, fmt, G, positions=pos)
    assert_same_packed(gr, orr, what + " residual")
    want = oracle.decode_residual(orr, R0o)
    if c["in_place"]:
        buf = R0g.clone()
        kvq.decode_residual(gr, buf, out=buf)
        got = buf
    else:
        got = kvq.decode_residual(gr, R0g)
    assert_bits_equal(to_host(got), want, what + " residual decode")


N_POOL_CASES = 80


def draw_pool_case(i):
    rng = np.random.default_rng(5000 + i)
    fmt, kind, G = [("int4", "key", int(rng.choice([16, 32, 64]))), ("int4", "value", int(rng.choice([8, 16, 64]))),
                    ("nvfp4", "key", 16), ("nvfp4_row", "value", 16), ("fp8_row", "key", 0)][i % 5]
    return dict(seed=5000 + i, fmt=fmt, kind=kind, G=G, P=int(rng.integers(1, 20)),
                S=int(rng.choice([1, 4, 16, 32, 48])), H=int(rng.integers(1, 5)), D=int(rng.choice([8, 24, 64, 128])),
                pad=int(rng.choice([0, 2])), local=bool(rng.integers(0, 2)), sink=int(rng.integers(0, 6)),
                recent=int(rng.integers(0, 40)))


@pytest.mark.parametrize("i", range(N_POOL_CASES))
def test_random_pool_window_and_slots(i):
    c = draw_pool_case(i)
    rng = np.random.default_rng(c["seed"])
    fmt, kind, G, P, S, H, D, pad = c["fmt"], c["kind"], c["G"], c["P"], c["S"], c["H"], c["D"], c["pad"]
    what = f"case {i} {c}"
    if fmt == "int4" and kind == "value" and D % G:
        G = 8
    # paged pack / unpack of a pool of P pages of S slots (padded page stride when pad > 0)
    T = P * S
    buf = values(rng, P * (S + pad), H, D).reshape(P, S + pad, H, D)
    bd = to_dev(buf)
    if pad and P > 1 and S & (S - 1):
        # a padded page stride needs a power-of-two page size (the ABI says so): rejected, then
        # the same pages without padding
        with pytest.raises(kvq.KvqError):
            kvq.pack_paged(bd[:, :S], kind, fmt, G)
        pad = 0
        buf = np.ascontiguousarray(buf[:, :S])
        bd = to_dev(buf)
    local = c["local"]
    # page-local KEY groups must tile a page: INT4 G | S or S | G, NVFP4 16 | S
    if local and kind == "key" and ((fmt == "int4" and G % S and S % G) or (fmt == "nvfp4" and S % 16)):
        with pytest.raises(kvq.KvqError):
            kvq.pack_paged(bd[:, :S], kind, fmt, G, page_local=True)
        local = False
    gp = kvq.pack_paged(bd[:, :S], kind, fmt, G, page_local=local)
    op = oracle.pack_paged(buf[:, :S], kind, fmt, G, page_local=local)
    g, o = planes(gp), planes(op)  # page-local KEY groups: the descriptor records min(G, S), the oracle G
    assert set(g) == set(o), what
    for k in o:
        assert_bits_equal(g[k], o[k], f"{what} pack_paged {k}")
    assert (gp.rows, gp.H, gp.D) == (T, H, D)
    out = torch.zeros((P, S + pad, H, D), dtype=torch.bfloat16, device=dev())
    kvq.unpack_paged(gp, out[:, :S])
    assert_bits_equal(to_host(out)[:, :S], oracle.unpack_paged(op, P, S), what + " unpack_paged")
    # the same tokens as one tensor with a BF16 window
    x = np.ascontiguousarray(buf[:, :S]).reshape(T, H, D)
    gw = kvq.encode_window(to_dev(x), kind, fmt, G, c["sink"], c["recent"])
    ow = oracle.encode_window(x, kind, fmt, G, c["sink"], c["recent"])
    assert_same_packed(gw.packed, ow.packed, what + " window payload")
    assert_bits_equal(to_host(gw.window), ow.window, what + " window rows")
    assert_bits_equal(to_host(kvq.decode_window(gw)), oracle.decode_window(ow), what + " window decode")
    # slot writes and reads where every row carries its own metadata
    if (fmt, kind) in (("int4", "value"), ("nvfp4_row", "value"), ("fp8_row", "key")):
        cache = kvq.pack(to_dev(x), kind, fmt, G)
        ocache = oracle.pack(x, kind, fmt, G)
        N = int(rng.integers(1, T + 1))
        slots = rng.permutation(T)[:N].astype(np.int32)
        new = values(rng, N, H, D)
        kvq.store_rows(cache, to_dev(new), torch.from_numpy(slots).to(dev()))
        oracle.store_rows(ocache, new, slots)
        assert_same_packed(cache, ocache, what + " store_rows")
        rd = rng.integers(0, T, int(rng.integers(1, 2 * T + 1))).astype(np.int32)
        got = to_host(kvq.load_rows(cache, torch.from_numpy(rd).to(dev())))
        assert_bits_equal(got, oracle.load_rows(ocache, rd), what + " load_rows")
