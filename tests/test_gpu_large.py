"""GPU parity past the 32-bit element counts: a [4194404, 8, 128] bf16 tensor (4 295 069 696
elements, 8.6 GB, more than 2^32 elements and 2^33 bytes).

The whole tensor goes through pack and unpack (INT4 G64 and NVFP4 G16, K and V) and, for INT4, a
dense residual encode against the reconstruction and its decode, in the launch configuration of
the bulk workload (contiguous rows, the vector kernels). The oracle then checks the token windows
where 32-bit indexing would break: the start, the rows around element 2^31 (token 2^21), and
the rows from just before element 2^32 (token 2^22) to the end, whose last KEY group is partial
(36 tokens). Windows start on group boundaries, so the oracle's pack of a window forms the same
groups; NVFP4 windows are packed with the multiplier the oracle computes from the whole tensor's
amax. Every code, metadata and reconstructed element of the windows must agree bit for bit.

A second test sends the same tensor through the generic kernels (one work item per thread),
which run in launches of at most 2^31 work items: an unpack into a view whose token pitch is
not 16-byte aligned (2^31 + 51 200 work items, two launches) and the out-of-place decode of a
sparse residual into such a view, which first copies every element of the predecessor (2^32 +
102 400 work items, three launches) and then scatters the kept rows.
"""

import numpy as np
import pytest
import torch

import kv_cache_quantization_kvq_amd as kvq
import oracle
from gpu_util import assert_bits_equal, dev, to_host

pytestmark = pytest.mark.gpu

T, H, D = (1 << 22) + 100, 8, 128
WINDOWS = ((0, 64), ((1 << 21) - 64, (1 << 21) + 64), ((1 << 22) - 64, T))


@pytest.fixture(scope="module")
def tensors():
    assert T * H * D > 1 << 32
    gen = torch.Generator(device=dev()).manual_seed(2024)
    x0 = torch.randn((T, H, D), generator=gen, dtype=torch.bfloat16, device=dev())
    x1 = torch.empty_like(x0)
    for t in range(0, T, 1 << 20):  # x1 = bf16(x0 + 0.1 N(0, 1)), in chunks
        c = slice(t, min(T, t + (1 << 20)))
        x1[c] = (x0[c].float() + 0.1 * torch.randn(x0[c].shape, generator=gen, device=dev())).bfloat16()
    torch.cuda.synchronize()
    X0, X1 = to_host(x0), to_host(x1)
    prev = oracle.set_threaded(True)
    g = oracle.nvfp4_global(oracle.tensor_amax(X0))
    oracle.set_threaded(prev)
    yield x0, x1, X0, X1, g


def host(t):
    a = t.cpu().numpy()
    return a.view(np.uint16) if a.dtype == np.int16 else a


def window_planes(p, kind, G, t0, t1):
    """The GPU planes that hold rows t0:t1 (KEY metadata: their token groups)."""
    m = slice(t0 // G, -(-t1 // G)) if kind == "key" else slice(t0, t1)
    out = {"codes": host(p.codes[t0:t1])}
    for name in ("meta0", "meta1"):
        a = getattr(p, name)
        if a is not None:
            out[name] = host(a[m])
    return out


def assert_window(gp, op, kind, G, t0, t1, what):
    got = window_planes(gp, kind, G, t0, t1)
    for name in got:
        want = getattr(op, name)
        want = want.view(np.uint16) if want.dtype == np.int16 else want
        assert_bits_equal(got[name], want, f"{what} {name} rows {t0}:{t1}")


@pytest.mark.parametrize("fmt,G", [("int4", 64), ("nvfp4", 16)])
@pytest.mark.parametrize("kind", ["key", "value"])
def test_beyond_32bit_elements(tensors, fmt, G, kind):
    x0, x1, X0, X1, g = tensors
    gp = kvq.pack(x0, kind, fmt, G)
    R0 = kvq.unpack(gp)
    gr = R1 = None
    if fmt == "int4":
        gr = kvq.encode_residual(x1, R0, kind, fmt, G)
        R1 = kvq.decode_residual(gr, R0)
    torch.cuda.synchronize()
    if fmt == "nvfp4":
        assert float(gp.global_scale.cpu()[0]) == g
    for t0, t1 in WINDOWS:
        what = f"{fmt} {kind}"
        op = oracle.pack(X0[t0:t1], kind, fmt, G, global_scale=g if fmt == "nvfp4" else None)
        assert_window(gp, op, kind, G, t0, t1, what + " pack")
        oR0 = oracle.unpack(op)
        assert_bits_equal(to_host(R0[t0:t1]), oR0, f"{what} unpack rows {t0}:{t1}")
        if gr is not None:
            orr = oracle.encode_residual(X1[t0:t1], oR0, kind, fmt, G)
            assert_window(gr, orr, kind, G, t0, t1, what + " residual")
            assert_bits_equal(to_host(R1[t0:t1]), oracle.decode_residual(orr, oR0),
                              f"{what} residual decode rows {t0}:{t1}")
    del gp, R0, gr, R1
    torch.cuda.empty_cache()


def odd_pitch(T_, H_, D_):
    """An uninitialized bf16 [T, H, D] view whose token pitch (H*D + 3) breaks 16-byte rows."""
    buf = torch.empty((T_, H_ * D_ + 3), dtype=torch.bfloat16, device=dev())
    return buf[:, :H_ * D_].unflatten(1, (H_, D_))


def test_generic_kernels_beyond_32bit_work_items(tensors):
    x0, x1, X0, X1, _ = tensors
    kind, fmt, G = "key", "int4", 64
    gp = kvq.pack(x0, kind, fmt, G)
    out = odd_pitch(T, H, D)
    kvq.unpack(gp, out=out)
    R0 = kvq.unpack(gp)
    pos_list = [0, (1 << 21) + 5, (1 << 22) + 7, T - 1]
    r = kvq.encode_residual(x1, R0, kind, fmt, G,
                            positions=torch.tensor(pos_list, dtype=torch.int32, device=dev()))
    out2 = odd_pitch(T, H, D)
    kvq.decode_residual(r, R0, out=out2)
    torch.cuda.synchronize()
    oR0 = {}
    for t0, t1 in WINDOWS:
        w = oracle.unpack(oracle.pack(X0[t0:t1], kind, fmt, G))
        assert_bits_equal(to_host(out[t0:t1]), w, f"generic unpack rows {t0}:{t1}")
        for t in range(t0, t1):
            oR0[t] = w[t - t0]
    # the kept rows: the oracle's residual of those rows alone (KEY groups run over the compact
    # rows), added to the oracle's reconstruction
    P = np.stack([oR0[t] for t in pos_list])
    orr = oracle.encode_residual(np.ascontiguousarray(X1[pos_list]), P, kind, fmt, G)
    want_kept = oracle.decode_residual(orr, P)
    got = to_host(out2[torch.tensor(pos_list, device=dev())])
    assert_bits_equal(got, want_kept, "sparse decode kept rows")
    kept = set(pos_list)
    for t0, t1 in WINDOWS:
        rows = [t for t in range(t0, t1) if t not in kept]
        got = to_host(out2[torch.tensor(rows, device=dev())])
        assert_bits_equal(got, np.stack([oR0[t] for t in rows]), f"sparse decode copied rows {t0}:{t1}")
