"""Guard bands and poisoned outputs.

An exact-code comparison is the check that catches a wrong row pitch, and a tool that misses
uninitialised reads can hide a kernel that leaves part of its output unwritten (FreeToken PR #408,
the V row-pitch and initcheck findings). Here every output plane of pack / encode_residual and
every decoded tensor of unpack / decode_residual is a view into a larger buffer: the bytes on both
sides hold a canary pattern and the view itself is filled with a poison pattern before the call.
After the call the canaries must be intact (no write outside the output) and every output byte
must equal the oracle's (no byte left unwritten). The shapes cover the vector kernels (ragged token
counts, partial KEY groups), lane groups of short rows, a slab with idle lanes, and the generic
path; the formats cover INT4 at four group sizes, NVFP4 and the two per-row formats, dense and
sparse residuals.
"""

import dataclasses

import numpy as np
import pytest
import torch

import kv_cache_quantization_kvq_amd as kvq
import oracle
from gpu_util import assert_bits_equal, assert_same_packed, to_dev, to_host
from workloads import normal_kv

pytestmark = pytest.mark.gpu

GUARD = 4096  # bytes on each side; a multiple of 256 keeps the planes' alignment
CANARY = 0xA5
POISON = 0x5A

FORMS = [("int4", 64), ("int4", 16), ("int4", 32), ("int4", 128), ("nvfp4", 16), ("nvfp4_row", 16), ("fp8_row", 0)]
SHAPES = [
    (1000, 4, 256),  # vector path, 1000 = 15*64 + 40 tokens: partial KEY groups
    (333, 1, 128),   # 16 chunks per row: lane groups
    (77, 3, 64),     # 24 chunks per row: a slab with idle lanes
    (50, 2, 40),     # D = 40: generic path for most forms
]


class Guarded:
    """Tensors that are views into canary-bordered, poison-filled buffers."""

    def __init__(self, dev):
        self.dev = dev
        self.bufs = []

    def like(self, shape, dtype):
        n = int(np.prod(shape)) * torch.empty(0, dtype=dtype).element_size()
        buf = torch.full((n + 2 * GUARD,), CANARY, dtype=torch.uint8, device=self.dev)
        buf[GUARD:GUARD + n] = POISON
        self.bufs.append((buf, n))
        return buf[GUARD:GUARD + n].view(dtype).view(shape)

    def packed(self, fmt, kind, G, rows, H, D, full_T, sparse=False):
        p = kvq.alloc_packed(fmt, kind, G, rows, H, D, full_T, self.dev, sparse=sparse)
        repl = {}
        for name in ("codes", "meta0", "meta1", "global_scale"):
            t = getattr(p, name)
            if t is not None:
                repl[name] = self.like(tuple(t.shape), t.dtype)
        return dataclasses.replace(p, **repl)

    def check(self, what):
        torch.cuda.synchronize()
        for buf, n in self.bufs:
            head, tail = buf[:GUARD], buf[GUARD + n:]
            assert bool((head == CANARY).all()) and bool((tail == CANARY).all()), f"{what}: write outside an output"


@pytest.mark.parametrize("T,H,D", SHAPES)
@pytest.mark.parametrize("fmt,G", FORMS)
@pytest.mark.parametrize("kind", ["key", "value"])
def test_outputs_written_exactly_and_only(T, H, D, fmt, G, kind):
    dev = torch.device("cuda")
    rng = np.random.default_rng(T * 7 + H * 5 + D)
    x0 = normal_kv(rng, T, H, D)
    x1 = normal_kv(rng, T, H, D)
    pos = np.sort(rng.choice(T, T // 3, replace=False)).astype(np.int32)
    g = Guarded(dev)

    # pack / unpack
    p = g.packed(fmt, kind, G, T, H, D, T)
    kvq.pack(to_dev(x0), kind, fmt, G, out=p)
    op = oracle.pack(x0, kind, fmt, G)
    g.check("pack")
    assert_same_packed(p, op, "pack")
    r0 = g.like((T, H, D), torch.bfloat16)
    kvq.unpack(p, out=r0)
    o0 = oracle.unpack(op)
    g.check("unpack")
    assert_bits_equal(to_host(r0), o0, "unpack")

    # dense residual
    res = g.packed(fmt, kind, G, T, H, D, T)
    kvq.encode_residual(to_dev(x1), r0, kind, fmt, G, out=res)
    ores = oracle.encode_residual(x1, o0, kind, fmt, G)
    g.check("encode_residual")
    assert_same_packed(res, ores, "encode_residual")
    r1 = g.like((T, H, D), torch.bfloat16)
    kvq.decode_residual(res, r0, out=r1)
    g.check("decode_residual")
    assert_bits_equal(to_host(r1), oracle.decode_residual(ores, o0), "decode_residual")

    # sparse residual: compact rows, and an out-of-place decode that copies the absent rows
    sp = g.packed(fmt, kind, G, len(pos), H, D, T, sparse=True)
    kvq.encode_residual(to_dev(x1), r0, kind, fmt, G, positions=torch.from_numpy(pos).to(dev), out=sp)
    osp = oracle.encode_residual(x1, o0, kind, fmt, G, positions=pos)
    g.check("sparse encode_residual")
    assert_same_packed(sp, osp, "sparse encode_residual")
    r2 = g.like((T, H, D), torch.bfloat16)
    kvq.decode_residual(sp, r0, out=r2)
    g.check("sparse decode_residual")
    assert_bits_equal(to_host(r2), oracle.decode_residual(osp, o0), "sparse decode_residual")
