"""The OpenMP build of the oracle gives the same bits as the single-threaded build (CPU only).

Both libraries are compiled from the same source; the threaded one runs its loops over
independent groups and rows on all threads and takes the tensor amax as a max of per-thread
maxima. This checks every entry point on ragged shapes whose groups spread over the threads.
"""

import numpy as np
import pytest

import oracle
from workloads import bf16_bits


@pytest.fixture
def both():
    """Run a callable under each build; returns (single-threaded result, threaded result)."""
    def run(fn):
        prev = oracle.set_threaded(False)
        try:
            a = fn()
            oracle.set_threaded(True)
            b = fn()
        finally:
            oracle.set_threaded(prev)
        return a, b
    return run


def same_packed(a, b):
    for f in ("codes", "meta0", "meta1", "global_scale", "positions"):
        x, y = getattr(a, f), getattr(b, f)
        assert (x is None) == (y is None), f
        if x is not None:
            np.testing.assert_array_equal(x.view(np.uint8), y.view(np.uint8), err_msg=f)


def inputs(seed=0, T=333, H=3, D=72):
    rng = np.random.default_rng(seed)
    x0 = rng.standard_t(3, (T, H, D))
    x0[rng.random((T, H, D)) < 0.01] = -0.0
    x1 = x0 + 0.1 * rng.standard_normal((T, H, D))
    return bf16_bits(x0), bf16_bits(x1), np.sort(rng.choice(T, T // 4, replace=False)).astype(np.int32)


def test_threaded_build_uses_threads():
    prev = oracle.set_threaded(True)
    try:
        assert oracle.threads() >= 1
    finally:
        oracle.set_threaded(prev)
    assert oracle.threads() == 1


@pytest.mark.parametrize("fmt,G", [("int4", 64), ("int4", 16), ("int4", 5), ("nvfp4", 16), ("nvfp4_row", 16),
                                   ("fp8_row", 0)])
@pytest.mark.parametrize("kind", ["key", "value"])
def test_codec_ops_bit_identical(both, fmt, G, kind):
    x0, x1, pos = inputs()
    a, b = both(lambda: oracle.pack(x0, kind, fmt, G))
    same_packed(a, b)
    ya, yb = both(lambda: oracle.unpack(a))
    np.testing.assert_array_equal(ya, yb)
    for positions in (None, pos):
        ra, rb = both(lambda: oracle.encode_residual(x1, ya, kind, fmt, G, positions=positions))
        same_packed(ra, rb)
        da, db = both(lambda: oracle.decode_residual(ra, ya))
        np.testing.assert_array_equal(da, db)
    ta, tb = both(lambda: oracle.tensor_amax(x1, ya, pos))
    assert ta == tb


def test_paged_slots_window_bit_identical(both):
    x0, x1, pos = inputs(1, T=256, H=2, D=64)
    pa, pb = both(lambda: oracle.pack_paged(x0.reshape(16, 16, 2, 64), "key", "int4", 16, page_local=True))
    same_packed(pa, pb)
    ua, ub = both(lambda: oracle.unpack_paged(pa, 16, 16))
    np.testing.assert_array_equal(ua, ub)
    wa, wb = both(lambda: oracle.encode_window(x1, "key", "nvfp4", prev=x0))
    same_packed(wa.packed, wb.packed)
    np.testing.assert_array_equal(wa.window, wb.window)
    da, db = both(lambda: oracle.decode_window(wa, prev=x0))
    np.testing.assert_array_equal(da, db)

    def slots():
        cache = oracle.pack(x0, "value", "fp8_row", 0)
        oracle.store_rows(cache, x1[:40], pos[:40])
        return cache, oracle.load_rows(cache, pos[:40])
    (ca, la), (cb, lb) = both(slots)
    same_packed(ca, cb)
    np.testing.assert_array_equal(la, lb)
