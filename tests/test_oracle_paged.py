"""Pins of the oracle's paged adapter and slot writes (CPU only).

pack_paged / unpack_paged work on a paged view [pages, page_size, heads, dim] (vllm-rlt pull
request #166: interface review, item 3, and the stacked-PR follow-up); store_rows / load_rows
quantize rows into, and decode rows out of, cache slots named by an index array (FreeToken pull
request #408, fp8 commit: fused quantize + scatter with slot ids).

What pins them:
  * flat pack_paged is bitwise pack() of the page-major token sequence, for contiguous and for
    padded page strides (pad contents never read), and unpack_paged inverts it in place;
  * page-local KEY grouping equals pack() with G = page_size when G is a multiple of the page
    size, and flat packing when the page size is a multiple of G; for other sizes every page
    depends on its own rows only (changing one page changes no other page's bits);
  * the NVFP4 multiplier of a page-local packing is the one of the whole paged tensor;
  * store_rows writes exactly pack()'s bits of the new rows into their slots and leaves every
    other slot bitwise as it was; load_rows returns exactly unpack() of those rows; for a
    token-grouped KEY cache load_rows equals unpack() indexed by the slots;
  * out-of-range and repeated slots, and formats whose rows are not independent, are rejected.
"""

import numpy as np
import pytest

import oracle
from workloads import bf16_bits, normal_kv


def paged(seed, P, S, H, D, pad=0):
    rng = np.random.default_rng(seed)
    buf = normal_kv(rng, P * (S + pad), H, D).reshape(P, S + pad, H, D)
    if pad:
        buf[:, S:] = 0x7FC0  # bf16 NaN in the padding: never read
    return buf[:, :S]


def same(a, b):
    for f in ("codes", "meta0", "meta1", "global_scale"):
        x, y = getattr(a, f), getattr(b, f)
        assert (x is None) == (y is None), f
        if x is not None:
            np.testing.assert_array_equal(x.reshape(-1), y.reshape(-1), err_msg=f)


FORMS = [("int4", 64), ("int4", 16), ("nvfp4", 16), ("nvfp4_row", 16), ("fp8_row", 0)]


@pytest.mark.parametrize("fmt,G", FORMS)
@pytest.mark.parametrize("kind", ["key", "value"])
@pytest.mark.parametrize("pad", [0, 3])
def test_flat_pack_paged_is_pack_of_token_sequence(fmt, G, kind, pad):
    x4 = paged(1, 5, 16, 2, 40, pad)
    flat = np.ascontiguousarray(x4).reshape(80, 2, 40)
    a = oracle.pack_paged(x4, kind, fmt, G)
    same(a, oracle.pack(flat, kind, fmt, G))
    y4 = oracle.unpack_paged(a, 5, 16)
    np.testing.assert_array_equal(y4.reshape(80, 2, 40), oracle.unpack(oracle.pack(flat, kind, fmt, G)))


@pytest.mark.parametrize("S,G", [(16, 64), (16, 32), (32, 32), (8, 128)])
def test_page_local_key_groups_of_whole_pages(S, G):
    x4 = paged(2, 6, S, 3, 24)
    flat = np.ascontiguousarray(x4).reshape(6 * S, 3, 24)
    a = oracle.pack_paged(x4, "key", "int4", G, page_local=True)
    b = oracle.pack(flat, "key", "int4", S)  # one group per page
    same(a, b)
    np.testing.assert_array_equal(oracle.unpack_paged(a, 6, S).reshape(6 * S, 3, 24), oracle.unpack(b))


@pytest.mark.parametrize("fmt,G", [("int4", 16), ("int4", 8), ("nvfp4", 16)])
def test_page_local_equals_flat_when_groups_tile_pages(fmt, G):
    x4 = paged(3, 4, 32, 2, 16)
    a = oracle.pack_paged(x4, "key", fmt, G, page_local=True)
    b = oracle.pack_paged(x4, "key", fmt, G, page_local=False)
    same(a, b)


@pytest.mark.parametrize("fmt,G", [("int4", 16), ("nvfp4", 16)])
def test_page_local_ragged_pages_are_independent(fmt, G):
    P, S = 4, 24  # 24 = 16 + 8: one full and one partial group per page
    x4 = paged(4, P, S, 2, 16).copy()
    x4[0, 0, 0, 0] = bf16_bits(np.array(100.0))  # the tensor amax sits in page 0 (fixes NVFP4's g)
    a = oracle.pack_paged(x4, "key", fmt, G, page_local=True)
    assert a.meta0.shape == (P * 2, 2, 16)
    x4b = x4.copy()
    x4b[2] = bf16_bits(np.random.default_rng(9).standard_normal((S, 2, 16)) * 0.5)
    b = oracle.pack_paged(x4b, "key", fmt, G, page_local=True)
    if fmt == "nvfp4":
        assert a.global_scale[0] == b.global_scale[0] == oracle.nvfp4_global(100.0)
    ya, yb = oracle.unpack_paged(a, P, S), oracle.unpack_paged(b, P, S)
    for p in (0, 1, 3):
        np.testing.assert_array_equal(a.codes[p * S:(p + 1) * S], b.codes[p * S:(p + 1) * S])
        np.testing.assert_array_equal(a.meta0[p * 2:(p + 1) * 2], b.meta0[p * 2:(p + 1) * 2])
        np.testing.assert_array_equal(ya[p], yb[p])
    # each page alone: groups over its slots [0, 16) and [16, 24)
    for p in range(P):
        one = oracle.pack(np.ascontiguousarray(x4[p]), "key", fmt, G,
                          global_scale=None if fmt == "int4" else float(a.global_scale[0]))
        np.testing.assert_array_equal(a.codes[p * S:(p + 1) * S], one.codes)
        np.testing.assert_array_equal(a.meta0[p * 2:(p + 1) * 2], one.meta0)
        np.testing.assert_array_equal(ya[p], oracle.unpack(one))


ROW_LOCAL = [("int4", "value", 64), ("int4", "value", 16), ("nvfp4_row", "key", 16), ("nvfp4_row", "value", 16),
             ("fp8_row", "key", 0), ("fp8_row", "value", 0)]


@pytest.mark.parametrize("fmt,kind,G", ROW_LOCAL)
def test_store_rows_writes_pack_bits_into_slots(fmt, kind, G):
    rng = np.random.default_rng(5)
    n_slots, H, D = 96, 2, 128
    cache = oracle.pack(normal_kv(rng, n_slots, H, D), kind, fmt, G)
    before = {f: getattr(cache, f).copy() for f in ("codes", "meta0", "meta1") if getattr(cache, f) is not None}
    new = normal_kv(rng, 13, H, D)
    slots = rng.choice(n_slots, 13, replace=False).astype(np.int32)
    oracle.store_rows(cache, new, slots)
    ref = oracle.pack(new, kind, fmt, G)
    others = np.setdiff1d(np.arange(n_slots), slots)
    for f, old in before.items():
        got = getattr(cache, f)
        np.testing.assert_array_equal(got[slots], getattr(ref, f))
        np.testing.assert_array_equal(got[others], old[others])
    np.testing.assert_array_equal(oracle.load_rows(cache, slots), oracle.unpack(ref))
    np.testing.assert_array_equal(oracle.load_rows(cache, others), oracle.unpack(oracle.pack(
        normal_kv(np.random.default_rng(5), n_slots, H, D), kind, fmt, G))[others])


@pytest.mark.parametrize("fmt,G", [("int4", 64), ("nvfp4", 16)])
def test_load_rows_of_token_grouped_key_cache(fmt, G):
    rng = np.random.default_rng(6)
    cache = oracle.pack(normal_kv(rng, 200, 2, 32), "key", fmt, G)
    slots = rng.choice(200, 37, replace=False).astype(np.int32)
    np.testing.assert_array_equal(oracle.load_rows(cache, slots), oracle.unpack(cache)[slots])


def test_store_rows_rejections():
    rng = np.random.default_rng(7)
    new = normal_kv(rng, 3, 1, 32)
    c = oracle.pack(normal_kv(rng, 10, 1, 32), "value", "fp8_row", 0)
    for bad in ([0, 1, 10], [0, -1, 2], [4, 4, 5]):
        with pytest.raises(ValueError):
            oracle.store_rows(c, new, np.array(bad, np.int32))
    for fmt, kind, G in (("int4", "key", 64), ("nvfp4", "value", 16), ("nvfp4", "key", 16)):
        c = oracle.pack(normal_kv(rng, 10, 1, 32), kind, fmt, G)
        with pytest.raises(ValueError):
            oracle.store_rows(c, new, np.array([0, 1, 2], np.int32))
    with pytest.raises(ValueError):
        oracle.load_rows(c, np.array([10], np.int32))
