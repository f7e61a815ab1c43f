"""Pins of the oracle's BF16 protected window (CPU only): the first `sink` and the latest
`recent` tokens kept in BF16, the rest quantized (vllm-rlt pull request #166, "Real Ouro
numerical comparison": first 4 / latest 16 kept BF16; protected rows excluded from the
quantized payload; BF16 passthrough bitwise equal).

What pins it:
  * passthrough: every protected row decodes bitwise equal to the input row (plain and
    residual: a residual's protected rows reconstruct to the current values exactly);
  * the quantized payload is exactly pack() of the middle rows [sink, T - recent) as their own
    tensor (every format, both kinds, partial groups), and its decode is unpack() of it;
  * a windowed residual's payload is exactly the sparse residual whose positions are the middle
    range (the window composes with the position maps), and its middle rows decode to
    bf16(prev + unpack);
  * edge cases: T <= sink + recent keeps every row (empty payload, NVFP4 multiplier 1), and a
    zero window is plain pack/unpack.
"""

import numpy as np
import pytest

import oracle
from workloads import bf16_bits, bf16_to_f32, normal_kv

FORMS = [("int4", 64), ("int4", 16), ("nvfp4", 16), ("nvfp4_row", 16), ("fp8_row", 0)]


def same_payload(a, b):
    for f in ("codes", "meta0", "meta1", "global_scale"):
        x, y = getattr(a, f), getattr(b, f)
        assert (x is None) == (y is None), f
        if x is not None:
            np.testing.assert_array_equal(x, y, err_msg=f)


@pytest.mark.parametrize("fmt,G", FORMS)
@pytest.mark.parametrize("kind", ["key", "value"])
@pytest.mark.parametrize("T,sink,recent", [(150, 4, 16), (97, 4, 16), (40, 0, 16), (40, 4, 0), (64, 7, 3)])
def test_window_pack(fmt, G, kind, T, sink, recent):
    x = normal_kv(np.random.default_rng(T + sink), T, 3, 40)
    w = oracle.encode_window(x, kind, fmt, G, sink, recent)
    ns, nr = oracle.window_split(T, sink, recent)
    mid = np.ascontiguousarray(x[ns:T - nr])
    ref = oracle.pack(mid, kind, fmt, G)
    same_payload(w.packed, ref)
    np.testing.assert_array_equal(w.window, np.concatenate([x[:ns], x[T - nr:]]))
    y = oracle.decode_window(w)
    np.testing.assert_array_equal(y[:ns], x[:ns])          # passthrough, bitwise
    np.testing.assert_array_equal(y[T - nr:], x[T - nr:])
    np.testing.assert_array_equal(y[ns:T - nr], oracle.unpack(ref))


@pytest.mark.parametrize("fmt,G", FORMS)
@pytest.mark.parametrize("kind", ["key", "value"])
def test_window_residual_is_sparse_residual_over_middle(fmt, G, kind):
    rng = np.random.default_rng(4)
    T, sink, recent = 130, 4, 16
    prev = normal_kv(rng, T, 2, 64)
    cur = bf16_bits(bf16_to_f32(prev).astype(np.float64) + 0.1 * rng.standard_normal(prev.shape))
    w = oracle.encode_window(cur, kind, fmt, G, sink, recent, prev=prev)
    pos = np.arange(sink, T - recent, dtype=np.int32)
    sp = oracle.encode_residual(cur, prev, kind, fmt, G, positions=pos)
    same_payload(w.packed, sp)
    y = oracle.decode_window(w, prev=prev)
    np.testing.assert_array_equal(y[:sink], cur[:sink])
    np.testing.assert_array_equal(y[T - recent:], cur[T - recent:])
    want = oracle.decode_residual(sp, prev)  # absent rows are prev; kept rows bf16(prev + delta)
    np.testing.assert_array_equal(y[sink:T - recent], want[sink:T - recent])


@pytest.mark.parametrize("fmt,G", FORMS)
@pytest.mark.parametrize("T", [0, 1, 5, 20])
def test_window_covers_everything(fmt, G, T):
    x = normal_kv(np.random.default_rng(T), T, 2, 32)
    w = oracle.encode_window(x, "key", fmt, G, 4, 16)
    assert w.packed.rows == 0 and w.window.shape[0] == T
    if fmt == "nvfp4":
        assert w.packed.global_scale[0] == 1.0
    np.testing.assert_array_equal(oracle.decode_window(w), x)


@pytest.mark.parametrize("fmt,G", FORMS)
def test_zero_window_is_plain_codec(fmt, G):
    x = normal_kv(np.random.default_rng(8), 70, 2, 32)
    w = oracle.encode_window(x, "key", fmt, G, 0, 0)
    same_payload(w.packed, oracle.pack(x, "key", fmt, G))
    np.testing.assert_array_equal(oracle.decode_window(w), oracle.unpack(oracle.pack(x, "key", fmt, G)))


def test_window_rejects_negative_sizes():
    x = normal_kv(np.random.default_rng(0), 8, 1, 16)
    with pytest.raises(ValueError):
        oracle.encode_window(x, "key", "int4", 64, -1, 16)
