"""Pins of the oracle's cross-loop residual layer (CPU only).

What pins it:
  * identity: current == previous gives a zero residual and a decode equal to previous (up to
    -0.0 becoming +0.0, which IEEE addition of +0 implies);
  * decode composes with unpack: decode_residual(R, P) == bf16(P + unpack(R)) computed with
    numpy/torch arithmetic, dense and sparse, for every format pairing (mixed chains);
  * sparse with every position, in order, is bitwise the dense residual;
  * absent rows are bitwise copies of previous; the position map is an owned copy;
  * the chain on reconstructed predecessors does not compound error, while encoding deltas of
    the original states does (the codec page's first review names this property);
  * K groups of a sparse residual follow compact row order.
"""

import numpy as np
import pytest

import oracle
from workloads import bf16_bits, bf16_to_f32, c3_chain_inputs, normal_kv


def add_bf16(prev_bits, delta_bits):
    s = bf16_to_f32(prev_bits) + bf16_to_f32(delta_bits)  # one binary32 addition
    return bf16_bits(s)


FORMS = [("int4", 64), ("int4", 16), ("nvfp4", 16), ("nvfp4_row", 16), ("fp8_row", 0)]


@pytest.mark.parametrize("fmt,G", FORMS)
@pytest.mark.parametrize("kind", ["key", "value"])
def test_identity_residual(fmt, G, kind):
    rng = np.random.default_rng(0)
    P = normal_kv(rng, 70, 2, 24)
    P[0, 0, 0] = 0x8000
    R = oracle.encode_residual(P, P, kind, fmt, G)
    out = oracle.decode_residual(R, P)
    want = P.copy()
    want[want == 0x8000] = 0
    np.testing.assert_array_equal(out, want)


@pytest.mark.parametrize("base_fmt,base_G", FORMS)
@pytest.mark.parametrize("res_fmt,res_G", FORMS + [("int4", 32)])
@pytest.mark.parametrize("kind", ["key", "value"])
def test_decode_is_prev_plus_unpack(base_fmt, base_G, res_fmt, res_G, kind):
    rng = np.random.default_rng(1)
    X0 = normal_kv(rng, 50, 2, 40)
    X1 = bf16_bits(bf16_to_f32(X0).astype(np.float64) + 0.1 * rng.standard_normal(X0.shape))
    R0 = oracle.unpack(oracle.pack(X0, kind, base_fmt, base_G))
    Rr = oracle.encode_residual(X1, R0, kind, res_fmt, res_G)
    np.testing.assert_array_equal(oracle.decode_residual(Rr, R0), add_bf16(R0, oracle.unpack(Rr)))
    # the encoded rows are bf16(X1 - R0): encoding them directly gives the same payload
    delta = bf16_bits(bf16_to_f32(X1) - bf16_to_f32(R0))
    direct = oracle.pack(delta, kind, res_fmt, res_G)
    np.testing.assert_array_equal(direct.codes, Rr.codes)
    np.testing.assert_array_equal(direct.meta0, Rr.meta0)
    # sparse
    pos = np.sort(rng.choice(50, 13, replace=False)).astype(np.int32)
    Rs = oracle.encode_residual(X1, R0, kind, res_fmt, res_G, positions=pos)
    assert Rs.rows == 13 and Rs.positions is not None
    dec = oracle.decode_residual(Rs, R0)
    want = R0.copy()
    want[pos] = add_bf16(R0[pos], oracle.unpack(Rs))
    np.testing.assert_array_equal(dec, want)


@pytest.mark.parametrize("fmt,G", FORMS)
@pytest.mark.parametrize("kind", ["key", "value"])
def test_sparse_all_positions_equals_dense(fmt, G, kind):
    rng = np.random.default_rng(2)
    C = normal_kv(rng, 40, 3, 16)
    P = normal_kv(rng, 40, 3, 16)
    d = oracle.encode_residual(C, P, kind, fmt, G)
    s = oracle.encode_residual(C, P, kind, fmt, G, positions=np.arange(40, dtype=np.int32))
    for a in ("codes", "meta0", "meta1", "global_scale"):
        if getattr(d, a) is not None:
            np.testing.assert_array_equal(getattr(d, a), getattr(s, a))
    np.testing.assert_array_equal(oracle.decode_residual(d, P), oracle.decode_residual(s, P))


def test_sparse_absent_rows_and_owned_positions():
    rng = np.random.default_rng(3)
    C = normal_kv(rng, 64, 2, 32)
    P = normal_kv(rng, 64, 2, 32)
    pos = np.array([60, 3, 17, 40, 41], np.int32)  # any order: the given order is compact order
    R = oracle.encode_residual(C, P, "key", "int4", 4, positions=pos)
    pos[0] = 0  # the residual keeps its own copy
    assert R.positions.tolist() == [60, 3, 17, 40, 41]
    out = oracle.decode_residual(R, P)
    absent = np.setdiff1d(np.arange(64), R.positions)
    np.testing.assert_array_equal(out[absent], P[absent])
    # compact K groups: rows (60, 3, 17, 40) form group 0, row 41 group 1
    delta = bf16_bits(bf16_to_f32(C[R.positions]) - bf16_to_f32(P[R.positions]))
    direct = oracle.pack(delta, "key", "int4", 4)
    np.testing.assert_array_equal(direct.codes, R.codes)
    np.testing.assert_array_equal(direct.meta0, R.meta0)
    # in place (out is prev): only kept rows change
    P2 = P.copy()
    oracle.decode_residual(R, P2, out=P2)
    np.testing.assert_array_equal(P2, out)


def test_chain_does_not_compound():
    ch = c3_chain_inputs(0)
    XK = [x[:256] for x in ch["XK"]]
    R = oracle.unpack(oracle.pack(XK[0], "key", "int4", 64))
    errs = []
    for k in range(1, 4):
        res = oracle.encode_residual(XK[k], R, "key", "int4", 64)
        R = oracle.decode_residual(res, R)
        errs.append(np.linalg.norm(bf16_to_f32(R) - bf16_to_f32(XK[k])))
    # drifting alternative: encode the deltas of the original states and accumulate
    Rd = oracle.unpack(oracle.pack(XK[0], "key", "int4", 64))
    derrs = []
    for k in range(1, 4):
        res = oracle.encode_residual(XK[k], XK[k - 1], "key", "int4", 64)
        Rd = oracle.decode_residual(res, Rd)
        derrs.append(np.linalg.norm(bf16_to_f32(Rd) - bf16_to_f32(XK[k])))
    assert max(errs) < 1.2 * errs[0]
    assert derrs[-1] > 3 * errs[-1]


def test_positions_out_of_range_rejected():
    P = np.zeros((8, 1, 4), np.uint16)
    with pytest.raises(ValueError):
        oracle.encode_residual(P, P, "key", "int4", 4, positions=np.array([8], np.int32))
