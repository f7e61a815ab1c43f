"""The C ABI used from a plain C++ program (tests/c_abi/kvq_c_chain.cpp, built by
__graft_entry__.build()), with no Python binding in between: it packs an INT4 G64 KEY tensor,
unpacks it, encodes a sparse NVFP4 VALUE residual of a second tensor against that
reconstruction and decodes it out of place, allocating every plane itself from kvq_plane_bytes.
Its inputs and outputs are compared with the CPU oracle bit for bit."""

import os
import subprocess

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "kvq_c_chain")


def load(d, name, dtype):
    return np.fromfile(os.path.join(d, name), dtype=dtype)


def same_bytes(got, want, what):
    want = np.ascontiguousarray(want).view(np.uint8).ravel()
    assert got.size == want.size, f"{what}: {got.size} bytes vs {want.size}"
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{what}: {bad.size} bytes differ, first at {bad[0]}"


@pytest.mark.parametrize("T,H,D", [(1000, 4, 128), (64, 1, 256), (129, 3, 64)])
def test_c_program_chain_matches_oracle(T, H, D, tmp_path):
    assert os.path.exists(EXE), "tests/c_abi/kvq_c_chain is missing: run __graft_entry__.build()"
    d = str(tmp_path)
    r = subprocess.run([EXE, d, str(T), str(H), str(D)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    x0 = load(d, "x0.bin", np.uint16).reshape(T, H, D)
    x1 = load(d, "x1.bin", np.uint16).reshape(T, H, D)
    pos = load(d, "positions.bin", np.int32)
    op = oracle.pack(x0, "key", "int4", 64)
    same_bytes(load(d, "pack_codes.bin", np.uint8), op.codes, "pack codes")
    same_bytes(load(d, "pack_meta0.bin", np.uint8), op.meta0, "pack minimums")
    same_bytes(load(d, "pack_meta1.bin", np.uint8), op.meta1, "pack scales")
    r0 = oracle.unpack(op)
    same_bytes(load(d, "r0.bin", np.uint8), r0, "unpack")
    orr = oracle.encode_residual(x1, r0, "value", "nvfp4", 16, positions=pos)
    same_bytes(load(d, "residual_codes.bin", np.uint8), orr.codes, "residual codes")
    same_bytes(load(d, "residual_meta0.bin", np.uint8), orr.meta0, "residual block scales")
    same_bytes(load(d, "residual_global.bin", np.uint8), orr.global_scale, "residual global scale")
    same_bytes(load(d, "residual_positions.bin", np.uint8), pos, "residual positions")
    same_bytes(load(d, "r1.bin", np.uint8), oracle.decode_residual(orr, r0), "residual decode")
