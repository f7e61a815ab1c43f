"""Host logic of the bench: the algorithmic bytes behind every GB/s and roofline figure.

Each op's bytes are derived here independently of bench.py: the bf16 tensors it must read or write
(2 bytes per element each), the packed payload it must read or write (the oracle's storage
accounting), and for NVFP4 encodes the extra full read of the encoded rows that the per-tensor
multiplier forces before any code can be written (vllm-rlt PR #166, "Purpose": the scalar FP32
multiplier is computed from the whole encoded tensor on every call).
"""

import pytest

import bench
import oracle

T, H, D = 131072, 8, 128
N = T * H * D


def independent(op, fmt, kind, G):
    payload = oracle.storage_bytes(fmt, kind, G, T, H, D)
    bf16 = 2 * N
    if op == "pack":
        return bf16 + payload + (bf16 if fmt == "nvfp4" else 0)
    if op == "unpack":
        return payload + bf16
    if op == "encode_residual":
        return 2 * bf16 + payload + (2 * bf16 if fmt == "nvfp4" else 0)
    if op == "decode_residual":
        return payload + 2 * bf16
    raise ValueError(op)


@pytest.mark.parametrize("op", ["pack", "unpack", "encode_residual", "decode_residual"])
@pytest.mark.parametrize("fmt,G", [("int4", 64), ("nvfp4", 16)])
@pytest.mark.parametrize("kind", ["key", "value"])
def test_algorithmic_bytes_match_payload_accounting(op, fmt, G, kind):
    assert bench.algo_bytes(op, fmt, N) == independent(op, fmt, kind, G)


def test_bulk_step_totals():
    # per tensor of the bulk workload: INT4 G64 and NVFP4 G16 payloads differ by the 4-byte multiplier
    assert oracle.storage_bytes("int4", "key", 64, T, H, D) == 75497472
    assert oracle.storage_bytes("nvfp4", "value", 16, T, H, D) == 75497476
    want = {("pack", "int4"): 343932928, ("pack", "nvfp4"): 612368388,
            ("unpack", "int4"): 343932928, ("unpack", "nvfp4"): 343932932,
            ("encode_residual", "int4"): 612368384, ("encode_residual", "nvfp4"): 1149239300,
            ("decode_residual", "int4"): 612368384, ("decode_residual", "nvfp4"): 612368388}
    for (op, fmt), b in want.items():
        assert bench.algo_bytes(op, fmt, N) == b
    # one step: the eight ops of both formats, for K and V
    assert sum(2 * b for b in want.values()) == 9261023264


def test_multi_gpu_request_is_refused(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    assert bench.main() == 2
    assert "one GPU" in capsys.readouterr().err
