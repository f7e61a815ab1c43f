"""Helpers for the GPU parity tests: move bf16 bit arrays to and from the device and compare a
packed tensor from the HIP library with the oracle's, plane by plane, bit for bit."""

from __future__ import annotations

import numpy as np
import torch

import oracle


def dev() -> torch.device:
    return torch.device("cuda:0")


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bits (any numpy layout) -> contiguous bf16 tensor on the GPU."""
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev())


def to_host(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor (any layout) -> uint16 bits."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def planes(p) -> dict:
    """Host copies of a packed tensor's planes (GPU Packed or oracle Packed)."""
    out = {}
    for name in ("codes", "meta0", "meta1", "global_scale", "positions"):
        a = getattr(p, name)
        if a is None:
            continue
        if isinstance(a, torch.Tensor):
            a = a.cpu().numpy()
        if name in ("meta0", "meta1") and a.dtype == np.int16:
            a = a.view(np.uint16)
        if name in ("meta0", "meta1") and a.dtype == np.float32:
            a = np.ascontiguousarray(a).view(np.uint32)  # FP32 row scales compare as bits
        if name == "global_scale":
            a = np.asarray(a, np.float32).view(np.uint32)
        out[name] = np.asarray(a)
    return out


def first_mismatch(a: np.ndarray, b: np.ndarray) -> str:
    bad = np.argwhere(a != b)
    return f"{len(bad)} of {a.size} differ; first at {tuple(bad[0])}: got {a[tuple(bad[0])]} want {b[tuple(bad[0])]}"


def assert_bits_equal(got: np.ndarray, want: np.ndarray, what: str) -> None:
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    if not np.array_equal(got, want):
        raise AssertionError(f"{what}: {first_mismatch(got, want)}")


def assert_same_packed(gp, op, what: str = "") -> None:
    g, o = planes(gp), planes(op)
    assert set(g) == set(o), f"{what}: planes {sorted(g)} vs {sorted(o)}"
    for k in o:
        assert_bits_equal(g[k], o[k], f"{what} {k}")
    assert (gp.format, gp.kind, gp.group_size, gp.rows, gp.H, gp.D) == (op.format, op.kind, op.group_size, op.rows,
                                                                       op.H, op.D)


def rel_l2(y_bits: np.ndarray, x_bits: np.ndarray) -> float:
    y = oracle.bf16_to_f32(y_bits).astype(np.float64)
    x = oracle.bf16_to_f32(x_bits).astype(np.float64)
    n = np.linalg.norm(x)
    return float(np.linalg.norm(y - x) / n) if n else 0.0
