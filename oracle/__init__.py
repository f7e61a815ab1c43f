"""CPU oracle of the KV-cache quantization codec (Python side).

TEST INFRASTRUCTURE ONLY. This package wraps ``kvq_oracle.c``, the plain scalar C statement of
what the codec computes. Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import it. The product path (``kv_cache_quantization_kvq_amd``) never
imports, links or calls anything here, and the two share no code.

Arrays: bf16 tensors are ``numpy.uint16`` arrays of bf16 bit patterns with shape ``[T, H, D]``
and unit channel stride (any token/head strides, e.g. a view into a fused QKV buffer).

Parity pins live in ``tests/test_oracle_*.py``; every function here is pinned there except
where the module docstring of that test says "parity unpinned".
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "libkvq_oracle.so")

KIND = {"key": 0, "value": 1}
FORMAT = {"int4": 0, "nvfp4": 1}

# -O2 without -march=native; -ffp-contract=off so that no multiply-add is fused.
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/libkvq_oracle.so``."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int32
        ci = ctypes.c_int
        lib.kvq_oracle_pack.argtypes = [p, i64, i64, i64, i64, i64, ci, ci, i32, p, p, p, p, ctypes.c_float]
        lib.kvq_oracle_pack.restype = ci
        lib.kvq_oracle_unpack.argtypes = [ci, ci, i32, i64, i64, i64, p, p, p, p, p, i64, i64]
        lib.kvq_oracle_unpack.restype = ci
        lib.kvq_oracle_encode_residual.argtypes = [p, i64, i64, p, i64, i64, i64, i64, i64, p, i64, ci, ci, i32,
                                                   p, p, p, p, p, ctypes.c_float]
        lib.kvq_oracle_tensor_amax.argtypes = [p, i64, i64, p, i64, i64, i64, i64, i64, p, i64]
        lib.kvq_oracle_tensor_amax.restype = ctypes.c_float
        lib.kvq_oracle_encode_residual.restype = ci
        lib.kvq_oracle_decode_residual.argtypes = [ci, ci, i32, i64, i64, i64, p, p, p, p, p, p, i64, i64, i64,
                                                   p, i64, i64]
        lib.kvq_oracle_decode_residual.restype = ci
        lib.kvq_oracle_storage_bytes.argtypes = [ci, ci, i32, i64, i64, i64, ci]
        lib.kvq_oracle_storage_bytes.restype = i64
        lib.kvq_oracle_nvfp4_global.argtypes = [ctypes.c_float]
        lib.kvq_oracle_nvfp4_global.restype = ctypes.c_float
        for name, outt in (("kvq_oracle_f32_to_bf16_n", None), ("kvq_oracle_f32_to_f16_n", None),
                           ("kvq_oracle_f32_to_e4m3_n", None), ("kvq_oracle_e2m1_encode_n", None)):
            fn = getattr(lib, name)
            fn.argtypes = [p, p, i64]
            fn.restype = outt
        lib.kvq_oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
        lib.kvq_oracle_f16_to_f32.restype = ctypes.c_float
        lib.kvq_oracle_e4m3_to_f32.argtypes = [ctypes.c_uint8]
        lib.kvq_oracle_e4m3_to_f32.restype = ctypes.c_float
        lib.kvq_oracle_e2m1_to_f32.argtypes = [ctypes.c_uint8]
        lib.kvq_oracle_e2m1_to_f32.restype = ctypes.c_float
        _lib_handle = lib
    return _lib_handle


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _view_strides(x: np.ndarray):
    if x.dtype != np.uint16 or x.ndim != 3:
        raise ValueError("expected a uint16 [T, H, D] array of bf16 bits")
    st, sh, sd = (s // 2 for s in x.strides)
    if x.size and x.shape[2] > 1 and sd != 1:
        raise ValueError("channel stride must be 1")
    return st, sh


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


@dataclass
class Packed:
    """One encoded tensor: codes [rows, H, ceil(D/2)] u8, metadata planes, global scale, positions."""

    format: str
    kind: str
    group_size: int
    rows: int
    H: int
    D: int
    codes: np.ndarray
    meta0: np.ndarray  # int4: f16 minimum bits (uint16); nvfp4: E4M3 block scale bytes (uint8)
    meta1: Optional[np.ndarray]  # int4: f16 scale bits (uint16); nvfp4: None
    global_scale: Optional[np.ndarray]  # nvfp4: float32[1]
    positions: Optional[np.ndarray] = field(default=None)  # sparse residual: owned int32 copy


def meta_shape(kind: str, G: int, rows: int, H: int, D: int):
    return (ceil_div(rows, G), H, D) if kind == "key" else (rows, H, ceil_div(D, G))


def _alloc(fmt: str, kind: str, G: int, rows: int, H: int, D: int) -> Packed:
    codes = np.zeros((rows, H, ceil_div(D, 2)), np.uint8)
    ms = meta_shape(kind, G, rows, H, D)
    if fmt == "int4":
        return Packed(fmt, kind, G, rows, H, D, codes, np.zeros(ms, np.uint16), np.zeros(ms, np.uint16), None)
    return Packed(fmt, kind, G, rows, H, D, codes, np.zeros(ms, np.uint8), None, np.zeros(1, np.float32))


def default_group(fmt: str) -> int:
    return 64 if fmt == "int4" else 16


def pack(x: np.ndarray, kind: str, fmt: str = "int4", G: Optional[int] = None,
         global_scale: Optional[float] = None) -> Packed:
    """pack_kv of a bf16 [T, H, D] view. ``global_scale`` (NVFP4 only) encodes these rows with
    the multiplier of a larger tensor they are a slice of; by default the rows are the whole
    encoded tensor and the multiplier is computed from their own amax."""
    G = G or default_group(fmt)
    st, sh = _view_strides(x)
    T, H, D = x.shape
    out = _alloc(fmt, kind, G, T, H, D)
    rc = _lib().kvq_oracle_pack(_ptr(x), T, H, D, st, sh, KIND[kind], FORMAT[fmt], G, _ptr(out.codes),
                                _ptr(out.meta0), _ptr(out.meta1), _ptr(out.global_scale),
                                -1.0 if global_scale is None else float(global_scale))
    if rc:
        raise ValueError(f"oracle pack failed ({rc})")
    return out


def unpack(p: Packed, out: Optional[np.ndarray] = None) -> np.ndarray:
    """unpack_kv: decoded bf16 bits [rows, H, D]."""
    if out is None:
        out = np.zeros((p.rows, p.H, p.D), np.uint16)
    st, sh = _view_strides(out)
    rc = _lib().kvq_oracle_unpack(KIND[p.kind], FORMAT[p.format], p.group_size, p.rows, p.H, p.D, _ptr(p.codes),
                                  _ptr(p.meta0), _ptr(p.meta1), _ptr(p.global_scale), _ptr(out), st, sh)
    if rc:
        raise ValueError(f"oracle unpack failed ({rc})")
    return out


def encode_residual(cur: np.ndarray, prev: np.ndarray, kind: str, fmt: str = "int4", G: Optional[int] = None,
                    positions: Optional[np.ndarray] = None, global_scale: Optional[float] = None) -> Packed:
    """encode_residual of cur against the reconstructed predecessor prev (both [T, H, D]).
    ``global_scale`` as in ``pack``."""
    G = G or default_group(fmt)
    cst, csh = _view_strides(cur)
    pst, psh = _view_strides(prev)
    if cur.shape != prev.shape:
        raise ValueError("cur/prev shape mismatch")
    T, H, D = cur.shape
    pos = None
    M = 0
    if positions is not None:
        pos = np.ascontiguousarray(positions, dtype=np.int32)
        M = int(pos.shape[0])
    rows = M if pos is not None else T
    out = _alloc(fmt, kind, G, rows, H, D)
    if pos is not None:
        out.positions = np.zeros(M, np.int32)
    rc = _lib().kvq_oracle_encode_residual(_ptr(cur), cst, csh, _ptr(prev), pst, psh, T, H, D, _ptr(pos), M,
                                           KIND[kind], FORMAT[fmt], G, _ptr(out.codes), _ptr(out.meta0),
                                           _ptr(out.meta1), _ptr(out.global_scale), _ptr(out.positions),
                                           -1.0 if global_scale is None else float(global_scale))
    if rc:
        raise ValueError(f"oracle encode_residual failed ({rc})")
    return out


def decode_residual(r: Packed, prev: np.ndarray, out: Optional[np.ndarray] = None) -> np.ndarray:
    """decode_residual: prev + unpack(r) in the input dtype; absent sparse rows copy prev."""
    if out is None:
        out = np.zeros(prev.shape, np.uint16)
    pst, psh = _view_strides(prev)
    ost, osh = _view_strides(out)
    T = prev.shape[0]
    rc = _lib().kvq_oracle_decode_residual(KIND[r.kind], FORMAT[r.format], r.group_size, r.rows, r.H, r.D,
                                           _ptr(r.codes), _ptr(r.meta0), _ptr(r.meta1), _ptr(r.global_scale),
                                           _ptr(r.positions), _ptr(prev), pst, psh, T, _ptr(out), ost, osh)
    if rc:
        raise ValueError(f"oracle decode_residual failed ({rc})")
    return out


def tensor_amax(cur: np.ndarray, prev: Optional[np.ndarray] = None, positions: Optional[np.ndarray] = None) -> float:
    """max |x| over the rows an encode of (cur[, prev][, positions]) sees."""
    cst, csh = _view_strides(cur)
    pst, psh = _view_strides(prev) if prev is not None else (0, 0)
    T, H, D = cur.shape
    pos = None if positions is None else np.ascontiguousarray(positions, dtype=np.int32)
    M = 0 if pos is None else int(pos.shape[0])
    return float(_lib().kvq_oracle_tensor_amax(_ptr(cur), cst, csh, _ptr(prev), pst, psh, T, H, D, _ptr(pos), M))


def storage_bytes(fmt: str, kind: str, G: int, rows: int, H: int, D: int, sparse: bool = False) -> int:
    return int(_lib().kvq_oracle_storage_bytes(FORMAT[fmt], KIND[kind], G, rows, H, D, int(bool(sparse))))


# ---- scalar conversions, vectorized over numpy arrays (for the pin tests) ----

def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    y = np.empty(x.shape, np.uint16)
    _lib().kvq_oracle_f32_to_bf16_n(_ptr(x), _ptr(y), x.size)
    return y


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    y = np.empty(x.shape, np.uint16)
    _lib().kvq_oracle_f32_to_f16_n(_ptr(x), _ptr(y), x.size)
    return y


def f32_to_e4m3(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32)
    y = np.empty(x.shape, np.uint8)
    _lib().kvq_oracle_f32_to_e4m3_n(_ptr(x), _ptr(y), x.size)
    return y


def e2m1_encode(q: np.ndarray) -> np.ndarray:
    """E2M1 code of each value (sign from the value itself)."""
    q = np.ascontiguousarray(q, np.float32)
    y = np.empty(q.shape, np.uint8)
    _lib().kvq_oracle_e2m1_encode_n(_ptr(q), _ptr(y), q.size)
    return y


def f16_to_f32(h: int) -> float:
    return float(_lib().kvq_oracle_f16_to_f32(h))


def e4m3_to_f32(b: int) -> float:
    return float(_lib().kvq_oracle_e4m3_to_f32(b))


def e2m1_to_f32(c: int) -> float:
    return float(_lib().kvq_oracle_e2m1_to_f32(c))


def nvfp4_global(amax: float) -> float:
    return float(_lib().kvq_oracle_nvfp4_global(amax))


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32 (upper half of the binary32 word)."""
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)
