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
_LIB_OMP = os.path.join(_HERE, "libkvq_oracle_omp.so")

KIND = {"key": 0, "value": 1}
FORMAT = {"int4": 0, "nvfp4": 1, "nvfp4_row": 2, "fp8_row": 3}

# -O2 without -march=native; -ffp-contract=off so that no multiply-add is fused.
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: ``oracle/libkvq_oracle.so`` (single-threaded) and
    ``oracle/libkvq_oracle_omp.so`` (the same source with -fopenmp: loops over independent
    groups and rows on all threads, same bits)."""
    for path, extra in ((_LIB, []), (_LIB_OMP, ["-fopenmp"])):
        if force or not os.path.exists(path):
            tmp = path + ".tmp"
            subprocess.run(["gcc", *CFLAGS, *extra, _SRC, "-o", tmp, "-lm"], check=True)
            os.replace(tmp, path)
    return _LIB


_handles = {}
_threaded = False


def set_threaded(on: bool) -> bool:
    """Route every call below to the OpenMP build (True) or the single-threaded build (False).
    Returns the previous setting."""
    global _threaded
    prev, _threaded = _threaded, bool(on)
    return prev


def threads() -> int:
    """Threads the active build runs its loops on (1 for the single-threaded build)."""
    return int(_lib().kvq_oracle_threads())


def _lib():
    path = _LIB_OMP if _threaded else _LIB
    if path not in _handles:
        if not os.path.exists(path):
            build(force=False)
        lib = ctypes.CDLL(path)
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
        lib.kvq_oracle_pack_paged.argtypes = [p, i64, i64, i64, i64, i64, i64, i64, ci, ci, i32, ci, p, p, p, p]
        lib.kvq_oracle_pack_paged.restype = ci
        lib.kvq_oracle_unpack_paged.argtypes = [ci, ci, i32, ci, i64, i64, i64, i64, p, p, p, p, p, i64, i64, i64]
        lib.kvq_oracle_unpack_paged.restype = ci
        lib.kvq_oracle_store_rows.argtypes = [p, i64, i64, i64, i64, i64, p, ci, ci, i32, i64, p, p, p]
        lib.kvq_oracle_store_rows.restype = ci
        lib.kvq_oracle_load_rows.argtypes = [ci, ci, i32, i64, i64, i64, p, p, p, p, p, i64, p, i64, i64]
        lib.kvq_oracle_load_rows.restype = ci
        lib.kvq_oracle_encode_window.argtypes = [p, i64, i64, p, i64, i64, i64, i64, i64, i64, i64, ci, ci, i32,
                                                 p, p, p, p, p]
        lib.kvq_oracle_encode_window.restype = ci
        lib.kvq_oracle_decode_window.argtypes = [ci, ci, i32, i64, i64, i64, i64, i64, p, p, p, p, p, p, i64, i64,
                                                 p, i64, i64]
        lib.kvq_oracle_decode_window.restype = ci
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
        lib.kvq_oracle_threads.argtypes = []
        lib.kvq_oracle_threads.restype = ci
        _handles[path] = lib
    return _handles[path]


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
    """One encoded tensor: codes, metadata planes, global scale, positions.

    codes: [rows, H, ceil(D/2)] u8 nibbles ([rows, H, D] one byte per element for fp8_row).
    meta0: int4 f16 minimum bits (uint16); nvfp4 and nvfp4_row E4M3 block scales (uint8);
           fp8_row FP32 row scales [rows, H].
    meta1: int4 f16 scale bits (uint16); nvfp4_row FP32 row multipliers [rows, H]; else None.
    global_scale: nvfp4 float32[1]; else None.
    page_local / page_size: set by pack_paged when KEY groups were kept inside pages (the KEY
    metadata then has ceil(page_size/G) rows per page)."""

    format: str
    kind: str
    group_size: int
    rows: int
    H: int
    D: int
    codes: np.ndarray
    meta0: np.ndarray
    meta1: Optional[np.ndarray]
    global_scale: Optional[np.ndarray]
    positions: Optional[np.ndarray] = field(default=None)  # sparse residual: owned int32 copy
    page_local: bool = False
    page_size: int = 0


def meta_shape(kind: str, G: int, rows: int, H: int, D: int, fmt: str = "int4"):
    if fmt == "nvfp4_row":
        return (rows, H, ceil_div(D, 16))
    if fmt == "fp8_row":
        return (rows, H)
    return (ceil_div(rows, G), H, D) if kind == "key" else (rows, H, ceil_div(D, G))


def _alloc(fmt: str, kind: str, G: int, rows: int, H: int, D: int, key_meta_rows: Optional[int] = None) -> Packed:
    codes = np.zeros((rows, H, D if fmt == "fp8_row" else ceil_div(D, 2)), np.uint8)
    ms = meta_shape(kind, G, rows, H, D, fmt)
    if key_meta_rows is not None:
        ms = (key_meta_rows, H, D)
    if fmt == "int4":
        return Packed(fmt, kind, G, rows, H, D, codes, np.zeros(ms, np.uint16), np.zeros(ms, np.uint16), None)
    if fmt == "nvfp4":
        return Packed(fmt, kind, G, rows, H, D, codes, np.zeros(ms, np.uint8), None, np.zeros(1, np.float32))
    if fmt == "nvfp4_row":
        return Packed(fmt, kind, G, rows, H, D, codes, np.zeros(ms, np.uint8), np.zeros((rows, H), np.float32), None)
    return Packed(fmt, kind, G, rows, H, D, codes, np.zeros(ms, np.float32), None, None)


def default_group(fmt: str) -> int:
    return {"int4": 64, "nvfp4": 16, "nvfp4_row": 16, "fp8_row": 0}[fmt]


def _group(fmt: str, G: Optional[int]) -> int:
    return default_group(fmt) if G is None or (G == 0 and fmt != "fp8_row") else int(G)


def pack(x: np.ndarray, kind: str, fmt: str = "int4", G: Optional[int] = None,
         global_scale: Optional[float] = None) -> Packed:
    """pack_kv of a bf16 [T, H, D] view. ``global_scale`` (NVFP4 only) encodes these rows with
    the multiplier of a larger tensor they are a slice of; by default the rows are the whole
    encoded tensor and the multiplier is computed from their own amax."""
    G = _group(fmt, G)
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
    G = _group(fmt, G)
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


def _paged_strides(x: np.ndarray):
    if x.dtype != np.uint16 or x.ndim != 4:
        raise ValueError("expected a uint16 [P, S, H, D] array of bf16 bits")
    sp, ss, sh, sd = (s // 2 for s in x.strides)
    if x.size and x.shape[3] > 1 and sd != 1:
        raise ValueError("channel stride must be 1")
    return sp, ss, sh


def pack_paged(x: np.ndarray, kind: str, fmt: str = "int4", G: Optional[int] = None, page_local: bool = False) -> Packed:
    """pack_paged of a bf16 paged view [P, S, H, D] (pages in page-major token order)."""
    G = _group(fmt, G)
    sp, ss, sh = _paged_strides(x)
    P, S, H, D = x.shape
    local = bool(page_local) and kind == "key" and fmt in ("int4", "nvfp4")
    out = _alloc(fmt, kind, G, P * S, H, D, key_meta_rows=P * ceil_div(S, G) if local else None)
    out.page_local, out.page_size = local, S
    rc = _lib().kvq_oracle_pack_paged(_ptr(x), P, S, H, D, sp, ss, sh, KIND[kind], FORMAT[fmt], G, int(local),
                                      _ptr(out.codes), _ptr(out.meta0), _ptr(out.meta1), _ptr(out.global_scale))
    if rc:
        raise ValueError(f"oracle pack_paged failed ({rc})")
    return out


def unpack_paged(p: Packed, P: int, S: int, out: Optional[np.ndarray] = None) -> np.ndarray:
    """unpack_paged: decoded bf16 bits written into a paged view [P, S, H, D]."""
    if P * S != p.rows:
        raise ValueError("pages x page_size != rows")
    if out is None:
        out = np.zeros((P, S, p.H, p.D), np.uint16)
    sp, ss, sh = _paged_strides(out)
    rc = _lib().kvq_oracle_unpack_paged(KIND[p.kind], FORMAT[p.format], p.group_size, int(p.page_local), P, S, p.H,
                                        p.D, _ptr(p.codes), _ptr(p.meta0), _ptr(p.meta1), _ptr(p.global_scale),
                                        _ptr(out), sp, ss, sh)
    if rc:
        raise ValueError(f"oracle unpack_paged failed ({rc})")
    return out


def store_rows(cache: Packed, x: np.ndarray, slots: np.ndarray) -> None:
    """Quantize the rows x[N, H, D] and write row i into cache row slots[i] (in place)."""
    st, sh = _view_strides(x)
    N, H, D = x.shape
    if (H, D) != (cache.H, cache.D):
        raise ValueError("row shape mismatch")
    sl = np.ascontiguousarray(slots, dtype=np.int32)
    if sl.shape != (N,):
        raise ValueError("one slot per row")
    rc = _lib().kvq_oracle_store_rows(_ptr(x), N, H, D, st, sh, _ptr(sl), KIND[cache.kind], FORMAT[cache.format],
                                      cache.group_size, cache.rows, _ptr(cache.codes), _ptr(cache.meta0),
                                      _ptr(cache.meta1))
    if rc:
        raise ValueError(f"oracle store_rows failed ({rc})")


def load_rows(cache: Packed, slots: np.ndarray, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Decoded bf16 bits of cache rows slots[0..N) as [N, H, D]."""
    sl = np.ascontiguousarray(slots, dtype=np.int32)
    N = int(sl.shape[0])
    if out is None:
        out = np.zeros((N, cache.H, cache.D), np.uint16)
    st, sh = _view_strides(out)
    rc = _lib().kvq_oracle_load_rows(KIND[cache.kind], FORMAT[cache.format], cache.group_size, cache.rows, cache.H,
                                     cache.D, _ptr(cache.codes), _ptr(cache.meta0), _ptr(cache.meta1),
                                     _ptr(cache.global_scale), _ptr(sl), N, _ptr(out), st, sh)
    if rc:
        raise ValueError(f"oracle load_rows failed ({rc})")
    return out


def window_split(T: int, sink: int, recent: int):
    """(rows kept at the front, rows kept at the end) of a BF16 window over T tokens."""
    ns = min(sink, T)
    return ns, min(recent, T - ns)


@dataclass
class Windowed:
    """A tensor encoded with a BF16 window: the quantized middle rows and the raw protected rows."""

    packed: Packed
    window: np.ndarray  # uint16 bf16 bits [n_sink + n_recent, H, D]
    T: int
    sink: int
    recent: int


def encode_window(cur: np.ndarray, kind: str, fmt: str = "int4", G: Optional[int] = None, sink: int = 4,
                  recent: int = 16, prev: Optional[np.ndarray] = None) -> Windowed:
    """Pack (prev None) or residual-encode cur with its first `sink` and latest `recent` rows kept
    in BF16."""
    G = _group(fmt, G)
    cst, csh = _view_strides(cur)
    pst, psh = _view_strides(prev) if prev is not None else (0, 0)
    if prev is not None and prev.shape != cur.shape:
        raise ValueError("cur/prev shape mismatch")
    T, H, D = cur.shape
    ns, nr = window_split(T, sink, recent)
    out = _alloc(fmt, kind, G, T - ns - nr, H, D)
    win = np.zeros((ns + nr, H, D), np.uint16)
    rc = _lib().kvq_oracle_encode_window(_ptr(cur), cst, csh, _ptr(prev), pst, psh, T, H, D, sink, recent,
                                         KIND[kind], FORMAT[fmt], G, _ptr(out.codes), _ptr(out.meta0),
                                         _ptr(out.meta1), _ptr(out.global_scale), _ptr(win))
    if rc:
        raise ValueError(f"oracle encode_window failed ({rc})")
    return Windowed(out, win, T, sink, recent)


def decode_window(w: Windowed, prev: Optional[np.ndarray] = None, out: Optional[np.ndarray] = None) -> np.ndarray:
    """Decode a windowed tensor (adding to prev for a residual) into bf16 bits [T, H, D]."""
    p = w.packed
    if out is None:
        out = np.zeros((w.T, p.H, p.D), np.uint16)
    ost, osh = _view_strides(out)
    pst, psh = _view_strides(prev) if prev is not None else (0, 0)
    win = np.ascontiguousarray(w.window)  # kept alive across the call
    rc = _lib().kvq_oracle_decode_window(KIND[p.kind], FORMAT[p.format], p.group_size, w.T, p.H, p.D, w.sink,
                                         w.recent, _ptr(p.codes), _ptr(p.meta0), _ptr(p.meta1),
                                         _ptr(p.global_scale), _ptr(win), _ptr(prev), pst, psh, _ptr(out), ost, osh)
    if rc:
        raise ValueError(f"oracle decode_window failed ({rc})")
    return out


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
