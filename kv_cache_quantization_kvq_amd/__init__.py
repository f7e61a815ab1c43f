"""kvq -- KV-cache quantization codec for AMD MI355X (gfx950): Python binding.

A thin ctypes binding over ``libkvq.so`` (the C ABI in ``include/kvq.h``). It marshals torch
device tensors into ``kvq_tensor`` / ``kvq_packed`` descriptors and allocates the packed planes
with torch; every step of the codec runs in the library's HIP kernels on the current stream.
There is no CPU fallback: importing works anywhere, but the first call that needs the library
raises if ``libkvq.so`` is missing, and compute calls require tensors on a ROCm device.

Usage (the four-call form of the codec page's usage example)::

    packed = kvq.pack(values, kind="key", format="nvfp4")
    previous = kvq.unpack(packed)
    residual = kvq.encode_residual(current, previous, kind="key", format="nvfp4")
    rebuilt = kvq.decode_residual(residual, previous)

Paged caches: ``pack_paged`` / ``unpack_paged`` take [pages, page_size, H, D] views;
``store_rows`` quantizes new rows straight into cache slots named by a device int32 tensor
(row formats and INT4 VALUE) and ``load_rows`` decodes rows by slot.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIBRARY may point at another build of the same library (e.g. a tuning variant); it must
# exist like the default one does -- there is no fallback.
LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(_PKG, "libkvq.so")

KIND = {"key": 0, "value": 1}
FORMAT = {"int4": 0, "nvfp4": 1, "nvfp4_row": 2, "fp8_row": 3}
KIND_NAME = {v: k for k, v in KIND.items()}
FORMAT_NAME = {v: k for k, v in FORMAT.items()}
STATUS = {0: "KVQ_OK", 1: "KVQ_ERR_NULL", 2: "KVQ_ERR_SHAPE", 3: "KVQ_ERR_LAYOUT", 4: "KVQ_ERR_FORMAT",
          5: "KVQ_ERR_GROUP", 6: "KVQ_ERR_DTYPE", 7: "KVQ_ERR_MISMATCH", 8: "KVQ_ERR_HIP", 9: "KVQ_ERR_WORKSPACE",
          10: "KVQ_ERR_SCRATCH"}
PLANES = ("codes", "meta0", "meta1", "global_scale", "positions")
EXPORTS = ("kvq_version", "kvq_status_string", "kvq_storage_bytes", "kvq_plane_bytes", "kvq_workspace_bytes",
           "kvq_pack", "kvq_unpack", "kvq_encode_residual", "kvq_decode_residual", "kvq_validate_positions",
           "kvq_pack_paged", "kvq_unpack_paged", "kvq_store_rows", "kvq_load_rows", "kvq_encode_window",
           "kvq_decode_window", "kvq_attention_workspace_bytes", "kvq_decode_attention",
           "kvq_decode_attention_noalloc", "kvq_nvfp4_global_scale")


class KvqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {STATUS.get(status, status)}")
        self.status = status


class KvqTensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("T", ctypes.c_int64), ("H", ctypes.c_int64), ("D", ctypes.c_int64),
                ("stride_t", ctypes.c_int64), ("stride_h", ctypes.c_int64)]


class KvqPaged(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("pages", ctypes.c_int64), ("page_size", ctypes.c_int64), ("H", ctypes.c_int64),
                ("D", ctypes.c_int64), ("stride_page", ctypes.c_int64), ("stride_slot", ctypes.c_int64),
                ("stride_h", ctypes.c_int64)]


class KvqPacked(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("kind", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("rows", ctypes.c_int64), ("H", ctypes.c_int64), ("D", ctypes.c_int64),
                ("full_T", ctypes.c_int64), ("codes", ctypes.c_void_p), ("meta0", ctypes.c_void_p),
                ("meta1", ctypes.c_void_p), ("global_scale", ctypes.c_void_p), ("positions", ctypes.c_void_p)]


_lib = None


def library() -> ctypes.CDLL:
    """Load ``libkvq.so`` (built in-tree by ``__graft_entry__.build()``). Raises if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"kvq: {LIB_PATH} is not built; run __graft_entry__.build() first "
                               "(there is no fallback implementation)")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, I64, U64P = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_uint64)
        lib.kvq_version.restype = ctypes.c_char_p
        lib.kvq_version.argtypes = []
        lib.kvq_status_string.restype = ctypes.c_char_p
        lib.kvq_status_string.argtypes = [ctypes.c_int]
        lib.kvq_storage_bytes.argtypes = [ctypes.c_int, ctypes.c_int, I32, I64, I64, I64, I32, U64P]
        lib.kvq_storage_bytes.restype = ctypes.c_int
        lib.kvq_plane_bytes.argtypes = [ctypes.c_int, ctypes.c_int, I32, I64, I64, I64, I32, U64P]
        lib.kvq_plane_bytes.restype = ctypes.c_int
        lib.kvq_workspace_bytes.argtypes = []
        lib.kvq_workspace_bytes.restype = ctypes.c_size_t
        TP, PP = ctypes.POINTER(KvqTensor), ctypes.POINTER(KvqPacked)
        lib.kvq_pack.argtypes = [TP, ctypes.c_int, ctypes.c_int, I32, PP, P, P]
        lib.kvq_pack.restype = ctypes.c_int
        lib.kvq_unpack.argtypes = [PP, TP, P]
        lib.kvq_unpack.restype = ctypes.c_int
        lib.kvq_encode_residual.argtypes = [TP, TP, P, I64, ctypes.c_int, ctypes.c_int, I32, PP, P, P]
        lib.kvq_encode_residual.restype = ctypes.c_int
        lib.kvq_decode_residual.argtypes = [PP, TP, TP, P]
        lib.kvq_decode_residual.restype = ctypes.c_int
        lib.kvq_validate_positions.argtypes = [P, I64, I64, P, P, P]
        lib.kvq_validate_positions.restype = ctypes.c_int
        GP = ctypes.POINTER(KvqPaged)
        lib.kvq_pack_paged.argtypes = [GP, ctypes.c_int, ctypes.c_int, I32, I32, PP, P, P]
        lib.kvq_pack_paged.restype = ctypes.c_int
        lib.kvq_unpack_paged.argtypes = [PP, GP, P]
        lib.kvq_unpack_paged.restype = ctypes.c_int
        lib.kvq_store_rows.argtypes = [TP, P, PP, P]
        lib.kvq_store_rows.restype = ctypes.c_int
        lib.kvq_load_rows.argtypes = [PP, P, TP, P]
        lib.kvq_load_rows.restype = ctypes.c_int
        lib.kvq_encode_window.argtypes = [TP, TP, I64, I64, ctypes.c_int, ctypes.c_int, I32, PP, P, P, P]
        lib.kvq_encode_window.restype = ctypes.c_int
        lib.kvq_decode_window.argtypes = [PP, P, I64, I64, TP, TP, P]
        lib.kvq_decode_window.restype = ctypes.c_int
        lib.kvq_attention_workspace_bytes.argtypes = [I64, I64, I64, I64]
        lib.kvq_attention_workspace_bytes.restype = ctypes.c_size_t
        lib.kvq_decode_attention.argtypes = [P, I64, PP, PP, PP, PP, ctypes.c_float, P, P, ctypes.c_size_t, P]
        lib.kvq_decode_attention.restype = ctypes.c_int
        lib.kvq_decode_attention_noalloc.argtypes = [P, I64, PP, PP, PP, PP, ctypes.c_float, P, P]
        lib.kvq_decode_attention_noalloc.restype = ctypes.c_int
        lib.kvq_nvfp4_global_scale.argtypes = [TP, TP, P, I64, P, P, P]
        lib.kvq_nvfp4_global_scale.restype = ctypes.c_int
        _lib = lib
    return _lib


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise KvqError(fn, status)


def version() -> str:
    return library().kvq_version().decode()


def default_group(fmt: str) -> int:
    return {"int4": 64, "nvfp4": 16, "nvfp4_row": 16, "fp8_row": 0}[fmt]


def plane_bytes(fmt: str, kind: str, group_size: int, rows: int, H: int, D: int, sparse: bool = False) -> Dict[str, int]:
    sizes = (ctypes.c_uint64 * 5)()
    _check("kvq_plane_bytes", library().kvq_plane_bytes(FORMAT[fmt], KIND[kind], group_size, rows, H, D,
                                                         int(bool(sparse)), sizes))
    return dict(zip(PLANES, (int(s) for s in sizes)))


def storage_bytes(fmt: str, kind: str, group_size: int, rows: int, H: int, D: int, sparse: bool = False) -> int:
    out = ctypes.c_uint64()
    _check("kvq_storage_bytes", library().kvq_storage_bytes(FORMAT[fmt], KIND[kind], group_size, rows, H, D,
                                                             int(bool(sparse)), ctypes.byref(out)))
    return int(out.value)


def meta_shape(kind: str, G: int, rows: int, H: int, D: int, fmt: str = "int4") -> Tuple[int, ...]:
    if fmt == "nvfp4_row":
        return (rows, H, -(-D // 16))
    if fmt == "fp8_row":
        return (rows, H)
    return (-(-rows // G), H, D) if kind == "key" else (rows, H, -(-D // G))


@dataclass
class Packed:
    """An encoded tensor: torch planes on the device plus the descriptor fields."""

    format: str
    kind: str
    group_size: int
    rows: int
    H: int
    D: int
    full_T: int
    codes: torch.Tensor  # uint8 [rows, H, ceil(D/2)] ([rows, H, D] for fp8_row)
    meta0: torch.Tensor  # int4: f16 minimums (int16 view); nvfp4(_row): E4M3 bytes; fp8_row: float32 [rows, H]
    meta1: Optional[torch.Tensor]  # int4: f16 scales (int16 view); nvfp4_row: float32 row multipliers [rows, H]
    global_scale: Optional[torch.Tensor]  # nvfp4: float32 [1]
    positions: Optional[torch.Tensor] = None  # sparse residual: owned int32 [rows]
    # storage behind `positions`, at least one element so that a sparse residual with no rows
    # still has the non-NULL position pointer that marks it sparse
    pos_buf: Optional[torch.Tensor] = None

    def descriptor(self) -> KvqPacked:
        return KvqPacked(FORMAT[self.format], KIND[self.kind], self.group_size, 0, self.rows, self.H, self.D,
                         self.full_T, _ptr(self.codes), _ptr(self.meta0), _ptr(self.meta1), _ptr(self.global_scale),
                         _ptr(self.pos_buf if self.pos_buf is not None else self.positions))

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.codes, self.meta0, self.meta1, self.global_scale,
                                                          self.positions) if t is not None)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _view(x: torch.Tensor) -> KvqTensor:
    if x.dtype != torch.bfloat16:
        raise TypeError("kvq: tensors must be bfloat16")
    if x.dim() != 3:
        raise ValueError("kvq: tensors must be [T, H, D]")
    T, H, D = x.shape
    if D > 1 and x.stride(2) != 1 and x.numel() > 0:
        raise ValueError("kvq: channel stride must be 1")
    return KvqTensor(ctypes.c_void_p(x.data_ptr()), 0, 0, T, H, D, x.stride(0), x.stride(1))


def _device_of(x: torch.Tensor) -> torch.device:
    if x.device.type != "cuda":
        raise ValueError("kvq: tensors must be on a ROCm device (no CPU path)")
    return x.device


def _stream(dev: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


_workspaces: Dict[Tuple[int, int], torch.Tensor] = {}
_empty_maps: Dict[int, torch.Tensor] = {}


def _empty_map(dev: torch.device) -> torch.Tensor:
    """A one-element device int32 tensor whose (non-NULL) address stands for an empty position
    map: the library never reads it when M == 0."""
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    t = _empty_maps.get(key)
    if t is None:
        t = torch.zeros(1, dtype=torch.int32, device=dev)
        _empty_maps[key] = t
    return t


def workspace(dev: torch.device) -> torch.Tensor:
    """Workspace for NVFP4 encodes (per-block partial maxima), one per (device, current stream),
    allocated once."""
    key = (dev.index if dev.index is not None else torch.cuda.current_device(), torch.cuda.current_stream(dev).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None:
        ws = torch.zeros(int(library().kvq_workspace_bytes()), dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    return ws


def alloc_packed(fmt: str, kind: str, group_size: int, rows: int, H: int, D: int, full_T: int,
                 dev: torch.device, sparse: bool = False) -> Packed:
    G = group_size or default_group(fmt)
    sizes = plane_bytes(fmt, kind, G, rows, H, D, sparse)
    ms = meta_shape(kind, G, rows, H, D, fmt)
    codes = torch.empty((rows, H, D if fmt == "fp8_row" else -(-D // 2)), dtype=torch.uint8, device=dev)
    meta1, gs = None, None
    if fmt == "int4":
        meta0 = torch.empty(ms, dtype=torch.int16, device=dev)
        meta1 = torch.empty(ms, dtype=torch.int16, device=dev)
    elif fmt == "nvfp4":
        meta0 = torch.empty(ms, dtype=torch.uint8, device=dev)
        gs = torch.empty(1, dtype=torch.float32, device=dev)
    elif fmt == "nvfp4_row":
        meta0 = torch.empty(ms, dtype=torch.uint8, device=dev)
        meta1 = torch.empty((rows, H), dtype=torch.float32, device=dev)
    else:
        meta0 = torch.empty(ms, dtype=torch.float32, device=dev)
    pos_buf = torch.empty(max(rows, 1), dtype=torch.int32, device=dev) if sparse else None
    pos = pos_buf[:rows] if sparse else None
    p = Packed(fmt, kind, G, rows, H, D, full_T, codes, meta0, meta1, gs, pos, pos_buf)
    assert p.nbytes() == sum(sizes.values())
    return p


def pack(x: torch.Tensor, kind: str = "key", format: str = "int4", group_size: int = 0,
         out: Optional[Packed] = None) -> Packed:
    """pack_kv: encode a bf16 [T, H, D] view (any token/head strides, channel stride 1)."""
    dev = _device_of(x)
    T, H, D = x.shape
    G = group_size or default_group(format)
    if out is None:
        out = alloc_packed(format, kind, G, T, H, D, T, dev)
    desc = out.descriptor()
    ws = workspace(dev) if format == "nvfp4" else None
    _check("kvq_pack", library().kvq_pack(ctypes.byref(_view(x)), KIND[kind], FORMAT[format], G, ctypes.byref(desc),
                                          _ptr(ws), _stream(dev)))
    return out


def unpack(p: Packed, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """unpack_kv: decode to a bf16 [rows, H, D] tensor (or into the view `out`)."""
    dev = p.codes.device
    if out is None:
        out = torch.empty((p.rows, p.H, p.D), dtype=torch.bfloat16, device=dev)
    desc = p.descriptor()
    _check("kvq_unpack", library().kvq_unpack(ctypes.byref(desc), ctypes.byref(_view(out)), _stream(dev)))
    return out


def encode_residual(current: torch.Tensor, previous: torch.Tensor, kind: str = "key", format: str = "int4",
                    group_size: int = 0, positions: Optional[torch.Tensor] = None,
                    out: Optional[Packed] = None) -> Packed:
    """encode_residual of `current` against the reconstructed predecessor `previous`; with
    `positions` (device int32 [M]) only those rows are encoded, in that order."""
    dev = _device_of(current)
    T, H, D = current.shape
    G = group_size or default_group(format)
    M = 0
    pos_ptr = None
    if positions is not None:
        if positions.dtype != torch.int32 or positions.device != current.device or positions.dim() != 1:
            raise ValueError("kvq: positions must be a 1-D int32 tensor on the tensors' device")
        positions = positions.contiguous()
        M = positions.numel()
        pos_ptr = _ptr(positions if M > 0 else _empty_map(dev))
    rows = M if positions is not None else T
    if out is None:
        out = alloc_packed(format, kind, G, rows, H, D, T, dev, sparse=positions is not None)
    desc = out.descriptor()
    ws = workspace(dev) if format == "nvfp4" else None
    _check("kvq_encode_residual",
           library().kvq_encode_residual(ctypes.byref(_view(current)), ctypes.byref(_view(previous)), pos_ptr, M,
                                         KIND[kind], FORMAT[format], G, ctypes.byref(desc), _ptr(ws), _stream(dev)))
    out.full_T = T
    return out


def nvfp4_global_scale(current: torch.Tensor, previous: Optional[torch.Tensor] = None,
                       positions: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The NVFP4 multiplier fl(2688 / amax) that an NVFP4 pack (previous None) or residual
    encode of the same arguments stores, as a device float32 [1] tensor."""
    dev = _device_of(current)
    M = 0
    pos_ptr = None
    if positions is not None:
        if positions.dtype != torch.int32 or positions.device != current.device or positions.dim() != 1:
            raise ValueError("kvq: positions must be a 1-D int32 tensor on the tensors' device")
        positions = positions.contiguous()
        M = positions.numel()
        pos_ptr = _ptr(positions if M > 0 else _empty_map(dev))
    if out is None:
        out = torch.empty(1, dtype=torch.float32, device=dev)
    prev = ctypes.byref(_view(previous)) if previous is not None else None
    _check("kvq_nvfp4_global_scale", library().kvq_nvfp4_global_scale(
        ctypes.byref(_view(current)), prev, pos_ptr, M, _ptr(out), _ptr(workspace(dev)), _stream(dev)))
    return out


def decode_residual(r: Packed, previous: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """decode_residual: previous + unpack(r) in the input dtype; absent sparse rows copy
    `previous`. `out` may be `previous` itself (in place)."""
    dev = r.codes.device
    if out is None:
        out = torch.empty(previous.shape, dtype=torch.bfloat16, device=dev)
    desc = r.descriptor()
    _check("kvq_decode_residual", library().kvq_decode_residual(ctypes.byref(desc), ctypes.byref(_view(previous)),
                                                                ctypes.byref(_view(out)), _stream(dev)))
    return out


def _paged_view(x: torch.Tensor) -> KvqPaged:
    if x.dtype != torch.bfloat16:
        raise TypeError("kvq: tensors must be bfloat16")
    if x.dim() != 4:
        raise ValueError("kvq: paged tensors must be [pages, page_size, H, D]")
    P, S, H, D = x.shape
    if D > 1 and x.stride(3) != 1 and x.numel() > 0:
        raise ValueError("kvq: channel stride must be 1")
    return KvqPaged(ctypes.c_void_p(x.data_ptr()), 0, 0, P, S, H, D, x.stride(0), x.stride(1), x.stride(2))


def page_local_group(fmt: str, kind: str, group_size: int, page_size: int) -> int:
    """Group size a page-local packing records: INT4 KEY groups shrink to the page."""
    G = group_size or default_group(fmt)
    if fmt == "int4" and kind == "key" and 0 < page_size < G:
        return page_size
    return G


def pack_paged(x: torch.Tensor, kind: str = "key", format: str = "int4", group_size: int = 0,
               page_local: bool = False, out: Optional[Packed] = None) -> Packed:
    """pack_paged: encode a bf16 [pages, page_size, H, D] view in page-major token order.
    ``page_local`` keeps KEY groups inside pages."""
    dev = _device_of(x)
    P, S, H, D = x.shape
    G = group_size or default_group(format)
    Ge = page_local_group(format, kind, G, S) if page_local else G
    if out is None:
        out = alloc_packed(format, kind, Ge, P * S, H, D, P * S, dev)
    desc = out.descriptor()
    ws = workspace(dev) if format == "nvfp4" else None
    _check("kvq_pack_paged", library().kvq_pack_paged(ctypes.byref(_paged_view(x)), KIND[kind], FORMAT[format], G,
                                                      int(bool(page_local)), ctypes.byref(desc), _ptr(ws),
                                                      _stream(dev)))
    out.group_size = desc.group_size
    return out


def unpack_paged(p: Packed, out: Optional[torch.Tensor] = None, page_size: Optional[int] = None) -> torch.Tensor:
    """unpack_paged: decode into a bf16 [pages, page_size, H, D] view (allocated when `out` is
    None, from `page_size`)."""
    dev = p.codes.device
    if out is None:
        if not page_size or p.rows % page_size:
            raise ValueError("kvq: give `out` or a page_size dividing the row count")
        out = torch.empty((p.rows // page_size, page_size, p.H, p.D), dtype=torch.bfloat16, device=dev)
    desc = p.descriptor()
    _check("kvq_unpack_paged", library().kvq_unpack_paged(ctypes.byref(desc), ctypes.byref(_paged_view(out)),
                                                          _stream(dev)))
    return out


def alloc_cache(fmt: str, kind: str, group_size: int, n_slots: int, H: int, D: int, dev: torch.device) -> Packed:
    """Planes of a slot cache of n_slots rows (contents undefined until written)."""
    return alloc_packed(fmt, kind, group_size, n_slots, H, D, n_slots, dev)


def _slots(slots: torch.Tensor, like: torch.Tensor, n: int) -> torch.Tensor:
    if slots.dtype != torch.int32 or slots.device != like.device or slots.dim() != 1 or slots.numel() != n:
        raise ValueError("kvq: slots must be a 1-D int32 tensor with one entry per row, on the cache's device")
    return slots.contiguous()


def store_rows(cache: Packed, rows: torch.Tensor, slots: torch.Tensor) -> Packed:
    """Quantize rows [N, H, D] and write row i into cache slot slots[i] (one launch; slots are a
    device int32 tensor, distinct and in range)."""
    dev = _device_of(rows)
    slots = _slots(slots, cache.codes, rows.shape[0])
    desc = cache.descriptor()
    _check("kvq_store_rows", library().kvq_store_rows(ctypes.byref(_view(rows)), _ptr(slots), ctypes.byref(desc),
                                                      _stream(dev)))
    return cache


def load_rows(cache: Packed, slots: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode cache rows slots[0..N) into a bf16 [N, H, D] tensor (or the view `out`)."""
    dev = cache.codes.device
    N = slots.numel()
    slots = _slots(slots, cache.codes, N)
    if out is None:
        out = torch.empty((N, cache.H, cache.D), dtype=torch.bfloat16, device=dev)
    desc = cache.descriptor()
    _check("kvq_load_rows", library().kvq_load_rows(ctypes.byref(desc), _ptr(slots), ctypes.byref(_view(out)),
                                                    _stream(dev)))
    return out


def window_split(T: int, sink: int, recent: int) -> Tuple[int, int]:
    """(rows kept in front, rows kept at the end) of a BF16 window over T tokens."""
    ns = min(sink, T)
    return ns, min(recent, T - ns)


@dataclass
class Windowed:
    """A tensor encoded with a BF16 window: the quantized middle rows and the raw protected rows."""

    packed: Packed
    window: torch.Tensor  # bf16 [n_sink + n_recent, H, D]
    T: int
    sink: int
    recent: int


def encode_window(current: torch.Tensor, kind: str = "key", format: str = "int4", group_size: int = 0,
                  sink: int = 4, recent: int = 16, previous: Optional[torch.Tensor] = None,
                  out: Optional[Windowed] = None) -> Windowed:
    """Pack (previous None) or residual-encode `current` with its first `sink` and latest `recent`
    rows kept in BF16."""
    dev = _device_of(current)
    T, H, D = current.shape
    G = group_size or default_group(format)
    ns, nr = window_split(T, sink, recent)
    if out is None:
        out = Windowed(alloc_packed(format, kind, G, T - ns - nr, H, D, T, dev),
                       torch.empty((ns + nr, H, D), dtype=torch.bfloat16, device=dev), T, sink, recent)
    desc = out.packed.descriptor()
    ws = workspace(dev) if format == "nvfp4" else None
    pv = ctypes.byref(_view(previous)) if previous is not None else None
    _check("kvq_encode_window", library().kvq_encode_window(ctypes.byref(_view(current)), pv, sink, recent, KIND[kind],
                                                            FORMAT[format], G, ctypes.byref(desc), _ptr(out.window),
                                                            _ptr(ws), _stream(dev)))
    return out


def decode_window(w: Windowed, previous: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode a windowed tensor into bf16 [T, H, D] (adding to `previous` for a residual)."""
    p = w.packed
    dev = p.codes.device
    if out is None:
        out = torch.empty((w.T, p.H, p.D), dtype=torch.bfloat16, device=dev)
    desc = p.descriptor()
    pv = ctypes.byref(_view(previous)) if previous is not None else None
    _check("kvq_decode_window", library().kvq_decode_window(ctypes.byref(desc), _ptr(w.window), w.sink, w.recent, pv,
                                                            ctypes.byref(_view(out)), _stream(dev)))
    return out


_attn_ws: Dict[Tuple[int, int], torch.Tensor] = {}


def decode_attention(q: torch.Tensor, k: Packed, v: Packed, k_res: Optional[Packed] = None,
                     v_res: Optional[Packed] = None, scale: Optional[float] = None,
                     out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step of attention over the packed cache (K, V, optionally one residual each):
    q bf16 [Hq, D] -> float32 [Hq, D] (D = 64, 128 or 256); query head hq reads KV head
    hq // (Hq // H)."""
    dev = _device_of(q)
    if q.dtype != torch.bfloat16 or q.dim() != 2:
        raise ValueError("kvq: q must be a bf16 [Hq, head_dim] tensor")
    q = q.contiguous()
    Hq, Dq = q.shape
    if out is None:
        out = torch.empty((Hq, Dq), dtype=torch.float32, device=dev)
    need = int(library().kvq_attention_workspace_bytes(k.rows, k.H, Hq, k.D))
    key = (dev.index if dev.index is not None else torch.cuda.current_device(), torch.cuda.current_stream(dev).cuda_stream)
    ws = _attn_ws.get(key)
    if ws is None or ws.numel() < max(need, 4):
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=dev)
        _attn_ws[key] = ws
    dk, dv = k.descriptor(), v.descriptor()
    drk = k_res.descriptor() if k_res is not None else None
    drv = v_res.descriptor() if v_res is not None else None
    scale = (1.0 / Dq ** 0.5) if scale is None else float(scale)
    _check("kvq_decode_attention", library().kvq_decode_attention(
        _ptr(q), Hq, ctypes.byref(dk), ctypes.byref(dv), ctypes.byref(drk) if drk is not None else None,
        ctypes.byref(drv) if drv is not None else None, scale, _ptr(out), _ptr(ws), ws.numel(), _stream(dev)))
    return out


def decode_attention_noalloc(q: torch.Tensor, k: Packed, v: Packed, k_res: Optional[Packed] = None,
                             v_res: Optional[Packed] = None, scale: Optional[float] = None,
                             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """decode_attention through the entry point that takes no workspace: its partials go to the
    library's static per-GPU scratch (calls overlapping on one GPU race). Pass ``out`` to make
    the call allocate nothing at all."""
    dev = _device_of(q)
    if q.dtype != torch.bfloat16 or q.dim() != 2 or not q.is_contiguous():
        raise ValueError("kvq: q must be a contiguous bf16 [Hq, head_dim] tensor")
    Hq, Dq = q.shape
    if out is None:
        out = torch.empty((Hq, Dq), dtype=torch.float32, device=dev)
    dk, dv = k.descriptor(), v.descriptor()
    drk = k_res.descriptor() if k_res is not None else None
    drv = v_res.descriptor() if v_res is not None else None
    scale = (1.0 / Dq ** 0.5) if scale is None else float(scale)
    _check("kvq_decode_attention_noalloc", library().kvq_decode_attention_noalloc(
        _ptr(q), Hq, ctypes.byref(dk), ctypes.byref(dv), ctypes.byref(drk) if drk is not None else None,
        ctypes.byref(drv) if drv is not None else None, scale, _ptr(out), _stream(dev)))
    return out


def validate_positions(positions: torch.Tensor, T: int) -> torch.Tensor:
    """Device-side check of a position map; returns a device int32 status (0 = valid, bit 0 =
    out of range, bit 1 = repeated) without synchronizing."""
    dev = _device_of(positions)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    scratch = torch.empty(max(1, -(-T // 32)), dtype=torch.int32, device=dev)
    _check("kvq_validate_positions", library().kvq_validate_positions(_ptr(positions.contiguous()), positions.numel(),
                                                                      T, _ptr(scratch), _ptr(status), _stream(dev)))
    return status


__all__ = ["pack", "unpack", "encode_residual", "decode_residual", "storage_bytes", "plane_bytes",
           "validate_positions", "pack_paged", "unpack_paged", "store_rows", "load_rows", "alloc_cache",
           "encode_window", "decode_window", "Windowed", "decode_attention", "decode_attention_noalloc",
           "nvfp4_global_scale",
           "Packed", "KvqError", "library", "version", "workspace", "alloc_packed"]
