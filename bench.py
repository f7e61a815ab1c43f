#!/usr/bin/env python3
"""Bench of the KV codec's hot path on one MI355X.

One step = every row of the hot path over one batch of the bulk workload (T=131072 tokens,
H_kv=8, D=128, bf16 Student-t nu=3, ~268 MB per K or V tensor), for both formats (INT4 G64 and
NVFP4 G16) and both kinds (K, V):
    R0 = unpack(pack(X0)); R = encode_residual(X1, R0); R1 = decode_residual(R, R0)
with X1 = bf16(X0 + 0.1 N(0,1)). Inputs are resident in HBM before the timed region; output
planes are preallocated, so the timed region holds only kernel launches.

value = algorithmic bytes of the whole step / step time (GB/s). Algorithmic bytes per element
(n = T*H*D): pack INT4 2.5625, NVFP4 4.5625 (+4 B); unpack 2.5625 (+4 B); residual encode
INT4 4.5625, NVFP4 8.5625 (+4 B); residual decode 4.5625 (+4 B). NVFP4 encodes read their input
twice (tensor amax first, then the codes), which the method's per-tensor scale requires.

Prints one JSON line on stdout; per-op timings go to stderr (and --detail FILE).

After the timed region, "extras" times the rows beyond the bulk step on the same K/V tensors
(p50 of 20 event-timed calls each, not part of `value`): the row formats NVFP4-row and FP8-row
(one FP32 scale per token and head; pack, unpack, residual encode/decode), pack_paged /
unpack_paged of K with page-local groups (16-token pages of a pool that interleaves K and V per
page, so the page stride is padded), and store_rows / load_rows of 16384 rows into and out of
a 131072-slot cache, and the BF16 window (first 4 / latest 16 rows raw) around INT4 G64 K
pack and residual encode/decode, and decode attention of 64 query heads over the packed K/V
(all four formats; INT4 G64 also with one fused residual), whose algorithmic bytes are the
packed planes it reads. Context lines: INT4 and NVFP4 K ops on one KV head's shard
([T, 1, 128], the per-GPU shape of head sharding over 8 GPUs); the 268 MB tensor copied by this
library's row-copy kernel and by the runtime's device-to-device copy (read + write bytes).

Every op (the 16 of the step and the extras) is also timed on a clean cache: a 1 GiB write, then
a 1 GiB read, before each call evict the 256 MB Infinity Cache without leaving dirty lines (10
calls per op, rotating over the ops). Inside the step an op follows the op that wrote one of
its inputs, part of which it may then read from that cache.

Parity and CPU baseline: the oracle runs the whole step at full size (its OpenMP build, all
threads) and every plane and every decoded tensor the timed step produced is compared with it
bit for bit; that run is the all-cores baseline. The single-threaded oracle runs the same 16
ops on the leading 32768 tokens. Algorithmic bytes per element for a
row format with c code bytes and m = block-scale bytes + 4/D row-scale bytes per element: pack
and unpack 2 + c + m, residual
encode and decode 4 + c + m; page-local INT4 G16 K 2.75; a slot write or read of N rows moves
N*H*D*(2 + c + m) bytes plus 4 B per slot id; a windowed op moves the codec bytes of its
T - 20 middle rows plus the 20 protected rows read and written in bf16.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, AMD public spec
T_FULL, H, D = 131072, 8, 128
FORMS = (("int4", 64), ("nvfp4", 16))
KINDS = ("key", "value")
OPS = ("pack", "unpack", "encode_residual", "decode_residual")


def algo_bytes(op: str, fmt: str, n: int) -> float:
    """Bytes the method must move for one op on n elements (see module docstring)."""
    meta = 0.0625  # 4 B per 64 values (INT4 G64) = 1 B per 16 values (NVFP4 G16)
    code = 0.5
    extra = 4 if fmt == "nvfp4" else 0
    if op == "pack":
        return n * (2 + code + meta) + (n * 2 if fmt == "nvfp4" else 0) + extra
    if op == "unpack":
        return n * (code + meta + 2) + extra
    if op == "encode_residual":
        return n * (4 + code + meta) + (n * 4 if fmt == "nvfp4" else 0) + extra
    if op == "decode_residual":
        return n * (code + meta + 2 + 2) + extra
    raise ValueError(op)


def row_format_bytes(fmt: str) -> tuple:
    """(code bytes, metadata bytes) per element of a row format at head_dim D."""
    if fmt == "nvfp4_row":
        return 0.5, 1.0 / 16 + 4.0 / D
    return 1.0, 4.0 / D


def make_evict(torch, dev):
    """A 1 GiB write, then a 1 GiB read: evicts the 256 MB Infinity Cache and leaves no dirty
    lines to be written back during the next op."""
    flush = torch.empty(1 << 29, dtype=torch.int16, device=dev)

    def evict():
        flush.fill_(1)
        torch.amax(flush)
    return evict


def time_clean(torch, stream, ops, evict, reps: int = 10) -> dict:
    """p50 in us of each (name, fn) of `ops`, each call on a clean cache; the reps rotate over
    the ops."""
    ev = {name: [] for name, _ in ops}
    for _ in range(reps):
        for name, fn in ops:
            evict()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ev[name].append((e0, e1))
    torch.cuda.synchronize()
    return {name: float(np.percentile([a.elapsed_time(b) for a, b in v], 50) * 1e3) for name, v in ev.items()}


def run_extras(kvq, torch, X, T: int, dev, evict, reps: int = 20) -> dict:
    """Row formats, paged views, slot writes/reads, windows, decode attention and the context
    lines on the bulk tensors (see the module docstring); returns {name: {us, GBps, pct_peak}}."""
    n = T * H * D
    x0, x1 = X["key"]
    calls = []
    for fmt, G in (("nvfp4_row", 16), ("fp8_row", 0)):
        c, m = row_format_bytes(fmt)
        p = kvq.alloc_packed(fmt, "key", G, T, H, D, T, dev)
        r = kvq.alloc_packed(fmt, "key", G, T, H, D, T, dev)
        R0 = torch.empty_like(x0)
        R1 = torch.empty_like(x0)
        calls += [
            (f"{fmt}-key-pack", n * (2 + c + m), lambda p=p, fmt=fmt, G=G: kvq.pack(x0, "key", fmt, G, out=p)),
            (f"{fmt}-key-unpack", n * (2 + c + m), lambda p=p, R0=R0: kvq.unpack(p, out=R0)),
            (f"{fmt}-key-encode_residual", n * (4 + c + m),
             lambda r=r, R0=R0, fmt=fmt, G=G: kvq.encode_residual(x1, R0, "key", fmt, G, out=r)),
            (f"{fmt}-key-decode_residual", n * (4 + c + m), lambda r=r, R0=R0, R1=R1: kvq.decode_residual(r, R0, out=R1)),
        ]
    # paged: a pool [pages, 2 (K, V), 16, H, D]; K pages are 2*16 rows apart
    S = 16
    pool = torch.empty((T // S, 2, S, H, D), dtype=torch.bfloat16, device=dev)
    pool[:, 0] = x0.view(T // S, S, H, D)
    pool[:, 1] = X["value"][0].view(T // S, S, H, D)
    pp = kvq.alloc_packed("int4", "key", 16, T, H, D, T, dev)
    pout = torch.empty_like(pool)
    calls += [
        ("int4-key-pack_paged-page_local", n * 2.75,
         lambda: kvq.pack_paged(pool[:, 0], "key", "int4", 64, page_local=True, out=pp)),
        ("int4-key-unpack_paged-page_local", n * 2.75, lambda: kvq.unpack_paged(pp, out=pout[:, 0])),
    ]
    # BF16 window (first 4 / latest 16 rows raw): INT4 G64 K pack, residual encode, residual decode
    nmid = (T - 20) * H * D
    nwin = 20 * H * D * 4  # window rows read and written
    wp = kvq.encode_window(x0, "key", "int4", 64, 4, 16)
    wr = kvq.encode_window(x1, "key", "int4", 64, 4, 16, previous=x0)
    wout = torch.empty_like(x0)
    calls += [
        ("int4-key-window_pack", nmid * 2.5625 + nwin, lambda: kvq.encode_window(x0, "key", "int4", 64, 4, 16, out=wp)),
        ("int4-key-window_encode_residual", nmid * 4.5625 + nwin,
         lambda: kvq.encode_window(x1, "key", "int4", 64, 4, 16, previous=x0, out=wr)),
        ("int4-key-window_decode_residual", nmid * 4.5625 + nwin,
         lambda: kvq.decode_window(wr, previous=x0, out=wout)),
    ]
    # decode attention over the packed cache: 64 query heads (GQA 8) over all T tokens, K/V
    # reconstructed in registers; algorithmic bytes = the packed K and V planes (+ residuals)
    Hq = 64
    qv = torch.randn((Hq, D), generator=torch.Generator(device="cpu").manual_seed(3)).to(torch.bfloat16).to(dev)
    aout = torch.empty((Hq, D), dtype=torch.float32, device=dev)
    for fmt, G in (("int4", 64), ("nvfp4", 16), ("nvfp4_row", 16), ("fp8_row", 0)):
        pk = kvq.pack(x0, "key", fmt, G)
        pv = kvq.pack(X["value"][0], "value", fmt, G)
        pbytes = pk.nbytes() + pv.nbytes()
        calls.append((f"{fmt}-decode_attention-Hq64", pbytes,
                      lambda pk=pk, pv=pv: kvq.decode_attention(qv, pk, pv, out=aout)))
        if fmt == "int4":
            rk = kvq.encode_residual(x1, kvq.unpack(pk), "key", fmt, G)
            rv = kvq.encode_residual(X["value"][1], kvq.unpack(pv), "value", fmt, G)
            calls.append((f"{fmt}-decode_attention-residual-Hq64", pbytes + rk.nbytes() + rv.nbytes(),
                          lambda pk=pk, pv=pv, rk=rk, rv=rv: kvq.decode_attention(qv, pk, pv, rk, rv, out=aout)))
    # slot writes and reads: 16384 rows into / out of a 131072-slot cache
    N = min(16384, T)
    g = torch.Generator(device="cpu").manual_seed(7)
    slots = torch.randperm(T, generator=g)[:N].to(torch.int32).to(dev)
    rows = x1[:N]
    for fmt, G in (("nvfp4_row", 16), ("fp8_row", 0)):
        c, m = row_format_bytes(fmt)
        cache = kvq.pack(x0, "key", fmt, G)
        outr = torch.empty((N, H, D), dtype=torch.bfloat16, device=dev)
        nb = N * H * D * (2 + c + m) + 4 * N
        calls += [
            (f"{fmt}-store_rows-16384", nb, lambda cache=cache: kvq.store_rows(cache, rows, slots)),
            (f"{fmt}-load_rows-16384", nb, lambda cache=cache, outr=outr: kvq.load_rows(cache, slots, out=outr)),
        ]
    # one KV head's shard of the same tensors ([T, 1, 128], contiguous): the per-GPU shape of head
    # (tensor-parallel) sharding over 8 GPUs
    xs0, xs1 = x0[:, :1].contiguous(), x1[:, :1].contiguous()
    ns = xs0.numel()
    ps = kvq.alloc_packed("int4", "key", 64, T, 1, D, T, dev)
    pn = kvq.alloc_packed("nvfp4", "key", 16, T, 1, D, T, dev)
    rs = kvq.alloc_packed("int4", "key", 64, T, 1, D, T, dev)
    Rs = kvq.unpack(kvq.pack(xs0, "key", "int4", 64))
    calls += [
        ("int4-key-pack-shard_H1", ns * 2.5625, lambda: kvq.pack(xs0, "key", "int4", 64, out=ps)),
        ("int4-key-encode_residual-shard_H1", ns * 4.5625,
         lambda: kvq.encode_residual(xs1, Rs, "key", "int4", 64, out=rs)),
        ("nvfp4-key-pack-shard_H1", ns * 4.5625 + 4, lambda: kvq.pack(xs0, "key", "nvfp4", 16, out=pn)),
    ]
    # context: the same 268 MB copied by a plain row-copy kernel of this library (a sparse residual
    # with no rows decodes out of place as one copy) and by the runtime's device-to-device copy
    cdst = torch.empty_like(x0)
    empty = kvq.encode_residual(x0, x0, "key", "int4", 64, positions=torch.zeros(0, dtype=torch.int32, device=dev))
    calls += [
        ("context-copy_kernel-268MB", 4 * n, lambda: kvq.decode_residual(empty, x0, out=cdst)),
        ("context-d2d_copy-268MB", 4 * n, lambda: cdst.copy_(x0)),
    ]
    stream = torch.cuda.current_stream(dev)
    for _, _, fn in calls:  # warmup
        fn()
    torch.cuda.synchronize()
    out = {}
    for name, nbytes, fn in calls:  # back-to-back calls of one op
        ev = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            ev.append((e0, e1))
        torch.cuda.synchronize()
        us = float(np.percentile([a.elapsed_time(b) for a, b in ev], 50) * 1e3)
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name] = {"us": round(us, 2), "GBps": round(gbs, 1), "pct_peak": round(100 * gbs / PEAK_HBM_GBS, 1)}
    clean = time_clean(torch, stream, [(name, fn) for name, _, fn in calls], evict)
    for name, nbytes, _ in calls:
        us = clean[name]
        gbs = nbytes / (us * 1e-6) / 1e9
        out[name].update(clean_us=round(us, 2), clean_pct_peak=round(100 * gbs / PEAK_HBM_GBS, 1))
        o = out[name]
        print(f"extra {name:38s} p50 {o['us']:8.1f} us {o['pct_peak']:5.1f}%   clean cache {us:8.1f} us "
              f"{o['clean_pct_peak']:5.1f}% of peak", file=sys.stderr)
    return out


TRAFFIC_SOURCES = ("csrc/kvq_device.hpp", "csrc/kvq_encode.hip", "csrc/kvq_decode.hip", "csrc/kvq_launch.hpp",
                   "_build.py")


def measured_traffic(op_name: str):
    """HBM bytes per launch of the single-launch op `op_name` from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE runs (profiles/traffic.json, copy-kernel scaled), or None if those
    counters were taken on other kernel sources or do not cover the op."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for rel in TRAFFIC_SOURCES:  # the bulk kernels' sources and their build flags
        with open(os.path.join(ROOT, "kv_cache_quantization_kvq_amd", rel), "rb") as f:
            h.update(f.read())
    op = rec.get("ops", {}).get(op_name)
    if rec.get("source_sha256") != h.hexdigest() or op is None:
        return None
    return float(op["traffic_bytes"])


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rmse_np(y_bits: np.ndarray, x_bits: np.ndarray, chunk: int = 8192) -> float:
    """Root-mean-square of y - x (bf16 bits [T, H, D]), accumulated in float64 over row chunks."""
    acc = 0.0
    for t in range(0, y_bits.shape[0], chunk):
        d = bf16_to_f64(y_bits[t:t + chunk]) - bf16_to_f64(x_bits[t:t + chunk])
        acc += float((d * d).sum())
    return (acc / max(y_bits.size, 1)) ** 0.5


def rmse_dev(torch, y, x, chunk: int = 8192) -> float:
    """Root-mean-square of y - x (bf16 [T, H, D] device tensors), accumulated in float64."""
    acc, n = 0.0, 0
    for t in range(0, y.shape[0], chunk):
        d = y[t:t + chunk].double() - x[t:t + chunk].double()
        acc += float((d * d).sum())
        n += d.numel()
    return (acc / max(n, 1)) ** 0.5


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        return ""


def oracle_step(oracle, data: dict, n: int, on_result=None):
    """The 16 ops of one step through the oracle; returns (seconds in oracle calls, algorithmic
    bytes). on_result(fmt, kind, p, R0, r, R1) sees each chain's outputs outside the timing."""
    secs, total = 0.0, 0.0
    for fmt, G in FORMS:
        for kind in KINDS:
            X0, X1 = data[kind]
            t0 = time.perf_counter()
            p = oracle.pack(X0, kind, fmt, G)
            R0 = oracle.unpack(p)
            r = oracle.encode_residual(X1, R0, kind, fmt, G)
            R1 = oracle.decode_residual(r, R0)
            secs += time.perf_counter() - t0
            total += sum(algo_bytes(op, fmt, n) for op in OPS)
            if on_result is not None:
                on_result(fmt, kind, p, R0, r, R1)
    return secs, total


def oracle_single_thread(T_sample: int) -> dict:
    """The single-threaded oracle on the leading T_sample rows of the same workload."""
    import oracle
    from workloads import c4_residual_target, c4_tensors

    oracle.build(force=False)
    prev = oracle.set_threaded(False)
    try:
        d = c4_tensors(0, T=T_sample)
        data = {"key": (d["K"], c4_residual_target(d["K"], stream=0)),
                "value": (d["V"], c4_residual_target(d["V"], stream=1))}
        secs, nbytes = oracle_step(oracle, data, T_sample * H * D)
    finally:
        oracle.set_threaded(prev)
    return {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": 1, "seconds": round(secs, 2),
            "sample": f"leading {T_sample} of {T_FULL} tokens (H=8, D=128), all 16 ops of one step"}


def host_planes(p) -> dict:
    """Host bit patterns of a packed tensor's planes (device or oracle)."""
    out = {}
    for name in ("codes", "meta0", "meta1", "global_scale"):
        a = getattr(p, name)
        if a is None:
            continue
        if not isinstance(a, np.ndarray):
            a = a.cpu().numpy()
        out[name] = np.ascontiguousarray(a).view({1: np.uint8, 2: np.uint16, 4: np.uint32}[a.dtype.itemsize])
    return out


def oracle_all_cores(host: dict, bufs: dict, T: int, torch):
    """The oracle's OpenMP build on the whole step at full size, compared bit for bit with what
    the timed step left in `bufs`. Returns the baseline record, the parity verdicts and the
    oracle's reconstruction RMSEs."""
    import oracle

    oracle.build(force=False)
    prev = oracle.set_threaded(True)
    parity, ormse = {}, {}

    def dev_bits(t):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    def check(fmt, kind, p, R0, r, R1):
        b = bufs[(fmt, kind)]
        ok = True
        for dp, op in ((b["p"], p), (b["r"], r)):
            g, o = host_planes(dp), host_planes(op)
            ok = ok and set(g) == set(o) and all(np.array_equal(g[k], o[k]) for k in o)
        ok = ok and np.array_equal(dev_bits(b["R0"]), R0) and np.array_equal(dev_bits(b["R1"]), R1)
        parity[f"{fmt}-{kind}"] = bool(ok)
        X0, X1 = host[kind]
        ormse[f"{fmt}-{kind}"] = (rmse_np(R0, X0), rmse_np(R1, X1))

    try:
        threads = oracle.threads()
        secs, nbytes = oracle_step(oracle, host, T * H * D, check)
    finally:
        oracle.set_threaded(prev)
    rec = {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "seconds": round(secs, 2),
           "sample": f"the whole step at full size (T={T}, H=8, D=128, all 16 ops), OpenMP build of the C oracle "
                     f"on {threads} threads (loops over independent groups and rows)",
           "cpu": cpu_model()}
    return rec, parity, ormse


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--tokens", type=int, default=T_FULL, help="T (default: the bulk workload)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=32768)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip the row-format / paged / slot timings")
    ap.add_argument("--detail", default="")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain copy kernel of a known size (268 MB) after warmup, for counter scaling")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the codec has no multi-GPU path "
              f"(got --gpus {args.gpus}, WORLD_SIZE {world})", file=sys.stderr)
        return 2

    import torch

    import kv_cache_quantization_kvq_amd as kvq
    from workloads import c4_residual_target, c4_tensors

    dev = torch.device("cuda:0")
    T = args.tokens
    n = T * H * D

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    t_gen = time.perf_counter()
    d = c4_tensors(0, T=T)
    X, host = {}, {}
    for kind, key, stream in (("key", "K", 0), ("value", "V", 1)):
        host[kind] = (d[key], c4_residual_target(d[key], stream=stream))
        X[kind] = tuple(to_dev(a) for a in host[kind])
    del d
    if args.no_cpu_baseline:
        host = None
    print(f"inputs ready in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    # preallocated outputs
    bufs = {}
    for fmt, G in FORMS:
        for kind in KINDS:
            bufs[(fmt, kind)] = dict(
                p=kvq.alloc_packed(fmt, kind, G, T, H, D, T, dev),
                r=kvq.alloc_packed(fmt, kind, G, T, H, D, T, dev),
                R0=torch.empty((T, H, D), dtype=torch.bfloat16, device=dev),
                R1=torch.empty((T, H, D), dtype=torch.bfloat16, device=dev),
            )
    stream = torch.cuda.current_stream(dev)

    calls = []  # (name, fmt, op, fn) in step order
    for fmt, G in FORMS:
        for kind in KINDS:
            b = bufs[(fmt, kind)]
            x0, x1 = X[kind]
            calls.append((f"{fmt}-{kind}-pack", fmt, "pack",
                          lambda x0=x0, kind=kind, fmt=fmt, G=G, b=b: kvq.pack(x0, kind, fmt, G, out=b["p"])))
            calls.append((f"{fmt}-{kind}-unpack", fmt, "unpack",
                          lambda b=b: kvq.unpack(b["p"], out=b["R0"])))
            calls.append((f"{fmt}-{kind}-encode_residual", fmt, "encode_residual",
                          lambda x1=x1, kind=kind, fmt=fmt, G=G, b=b: kvq.encode_residual(x1, b["R0"], kind, fmt, G,
                                                                                         out=b["r"])))
            calls.append((f"{fmt}-{kind}-decode_residual", fmt, "decode_residual",
                          lambda b=b: kvq.decode_residual(b["r"], b["R0"], out=b["R1"])))
    # kernel launches per op: NVFP4 encodes run amax, finalize and the encode kernel
    launches = {name: (3 if (fmt == "nvfp4" and op in ("pack", "encode_residual")) else 1)
                for name, fmt, op, _ in calls}

    def step(timed=None, events=None):
        for name, _fmt, _op, fn in calls:
            if events is not None and (timed is None or name == timed):
                events.append((name, torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
                events[-1][1].record(stream)
                fn()
                events[-1][2].record(stream)
            else:
                fn()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.copy_calibration:
        # a sparse residual with no rows decodes out of place as one row-copy kernel over the
        # whole tensor: T*H*D*2 bytes read and the same written
        x0 = X["key"][0]
        empty = kvq.encode_residual(x0, x0, "key", "int4", 64, positions=torch.zeros(0, dtype=torch.int32, device=dev))
        kvq.decode_residual(empty, x0, out=torch.empty_like(x0))
        torch.cuda.synchronize()
        print(f"copy calibration: {x0.numel() * 2} bytes read and written", file=sys.stderr)

    # per-op table from up to 20 instrumented steps (events around every op; not the timed region)
    prof = []
    for _ in range(min(20, max(1, args.steps))):
        step(events=prof)
    torch.cuda.synchronize()
    per_op = {}
    for name, fmt, op, _ in calls:
        ms = np.array([e0.elapsed_time(e1) for nm, e0, e1 in prof if nm == name])
        nbytes = algo_bytes(op, fmt, n)
        per_op[name] = dict(mean_us=float(ms.mean() * 1e3), p50_us=float(np.percentile(ms, 50) * 1e3),
                            p90_us=float(np.percentile(ms, 90) * 1e3), bytes=nbytes,
                            gbs=float(nbytes / (np.percentile(ms, 50) * 1e-3) / 1e9), launches=launches[name])
    # the dominant single-kernel op: the one-launch op with the largest share of the step
    dom_name = max((k for k in per_op if per_op[k]["launches"] == 1), key=lambda k: per_op[k]["mean_us"])

    # timed region: K steps; events only around the dominant op (for the roofline figure)
    dom_events = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(timed=dom_name, events=dom_events)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    dom_us = float(np.mean([e0.elapsed_time(e1) for _, e0, e1 in dom_events]) * 1e3)

    step_bytes = sum(v["bytes"] for v in per_op.values())
    ms_per_step = elapsed / args.steps * 1e3
    value = step_bytes / (elapsed / args.steps) / 1e9
    dom = per_op[dom_name]
    achieved = dom["bytes"] / (dom_us * 1e-6) / 1e9

    # every op of the step again, each call on a clean cache
    evict = make_evict(torch, dev)
    clean = time_clean(torch, stream, [(name, fn) for name, _f, _o, fn in calls], evict)
    for name, v in per_op.items():
        v["clean_p50_us"] = clean[name]
        v["clean_gbs"] = float(v["bytes"] / (clean[name] * 1e-6) / 1e9)
        print(f"{name:34s} mean {v['mean_us']:8.1f} us  p50 {v['p50_us']:8.1f}  p90 {v['p90_us']:8.1f}  "
              f"{100 * v['gbs'] / PEAK_HBM_GBS:5.1f}% of peak   clean cache p50 {v['clean_p50_us']:8.1f} us  "
              f"{100 * v['clean_gbs'] / PEAK_HBM_GBS:5.1f}%", file=sys.stderr)

    # the largest kernel by time per step: the NVFP4 residual encodes' tensor-amax pass over both
    # input tensors (two launches per step), timed alone through the entry point that runs only
    # that pass (plus its one-block finalize), on the step's own inputs
    amax_in = (X["key"][1], bufs[("nvfp4", "key")]["R0"])
    amax_out = torch.empty(1, dtype=torch.float32, device=dev)
    amax_fn = lambda: kvq.nvfp4_global_scale(*amax_in, out=amax_out)  # noqa: E731
    amax_ev = []
    for _ in range(20):
        amax_ev.append((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
        amax_ev[-1][0].record(stream)
        amax_fn()
        amax_ev[-1][1].record(stream)
    torch.cuda.synchronize()
    amax_us = float(np.mean([a.elapsed_time(b) for a, b in amax_ev]) * 1e3)
    amax_clean_us = time_clean(torch, stream, [("amax", amax_fn)], evict)["amax"]
    amax_bytes = 4.0 * n

    extras = None
    if not args.no_extras:
        extras = run_extras(kvq, torch, X, T, dev, evict)
        # context: the same step captured once as a HIP graph and replayed (every call only
        # enqueues kernels, so it can be captured); the difference to `value` is the launch gaps
        side = torch.cuda.Stream(dev)
        with torch.cuda.stream(side):
            step()  # the NVFP4 workspace of this stream exists before capture
            side.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=side):
                step()
            graph.replay()
            side.synchronize()
            t_g = time.perf_counter()
            for _ in range(args.steps):
                graph.replay()
            side.synchronize()
            g_step = (time.perf_counter() - t_g) / args.steps
        del graph
        g_gbs = step_bytes / g_step / 1e9
        extras["context-step_as_hip_graph"] = {"us": round(g_step * 1e6, 1), "GBps": round(g_gbs, 1),
                                               "pct_peak": round(100 * g_gbs / PEAK_HBM_GBS, 1)}
        print(f"extra {'context-step_as_hip_graph':38s} {g_step * 1e6:9.1f} us per step  {g_gbs:7.1f} GB/s  "
              f"{100 * g_gbs / PEAK_HBM_GBS:5.1f}% of peak", file=sys.stderr)

    # reconstruction RMSE of the full tensors: unpack (R0 - X0) and residual decode (R1 - X1)
    quality = {}
    for fmt, G in FORMS:
        for kind in KINDS:
            b = bufs[(fmt, kind)]
            x0, x1 = X[kind]
            quality[f"{fmt}-{kind}"] = dict(unpack=rmse_dev(torch, b["R0"], x0), residual=rmse_dev(torch, b["R1"], x1))

    cpu, parity = None, None
    if not args.no_cpu_baseline:
        cpu, parity, oracle_rmse = oracle_all_cores(host, bufs, T, torch)
        cpu["single_thread"] = oracle_single_thread(min(args.cpu_sample_tokens, T))
        worst = 0.0
        for key, (ou, orr) in oracle_rmse.items():
            q = quality[key]
            q["oracle_unpack"], q["oracle_residual"] = ou, orr
            worst = max(worst, abs(q["unpack"] - ou) / max(ou, 1e-300), abs(q["residual"] - orr) / max(orr, 1e-300))
        quality["max_rel_diff_vs_oracle"] = worst
        parity = {"bit_exact_full": all(parity.values()), **parity,
                  "what": "every plane (codes, metadata, global scale) and every decoded tensor of the timed step, "
                          "all 134M elements per tensor, against the oracle"}
        print(f"parity (full size, every output of the timed step vs the oracle): {parity}", file=sys.stderr)
        print(f"cpu baseline: all cores {cpu['value']} GB/s on {cpu['cores']} threads ({cpu['seconds']} s); "
              f"single thread {cpu['single_thread']['value']} GB/s ({cpu['single_thread']['seconds']} s)",
              file=sys.stderr)
    for key, q in quality.items():
        if isinstance(q, dict):
            print(f"rmse {key:12s} unpack {q['unpack']:.6e}  residual {q['residual']:.6e}"
                  + (f"  (oracle {q['oracle_unpack']:.6e} / {q['oracle_residual']:.6e})" if "oracle_unpack" in q
                     else ""), file=sys.stderr)

    line = {
        "metric": "codec GB/s and % HBM peak (pack/unpack/residual), INT4-G64 & NVFP4-G16",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "bulk codec: T=131072 tokens, H_kv=8, D=128, bf16 Student-t nu=3; INT4-G64 and "
                        "NVFP4-G16, K and V; pack, unpack, residual encode, residual decode per step",
            "T": T, "H_kv": H, "D": D, "bytes_per_step": step_bytes,
            "pct_hbm_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": dom_name,
            "kernel_avg_us": round(dom_us, 2),
            "bytes_per_launch": dom["bytes"],
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(dom_name),
            "clean_cache_us": round(per_op[dom_name]["clean_p50_us"], 2),
            "clean_cache_frac": round(per_op[dom_name]["clean_gbs"] / PEAK_HBM_GBS, 4),
            "largest_kernel": {
                "kernel": "k_amax_vec (NVFP4 residual tensor-amax pass over cur and prev, + one-block finalize)",
                "launches_per_step": 2,
                "bytes_per_launch": amax_bytes,
                "avg_us": round(amax_us, 2),
                "achieved": round(amax_bytes / (amax_us * 1e-6) / 1e9, 1),
                "frac": round(amax_bytes / (amax_us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
                "clean_cache_us": round(amax_clean_us, 2),
            },
        },
        "per_op": {k: {"mean_us": round(v["mean_us"], 2), "p50_us": round(v["p50_us"], 2),
                       "p90_us": round(v["p90_us"], 2), "pct_peak": round(100 * v["gbs"] / PEAK_HBM_GBS, 1),
                       "clean_p50_us": round(v["clean_p50_us"], 2),
                       "clean_pct_peak": round(100 * v["clean_gbs"] / PEAK_HBM_GBS, 1)}
                   for k, v in per_op.items()},
        "parity": parity,
        "cpu_baseline": cpu,
        "rmse": {k: ({kk: (vv if isinstance(vv, bool) else float(f"{vv:.7g}")) for kk, vv in v.items()}
                     if isinstance(v, dict) else float(f"{v:.3g}"))
                 for k, v in quality.items()},
        "extras": extras,
    }
    if args.detail:
        with open(args.detail, "w") as f:
            json.dump({"line": line, "per_op": per_op}, f, indent=1)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
