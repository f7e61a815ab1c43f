"""Seeded synthetic bf16 K/V tensors shaped like the pages' workloads.

Recipe (every config): ``numpy.random.default_rng(seed)``; draws are float64, rounded to
float32 (numpy cast, nearest-even) and then to bf16 (torch CPU cast, nearest-even). Arrays are
returned as ``numpy.uint16`` bf16 bit patterns with shape ``[T, H, D]``. Nothing here performs
codec arithmetic; where an input is defined from a reconstructed tensor (the mixed chain), the
caller passes that tensor in.

The five workloads:
  c1  T=128  H=2 D=64   N(0,1), 2 outlier channels per head x20 (INT4 G64 pack/unpack)
  c2  T=4096 H=8 D=128  N(0,1), 4 outlier channels per head x30, 1% exact +0.0 (NVFP4 G16)
  c3  T=8192 H=8 D=128  X0~N(0,1), Xk = bf16(X(k-1) + 0.1 N(0,1)), k=1..3; loop-3 positions:
                        sorted 25% sample of the rows, int32 (INT4 G64 residual chain)
  c4  T=131072 H=8 D=128  Student-t nu=3; X1 = bf16(X0 + 0.1 N(0,1)) (bulk, both formats)
  c5  T=1000 H=4 D=256  N(0,1) with signed zeros and tiny 32-aligned blocks; K is a strided
                        view of a fused QKV buffer (row pitch 3*H*D); mixed NVFP4/INT4-G32 chain
"""

from __future__ import annotations

import numpy as np
import torch

CONFIGS = {
    "c1": dict(T=128, H=2, D=64),
    "c2": dict(T=4096, H=8, D=128),
    "c3": dict(T=8192, H=8, D=128),
    "c4": dict(T=131072, H=8, D=128),
    "c5": dict(T=1000, H=4, D=256),
}


def bf16_bits(a) -> np.ndarray:
    """float64/float32 array -> float32 (nearest-even) -> bf16 bits (nearest-even)."""
    f32 = np.ascontiguousarray(np.asarray(a).astype(np.float32))
    t = torch.from_numpy(f32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).reshape(f32.shape)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


def _f32_with_outliers(base64: np.ndarray, rng: np.random.Generator, k: int, factor: float) -> np.ndarray:
    """Round to float32, then scale k outlier channels per head (picked without replacement) by
    `factor` in float32."""
    f32 = base64.astype(np.float32)
    T, H, D = f32.shape
    for h in range(H):
        ch = rng.choice(D, k, replace=False)
        f32[:, h, ch] *= np.float32(factor)
    return f32


def normal_kv(rng: np.random.Generator, T: int, H: int, D: int) -> np.ndarray:
    return bf16_bits(rng.standard_normal((T, H, D)))


def c1_tensors(seed: int = 0):
    c = CONFIGS["c1"]
    rng = np.random.default_rng(seed)
    k64 = rng.standard_normal((c["T"], c["H"], c["D"]))
    v64 = rng.standard_normal((c["T"], c["H"], c["D"]))
    K = bf16_bits(_f32_with_outliers(k64, rng, 2, 20.0))
    V = bf16_bits(_f32_with_outliers(v64, rng, 2, 20.0))
    return {"K": K, "V": V}


def c2_tensors(seed: int = 0):
    c = CONFIGS["c2"]
    rng = np.random.default_rng(seed)
    shape = (c["T"], c["H"], c["D"])
    k64 = rng.standard_normal(shape)
    v64 = rng.standard_normal(shape)
    kf = _f32_with_outliers(k64, rng, 4, 30.0)
    vf = _f32_with_outliers(v64, rng, 4, 30.0)
    kf[rng.random(shape) < 0.01] = 0.0
    vf[rng.random(shape) < 0.01] = 0.0
    return {"K": bf16_bits(kf), "V": bf16_bits(vf)}


def c3_chain_inputs(seed: int = 0):
    """Loop states X0..X3 for K and V (true values, independent of the codec) and the loop-3
    position map (sorted, distinct, 25% of the rows)."""
    c = CONFIGS["c3"]
    rng = np.random.default_rng(seed)
    shape = (c["T"], c["H"], c["D"])
    XK = [bf16_bits(rng.standard_normal(shape))]
    XV = [bf16_bits(rng.standard_normal(shape))]
    for _ in range(3):
        zk = rng.standard_normal(shape)
        zv = rng.standard_normal(shape)
        XK.append(bf16_bits(bf16_to_f32(XK[-1]).astype(np.float64) + 0.1 * zk))
        XV.append(bf16_bits(bf16_to_f32(XV[-1]).astype(np.float64) + 0.1 * zv))
    positions = np.sort(rng.choice(c["T"], c["T"] // 4, replace=False)).astype(np.int32)
    return {"XK": XK, "XV": XV, "positions": positions}


C4_CHUNK = 4096  # rows per independently seeded chunk of the bulk tensors


def _chunked(seed_words, T: int, H: int, D: int, draw) -> np.ndarray:
    """Rows in chunks of C4_CHUNK, chunk i drawn from its own generator
    default_rng(SeedSequence(seed_words).spawn(n)[i]); the first k chunks are therefore the
    same for any T >= k * C4_CHUNK. Chunks are drawn on a thread pool."""
    from concurrent.futures import ThreadPoolExecutor

    n = -(-T // C4_CHUNK)
    seqs = np.random.SeedSequence(seed_words).spawn(max(n, 1))
    out = np.empty((T, H, D), np.uint16)

    def work(i):
        r0 = i * C4_CHUNK
        r1 = min(T, r0 + C4_CHUNK)
        rng = np.random.default_rng(seqs[i])
        out[r0:r1] = bf16_bits(draw(rng, (r1 - r0, H, D), r0, r1))

    with ThreadPoolExecutor(max_workers=min(16, max(1, n))) as ex:
        list(ex.map(work, range(n)))
    return out


def c4_tensors(seed: int = 0, T: int | None = None):
    """Heavy-tailed bulk K and V (Student-t, nu = 3). A smaller T gives the leading rows of the
    full tensors (chunked seeding)."""
    c = CONFIGS["c4"]
    T = c["T"] if T is None else T
    t3 = lambda rng, shape, r0, r1: rng.standard_t(3, shape)  # noqa: E731
    K = _chunked([seed, 0], T, c["H"], c["D"], t3)
    V = _chunked([seed, 1], T, c["H"], c["D"], t3)
    return {"K": K, "V": V}


def c4_residual_target(X0: np.ndarray, seed: int = 1, stream: int = 0) -> np.ndarray:
    """Next-loop state X1 = bf16(X0 + 0.1 N(0,1)), with its own chunked seed."""
    T, H, D = X0.shape

    def draw(rng, shape, r0, r1):
        return bf16_to_f32(X0[r0:r1]).astype(np.float64) + 0.1 * rng.standard_normal(shape)

    return _chunked([seed, 2 + stream], T, H, D, draw)


def _block_factors(rng: np.random.Generator, n_blocks_shape) -> np.ndarray:
    """Per-block scale factor: 2% 2^-16, 2% 2^-100, 1% 2^-130, the rest 1."""
    u = rng.random(n_blocks_shape)
    f = np.ones(n_blocks_shape)
    f[u < 0.05] = 2.0 ** -130
    f[u < 0.04] = 2.0 ** -100
    f[u < 0.02] = 2.0 ** -16
    return f


def _expand_token_blocks(f: np.ndarray, T: int) -> np.ndarray:
    # f: [ceil(T/32), H, D] -> [T, H, D]
    return np.repeat(f, 32, axis=0)[:T]


def _expand_channel_blocks(f: np.ndarray, D: int) -> np.ndarray:
    # f: [T, H, ceil(D/32)] -> [T, H, D]
    return np.repeat(f, 32, axis=2)[:, :, :D]


def _c5_values(rng, shape, kind):
    T, H, D = shape
    x = rng.standard_normal(shape)
    if kind == "key":
        fac = _expand_token_blocks(_block_factors(rng, (-(-T // 32), H, D)), T)
    else:
        fac = _expand_channel_blocks(_block_factors(rng, (T, H, -(-D // 32))), D)
    x = x * fac
    u = rng.random(shape)
    f32 = x.astype(np.float32)
    f32[u < 0.02] = np.float32(0.0)
    f32[u < 0.01] = np.float32(-0.0)
    return bf16_bits(f32)


def c5_tensors(seed: int = 0):
    """Edge shapes. Returns the fused QKV buffer [T, 3*H*D], the K view into it ([T, H, D] with
    token stride 3*H*D and head stride D), and a contiguous V."""
    c = CONFIGS["c5"]
    T, H, D = c["T"], c["H"], c["D"]
    rng = np.random.default_rng(seed)
    qkv = bf16_bits(rng.standard_normal((T, 3 * H * D)))
    kvals = _c5_values(rng, (T, H, D), "key")
    V = _c5_values(rng, (T, H, D), "value")
    qkv[:, H * D:2 * H * D] = kvals.reshape(T, H * D)
    K = qkv[:, H * D:2 * H * D].reshape(T, H, D)  # a view: strides (3*H*D, D, 1) elements
    assert not K.flags["C_CONTIGUOUS"]
    return {"QKV": qkv, "K": K, "V": V}


def c5_residual_targets(R0K: np.ndarray, R0V: np.ndarray, seed: int = 5):
    """Next-loop states for the mixed chain, built from the reconstructed NVFP4 base R0:
    X1 = bf16(R0 + 0.1 N(0,1)); X1 := R0 on 2% of the 32-member residual groups (a zero
    residual); on 32-member blocks where R0 is exactly zero, X1 = bf16(2^-20 z) on half of them
    and bf16(2^-30 z) on the other half (tiny residual groups)."""
    rng = np.random.default_rng(seed)
    out = []
    for R0, kind in ((R0K, "key"), (R0V, "value")):
        T, H, D = R0.shape
        r0 = bf16_to_f32(R0).astype(np.float64)
        z = rng.standard_normal(R0.shape)
        x1 = r0 + 0.1 * z
        if kind == "key":
            nb = (-(-T // 32), H, D)
            expand = lambda a: _expand_token_blocks(a, T)  # noqa: E731
            zero_blk = np.ones(nb, bool)
            for b in range(nb[0]):
                zero_blk[b] = np.all((R0[b * 32:(b + 1) * 32] & 0x7FFF) == 0, axis=0)
        else:
            nb = (T, H, -(-D // 32))
            expand = lambda a: _expand_channel_blocks(a, D)  # noqa: E731
            zero_blk = np.ones(nb, bool)
            for c in range(nb[2]):
                zero_blk[:, :, c] = np.all((R0[:, :, c * 32:(c + 1) * 32] & 0x7FFF) == 0, axis=2)
        keep = expand(rng.random(nb) < 0.02)
        coin = rng.random(nb) < 0.5
        tiny20 = expand(zero_blk & coin)
        tiny30 = expand(zero_blk & ~coin)
        z2 = rng.standard_normal(R0.shape)
        x1 = np.where(tiny20, 2.0 ** -20 * z2, x1)
        x1 = np.where(tiny30, 2.0 ** -30 * z2, x1)
        X1 = bf16_bits(x1)
        X1 = np.where(keep, R0, X1).astype(np.uint16)
        out.append(X1)
    return {"XK1": out[0], "XV1": out[1]}


def tiny_tensor(seed: int = 7, T: int = 64, H: int = 2, D: int = 64):
    """A tensor whose amax is about 1e-35, with 16-member blocks scaled down by up to 2^-16 so
    that some NVFP4 decode scales fall below the binary32 normal range."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H, D)) * 1e-35
    # one factor per 16x16 tile covers both the token-axis and channel-axis block shapes
    fac = np.array([1.0, 2.0 ** -6, 2.0 ** -12, 2.0 ** -16])[rng.integers(0, 4, (-(-T // 16), H, -(-D // 16)))]
    fac = np.repeat(np.repeat(fac, 16, axis=0)[:T], 16, axis=2)[:, :, :D]
    return bf16_bits(x * fac)
