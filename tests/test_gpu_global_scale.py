"""GPU parity of the NVFP4 global multiplier entry point (kvq_nvfp4_global_scale) against the
oracle's rule g = fl(2688 / amax) over the rows an encode sees, and against the multiplier the
NVFP4 encoders themselves store ([PR166] "Purpose", second bullet)."""

import numpy as np
import pytest
import torch

import kv_cache_quantization_kvq_amd as kvq
import oracle
from gpu_util import dev, to_dev
from workloads import bf16_bits, c5_tensors, normal_kv, tiny_tensor

pytestmark = pytest.mark.gpu


def g_bits(t: torch.Tensor) -> int:
    return int(t.cpu().numpy().view(np.uint32)[0])


def want_bits(cur, prev=None, pos=None) -> int:
    return int(np.float32(oracle.nvfp4_global(oracle.tensor_amax(cur, prev, pos))).view(np.uint32))


@pytest.mark.parametrize("T,H,D", [(1, 1, 16), (333, 3, 48), (4096, 8, 128), (1000, 4, 256), (77, 2, 7)])
def test_global_scale_dense_residual_sparse(T, H, D):
    rng = np.random.default_rng(T + D)
    x0 = normal_kv(rng, T, H, D)
    x1 = bf16_bits(oracle.bf16_to_f32(x0) + 0.1 * rng.standard_normal((T, H, D)))
    pos = np.sort(rng.choice(T, max(1, T // 4), replace=False)).astype(np.int32)
    a0, a1, p = to_dev(x0), to_dev(x1), torch.from_numpy(pos).to(dev())
    assert g_bits(kvq.nvfp4_global_scale(a0)) == want_bits(x0)
    assert g_bits(kvq.nvfp4_global_scale(a1, a0)) == want_bits(x1, x0)
    assert g_bits(kvq.nvfp4_global_scale(a1, a0, p)) == want_bits(x1, x0, pos)
    # the same bits the encoders store
    assert g_bits(kvq.nvfp4_global_scale(a1, a0)) == g_bits(kvq.encode_residual(a1, a0, "key", "nvfp4").global_scale)
    assert g_bits(kvq.nvfp4_global_scale(a0)) == g_bits(kvq.pack(a0, "value", "nvfp4").global_scale)


def test_global_scale_edge_cases():
    # empty tensor and all zeros -> 1.0; a strided view; the tiny tensor (quotient near overflow)
    z = torch.zeros((0, 2, 16), dtype=torch.bfloat16, device=dev())
    assert g_bits(kvq.nvfp4_global_scale(z)) == 0x3F800000
    zz = torch.zeros((5, 2, 16), dtype=torch.bfloat16, device=dev())
    assert g_bits(kvq.nvfp4_global_scale(zz)) == 0x3F800000
    empty = torch.zeros(0, dtype=torch.int32, device=dev())
    assert g_bits(kvq.nvfp4_global_scale(zz, zz, empty)) == 0x3F800000
    c = c5_tensors(0)
    k = c["K"]  # a strided view into the fused QKV buffer (row pitch 3*H*D)
    T, H, D = k.shape
    kv = to_dev(c["QKV"])[:, H * D:2 * H * D].view(T, H, D)
    assert kv.stride(0) == 3 * H * D
    assert g_bits(kvq.nvfp4_global_scale(kv)) == want_bits(k)
    t = tiny_tensor()
    assert g_bits(kvq.nvfp4_global_scale(to_dev(t))) == want_bits(t)
