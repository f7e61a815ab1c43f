"""GPU parity at the bulk size (T=131072, H=8, D=128, Student-t nu=3), in full, in the launch
configuration the bench times.

For each format (INT4 G64, NVFP4 G16) and kind, the whole chain of the bulk workload runs on
the device and in the oracle (its OpenMP build, which gives the same bits as the
single-threaded one), and every output is compared bit for bit over all 134M elements:
    R0 = unpack(pack(X0));  R = encode_residual(X1, R0);  R1 = decode_residual(R, R0)
with X1 = bf16(X0 + 0.1 N(0,1)). The residual is encoded against the reconstructed predecessor
R0 ([PR166] "Purpose", fourth bullet), once the device's R0 has been shown equal to the
oracle's: both sides then encode the same input.
"""

import numpy as np
import pytest
import torch

import kv_cache_quantization_kvq_amd as kvq
import oracle
from gpu_util import assert_bits_equal, planes, to_dev, to_host
from workloads import c4_residual_target, c4_tensors

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bulk():
    d = c4_tensors(0)
    return {"key": (d["K"], c4_residual_target(d["K"], stream=0)),
            "value": (d["V"], c4_residual_target(d["V"], stream=1))}


@pytest.fixture(scope="module", autouse=True)
def threaded_oracle():
    prev = oracle.set_threaded(True)
    yield
    oracle.set_threaded(prev)


def assert_planes_equal(gp, op, what):
    g, o = planes(gp), planes(op)
    assert set(g) == set(o), what
    for name, want in o.items():
        assert_bits_equal(g[name], want, f"{what} {name}")


@pytest.mark.parametrize("fmt", ["int4", "nvfp4"])
@pytest.mark.parametrize("kind", ["key", "value"])
def test_bulk_full_size_chain(bulk, kind, fmt):
    X0, X1 = bulk[kind]
    assert X0.shape == (131072, 8, 128)
    G = 64 if fmt == "int4" else 16
    x0, x1 = to_dev(X0), to_dev(X1)
    gp = kvq.pack(x0, kind, fmt, G)
    R0 = kvq.unpack(gp)
    torch.cuda.synchronize()
    op = oracle.pack(X0, kind, fmt, G)
    oR0 = oracle.unpack(op)
    assert_planes_equal(gp, op, f"{fmt} {kind} pack")
    assert_bits_equal(to_host(R0), oR0, f"{fmt} {kind} unpack")
    del op
    gr = kvq.encode_residual(x1, R0, kind, fmt, G)
    R1 = kvq.decode_residual(gr, R0)
    torch.cuda.synchronize()
    orr = oracle.encode_residual(X1, oR0, kind, fmt, G)
    assert_planes_equal(gr, orr, f"{fmt} {kind} residual")
    assert_bits_equal(to_host(R1), oracle.decode_residual(orr, oR0), f"{fmt} {kind} residual decode")
    if fmt == "nvfp4":  # the multipliers are the oracle's full-tensor amax rule
        assert float(planes(gr)["global_scale"].view(np.float32)[0]) == oracle.nvfp4_global(
            oracle.tensor_amax(X1, oR0))
