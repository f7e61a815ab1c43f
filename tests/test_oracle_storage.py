"""Storage accounting pinned to the figures the pages print (tests/golden/pages_storage.txt).

The oracle counts exact payload bytes: codes rows*H*ceil(D/2), INT4 metadata 4 B per group
(f16 minimum + f16 scale), NVFP4 metadata 1 B per 16-member block plus one FP32 per tensor,
and 4 B per row of an owned sparse position map. The 76 B figure is the per-row-scale format of
the FreeToken page; in the per-tensor format it is one (token, head) row packed as its own
tensor (64 + 8 + 4), see test_76_bytes_row.
"""

import os

import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_storage.txt")


def golden():
    out = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        name, value, _src = (s.strip() for s in line.split("|"))
        out[name] = float(value)
    return out


G = golden()


def bits_per_element(fmt, kind, Gs, rows, H, D):
    b = oracle.storage_bytes(fmt, kind, Gs, rows, H, D)
    return 8.0 * b / (rows * H * D)


def test_bits_per_element_complete_groups():
    # large tensors, complete groups: the per-tensor 4 B of NVFP4 vanishes in the average
    assert bits_per_element("int4", "value", 64, 4096, 8, 128) == G["int4_g64_bits_per_element"]
    assert bits_per_element("int4", "key", 64, 4096, 8, 128) == G["int4_g64_bits_per_element_table"]
    assert bits_per_element("int4", "value", 16, 4096, 8, 128) == G["int4_g16_bits_per_element"]
    assert bits_per_element("int4", "key", 16, 4096, 8, 128) == G["int4_g16_bits_per_element"]
    n = 4096 * 8 * 128
    for kind in ("key", "value"):
        b = oracle.storage_bytes("nvfp4", kind, 16, 4096, 8, 128)
        assert b == n * G["nvfp4_g16_bits_per_element"] / 8 + G["nvfp4_bytes_per_tensor"]


def test_76_bytes_row():
    assert oracle.storage_bytes("nvfp4", "value", 16, 1, 1, 128) == G["nvfp4_row_bytes_d128"]
    assert 2 * oracle.storage_bytes("nvfp4", "value", 16, 1, 1, 128) == G["nvfp4_kv_pair_bytes_d128"]
    assert 1 * 1 * 128 * 2 == G["bf16_row_bytes_d128"]
    # a config-2 tensor [4096, 8, 128]: 72 B per row plus one 4 B tensor scale
    assert oracle.storage_bytes("nvfp4", "value", 16, 4096, 8, 128) == 4096 * 8 * 72 + 4 == 2359300
    assert oracle.storage_bytes("nvfp4", "key", 16, 4096, 8, 128) == 2359300


def test_per_token_layer_bytes():
    per_kind_16h = oracle.storage_bytes("int4", "value", 64, 1, 16, 128)
    assert 2 * per_kind_16h == G["bytes_per_token_layer_16h_4bit"]
    assert 2 * 16 * 128 * 2 == G["bytes_per_token_layer_16h_bf16"]
    assert round(G["bytes_per_token_layer_16h_bf16"] / (2 * per_kind_16h), 2) == G["compression_vs_bf16"]
    per_kind_8h = oracle.storage_bytes("int4", "value", 64, 1, 8, 128)
    assert per_kind_8h == G["bytes_per_kind_token_8h"]
    assert 2 * per_kind_8h == G["bytes_per_token_kv_8h"]
    codes = 8 * 64
    assert 100.0 * (per_kind_8h - codes) / codes == G["scale_fraction_d128_percent"]


def test_group_counts_at_T2048():
    def ngroups(kind, Gs, T, D):
        # metadata groups per (head, channel) for K, per (token, head) row for V
        return (oracle.storage_bytes("int4", kind, Gs, T, 1, D) - T * ((D + 1) // 2)) // 4 // (D if kind == "key" else T)

    assert ngroups("key", 16, 2048, 128) == G["k_g16_groups_T2048"]
    assert ngroups("value", 16, 2048, 128) == G["v_g16_groups_D128"]
    assert ngroups("key", 64, 2048, 128) == G["k_g64_groups_T2048"]


def test_sparse_and_partial():
    # owned position map: 4 B per compact row
    assert oracle.storage_bytes("int4", "key", 64, 2048, 8, 128, sparse=True) == 2048 * 8 * 72 + 4 * 2048
    # partial groups round up: T=1000, G=32 -> 32 token groups; D=7 -> 4 code bytes per row
    assert oracle.storage_bytes("int4", "key", 32, 1000, 4, 256) == 1000 * 4 * 128 + 32 * 4 * 256 * 4
    assert oracle.storage_bytes("int4", "value", 4, 3, 1, 7) == 3 * 4 + 3 * 2 * 4
    assert oracle.storage_bytes("nvfp4", "value", 16, 0, 8, 128) == 4
    assert oracle.storage_bytes("nvfp4", "key", 8, 4, 1, 16) == -1  # NVFP4 is G16 only


@pytest.mark.parametrize("fmt,Gs", [("int4", 64), ("int4", 16), ("nvfp4", 16)])
def test_storage_equals_real_array_bytes(fmt, Gs):
    """The pages' second review asks that storage_bytes match the real tensor bytes."""
    import numpy as np
    from workloads import normal_kv

    x = normal_kv(np.random.default_rng(0), 100, 3, 40)
    for kind in ("key", "value"):
        p = oracle.pack(x, kind, fmt, Gs)
        real = sum(a.nbytes for a in (p.codes, p.meta0, p.meta1, p.global_scale) if a is not None)
        assert real == oracle.storage_bytes(fmt, kind, Gs, 100, 3, 40)


def test_row_format_bytes():
    # NVFP4 with one FP32 scale per (token, head) row: 64 + 8 + 4 = 76 B at D = 128, per row
    parts = G["nvfp4_row_code_bytes_d128"] + G["nvfp4_row_block_scale_bytes_d128"] + G["nvfp4_row_scale_bytes"]
    assert parts == G["nvfp4_row_bytes_d128"]
    for kind in ("key", "value"):
        assert oracle.storage_bytes("nvfp4_row", kind, 16, 1, 1, 128) == G["nvfp4_row_bytes_d128"]
        assert oracle.storage_bytes("nvfp4_row", kind, 16, 2, 1, 128) == G["nvfp4_kv_pair_bytes_d128"]
        # the per-row format scales linearly: no per-tensor term
        assert oracle.storage_bytes("nvfp4_row", kind, 16, 4096, 8, 128) == 4096 * 8 * 76
    # FP8 E4M3 with one FP32 scale per row: codes are half of bf16, plus a 4 B sidecar (~3%)
    b = oracle.storage_bytes("fp8_row", "value", 0, 1, 1, 128)
    assert b - G["fp8_row_scale_bytes"] == G["fp8_row_code_fraction_of_bf16"] * G["bf16_row_bytes_d128"]
    assert round(100 * G["fp8_row_scale_bytes"] / 128) == G["fp8_row_scale_percent_d128"]
    assert oracle.storage_bytes("fp8_row", "key", 0, 10, 4, 96, sparse=True) == 10 * 4 * (96 + 4) + 40
    # array bytes equal the formula
    from workloads import normal_kv
    import numpy as np
    x = normal_kv(np.random.default_rng(0), 9, 3, 40)
    for fmt, g in (("nvfp4_row", 16), ("fp8_row", 0)):
        p = oracle.pack(x, "value", fmt, g)
        nb = p.codes.nbytes + p.meta0.nbytes + (p.meta1.nbytes if p.meta1 is not None else 0)
        assert nb == oracle.storage_bytes(fmt, "value", g, 9, 3, 40)
