"""Exhaustive proof, on the GPU, that the gfx950 conversion instructions the codec may use
round exactly like the codec's software formulations.

Over all 2^32 binary32 inputs (NaNs skipped): v_cvt_pk_bf16_f32 vs the integer
round-to-nearest-even bf16 rounding, v_cvt_f16_f32 vs the software f16 rounding (with
subnormals), v_cvt_scalef32_pk_fp4_f32 (scale 1) vs the E2M1 threshold encoder with the sign
bit of the input; and for the 16 E2M1 codes v_cvt_scalef32_pk_f32_fp4 (scale 1) vs the
closed-form decode. The software formulations are themselves pinned on the CPU against the
oracle's definitions (test_kernel_formulas_host.py) and by the parity tests.
"""

import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(__file__), "probes", "libkvq_cvt_probe.so")
NAMES = ["bf16", "f16", "fp4 encode (all finite)", "fp4 encode (|x| <= 8)", "fp4 decode",
         "nibble order / f16 widening"]


def test_conversion_instructions_match_software_rounding():
    assert os.path.exists(LIB), "probe not built (run __graft_entry__.build())"
    lib = ctypes.CDLL(LIB)
    counts = (ctypes.c_ulonglong * 6)()
    first = (ctypes.c_uint32 * 6)()
    rc = lib.kvq_probe_cvt(counts, first)
    assert rc == 0
    report = {NAMES[i]: (int(counts[i]), hex(first[i])) for i in range(6)}
    print(report)
    for i in (0, 1, 2, 3, 4, 5):
        assert counts[i] == 0, f"{NAMES[i]}: {counts[i]} mismatches, first input bits {hex(first[i])}"
