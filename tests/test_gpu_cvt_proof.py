"""Exhaustive proof, on the GPU, that the gfx950 conversion instructions the codec may use
round exactly like the codec's software formulations.

Over all 2^32 binary32 inputs (NaNs skipped): v_cvt_pk_bf16_f32 vs the integer
round-to-nearest-even bf16 rounding, v_cvt_f16_f32 vs the software f16 rounding (with
subnormals), v_cvt_scalef32_pk_fp4_f32 (scale 1) vs the E2M1 threshold encoder with the sign
bit of the input; and for the 16 E2M1 codes v_cvt_scalef32_pk_f32_fp4 (scale 1) vs the
closed-form decode; plus the multiply-and-correct divisions by 15 and 6 against the IEEE
quotient (every finite non-negative input), v_rcp_f32 against the IEEE reciprocal (one-ulp
bound, normal range), its one-Newton-step refinement against the IEEE reciprocal (exact, every
scale in [2^-100, 2^100]), and the branch-free INT4 quotient against the IEEE division on
quotients at and next to every half-integer and float midpoint, for every scale significand at
eight exponents (about 1.5e11 cases); the E4M3 conversion instructions against the integer E4M3
rounding (every binary32 of magnitude up to 448) and decode (every finite code); and the
branch-free FP8-row quotient against the IEEE division on signed quotients at and next to float
midpoints from 2^-12 to 2^9 for every scale significand at eight exponents; and the NVFP4-row
row multiplier, block decode scale and its reciprocal computed without the IEEE division sequence
against the IEEE quotients for every finite positive bf16 row amax and every E4M3 scale code;
and v_cvt_pk_u8_f32 against round-to-nearest-even for every binary32 in [+0, 15.5] (the INT4
quotients it turns into codes).
The software formulations are written from the format definitions and are pinned
against the oracle end to end by the parity tests.
"""

import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(__file__), "probes", "libkvq_cvt_probe.so")
NAMES = ["bf16", "f16", "fp4 encode (all finite)", "fp4 encode (|x| <= 8)", "fp4 decode",
         "nibble order / f16 widening", "x/15 by FMA correction", "x/6 by FMA correction",
         "v_rcp_f32 within 1 ulp", "reciprocal + Newton step == RN(1/x)",
         "INT4 quotient (Markstein) == IEEE d / scale",
         "v_cvt_pk_fp8_f32 == E4M3 encode (|x| <= 448)", "v_cvt_pk_f32_fp8 == E4M3 decode",
         "FP8-row quotient (Markstein) == IEEE x / scale", "INT4 decode product exact (one FMA)",
         "NVFP4-row g = 2688 / amax without division (every bf16 amax)",
         "NVFP4-row s_dec = e4m3 / g without division (every amax x code)",
         "NVFP4-row 1 / s_dec without division (every amax x code)",
         "v_cvt_pk_u8_f32 rounds [0, 15.5] to nearest even",
         "NVFP4-row s_dec = e4m3 / g without division (every g significand x code)"]


def test_conversion_instructions_match_software_rounding():
    assert os.path.exists(LIB), "probe not built (run __graft_entry__.build())"
    lib = ctypes.CDLL(LIB)
    counts = (ctypes.c_ulonglong * len(NAMES))()
    first = (ctypes.c_uint32 * len(NAMES))()
    rc = lib.kvq_probe_cvt(counts, first)
    assert rc == 0
    report = {NAMES[i]: (int(counts[i]), hex(first[i])) for i in range(len(NAMES))}
    print(report)
    for i in range(len(NAMES)):
        assert counts[i] == 0, f"{NAMES[i]}: {counts[i]} mismatches, first input bits {hex(first[i])}"
