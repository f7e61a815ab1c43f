"""Build tests/c_abi/kvq_c_chain, a host program that uses libkvq through include/kvq.h only."""

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "kvq_c_chain")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    cmd = ["g++", "-O2", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
           "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "kvq_c_chain.cpp"), "-o", EXE + ".tmp",
           "-L", os.path.join(ROOT, "kv_cache_quantization_kvq_amd"), "-lkvq", "-L", os.path.join(ROCM, "lib"),
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/../../kv_cache_quantization_kvq_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("C ABI example build failed:\n" + r.stdout + r.stderr)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())
