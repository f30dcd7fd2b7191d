"""Build the C++ client of the C ABI (host code only, g++; no device code).

It links ``paged_kv_attention_03_amd/libpkv.so`` (the library under test) and
``oracle/liboracle.so`` (the float64 oracle, test infrastructure), both found
next to the binary through its run path, and the HIP runtime.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
EXE = os.path.join(HERE, "pkv_client")


def build(verbose: bool = False) -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = EXE + ".tmp"
    cmd = ["g++", "-O2", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           os.path.join(HERE, "pkv_client.cpp"), "-o", tmp,
           "-L", os.path.join(ROOT, "paged_kv_attention_03_amd"), "-lpkv",
           "-L", os.path.join(ROOT, "oracle"), "-loracle",
           "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../paged_kv_attention_03_amd",
           "-Wl,-rpath,$ORIGIN/../../oracle", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(verbose=True))
