"""Build the host sanitizer driver: the C-ABI layer (relative_bias_gqa_amd/csrc/abi.cpp) with
its HIP calls and kernel launches stubbed, and the CPU oracle (oracle/*.c), all compiled by
g++ / gcc for the host with AddressSanitizer and UndefinedBehaviorSanitizer (no device code
is built here).

Usage: ``python tests/host_sanitize/build.py OUT_DIR`` prints the driver's path.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "relative_bias_gqa_amd", "csrc")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
INC = ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-I", HERE]
HIP_HOST = ["-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include"]


def build(out_dir: str) -> str:
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in (os.path.join(CSRC, "abi.cpp"), os.path.join(HERE, "stubs.cpp"), os.path.join(HERE, "driver.cpp")):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        subprocess.run(["g++", "-std=c++17", *SAN, *HIP_HOST, *INC, "-c", src, "-o", obj], check=True)
        objs.append(obj)
    for src in ("rattn_oracle.c", "rattn_oracle_bwd.c"):
        obj = os.path.join(out_dir, src + ".o")
        subprocess.run(["gcc", "-std=c99", "-fopenmp", "-fno-fast-math", *SAN, *INC, "-c",
                        os.path.join(ROOT, "oracle", src), "-o", obj], check=True)
        objs.append(obj)
    exe = os.path.join(out_dir, "host_sanitize_driver")
    subprocess.run(["g++", *SAN, "-fopenmp", "-o", exe, *objs, "-lm"], check=True)
    return exe


if __name__ == "__main__":
    print(build(sys.argv[1] if len(sys.argv) > 1 else os.path.join(ROOT, "_build", "host_sanitize")))
