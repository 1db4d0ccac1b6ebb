"""In-tree build of the package's native libraries.

- libmoe_synth.so: the seeded input generator (plain C, host compiler).
- libmoe_mxfp4.so: the HIP kernels and the C-ABI entry points, for gfx950 only.
- libmoe_hbm.so: the streaming-read probe that bench.py runs beside the layer
  (measurement only).
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
ARCH = "gfx950"

HIP_SOURCES = ["moe_layer.hip", "k_pack.hip", "k_router.hip", "k_expert.hip", "k_shared.hip", "k_q2k.hip"]

# Packed-FP32 instructions are kept out of generated code on purpose.
HIP_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared", "-Wall",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-I", os.path.join(ROOT, "include")]


def build_synth() -> str:
    out = os.path.join(HERE, "libmoe_synth.so")
    subprocess.run(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-pthread", "-Wall", "-o", out,
                    os.path.join(CSRC, "synth.c"), "-lm"], check=True)
    return out


def build_hip(extra_flags=()) -> str:
    out = os.path.join(HERE, "libmoe_mxfp4.so")
    tmp = out + ".tmp"
    srcs = [os.path.join(CSRC, s) for s in HIP_SOURCES]
    subprocess.run(["hipcc", *HIP_FLAGS, *extra_flags, "-o", tmp, *srcs], check=True)
    os.replace(tmp, out)
    return out


def build_hbm_probe() -> str:
    out = os.path.join(HERE, "libmoe_hbm.so")
    tmp = out + ".tmp"
    subprocess.run(["hipcc", *HIP_FLAGS, "-o", tmp, os.path.join(CSRC, "hbm_probe.hip")], check=True)
    os.replace(tmp, out)
    return out


def build_all() -> None:
    build_synth()
    build_hip()
    build_hbm_probe()


if __name__ == "__main__":
    build_all()
