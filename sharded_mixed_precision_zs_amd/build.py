"""Build the in-tree shared libraries of the package.

  libzeroshard.so        the shard-step library (HIP, gfx950)  <- csrc/zeroshard.hip
                         + its host-side offload update (gcc) <- csrc/offload_cpu.cpp
  synth/libzssynth_dev.so   device twin of the input generator (HIP, gfx950)
  synth/libzssynth_host.so  host twin of the input generator (gcc)
  libzscopy.so           the plain copy the benchmark times as the HBM
                         ceiling (HIP, gfx950; measurement only) <- csrc/copy_ceiling.hip

Every call compiles from source. The libraries stay in the source tree so a
snapshot of the tree carries them to the GPU host.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libzeroshard.so")
SYNTH = os.path.join(PKG, "synth")
SYNTH_DEV = os.path.join(SYNTH, "libzssynth_dev.so")
SYNTH_HOST = os.path.join(SYNTH, "libzssynth_host.so")
COPY = os.path.join(PKG, "libzscopy.so")

ARCH = os.environ.get("ZS_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: each float operator rounds once, exactly as documented
#   (no fused multiply-add), so results match the op-by-op definition.
# No fast-math: IEEE division / sqrt and subnormals are required.
# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
HIP_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fPIC", "-shared", "-Wall", "-Wno-unused-result"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def _hip_lib(src, out, verbose, extra=()):
    tmp = out + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-I", INCLUDE, *extra, src, "-o", tmp], verbose)
    os.replace(tmp, out)


# Host half of the library (the ZeRO-Offload update): gcc, no contraction so
# vector mul/add stay separate IEEE operations; F16C for the fp16 convert.
CPU_FLAGS = ["-O3", "-std=c++17", "-ffp-contract=off", "-fno-fast-math", "-mf16c", "-fPIC",
             "-Wall", "-Wextra", "-pthread"]


def build_zeroshard(verbose=False):
    obj = os.path.join(PKG, "csrc", "offload_cpu.o")
    _run(["g++", *CPU_FLAGS, "-I", INCLUDE, "-c", os.path.join(PKG, "csrc", "offload_cpu.cpp"),
          "-o", obj], verbose)
    _hip_lib(os.path.join(PKG, "csrc", "zeroshard.hip"), LIB, verbose, extra=[obj, "-pthread"])
    os.remove(obj)
    return LIB


def build_synth_dev(verbose=False):
    _hip_lib(os.path.join(SYNTH, "synth_dev.hip"), SYNTH_DEV, verbose, extra=["-I", SYNTH])
    return SYNTH_DEV


def build_synth_host(verbose=False):
    tmp = SYNTH_HOST + ".tmp"
    _run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-I", SYNTH,
          os.path.join(SYNTH, "synth_host.c"), "-o", tmp], verbose)
    os.replace(tmp, SYNTH_HOST)
    return SYNTH_HOST


def build_copy(verbose=False):
    _hip_lib(os.path.join(PKG, "csrc", "copy_ceiling.hip"), COPY, verbose)
    return COPY


def build_all(verbose=False):
    return [build_zeroshard(verbose), build_synth_dev(verbose), build_synth_host(verbose),
            build_copy(verbose)]


if __name__ == "__main__":
    for p in build_all(verbose="-q" not in sys.argv):
        print(p)
