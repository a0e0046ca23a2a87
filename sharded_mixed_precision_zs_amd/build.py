"""Build the in-tree shared libraries of the package.

  libzeroshard.so        the shard-step library (HIP, gfx950)  <- csrc/zeroshard.hip
                         + its host-side offload update (gcc) <- csrc/offload_cpu.cpp
  synth/libzssynth_dev.so   device twin of the input generator (HIP, gfx950)
  synth/libzssynth_host.so  host twin of the input generator (gcc)
  libzscopy.so           the plain copy and the stream probes the benchmark
                         times as HBM ceilings (HIP, gfx950; measurement
                         only) <- csrc/copy_ceiling.hip
  libzsvariants.so       shapes of the fused kernel the benchmark times
                         against libzeroshard's (HIP, gfx950; measurement
                         only) <- csrc/fused_variants.hip

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
VARIANTS = os.path.join(PKG, "libzsvariants.so")

ARCH = os.environ.get("ZS_OFFLOAD_ARCH", "gfx950")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -ffp-contract=off: each float operator rounds once, exactly as documented
#   (no fused multiply-add), so results match the op-by-op definition.
# No fast-math: IEEE division / sqrt and subnormals are required.
# -packed-fp32-ops: keep the compiler from forming packed fp32 VALU ops.
HIP_FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-ffp-contract=off",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fPIC", "-shared", "-Wall", "-Wno-unused-result"]


# One HIP runtime per process, whichever is loaded first. torch ships its own
# copy of the HIP runtime (file libamdhip64.so, SONAME libamdhip64.so.7) and
# asks for it by file name; hipcc would link the libraries against the
# system copy (asked for as libamdhip64.so.7, found through
# LD_LIBRARY_PATH), so a library loaded before torch brought in a second
# runtime. Instead the libraries ask for "libamdhip64.so" -- the name torch
# asks for -- with torch's library directory first in their DT_RPATH (which
# precedes LD_LIBRARY_PATH): loaded first they map torch's runtime, which
# torch then finds by name; loaded after torch they find it the same way.
# Without torch the system directory supplies the runtime. The name comes
# from an import stub: an empty library whose SONAME is libamdhip64.so,
# linked in place of the runtime (-no-hip-rt); the HIP symbols are resolved
# when the library is loaded.
BUILD_DIR = os.path.join(ROOT, "_build")
HIP_STUB_DIR = os.path.join(BUILD_DIR, "hipstub")
ROCM_LIB = os.environ.get("ZS_ROCM_LIB", "/opt/rocm/lib")


def torch_lib_dir():
    """torch's library directory when it ships a HIP runtime, else None
    (found without importing torch)."""
    import importlib.util
    spec = importlib.util.find_spec("torch")
    if spec is None or not spec.submodule_search_locations:
        return None
    d = os.path.join(list(spec.submodule_search_locations)[0], "lib")
    return os.path.realpath(d) if os.path.exists(os.path.join(d, "libamdhip64.so")) else None


def hip_runtime_link_flags(verbose=False):
    """Link flags that bind a HIP library to the runtime as described above."""
    os.makedirs(HIP_STUB_DIR, exist_ok=True)
    src = os.path.join(HIP_STUB_DIR, "stub.c")
    with open(src, "w") as f:
        f.write("/* import stub: only its SONAME is used */\n")
    stub = os.path.join(HIP_STUB_DIR, "libamdhip64.so")
    _run(["gcc", "-shared", "-fPIC", "-Wl,-soname,libamdhip64.so", src, "-o", stub], verbose)
    path = ":".join(d for d in (torch_lib_dir(), ROCM_LIB) if d)
    return ["-no-hip-rt", f"-L{HIP_STUB_DIR}", "-Wl,--no-as-needed", "-lamdhip64",
            "-Wl,--disable-new-dtags", f"-Wl,-rpath,{path}"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def _hip_lib(src, out, verbose, extra=()):
    tmp = out + ".tmp"
    _run([HIPCC, *HIP_FLAGS, "-I", INCLUDE, *extra, src, *hip_runtime_link_flags(verbose),
          "-o", tmp], verbose)
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


def build_variants(verbose=False):
    _hip_lib(os.path.join(PKG, "csrc", "fused_variants.hip"), VARIANTS, verbose)
    return VARIANTS


def build_all(verbose=False):
    return [build_zeroshard(verbose), build_synth_dev(verbose), build_synth_host(verbose),
            build_copy(verbose), build_variants(verbose)]


if __name__ == "__main__":
    for p in build_all(verbose="-q" not in sys.argv):
        print(p)
