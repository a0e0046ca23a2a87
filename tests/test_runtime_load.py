"""One HIP runtime per process (CPU only: nothing here calls the GPU).

The libraries ask for libamdhip64.so.7 and carry the system ROCm directory
in their search path; torch ships its own copy of the runtime and asks for
it under another file name. Whichever enters the process first decides: a
library loaded before torch brings in the system copy and torch then maps a
second one beside it (launches from the library fail and torch can crash).
The package's loaders import torch first. Each case runs in a fresh
interpreter, since the order only matters before torch is imported.
"""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROBE = r"""
import ctypes, json, sys
sys.path.insert(0, {root!r})
{body}
maps = sorted({{line.split()[-1] for line in open('/proc/self/maps') if 'libamdhip64' in line}})
print(json.dumps(maps))
"""


def _hip_runtimes(body, hip_built):
    code = PROBE.format(root=ROOT, body=body)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    return json.loads(r.stdout.strip().splitlines()[-1])


def _torch_lib_dir():
    import torch
    return os.path.realpath(os.path.join(os.path.dirname(torch.__file__), "lib"))


def test_library_loaded_before_torch_maps_two_runtimes(hip_built):
    """The failure the loaders avoid: raw ctypes load first, torch second."""
    maps = _hip_runtimes(f"ctypes.CDLL({hip_built.LIB!r})\nimport torch", hip_built)
    assert len(maps) == 2, maps


def test_package_binding_shares_torchs_runtime(hip_built):
    """Importing the binding first still leaves one runtime: torch's."""
    body = ("from sharded_mixed_precision_zs_amd import zeroshard, synth\n"
            "synth._dev_lib()\n"
            "import torch")
    maps = _hip_runtimes(body, hip_built)
    assert len(maps) == 1, maps
    assert os.path.realpath(maps[0]).startswith(_torch_lib_dir()), maps
