"""One HIP runtime per process, whatever the load order (CPU only: nothing
here calls the GPU).

torch ships its own copy of the HIP runtime and asks for it by the file name
libamdhip64.so. The libraries ask for that same name and search torch's
library directory first (build.py), so whether a library or torch enters
the process first, exactly one runtime is mapped -- torch's, with its own
HSA runtime beside it -- and the library's launches share torch's streams
and allocations. Each case runs in a fresh interpreter, since the order only
matters before torch is imported.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROBE = r"""
import ctypes, json, sys
sys.path.insert(0, {root!r})
{body}
maps = {{}}
for line in open('/proc/self/maps'):
    path = line.split()[-1]
    for key in ('libamdhip64', 'libhsa-runtime64'):
        if key in path:
            maps.setdefault(key, set()).add(path)
print(json.dumps({{k: sorted(v) for k, v in maps.items()}}))
"""


def _mapped(body):
    code = PROBE.format(root=ROOT, body=body)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    return json.loads(r.stdout.strip().splitlines()[-1])


def _torch_lib_dir():
    import torch
    return os.path.realpath(os.path.join(os.path.dirname(torch.__file__), "lib"))


def _assert_one_runtime(maps):
    for key in ("libamdhip64", "libhsa-runtime64"):
        assert len(maps.get(key, [])) == 1, maps
        assert os.path.realpath(maps[key][0]).startswith(_torch_lib_dir()), maps


@pytest.mark.parametrize("which", ["LIB", "COPY", "SYNTH_DEV", "VARIANTS"])
def test_library_loaded_before_torch_shares_its_runtime(hip_built, which):
    """Raw ctypes load first, torch second: still one runtime, torch's."""
    path = getattr(hip_built, which)
    _assert_one_runtime(_mapped(f"ctypes.CDLL({path!r})\nimport torch"))


@pytest.mark.parametrize("which", ["LIB", "COPY", "SYNTH_DEV", "VARIANTS"])
def test_library_loaded_after_torch_shares_its_runtime(hip_built, which):
    path = getattr(hip_built, which)
    _assert_one_runtime(_mapped(f"import torch\nctypes.CDLL({path!r})"))


def test_package_binding_shares_torchs_runtime(hip_built):
    """Importing the binding and the generator first leaves one runtime."""
    body = ("from sharded_mixed_precision_zs_amd import zeroshard, synth\n"
            "synth._dev_lib()\n"
            "import torch")
    _assert_one_runtime(_mapped(body))


def test_libraries_ask_for_torchs_runtime_name(hip_built):
    """The dynamic section names libamdhip64.so (not the system SONAME) and
    searches torch's directory first."""
    out = subprocess.run(["readelf", "-d", hip_built.LIB], capture_output=True, text=True,
                         check=True).stdout
    needed = [ln for ln in out.splitlines() if "(NEEDED)" in ln and "amdhip" in ln]
    assert needed and all("[libamdhip64.so]" in ln for ln in needed), needed
    rpath = [ln for ln in out.splitlines() if "(RPATH)" in ln]
    assert rpath and _torch_lib_dir() in rpath[0].split("[", 1)[1], rpath
