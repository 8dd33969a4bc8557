"""The library and torch share one HIP runtime whatever the import order (CPU
only: checks the process's mapped libraries, no GPU call).

torch bundles a HIP runtime with the same soname as the system runtime the
library links; if the library were loaded first, the process would map both
and torch's streams and allocations would be foreign to the library's calls.
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROBE = """
import sys
sys.path.insert(0, {root!r})
{first}
import torch
maps = open('/proc/self/maps').read()
libs = sorted(set(l.split()[-1] for l in maps.splitlines()
                  if 'libamdhip64' in l or 'libhsa-runtime64' in l))
print('\\n'.join(libs))
"""


def _mapped(first):
    r = subprocess.run([sys.executable, "-c", PROBE.format(root=ROOT, first=first)], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    return [ln for ln in r.stdout.splitlines() if ln.strip()]


def test_one_hip_runtime_when_the_package_is_imported_first():
    libs = _mapped("import transformer_attention_04_amd")
    hip = [p for p in libs if "libamdhip64" in p]
    hsa = [p for p in libs if "libhsa-runtime64" in p]
    assert len(hip) == 1 and len(hsa) == 1, libs


def test_one_hip_runtime_when_torch_is_imported_first():
    libs = _mapped("import torch; import transformer_attention_04_amd")
    assert len([p for p in libs if "libamdhip64" in p]) == 1, libs
