"""Build libattn.so (the attention library) and libattn_clock.so (the
benchmark's shader-clock probe), gfx950 only, in-tree with hipcc, and record
the source revision they were built from in build_info.json."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "attn_fwd.hip")
SOURCES = [SRC, os.path.join(PKG, "csrc", "qkv_proj.hip")]  # all linked into libattn.so
OUT = os.path.join(PKG, "libattn.so")
CLOCK_SRC = os.path.join(PKG, "csrc", "clock_probe.hip")
CLOCK_OUT = os.path.join(PKG, "libattn_clock.so")
INFO = os.path.join(PKG, "build_info.json")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # device code only: NaN-free arithmetic lets v_max skip canonicalisation
    "-Xarch_device", "-fno-honor-nans",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src, out: str, extra: list[str] | None, verbose: bool) -> str:
    srcs = [src] if isinstance(src, str) else list(src)
    cmd = [HIPCC, *FLAGS, *(extra or []), "-o", out + ".tmp", *srcs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


def _git(*args: str) -> str | None:
    try:
        r = subprocess.run(["git", "-C", ROOT, *args], capture_output=True, text=True, timeout=10)
    except (OSError, subprocess.SubprocessError):
        return None
    return r.stdout.strip() if r.returncode == 0 else None


def write_info() -> dict:
    """The revision the libraries were built from (the GPU machine has no git
    history, so the benchmark reads it from here)."""
    import json
    import time
    status = _git("status", "--porcelain", "--untracked-files=no")
    ver = subprocess.run([HIPCC, "--version"], capture_output=True, text=True)
    info = {"git_rev": _git("rev-parse", "HEAD"), "tree_modified": bool(status) if status is not None else None,
            "hipcc": next((ln.strip() for ln in ver.stdout.splitlines() if "HIP version" in ln), None),
            "built_utc": time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime())}
    with open(INFO, "w") as f:
        json.dump(info, f, indent=1)
    return info


def build(out: str = OUT, extra: list[str] | None = None, verbose: bool = False) -> str:
    """Build the attention library (and, for the default output path, the
    clock probe and the build record)."""
    _compile(SOURCES, out, extra, verbose)
    if out == OUT:
        _compile(CLOCK_SRC, CLOCK_OUT, None, verbose)
        write_info()
    return out


if __name__ == "__main__":
    print(build(verbose=True))
