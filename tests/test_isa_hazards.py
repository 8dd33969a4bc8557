"""Checks on the gfx950 assembly of the attention kernels (CPU only: hipcc
cross-compiles).

The K/V tile copies are `global_load_lds_dwordx4` instructions written as inline
assembly, which the compiler's hazard recognizer does not look into, so their
operands are restricted to forms that need no wait states from it:

* the global address comes from a VGPR pair (`..., off` with an optional
  immediate offset), never from an SGPR base: a VMEM read of an SGPR written by a VALU instruction (v_readlane,
  v_readfirstlane, v_cmp) needs wait states the compiler cannot insert here;
* the one wait state an SALU write of M0 needs before an LDS-DMA instruction
  reads it is part of the assembly: no LDS-DMA instruction may directly follow
  an instruction whose destination is M0;
* M0 itself is written by scalar instructions only (a VALU write of an SGPR
  read by a VMEM instruction would need wait states as above).
"""
import os
import re
import subprocess

import pytest

from transformer_attention_04_amd import build as B


_ASM = {}


def _device_asm(tmp_path):
    """Device assembly of every kernel source of the library, concatenated
    (compiled once per test session)."""
    if not os.path.exists(B.HIPCC):
        pytest.skip("hipcc not available")
    if "asm" in _ASM:
        return _ASM["asm"]
    flags = [f for f in B.FLAGS if f not in ("-shared", "-fPIC")]
    text = []
    for src in B.SOURCES:
        out = tmp_path / (os.path.basename(src) + ".s")
        r = subprocess.run([B.HIPCC, *flags, "--cuda-device-only", "-S", "-o", str(out), src],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        text.append(out.read_text())
    _ASM["asm"] = "\n".join(text)
    return _ASM["asm"]


def _instructions(asm):
    for line in asm.splitlines():
        t = line.strip()
        if t and not t.startswith((";", ".")) and not t.endswith(":"):
            yield t


def test_no_lds_dma_directly_after_an_m0_write(tmp_path):
    asm = _device_asm(tmp_path)
    prev, n, bad = None, 0, []
    for ins in _instructions(asm):
        if ins.split()[0].startswith("global_load_lds"):
            n += 1
            parts = prev.split(None, 1) if prev else []
            if len(parts) > 1 and parts[1].split(",")[0].strip() == "m0":
                bad.append((prev, ins))
        prev = ins
    assert n > 0, "no LDS-DMA instruction found"
    assert not bad, f"{len(bad)} of {n} LDS-DMA instructions directly follow an M0 write, e.g. {bad[0]}"


def test_lds_dma_addresses_come_from_vgprs(tmp_path):
    asm = _device_asm(tmp_path)
    dma = [ins for ins in _instructions(asm) if ins.split()[0].startswith("global_load_lds")]
    assert dma, "no LDS-DMA instruction found"
    sgpr_based = [ins for ins in dma if ins.split(None, 1)[1].split(",")[1].split()[0] != "off"]
    assert not sgpr_based, f"{len(sgpr_based)} LDS-DMA instructions take an SGPR base, e.g. {sgpr_based[0]}"


def test_m0_for_lds_dma_written_by_scalar_instructions(tmp_path):
    # A VMEM instruction reading an SGPR (M0 included) that a VALU instruction
    # wrote needs wait states the assembly does not carry: M0 must come from
    # SALU (s_mov/s_add ...), never v_readfirstlane/v_readlane.
    asm = _device_asm(tmp_path)
    last_m0, n, bad = None, 0, []
    for ins in _instructions(asm):
        if ins.split()[0].startswith("global_load_lds"):
            n += 1
            if last_m0 is None or not last_m0.startswith("s_"):
                bad.append((last_m0, ins))
        parts = ins.split(None, 1)
        if len(parts) > 1 and parts[1].split(",")[0].strip() == "m0":
            last_m0 = ins
    assert n > 0, "no LDS-DMA instruction found"
    assert not bad, f"{len(bad)} LDS-DMA instructions take M0 from a non-scalar write, e.g. {bad[0]}"


def _functions(asm):
    """(name, body) of every kernel in the assembly."""
    out, name, body = [], None, []
    for line in asm.splitlines():
        label = re.match(r"^([A-Za-z_]\w*):\s*(;.*)?$", line)
        if label:
            if name:
                out.append((name, body))
            name, body = label.group(1), []
        elif name and line.strip().startswith(".Lfunc_end"):
            out.append((name, body))
            name, body = None, []
        elif name:
            body.append(line)
    return out


def test_attention_kernels_use_no_dot_instructions(tmp_path):
    # v_dot2* instructions wait for the matrix pipe on gfx950: beside another
    # wave's MFMA stream they stall this wave's in-order instruction stream,
    # so the softmax row sums are plain fp32 adds.
    asm = _device_asm(tmp_path)
    kernels = [(n, b) for n, b in _functions(asm) if "attn_fwd_kernel" in n]
    assert kernels, "no attention kernel found"
    bad = [(n, ins) for n, b in kernels for ins in _instructions("\n".join(b)) if ins.split()[0].startswith("v_dot")]
    assert not bad, f"{len(bad)} dot instructions in attention kernels, e.g. {bad[0]}"


def _kernel_meta(asm):
    """(name, vgpr, agpr, lds bytes, scratch bytes) of every kernel in the code object metadata."""
    meta = asm.split("amdhsa.kernels:")[1:]
    out = []
    for m in meta:
        for blk in re.split(r"\n  - ", m)[1:]:
            def g(k):
                x = re.search(r"\." + k + r":\s+(\S+)", blk)
                return x.group(1) if x else None
            if g("name") is None or g("vgpr_count") is None:
                continue
            out.append((g("name"), int(g("vgpr_count")), int(g("agpr_count") or 0),
                        int(g("group_segment_fixed_size")), int(g("private_segment_fixed_size"))))
    return out


# Workgroups each attention kernel instance must fit per CU: the launch
# geometry the schedule is built on (16-bit one-group tiles: three four-wave
# workgroups per CU; the eight-wave key split: one; 64-row key-split tiles:
# two; the two-wave decode tiles: at least two; fp32: one).  Keyed by
# (16-bit, KS, QG).
_WG_PER_CU = {(True, 1, 4): 3, (True, 2, 4): 1, (True, 2, 2): 2, (True, 2, 1): 2,
              (False, 1, 4): 1, (False, 2, 4): 1, (False, 2, 2): 1, (False, 2, 1): 1}


def test_attention_kernels_keep_their_occupancy(tmp_path):
    # 512 registers (VGPR + AGPR, allocated in granules of 8) per SIMD lane,
    # four SIMDs and 160 KB of LDS per CU; a kernel that outgrows its
    # launch bound spills instead, which the scratch limit catches.
    asm = _device_asm(tmp_path)
    pat = re.compile(r"attn_fwd_kernelI(DF16b|DF16_|f)Lb[01]ELi(\d)ELb[01]ELb[01]ELi(\d)E")
    seen = set()
    for name, vgpr, agpr, lds, scratch in _kernel_meta(asm):
        m = pat.search(name)
        if not m:
            continue
        key = (m.group(1) != "f", int(m.group(2)), int(m.group(3)))
        seen.add(key)
        regs = -(-(-(-vgpr // 4) * 4 + agpr) // 8) * 8
        waves_per_simd = 512 // regs
        waves = key[1] * key[2]  # waves per workgroup
        fit = min(4 * waves_per_simd // waves, (160 * 1024) // lds)
        assert fit >= _WG_PER_CU[key], (f"{name}: {vgpr} VGPR + {agpr} AGPR, {lds} B LDS fit {fit} workgroups "
                                         f"per CU, the schedule assumes {_WG_PER_CU[key]}")
        assert scratch <= 16, f"{name}: {scratch} bytes of scratch per lane (spills)"
    assert seen == set(_WG_PER_CU), f"kernel instances found: {sorted(seen)}"
