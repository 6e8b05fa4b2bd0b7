"""Builds libfa.so (the HIP kernels and the C ABI) in-tree for gfx950.

Every source is compiled by hipcc for gfx950 only; packed-fp32 instruction
selection is switched off for device code.  Objects go to ``_build/`` beside
this file; the library lands next to this file as ``libfa.so``.  The
compiler's per-kernel resource report (registers, spills, scratch, LDS,
occupancy) is kept as ``_build/resource_usage.json``.
"""
from __future__ import annotations

import concurrent.futures
import json
import os
import re
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfa.so")
# Measurement probe, a library of its own (not part of the attention ABI).
PROBE_SOURCE = "fa_probe.hip"
PROBE_LIB = os.path.join(PKG, "libfa_probe.so")
REPORT = os.path.join(BUILD, "resource_usage.json")
SOURCES = ["fa_api.hip", "fa_fwd.hip", "fa_bwd.hip", "fa_bwd_d128.hip", "fa_merge.hip",
           "fa_timing.hip"]
ARCH = "gfx950"
# Extra flags per source.  fa_bwd_d128.hip: MFMA results in VGPRs (the
# unmasked D = 128 dK/dV kernel otherwise moves its accumulators between
# register files on every tile).
EXTRA_FLAGS = {"fa_bwd_d128.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def hipcc():
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def compile_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


# Fields of the compiler's kernel-resource-usage remarks that are kept.
_FIELDS = {"TotalSGPRs": "sgprs", "VGPRs": "vgprs", "AGPRs": "agprs",
           "ScratchSize [bytes/lane]": "scratch_bytes", "Occupancy [waves/SIMD]": "occupancy",
           "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
           "LDS Size [bytes/block]": "lds_bytes"}
_REMARK = re.compile(r"remark:\s+(.*?):\s+(\S+)\s+\[-Rpass-analysis=kernel-resource-usage\]")


def parse_resource_remarks(text: str) -> dict:
    """{kernel symbol: {field: int}} from hipcc's kernel-resource-usage
    remarks (one "Function Name" line, then one line per field)."""
    out, cur = {}, None
    for key, val in _REMARK.findall(text):
        key = key.strip()
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None and key in _FIELDS:
            try:
                cur[_FIELDS[key]] = int(val)
            except ValueError:
                pass
    return out


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n"
                           f"{res.stdout}\n{res.stderr}")
    return res


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every source and link libfa.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *compile_flags(), *EXTRA_FLAGS.get(src, []),
                     "-Rpass-analysis=kernel-resource-usage", "-c",
                     os.path.join(CSRC, src), "-o", obj])
    usage = {}
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        for src, f in zip(SOURCES, [ex.submit(_run, c, verbose) for c in cmds]):
            for name, fields in parse_resource_remarks(f.result().stderr).items():
                usage[name] = dict(fields, source=src)
    with open(REPORT, "w") as fh:
        json.dump(usage, fh, indent=1, sort_keys=True)
    tmp = LIB + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    _run([cc, *compile_flags(), "-shared", "-o", tmp, os.path.join(CSRC, PROBE_SOURCE)], verbose)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
