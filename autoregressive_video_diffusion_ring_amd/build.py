"""Build librc.so (the C-ABI library with the gfx950 HIP kernels) in-tree.

    python -m autoregressive_video_diffusion_ring_amd.build

compiles every source under csrc/ with hipcc for gfx950 and links
``autoregressive_video_diffusion_ring_amd/librc.so``.  Object files go to
``_build/`` at the repository root.  hipcc cross-compiles without a GPU.

The compiler's per-kernel resource report (registers, spills, scratch bytes
per lane, occupancy, LDS) is kept in ``_build/kernel_resources.json``: a
kernel that silently moves an accumulator array to scratch memory still
computes the right result, only several times slower, so the report is
checked by the CPU tests.
"""
from __future__ import annotations

import json
import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "librc.so")

SOURCES = ["rc_host.cpp", "cache_write.hip", "chunk_attn.hip", "attn_fp8.hip", "memory.hip", "qkv_write.hip",
           "noalloc.hip"]

# Packed fp32 instructions are disabled for device code: they are generated
# only from ordinary float code and are not needed on any path here.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include")]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librc.so)")


# The attention kernels handle no NaN inputs specially; without NaN
# semantics their maxima compile to plain v_max3 instructions.
EXTRA = {"chunk_attn.hip": ["-fno-honor-nans"], "attn_fp8.hip": ["-fno-honor-nans"]}


RESOURCES = os.path.join(BUILD, "kernel_resources.json")
_REMARK = re.compile(r"remark: +(Function Name|[A-Za-z ]+?)(?: \[[^\]]*\])?: (\S+) \[-Rpass-analysis=kernel-resource-usage\]")


def parse_resource_remarks(text: str) -> dict:
    """{kernel symbol: {field: value}} from hipcc's kernel-resource-usage remarks."""
    out: dict = {}
    cur = None
    for line in text.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1).strip(), m.group(2)
        if key == "Function Name":
            cur = out.setdefault(val, {})
        elif cur is not None:
            cur[key] = int(val) if val.lstrip("-").isdigit() else val
    return out


def _compile(src: str, verbose: bool):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    device = src.endswith(".hip")
    report = ["-Rpass-analysis=kernel-resource-usage"] if device else []
    cmd = [hipcc(), *COMMON, *DEVICE_FLAGS, *EXTRA.get(src, []), *report, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    res = parse_resource_remarks(r.stderr) if device else {}
    out = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line and "kernel-resource-usage" not in line
                    and not line.lstrip().startswith(("|", "^")) and not re.match(r"\s*\d+ \|", line))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    if out.strip() and verbose:
        print(out, flush=True)
    return obj, {k: dict(v, source=src) for k, v in res.items()}


def build(verbose: bool = False) -> str:
    """Compile all sources and link librc.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    objs = [o for o, _ in results]
    resources: dict = {}
    for _, res in results:
        resources.update(res)
    with open(RESOURCES, "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *DEVICE_FLAGS, "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
