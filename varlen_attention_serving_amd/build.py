"""Build the gfx950 library ``libua.so`` in-tree with hipcc.

Every translation unit is compiled for gfx950 only, with packed-fp32 code
generation switched off, then linked into one shared object next to this file.
Run ``python -m varlen_attention_serving_amd.build`` or call ``build()``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libua.so")

SOURCES = ["ua_api.cpp", "ua_attn_d64.hip", "ua_attn_d128.hip", "ua_attn_d256.hip",
           "ua_merge.hip"]
HEADERS = ["ua_internal.h", "ua_attn_impl.h"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Wno-unused-result", "-Wno-unknown-pragmas",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _compile(src: str, extra=(), build_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    if err.strip():
        sys.stderr.write(err + "\n")
    return obj


def build(jobs: int = 0, verbose: bool = True, defines=(), out: str = LIB,
          build_dir: str = BUILD_DIR) -> str:
    """Compile all sources for gfx950 and link ``libua.so`` (always rebuilds).
    ``defines``/``out``/``build_dir`` serve experiment builds of variants."""
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, len(os.sched_getaffinity(0))))
    extra = [f"-D{d}" for d in defines]
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda src: _compile(src, extra, build_dir), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, out)
    if verbose:
        print(f"built {out}")
    return out


def resources(build_dir: str = BUILD_DIR) -> dict:
    """Per-kernel resources as the compiler reports them for gfx950 (VGPRs,
    AGPRs, SGPRs, spills, scratch, static LDS and its occupancy estimate,
    which ignores dynamic LDS), from a device-only compile of every kernel
    translation unit with the kernel-resource-usage remarks."""
    os.makedirs(build_dir, exist_ok=True)
    keys = {"TotalSGPRs": "sgpr", "VGPRs": "vgpr", "AGPRs": "agpr",
            "ScratchSize [bytes/lane]": "scratch", "Occupancy [waves/SIMD]": "occupancy",
            "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
            "LDS Size [bytes/block]": "lds_static"}
    out = {}
    for src in SOURCES:
        if not src.endswith(".hip"):
            continue
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".res.o")
        cmd = [HIPCC, *COMMON, "--offload-device-only", "-Rpass-analysis=kernel-resource-usage",
               "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
        cur = None
        for line in r.stderr.splitlines():
            if "remark:" not in line or "kernel-resource-usage" not in line:
                continue
            body = line.split("remark:", 1)[1].split("[-Rpass", 1)[0].strip()
            name, _, val = body.partition(":")
            name, val = name.strip(), val.strip()
            if name == "Function Name":
                cur = out.setdefault(val, {})
            elif cur is not None and name in keys:
                cur[keys[name]] = int(val) if val.isdigit() else val
    return out


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "--resources":
        pats = sys.argv[2:]
        for name, r in sorted(resources().items()):
            if pats and not any(s in name for s in pats):
                continue
            print(f"{name}  " + "  ".join(f"{k}={v}" for k, v in r.items()))
    else:
        build()
