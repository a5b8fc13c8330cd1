"""Build libtel.so for gfx950 with hipcc (in-tree: the library lands next to this file).

    python transformer_encoder_remove_amd/build.py [-v]

(Run as a script, not with -m: importing the package loads the library it builds.)

Every source under csrc/ is compiled to an object in <repo>/_build/ (parallel jobs),
then linked into transformer_encoder_remove_amd/libtel.so.
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import json
import os
import re
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtel.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ROCM_LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(HIPCC))), "lib")
MARKER_LIBS = ["-L", ROCM_LIB, f"-Wl,-rpath,{ROCM_LIB}", "-lrocprofiler-sdk-roctx"]

# Packed-fp32 VALU instructions are disabled for all device code.
COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", SRC, "-I", INCLUDE,
]


def sources() -> list[str]:
    return sorted(os.path.join(SRC, f) for f in os.listdir(SRC) if f.endswith((".hip", ".cpp")))


_FIELDS = {"TotalSGPRs": "sgpr", "VGPRs": "vgpr", "AGPRs": "agpr",
           "ScratchSize [bytes/lane]": "scratch", "Occupancy [waves/SIMD]": "occupancy",
           "SGPRs Spill": "sgpr_spill", "VGPRs Spill": "vgpr_spill",
           "LDS Size [bytes/block]": "lds"}


def parse_resource_usage(text: str) -> list[dict]:
    """Per-kernel figures from hipcc's -Rpass-analysis=kernel-resource-usage remarks."""
    kernels, cur = [], None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            kernels.append(cur)
            continue
        m = re.search(r"remark:\s+([^:]+(?:\[[^\]]*\])?): (\S+)", line)
        if m and cur is not None and m.group(1).strip() in _FIELDS:
            v = m.group(2)
            cur[_FIELDS[m.group(1).strip()]] = int(v) if v.lstrip("-").isdigit() else v
    return kernels


def source_digest(src: str) -> str:
    """SHA-256 over a source and every header under csrc/ and include/ (what it can include)."""
    h = hashlib.sha256()
    for f in [src] + sorted(os.path.join(d, n) for d in (SRC, INCLUDE) for n in os.listdir(d)
                            if n.endswith(".h")):
        h.update(open(f, "rb").read())
    return h.hexdigest()


def resource_report_path(src: str) -> str:
    return os.path.join(BUILD, os.path.basename(src) + ".resources.json")


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-c", src, "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
        cmd.append("-Rpass-analysis=kernel-resource-usage")   # per-kernel registers, scratch, LDS
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    out = r.stdout + r.stderr
    msg = "\n".join(l for l in out.splitlines()
                    if "packed-fp32-ops" not in l             # host pass does not know the feature
                    and "kernel-resource-usage" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    if verbose and msg.strip():
        print(msg)
    if src.endswith(".hip"):
        with open(resource_report_path(src), "w") as fh:
            json.dump({"source": os.path.basename(src), "sha256": source_digest(src),
                       "kernels": parse_resource_usage(out)}, fh, indent=1)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link libtel.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(8, len(srcs), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    # the host-timeline markers of api.cpp come from ROCm's marker library
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp,
           *MARKER_LIBS]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
