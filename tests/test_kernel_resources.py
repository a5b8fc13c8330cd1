"""Every kernel the library builds runs without scratch memory (no register spills to
memory, no private arrays), as the compiler reports it (-Rpass-analysis=
kernel-resource-usage). The build writes that report for each source; a source whose
report is missing or older than the source is compiled here once more to get it. CPU only."""
import importlib.util
import json
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location(
    "tel_build_script", os.path.join(ROOT, "transformer_encoder_remove_amd", "build.py"))
build = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(build)

HIP_SOURCES = [s for s in build.sources() if s.endswith(".hip")]


def _report(src: str) -> dict:
    path = build.resource_report_path(src)
    if os.path.exists(path):
        rep = json.load(open(path))
        if rep.get("sha256") == build.source_digest(src):
            return rep
    if not os.path.exists(build.HIPCC) and not shutil.which(build.HIPCC):
        pytest.skip("hipcc not available")
    cmd = [build.HIPCC, "-x", "hip", *build.COMMON, "-c", src, "-o", os.devnull,
           "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return {"kernels": build.parse_resource_usage(r.stdout + r.stderr)}


@pytest.mark.parametrize("src", HIP_SOURCES, ids=[os.path.basename(s) for s in HIP_SOURCES])
def test_no_scratch_no_spills(src):
    kernels = _report(src)["kernels"]
    if os.path.basename(src) not in ("noalloc.hip",):
        assert kernels, f"no kernel reported for {src}"
    for k in kernels:
        assert k.get("scratch") == 0, (k["name"], k)
        assert k.get("vgpr_spill") == 0 and k.get("sgpr_spill") == 0, (k["name"], k)


def test_parser_reads_the_remark_format():
    text = (
        "f.hip:1:1: remark: Function Name: _Z3fooPf [-Rpass-analysis=kernel-resource-usage]\n"
        "f.hip:1:1: remark:     TotalSGPRs: 14 [-Rpass-analysis=kernel-resource-usage]\n"
        "f.hip:1:1: remark:     VGPRs: 139 [-Rpass-analysis=kernel-resource-usage]\n"
        "f.hip:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n"
        "f.hip:1:1: remark:     Occupancy [waves/SIMD]: 3 [-Rpass-analysis=kernel-resource-usage]\n"
        "f.hip:1:1: remark:     VGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]\n"
        "f.hip:1:1: remark:     SGPRs Spill: 0 [-Rpass-analysis=kernel-resource-usage]\n"
        "f.hip:1:1: remark:     LDS Size [bytes/block]: 69632 [-Rpass-analysis=kernel-resource-usage]\n")
    (k,) = build.parse_resource_usage(text)
    assert k == {"name": "_Z3fooPf", "sgpr": 14, "vgpr": 139, "scratch": 0, "occupancy": 3,
                 "vgpr_spill": 0, "sgpr_spill": 0, "lds": 69632}
