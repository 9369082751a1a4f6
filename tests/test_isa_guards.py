"""Build-time checks on the gfx950 code libkda generates (CPU only; needs hipcc).

Results of the legacy v_mfma_f32_16x16x16_bf16 instruction, read at the wait
states the compiler inserts after it, came back stale on gfx950 (wrong output
rows in an otherwise correct kernel), so K = 16 bf16 products are issued as
16x16x32 with half the k-slots zeroed.  This test compiles every HIP source to
assembly and fails if the legacy instruction appears again.  It also checks
that no kernel spills to scratch.
"""
import os
import re
import shutil
import subprocess

import pytest

from chunked_gated_delta_12_amd import build as kbuild

CSRC = os.path.join(os.path.dirname(kbuild.__file__), "csrc")
HIP_SOURCES = [s for s in kbuild.SOURCES if s.endswith(".hip")]

@pytest.fixture(scope="module")
def assembly(tmp_path_factory):
    try:
        hipcc = kbuild.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    out = {}
    tmp = tmp_path_factory.mktemp("isa")
    for src in HIP_SOURCES:
        asm = tmp / (src + ".s")
        cmd = [hipcc] + kbuild._flags() + ["--cuda-device-only", "-S", os.path.join(CSRC, src),
                                           "-o", str(asm), "-Rpass-analysis=kernel-resource-usage"]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
        out[src] = (asm.read_text(), res.stderr)
    return out


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_legacy_16x16x16_bf16_mfma(assembly, src):
    text, _ = assembly[src]
    hits = [l.strip() for l in text.splitlines() if re.match(r"^\s*v_mfma_f32_16x16x16_?bf16", l)]
    assert not hits, f"{src} emits the legacy instruction: {hits[:3]}"


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_matrix_cores_used_where_expected(assembly, src):
    text, _ = assembly[src]
    n = len(re.findall(r"^\s*v_mfma_f32_16x16x32_bf16", text, flags=re.M))
    if src == "kda_chunk.hip":
        assert n > 0
    else:
        assert n == 0   # gate and decode are elementwise / bandwidth kernels


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_scratch_spills(assembly, src):
    _, remarks = assembly[src]
    sizes = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", remarks)]
    assert sizes and max(sizes) == 0, f"{src}: scratch use {max(sizes) if sizes else '?'} bytes/lane"
