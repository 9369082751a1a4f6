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


def _loop_bodies(text):
    """(function, lines) of every basic block the compiler annotates as part of a
    loop (its block label line carries "Loop Header" or "in Loop")."""
    fn, cur, in_loop, out = None, [], False, []
    for l in text.splitlines():
        if re.match(r"^_Z\S+:", l):
            fn = l.split(":")[0]
        starts = re.match(r"^(\.LBB\d+_\d+:|; %bb\.\d+:)", l)
        if starts or re.match(r"^_Z\S+:", l):
            if in_loop and cur:
                out.append((fn, cur))
            cur, in_loop = [], bool(starts) and "Loop" in l
        cur.append(l)
    if in_loop and cur:
        out.append((fn, cur))
    return out


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_spills_inside_loops(assembly, src):
    """Registers may spill around a kernel's prologue/epilogue (bounded below), but
    (almost) never inside a loop, where it costs memory traffic every iteration."""
    text, remarks = assembly[src]
    sizes = [int(x) for x in re.findall(r"ScratchSize \[bytes/lane\]: (\d+)", remarks)]
    assert sizes and max(sizes) <= 64, f"{src}: scratch use {max(sizes)} bytes/lane"
    bodies = _loop_bodies(text)
    if src == "kda_chunk.hip":
        assert bodies, "the per-chunk loops were not found"
    per_fn = {}
    for fn, body in bodies:
        per_fn[fn] = per_fn.get(fn, 0) + sum("scratch_" in l for l in body)
    # A stray reload or two per iteration is noise next to the loop's hundreds of
    # instructions; anything more means the kernel's registers no longer fit.
    bad = {fn: n for fn, n in per_fn.items() if n > 2}
    assert not bad, f"{src}: spills inside loops: {bad}"
