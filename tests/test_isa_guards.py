"""Build-time checks on the gfx950 code libkda generates (CPU only; needs hipcc).

Results of the legacy v_mfma_f32_16x16x16_bf16 instruction, read at the wait
states the compiler inserts after it, came back stale on gfx950 (wrong output
rows in an otherwise correct kernel), so K = 16 bf16 products are issued as
16x16x32 with half the k-slots zeroed.  This test compiles every HIP source to
assembly and fails if the legacy instruction appears again.  It also checks
that no kernel spills to scratch, with one stated exception: the gated
single-segment chunk kernel at d = 128 keeps one 4-byte value in scratch (8
bytes per lane) across its chunk loop, stored once before the loop and read
once after it.
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
    if src in ("kda_chunk.hip", "kda_map.hip", "kda_out.hip", "kda_bwd2.hip", "kda_gmap.hip"):
        assert n > 0
    elif src == "kda_bwd.hip":
        # the fp32 backward (fp32 inputs; bf16 at d = 16 and 32) runs on the fp32 matrix cores
        assert n == 0 and re.search(r"^\s*v_mfma_f32_16x16x4_?f32", text, flags=re.M)
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


# The one kernel allowed scratch: chunk_kernel<E, 128, 4, single segment, gated, bounded>.
_SCRATCH_ALLOWED = re.compile(r"_ZN3kda12chunk_kernelI(f|DF16b)Li128ELi4ELb0ELb1ELb0E")


def _scratch_per_function(remarks):
    out, fn = {}, None
    for l in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", l)
        if m:
            fn = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", l)
        if m and fn:
            out[fn] = int(m.group(1))
    return out


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_no_spills_inside_loops(assembly, src):
    """No kernel uses scratch, except the gated single-segment chunk kernel at d = 128
    (8 bytes per lane, outside its loops); and no loop body touches scratch."""
    text, remarks = assembly[src]
    per = _scratch_per_function(remarks)
    assert per, f"{src}: no resource-usage remarks"
    bad = {fn: n for fn, n in per.items() if n and not (_SCRATCH_ALLOWED.match(fn) and n <= 8)}
    assert not bad, f"{src}: scratch use (bytes/lane): {bad}"
    bodies = _loop_bodies(text)
    if src in ("kda_chunk.hip", "kda_map.hip", "kda_out.hip"):
        assert bodies, "the per-chunk loops were not found"
    per_fn = {}
    for fn, body in bodies:
        per_fn[fn] = per_fn.get(fn, 0) + sum("scratch_" in l for l in body)
    bad = {fn: n for fn, n in per_fn.items() if n}
    assert not bad, f"{src}: spills inside loops: {bad}"


# ----------------------------------------------------------------------------- matrix-core result hazards
# A matrix-core result must not be read before the instruction has retired; the
# compiler inserts the wait states, and within a basic block it uses 8 for
# 16x16x32 bf16 and 10 for 16x16x4 fp32 before a dependent read.  Across a
# loop back-edge it has been seen to insert fewer (two, for an fp32 state
# tile read right at the top of the next iteration), which returned stale
# values.  This walks every control-flow path after each MFMA and checks the
# distance to the first read of its result.
_WAITS = {"16x16x32_bf16": 8, "16x16x4_f32": 10, "16x16x4f32": 10}


def _regs(tok):
    tok = tok.strip().rstrip(",")
    m = re.match(r"^([va])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"^-?\|?([va])(\d+)\|?$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _blocks(lines):
    blocks, order, cur = {}, [], None
    for l in lines:
        m = re.match(r"^(\.LBB\d+_\d+):", l) or re.match(r"^; (%bb\.\d+):", l)
        if m:
            cur = m.group(1)
            blocks[cur], order = [], order + [cur]
            continue
        s = l.split(";")[0].strip()
        if s and not s.startswith(".") and cur is not None:
            blocks[cur].append(s)
    return blocks, order


def _successors(blocks, order, b):
    last = blocks[b][-1] if blocks[b] else ""
    op = last.split()[0] if last else ""
    if op == "s_branch":
        return [last.split()[1]]
    out = [last.split()[1]] if op.startswith("s_cbranch") else []
    if op == "s_endpgm":
        return out
    i = order.index(b)
    return out + ([order[i + 1]] if i + 1 < len(order) else [])


def _reads(ins):
    """(srcA/srcB or plain vector reads, srcC reads, vector registers written)."""
    op = ins.split()[0]
    ops = ins.split(None, 1)[1].split(",") if " " in ins else []
    if op.startswith("v_mfma"):
        return set().union(*(_regs(t) for t in ops[1:3])), _regs(ops[3]), _regs(ops[0])
    store = re.match(r"(ds_write|global_store|buffer_store|scratch_store|flat_store)", op)
    if op.startswith(("v_", "ds_", "global_", "buffer_", "scratch_", "flat_")):
        first = 0 if store else 1
        written = set() if store else _regs(ops[0]) if ops else set()
        return set().union(set(), *(_regs(t) for t in ops[first:])), set(), written
    return set(), set(), set()


def _early_reads(text):
    found = []
    for part in re.split(r"\n(?=_Z\S+:)", text):
        m = re.match(r"(_Z\S+):", part)
        if not m:
            continue
        blocks, order = _blocks(part[:part.find(".Lfunc_end")].split("\n"))
        for b in order:
            for idx, ins in enumerate(blocks[b]):
                if not ins.startswith("v_mfma"):
                    continue
                need = next((n for k, n in _WAITS.items() if k in ins), 10)
                dst0 = frozenset(_regs(ins.split(None, 1)[1].split(",")[0]))
                stack, seen = [(b, idx + 1, 0, dst0)], set()
                while stack:
                    bb, i, ws, dst = stack.pop()
                    if (bb, i, ws, dst) in seen or ws >= need or not dst:
                        continue
                    seen.add((bb, i, ws, dst))
                    if i >= len(blocks[bb]):
                        stack += [(s, 0, ws, dst) for s in _successors(blocks, order, bb) if s in blocks]
                        continue
                    x = blocks[bb][i]
                    ab, c, w = _reads(x)
                    # an accumulation into exactly the same registers is forwarded
                    if ab & dst or (c and c != dst0 and c & dst):
                        found.append(f"{m.group(1)[:50]} {b}: {ins[:40]} -> {bb}: {x[:40]} after {ws}")
                        continue
                    n = int(x.split()[1]) + 1 if x.startswith("s_nop") else 1
                    stack.append((bb, i + 1, ws + n, dst - frozenset(w)))
    return found


@pytest.mark.parametrize("src", HIP_SOURCES)
def test_matrix_results_not_read_early(assembly, src):
    text, _ = assembly[src]
    bad = _early_reads(text)
    assert not bad, f"{src}: matrix-core results read too early: {bad[:4]}"


def test_early_read_check_finds_a_planted_case():
    """The check itself: a fp32 result read two instructions after its
    producer, through a loop back-edge, is reported; with a pad it is not."""
    asm = ("_Zk:\n; %bb.0:\n.LBB0_1:\n\tv_mov_b32 v5, 0\n"
           "\tv_mfma_f32_16x16x4_f32 a[0:3], v23, a3, a[4:7]\n\ts_cbranch_vccz .LBB0_1\n"
           "; %bb.2:\n\ts_endpgm\n.Lfunc_end0:\n")
    assert _early_reads(asm)
    assert not _early_reads(asm.replace("\ts_cbranch_vccz", "\ts_nop 9\n\ts_cbranch_vccz"))
