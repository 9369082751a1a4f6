"""kda_chunk_fwd_noalloc (the prefill entry point that takes no workspace and uses
libkda's static per-device scratch) against kda_chunk_fwd with a caller workspace,
through the C ABI.

Both run the same kernels on the same inputs, so the outputs must agree bit for
bit.  Two calls in a row share the scratch: the first at the 64K-token, 16-head
prefill with its 16 segments (110 MiB of scratch), the second on a smaller input,
so the second reads nothing stale from the first.  The first is also checked
against the fp64 oracle on a few value columns, the second on the whole tensor.
"""
import sys

import numpy as np
import pytest
import torch

import chunked_gated_delta_12_amd as kda
from chunked_gated_delta_12_amd import inputs as kin

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_err(gpu, ref):
    gpu = gpu.detach().to("cpu").double().numpy()
    return float(np.abs(gpu - ref).max() / np.abs(ref).max())


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    kda.load_library()


def _pair(x, w, segments):
    """(o, S_T) of kda_chunk_fwd_noalloc and of kda_chunk_fwd, outputs pre-filled with NaN."""
    outs = []
    for fn in (kda.kda_chunk_fwd_noalloc, kda.kda_chunk_fwd):
        o = torch.full((w.B, w.T, w.H, w.dv), float("nan"), device=DEV, dtype=x["q"].dtype)
        S_T = torch.full((w.B, w.H, w.dk, w.dv), float("nan"), device=DEV)
        fn(x["q"], x["k"], x["v"], x["theta"], x["beta"], x["S0"], segments=segments, o=o, S_T=S_T)
        outs.append((o, S_T))
    torch.cuda.synchronize()
    return outs


def test_noalloc_equals_workspace_call_twice(oracle_mod):
    # first call: the 64K prefill at its automatic segment count (16), 110 MiB of scratch
    w1 = kin.WORKLOADS["prefill_64k"]
    seg1 = kda.kda_chunk_fwd_auto_segments(w1.B, w1.T, w1.H, w1.dk, w1.dv)
    need1 = kda.kda_chunk_fwd_workspace_size(w1.B, w1.T, w1.H, w1.dk, w1.dv, seg1)
    note(f"noalloc call 1: {w1} segments={seg1} scratch={need1} B")
    assert seg1 > 1 and 0 < need1 <= 128 << 20
    x1 = kin.chunk_inputs(w1, device=DEV)
    (o_n, s_n), (o_w, s_w) = _pair(x1, w1, seg1)
    assert torch.equal(o_n, o_w) and torch.equal(s_n, s_w)
    cols = [2, 21, 40, 59, 78, 97, 116, 127]
    cpu = lambda t: t[:, :, :4].contiguous().cpu()
    o_ref, s_ref = oracle_mod.chunk_fwd(cpu(x1["q"]), cpu(x1["k"]), cpu(x1["v"]), cpu(x1["theta"]),
                                        cpu(x1["beta"]), None, cols=cols)
    eo, es = rel_err(o_n[:, :, :4][..., cols], o_ref), rel_err(s_n[:, :4][..., cols], s_ref)
    note(f"  bit-equal to kda_chunk_fwd; heads 0-3, columns {cols}: err_o={eo:.3e} err_S={es:.3e}")
    assert eo <= 2e-2 and es <= 2e-2
    del x1, o_n, s_n, o_w, s_w

    # second call, smaller: bf16, d = 64, S0 != 0, ragged tail, 5 segments
    w2 = kin.scaled(kin.WORKLOADS["small"], T=1000 + 7)
    note(f"noalloc call 2: {w2} segments=5")
    x2c = kin.chunk_inputs(w2)
    x2 = {k: (v.to(DEV) if v is not None else None) for k, v in x2c.items()}
    (o_n, s_n), (o_w, s_w) = _pair(x2, w2, 5)
    assert torch.equal(o_n, o_w) and torch.equal(s_n, s_w)
    o_ref, s_ref = oracle_mod.chunk_fwd(x2c["q"], x2c["k"], x2c["v"], x2c["theta"], x2c["beta"], x2c["S0"])
    eo, es = rel_err(o_n, o_ref), rel_err(s_n, s_ref)
    note(f"  bit-equal to kda_chunk_fwd; whole tensor: err_o={eo:.3e} err_S={es:.3e}")
    assert eo <= 2e-2 and es <= 2e-2


def test_noalloc_single_segment():
    """One segment needs no scratch (the single-pass kernel runs alone)."""
    w = kin.scaled(kin.WORKLOADS["small"], T=300)
    x = {k: (v.to(DEV) if v is not None else None) for k, v in kin.chunk_inputs(w).items()}
    (o_n, s_n), (o_w, s_w) = _pair(x, w, 1)
    assert torch.equal(o_n, o_w) and torch.equal(s_n, s_w)
