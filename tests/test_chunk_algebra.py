"""The chunked form that the HIP kernels evaluate, written in fp64 numpy and pinned
against the token-by-token oracle (CPU only).

Within a 16-token chunk ("Kimi K3 Deep Dive...", "The Problem: The Diagonal-Block
Dilemma": intra-chunk and inter-chunk paths with decay products), with start state
S, inclusive chunk-local cumulative log-decay G and Gamma = exp(G) per channel:
    K+ = K*Gamma, K- = K/Gamma, Q+ = Q*Gamma, Kend = K*Gamma_C/Gamma
    A  = StrictLower(diag(beta) K+ K-^T),  T = (I + A)^-1
    W  = T diag(beta) K+,  Ut = T diag(beta) V,   U = Ut - W S
    O  = Q+ S + LowerIncl(Q+ K-^T) U
    S' = Diag(Gamma_C) S + Kend^T U
A chunk therefore maps S affinely, S' = M S + N with M = Diag(Gamma_C) - Kend^T W and
N = Kend^T Ut; a run of chunks (a segment) composes to one such map, which is how a
long sequence is split into independently scanned segments.  A ragged last chunk is
padded with identity tokens (g = 0, beta = 0, q = k = v = 0), which change nothing.
"""
import numpy as np
import pytest

from chunked_gated_delta_12_amd import inputs as kin

C = 16


def _chunks(q, k, v, g, beta):
    T = q.shape[0]
    n = -(-T // C)
    pad = n * C - T
    padf = lambda x: np.concatenate([x, np.zeros((pad,) + x.shape[1:])]) if pad else x
    return n, padf(q), padf(k), padf(v), padf(g), padf(beta)


def _intra(qc, kc, vc, gc, bc):
    G = np.cumsum(gc, axis=0)
    Gam = np.exp(G)
    Kp, Km, Qp = kc * Gam, kc / Gam, qc * Gam
    Kend = kc * (Gam[-1] / Gam)
    A = np.tril(bc[:, None] * (Kp @ Km.T), -1)
    Tm = np.linalg.inv(np.eye(C) + A)
    W = Tm @ (bc[:, None] * Kp)
    Ut = Tm @ (bc[:, None] * vc)
    Aqk = np.tril(Qp @ Km.T)
    return Gam[-1], Kend, W, Ut, Qp, Aqk


def chunked_head(q, k, v, g, beta, S0, segments=1):
    """One (batch, head) sequence; q,k,g [T,dk], v [T,dv], beta [T], S0 [dk,dv]."""
    T, dk = q.shape
    dv = v.shape[1]
    n, q, k, v, g, beta = _chunks(q, k, v, g, beta)
    intra = [_intra(q[i*C:(i+1)*C], k[i*C:(i+1)*C], v[i*C:(i+1)*C], g[i*C:(i+1)*C], beta[i*C:(i+1)*C])
             for i in range(n)]
    L = -(-n // segments)
    bounds = [(s * L, min(n, (s + 1) * L)) for s in range(segments) if s * L < n]
    # map of each segment but the last: widened state [N | M] from [0 | I]
    starts = [S0.copy()]
    for (c0, c1) in bounds[:-1]:
        X = np.concatenate([np.zeros((dk, dv)), np.eye(dk)], axis=1)
        for i in range(c0, c1):
            gC, Kend, W, Ut, _, _ = intra[i]
            Ufull = np.concatenate([Ut, np.zeros((C, dk))], axis=1) - W @ X
            X = gC[:, None] * X + Kend.T @ Ufull
        N, M = X[:, :dv], X[:, dv:]
        starts.append(M @ starts[-1] + N)
    O = np.zeros((n * C, dv))
    for s, (c0, c1) in enumerate(bounds):
        S = starts[s]
        for i in range(c0, c1):
            gC, Kend, W, Ut, Qp, Aqk = intra[i]
            U = Ut - W @ S
            O[i*C:(i+1)*C] = Qp @ S + Aqk @ U
            S = gC[:, None] * S + Kend.T @ U
    return O[:T], S


def chunked(q, k, v, g, beta, S0, segments=1):
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    O = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            s0 = S0[b, h] if S0 is not None else np.zeros((dk, dv))
            O[b, :, h], ST[b, h] = chunked_head(q[b, :, h], k[b, :, h], v[b, :, h], g[b, :, h],
                                                beta[b, :, h], s0, segments)
    return O, ST


def _case(name, **kw):
    w = kin.scaled(kin.WORKLOADS[name], **kw)
    x = kin.chunk_inputs(w)
    d = {n: (t.double().numpy() if t is not None else None) for n, t in x.items()}
    return d


@pytest.mark.parametrize("name,kw,segments", [
    ("tiny", {}, 1),
    ("tiny", {}, 3),
    ("small", dict(B=1, H=2, T=203), 1),          # ragged tail, S0 != 0
    ("small", dict(B=1, H=2, T=203), 4),
    ("decay_stress", dict(H=2, T=96, dk=32, dv=32), 1),   # g close to -5: exp(+-80) factors
    ("decay_stress", dict(H=2, T=96, dk=32, dv=32), 6),
])
def test_chunked_form_matches_oracle(oracle_mod, name, kw, segments):
    d = _case(name, **kw)
    g = oracle_mod.gate(d["theta"])
    o_ref, s_ref = oracle_mod.recurrence(d["q"], d["k"], d["v"], g, d["beta"], d["S0"])
    o, s = chunked(d["q"], d["k"], d["v"], g, d["beta"], d["S0"], segments)
    assert np.abs(o - o_ref).max() <= 1e-10 * np.abs(o_ref).max()
    assert np.abs(s - s_ref).max() <= 1e-10 * np.abs(s_ref).max()


def test_inverse_decay_within_bf16_in_stress_case(oracle_mod):
    """The largest factor the chunked form ever scales by is exp(-min G) <= exp(80)."""
    d = _case("decay_stress", H=2, T=256, dk=32, dv=32)
    G = oracle_mod.gate_cumsum(oracle_mod.gate(d["theta"]))
    assert np.exp(-G.min()) <= np.exp(80.0)
    assert np.exp(-G.min()) > 1e34      # and the case does come close to it
