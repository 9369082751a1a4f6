"""The chunked form of the backward pass, written in fp64 numpy and pinned against the
token-by-token backward oracle (CPU only).

Per 16-token chunk, with the forward quantities of tests/test_chunk_algebra.py (start
state S, K+ = K*Gamma, K- = K/Gamma, Q+ = Q*Gamma, Kend = K*Gamma_C/Gamma,
A = StrictLower(diag(beta) K+ K-^T), T = (I + A)^-1, Y = V - K+ S, U = T diag(beta) Y,
A_qk = LowerIncl(Q+ K-^T)), the incoming gradients dO of the chunk's outputs and dS' of
its end state give

    dU = A_qk^T dO + Kend dS'          Z = T^T dU,   dY = diag(beta) Z,   dV = dY
    dS = Diag(Gamma_C) dS' + Q+^T dO - K+^T dY        (carried to the previous chunk)
    dA_qk = LowerIncl(dO U^T),          dA = StrictLower(-Z U^T)
    dQ+ = dO S^T + dA_qk K-
    dK+ = -dY S^T + diag(beta) dA K-,  dK- = dA_qk^T Q+ + (diag(beta) dA)^T K+
    dKend = U dS'^T,   dGamma_C = rowsum(dS' * S)
    dbeta = rowsum(dA * K+ K-^T) + rowsum(Z * Y)

followed by the chain through the decay scalings to K, Q and the chunk-local cumulative
log-decay G, whose reverse prefix sum over the chunk gives dg.  The carried gradient
is the transposed chunk map of the forward (dS = M^T dS' + ...), so the segment
decomposition of the forward applies to it as well.
"""
import numpy as np
import pytest

C = 16


def chunked_backward_head(q, k, v, g, beta, S0, do, dS_T):
    """One (batch, head); q,k,g [T,dk], v,do [T,dv], beta [T], S0,dS_T [dk,dv]."""
    T, dk = q.shape
    dv = v.shape[1]
    n = -(-T // C)
    pad = n * C - T
    padf = lambda x: np.concatenate([x, np.zeros((pad,) + x.shape[1:])]) if pad else x
    q, k, v, g, beta, do = (padf(x) for x in (q, k, v, g, beta, do))

    # forward: chunk start states and the chunk quantities
    S = S0.copy()
    fw = []
    for i in range(n):
        sl = slice(i * C, (i + 1) * C)
        qc, kc, vc, gc, bc = q[sl], k[sl], v[sl], g[sl], beta[sl]
        G = np.cumsum(gc, axis=0)
        Gam = np.exp(G)
        gC = Gam[-1]
        Kp, Km, Qp, Kend = kc * Gam, kc / Gam, qc * Gam, kc * (gC / Gam)
        KK = Kp @ Km.T
        A = np.tril(bc[:, None] * KK, -1)
        Tm = np.linalg.inv(np.eye(C) + A)
        Y = vc - Kp @ S
        U = Tm @ (bc[:, None] * Y)
        Aqk = np.tril(Qp @ Km.T)
        fw.append((S.copy(), kc, qc, bc, Gam, gC, Kp, Km, Qp, Kend, KK, Tm, Y, U, Aqk))
        S = gC[:, None] * S + Kend.T @ U

    dq, dk_, dv_, dg, db = (np.zeros_like(x) for x in (q, k, v, g, beta))
    dS = dS_T.copy()
    for i in reversed(range(n)):
        S, kc, qc, bc, Gam, gC, Kp, Km, Qp, Kend, KK, Tm, Y, U, Aqk = fw[i]
        sl = slice(i * C, (i + 1) * C)
        dO = do[sl]
        dU = Aqk.T @ dO + Kend @ dS
        Z = Tm.T @ dU
        dY = bc[:, None] * Z
        dS_prev = gC[:, None] * dS + Qp.T @ dO - Kp.T @ dY
        dAqk = np.tril(dO @ U.T)
        dA = np.tril(-Z @ U.T, -1)
        dQp = dO @ S.T + dAqk @ Km
        dKp = -dY @ S.T + (bc[:, None] * dA) @ Km
        dKm = dAqk.T @ Qp + (bc[:, None] * dA).T @ Kp
        dKend = U @ dS.T
        dgC = np.sum(dS * S, axis=1)
        db[sl] = np.sum(dA * KK, axis=1) + np.sum(Z * Y, axis=1)
        dv_[sl] = dY
        # through K+ = K Gamma, K- = K / Gamma, Q+ = Q Gamma, Kend = K Gamma_C / Gamma, Gamma_C
        dk_[sl] = dKp * Gam + dKm / Gam + dKend * (gC / Gam)
        dq[sl] = dQp * Gam
        dG = dKp * Kp - dKm * Km + dQp * Qp - dKend * Kend
        dG[-1] += np.sum(dKend * Kend, axis=0) + dgC * gC
        dg[sl] = np.cumsum(dG[::-1], axis=0)[::-1]      # G = cumsum(g) within the chunk
        dS = dS_prev
    return {"dq": dq[:T], "dk": dk_[:T], "dv": dv_[:T], "dg": dg[:T], "dbeta": db[:T], "dS0": dS}


@pytest.mark.parametrize("T,gmin", [(53, -3.0), (64, -5.0), (7, -1.0)])
def test_chunked_backward_matches_token_oracle(oracle_mod, T, gmin):
    rng = np.random.default_rng(T)
    B, H, dk, dv = 1, 2, 6, 5
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = gmin * rng.random((B, T, H, dk))
    beta = rng.random((B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.3
    do = rng.standard_normal((B, T, H, dv))
    dS_T = rng.standard_normal((B, H, dk, dv))
    ref = oracle_mod.backward(q, k, v, g, beta, S0, do, dS_T)
    for h in range(H):
        got = chunked_backward_head(q[0, :, h], k[0, :, h], v[0, :, h], g[0, :, h], beta[0, :, h],
                                    S0[0, h], do[0, :, h], dS_T[0, h])
        for key, r in (("dq", ref["dq"][0, :, h]), ("dk", ref["dk"][0, :, h]), ("dv", ref["dv"][0, :, h]),
                       ("dg", ref["dg"][0, :, h]), ("dbeta", ref["dbeta"][0, :, h]), ("dS0", ref["dS0"][0, h])):
            scale = max(1.0, np.abs(r).max())
            np.testing.assert_allclose(got[key], r, rtol=0, atol=1e-10 * scale, err_msg=f"{key} head {h}")
