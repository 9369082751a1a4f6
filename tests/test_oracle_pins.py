"""Pins for the fp64 oracle (CPU only).

Each test checks the oracle against something other than itself: hand-derived
values, closed forms of special cases, invariants of the recurrence, an
independent parallel (attention-like) form solved with a triangular solver,
and the numeric bound the pages state for the gate.  The recurrence is the
gated delta rule of the "Kimi K3" explainer ("Across the sequence"); the gate
is the bounded scaled sigmoid of "Architecture Deep Dive: Kimi K3...",
section 3.2, equation 1.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
import torch

from chunked_gated_delta_12_amd import inputs as kin

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.json")


def _num(x):
    if isinstance(x, str):
        assert x == "-ln2"
        return -math.log(2.0)
    return float(x)


def _rand_case(rng, B, T, H, dk, dv, theta_sigma=2.0, s0=True, beta=None):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    theta = rng.standard_normal((B, T, H, dk)) * theta_sigma
    b = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H)))) if beta is None else np.full((B, T, H), beta)
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.3 if s0 else None
    return q, k, v, theta, b, S0


# ----------------------------------------------------------------------------- hand examples
@pytest.mark.parametrize("ex", json.load(open(GOLDEN))["examples"], ids=lambda e: e["name"])
def test_hand_examples(oracle_mod, ex):
    toks = ex["tokens"]
    T = len(toks)
    q = np.array([[t["q"]] for t in toks], dtype=np.float64)[None]      # [1, T, 1, 2]
    k = np.array([[t["k"]] for t in toks], dtype=np.float64)[None]
    v = np.array([[t["v"]] for t in toks], dtype=np.float64)[None]
    g = np.array([[[_num(x) for x in t["g"]]] for t in toks])[None]
    beta = np.array([[t["beta"]] for t in toks], dtype=np.float64)[None]
    o, S_T = oracle_mod.recurrence(q, k, v, g, beta)
    assert o.shape == (1, T, 1, 2)
    np.testing.assert_allclose(o[0, :, 0, :], np.array(ex["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(S_T[0, 0], np.array(ex["S_T"]), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- gate
def test_gate_special_values(oracle_mod):
    # sigmoid(0) = 1/2, sigmoid(+-ln 3) = 3/4 and 1/4 exactly; g = -5 * sigmoid.
    th = np.array([0.0, math.log(3.0), -math.log(3.0), 60.0, -60.0])
    g = oracle_mod.gate(th)
    np.testing.assert_allclose(g[:3], [-2.5, -3.75, -1.25], rtol=0, atol=1e-15)
    assert abs(g[3] + 5.0) < 1e-15          # saturates at the lower bound g_min = -5
    assert -1e-25 < g[4] <= 0.0             # and at 0 from below


def test_gate_range_and_monotone(oracle_mod):
    th = np.linspace(-30, 30, 2001)
    g = oracle_mod.gate(th)
    assert np.all(g <= 0.0) and np.all(g >= -5.0)
    assert np.all(np.diff(g) < 0)           # larger theta -> stronger forgetting
    # odd symmetry of the sigmoid about 1/2: g(x) + g(-x) = g_min
    np.testing.assert_allclose(g + g[::-1], -5.0, rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------- unbounded gate
# The ablation of the bound: the conventional log-decay -softplus(theta) ("Kimi K3 Deep
# Dive...", "The Design: Putting a Lower Bound on Log-Decay").
def test_softplus_gate_special_values(oracle_mod):
    # 1 + e^theta = 2, e, 4, 4/3 at theta = 0, ln(e - 1), ln 3, -ln 3
    th = np.array([0.0, math.log(math.e - 1.0), math.log(3.0), -math.log(3.0), 800.0, -800.0])
    g = oracle_mod.gate_softplus(th)
    np.testing.assert_allclose(g[:4], [-math.log(2.0), -1.0, -math.log(4.0), -math.log(4.0 / 3.0)],
                               rtol=0, atol=1e-15)
    assert g[4] == -800.0                   # no overflow of e^theta, and no lower bound
    assert -1e-300 < g[5] <= 0.0            # vanishing forgetting for very negative theta


def test_softplus_gate_identity_and_unbounded(oracle_mod):
    th = np.linspace(-40, 40, 1601)
    g = oracle_mod.gate_softplus(th)
    # softplus(x) - softplus(-x) = x
    np.testing.assert_allclose(g - g[::-1], -th, rtol=0, atol=1e-13)
    assert np.all(g <= 0.0) and np.all(np.diff(g) < 0)
    # below every bound: g <= -theta for theta > 0, and equal to -theta up to e^-theta
    pos = th > 0
    assert np.all(g[pos] <= -th[pos])
    np.testing.assert_allclose(g[th >= 35], -th[th >= 35], rtol=0, atol=1e-14)
    # agrees with an independent library softplus, ln(e^0 + e^theta)
    np.testing.assert_allclose(g, -np.logaddexp(0.0, th), rtol=1e-15, atol=1e-15)


def test_unbounded_gate_breaks_the_bf16_bound(oracle_mod):
    """With the unbounded gate a 16-token inverse decay exceeds bf16 on the decay-stress
    workload's gate inputs (theta ~ N(8, 1), g ~ -8 per token), which is why its diagonal
    tiles need the position-wise path; the bounded gate keeps the same inputs within e^80."""
    w = kin.scaled(kin.WORKLOADS["decay_stress"], T=512, H=4)
    th = kin.chunk_inputs(w)["theta"]
    G = oracle_mod.gate_cumsum(oracle_mod.gate_softplus(th))
    assert -G.min() > math.log(torch.finfo(torch.bfloat16).max)
    assert oracle_mod.gate_cumsum(oracle_mod.gate(th)).min() >= -80.0


def test_unbounded_beta_zero_is_pure_decay(oracle_mod):
    # beta = 0: o_t = S0^T (exp(Ghat_t) * q_t), Ghat the sum of -softplus(theta) from the
    # sequence start (numpy's logaddexp as the softplus)
    rng = np.random.default_rng(33)
    B, T, H, d = 1, 40, 2, 6
    q, k = rng.standard_normal((B, T, H, d)), rng.standard_normal((B, T, H, d))
    v, th = rng.standard_normal((B, T, H, d)), rng.standard_normal((B, T, H, d))
    S0 = rng.standard_normal((B, H, d, d))
    o, S_T = oracle_mod.chunk_fwd_unbounded(q, k, v, th, np.zeros((B, T, H)), S0)
    Gh = np.cumsum(-np.logaddexp(0.0, th), axis=1)
    ref = np.einsum("bhcj,bthc->bthj", S0, np.exp(Gh) * q)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S_T, np.exp(Gh[:, -1])[..., None] * S0, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------- output gate
# "Kimi K3" explainer, "Across the sequence": each attention output is scaled per
# channel and token by a sigmoid gate, o' = o * sigmoid(z).
def test_output_gate_special_values(oracle_mod):
    # sigmoid(0) = 1/2 and sigmoid(+-ln 3) = 3/4, 1/4; the far tails give o and 0
    o = np.array([2.0, -4.0, 8.0, 3.0, -7.0])
    z = np.array([0.0, math.log(3.0), -math.log(3.0), 800.0, -800.0])
    out = oracle_mod.output_gate(o, z)
    np.testing.assert_allclose(out, [1.0, -3.0, 2.0, 3.0, 0.0], rtol=0, atol=1e-14)
    assert out[0] == 1.0 and out[3] == 3.0 and out[4] == 0.0


def test_output_gate_symmetry_and_monotone(oracle_mod):
    rng = np.random.default_rng(21)
    o = rng.standard_normal((3, 5, 2, 8))
    z = rng.standard_normal((3, 5, 2, 8)) * 4.0
    # sigmoid(z) + sigmoid(-z) = 1, so the two gated outputs add back to o
    np.testing.assert_allclose(oracle_mod.output_gate(o, z) + oracle_mod.output_gate(o, -z), o,
                               rtol=0, atol=1e-14)
    # for a fixed positive output the gated value rises with z and stays in (0, o)
    zs = np.linspace(-30, 30, 601)
    g = oracle_mod.output_gate(np.full_like(zs, 2.5), zs)
    assert np.all(np.diff(g) > 0) and np.all(g > 0) and np.all(g < 2.5)


def test_output_gate_after_one_token_by_hand(oracle_mod):
    # One token, d_k = d_v = 2, S0 = I, g = 0, beta = 1, k = (1, 0), v = (3, 5),
    # q = (1, 1):  u = v - S^T k = (2, 5);  S = I + k u^T = [[3, 5], [0, 1]];
    # o = S^T q = (3, 6).  With z = (0, ln 3) the gated output is (1.5, 4.5); the
    # state is the gate-free one.
    q = np.array([1.0, 1.0]).reshape(1, 1, 1, 2)
    k = np.array([1.0, 0.0]).reshape(1, 1, 1, 2)
    v = np.array([3.0, 5.0]).reshape(1, 1, 1, 2)
    g = np.zeros((1, 1, 1, 2))
    beta = np.ones((1, 1, 1))
    S0 = np.eye(2).reshape(1, 1, 2, 2)
    o, S_T = oracle_mod.recurrence(q, k, v, g, beta, S0)
    z = np.array([0.0, math.log(3.0)]).reshape(1, 1, 1, 2)
    np.testing.assert_allclose(oracle_mod.output_gate(o, z)[0, 0, 0], [1.5, 4.5], rtol=0, atol=1e-14)
    np.testing.assert_allclose(S_T[0, 0], [[3.0, 5.0], [0.0, 1.0]], rtol=0, atol=1e-15)


def test_gate_cumsum_restarts_every_16(oracle_mod):
    B, T, H, dk = 2, 40, 3, 4          # 2.5 chunks: ragged tail
    g = -np.ones((B, T, H, dk))
    G = oracle_mod.gate_cumsum(g)
    expect = -(np.arange(T) % 16 + 1.0)
    np.testing.assert_array_equal(G, np.broadcast_to(expect[None, :, None, None], G.shape))
    rng = np.random.default_rng(0)
    g = -5 * rng.random((B, T, H, dk))
    G = oracle_mod.gate_cumsum(g)
    starts = np.arange(0, T, 16)
    np.testing.assert_array_equal(G[:, starts], g[:, starts])
    inner = np.array([t for t in range(T) if t % 16])
    np.testing.assert_allclose(G[:, inner] - G[:, inner - 1], g[:, inner], atol=1e-14)


# ----------------------------------------------------------------------------- closed forms
def test_beta_zero_is_pure_decay(oracle_mod):
    """beta = 0: nothing is written; o_t = S0^T (exp(Gh_t) * q_t), S_T = Diag(exp(Gh_T)) S0,
    with Gh the cumulative log-decay from the sequence start."""
    rng = np.random.default_rng(1)
    q, k, v, theta, _, S0 = _rand_case(rng, 2, 23, 3, 8, 5)
    beta = np.zeros(q.shape[:3])
    o, S_T = oracle_mod.chunk_fwd(q, k, v, theta, beta, S0)
    Gh = np.cumsum(-5.0 / (1.0 + np.exp(-theta)), axis=1)            # [B,T,H,dk]
    o_cf = np.einsum("bhij,bthi->bthj", S0, np.exp(Gh) * q)
    S_cf = np.exp(Gh[:, -1])[..., None] * S0
    np.testing.assert_allclose(o, o_cf, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S_T, S_cf, rtol=1e-12, atol=1e-13)


def test_disjoint_onehot_keys_reduce_to_decayed_linear_attention(oracle_mod):
    """k_s = e_{c_s} with distinct channels and S0 = 0: the delta correction vanishes and
    o_t = sum_{s<=t} beta_s q_t[c_s] exp(Gh_t[c_s] - Gh_s[c_s]) v_s."""
    rng = np.random.default_rng(2)
    B, T, H, dk, dv = 1, 12, 2, 16, 6
    q, _, v, theta, beta, _ = _rand_case(rng, B, T, H, dk, dv, s0=False)
    k = np.zeros((B, T, H, dk))
    chans = np.stack([rng.permutation(dk)[:T] for _ in range(H)], axis=1)   # [T, H]
    for t in range(T):
        for h in range(H):
            k[0, t, h, chans[t, h]] = 1.0
    o, _ = oracle_mod.chunk_fwd(q, k, v, theta, beta)
    Gh = np.cumsum(-5.0 / (1.0 + np.exp(-theta)), axis=1)
    o_cf = np.zeros_like(o)
    for h in range(H):
        for t in range(T):
            for s in range(t + 1):
                c = chans[s, h]
                w = beta[0, s, h] * q[0, t, h, c] * math.exp(Gh[0, t, h, c] - Gh[0, s, h, c])
                o_cf[0, t, h] += w * v[0, s, h]
    np.testing.assert_allclose(o, o_cf, rtol=1e-12, atol=1e-13)


def test_k_orthogonal_components_only_decay(oracle_mod):
    """Channels that no key touches are only forgotten: row c of S_T = exp(Gh_T[c]) S0[c]."""
    rng = np.random.default_rng(3)
    q, k, v, theta, beta, S0 = _rand_case(rng, 1, 30, 2, 10, 7)
    untouched = [1, 4, 8]
    k[..., untouched] = 0.0
    _, S_T = oracle_mod.chunk_fwd(q, k, v, theta, beta, S0)
    Gh = np.cumsum(-5.0 / (1.0 + np.exp(-theta)), axis=1)
    for c in untouched:
        np.testing.assert_allclose(S_T[:, :, c, :], np.exp(Gh[:, -1, :, c])[..., None] * S0[:, :, c, :],
                                   rtol=1e-12, atol=1e-14)


def test_single_step_orthogonal_direction(oracle_mod):
    """For one token and any x orthogonal to k: x^T S_1 = x^T Diag(exp(g)) S0."""
    rng = np.random.default_rng(4)
    q, k, v, theta, beta, S0 = _rand_case(rng, 1, 1, 1, 9, 4)
    kk = k[0, 0, 0]
    x = rng.standard_normal(9)
    x -= kk * (x @ kk)
    _, S1 = oracle_mod.chunk_fwd(q, k, v, theta, beta, S0)
    a = np.exp(-5.0 / (1.0 + np.exp(-theta[0, 0, 0])))
    np.testing.assert_allclose(x @ S1[0, 0], x @ (a[:, None] * S0[0, 0]), rtol=1e-12, atol=1e-13)


def test_single_step_closed_form(oracle_mod):
    """T = 1: o = (D S0)^T q + beta (k.q) (v - (D S0)^T k), D = Diag(exp(g))."""
    rng = np.random.default_rng(5)
    q, k, v, theta, beta, S0 = _rand_case(rng, 3, 1, 2, 6, 5)
    o, _ = oracle_mod.chunk_fwd(q, k, v, theta, beta, S0)
    for b in range(3):
        for h in range(2):
            D = np.exp(-5.0 / (1.0 + np.exp(-theta[b, 0, h])))
            DS = D[:, None] * S0[b, h]
            qq, kk, vv, bb = q[b, 0, h], k[b, 0, h], v[b, 0, h], beta[b, 0, h]
            expect = DS.T @ qq + bb * (kk @ qq) * (vv - DS.T @ kk)
            np.testing.assert_allclose(o[b, 0, h], expect, rtol=1e-12, atol=1e-13)


def test_read_back_after_full_write(oracle_mod):
    """beta = 1 and |k| = 1: the state returns v_t for k_t right after writing it (q_t = k_t)."""
    rng = np.random.default_rng(6)
    _, k, v, theta, _, S0 = _rand_case(rng, 2, 25, 2, 12, 6)
    beta = np.ones(k.shape[:3])
    o, _ = oracle_mod.chunk_fwd(k, k, v, theta, beta, S0)
    np.testing.assert_allclose(o, v, rtol=1e-11, atol=1e-12)


def test_associative_recall_orthonormal_keys(oracle_mod):
    """No forgetting (g = 0), beta = 1, orthonormal keys: S_m^T k_j = v_j for every j."""
    rng = np.random.default_rng(7)
    dk, dv, m = 16, 5, 11
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:, :m].T                                   # m orthonormal rows
    k = keys[None, :, None, :]
    v = rng.standard_normal((1, m, 1, dv))
    q = rng.standard_normal((1, m, 1, dk))
    g = np.zeros((1, m, 1, dk))
    beta = np.ones((1, m, 1))
    _, S_T = oracle_mod.recurrence(q, k, v, g, beta)
    np.testing.assert_allclose(keys @ S_T[0, 0], v[0, :, 0, :], rtol=1e-12, atol=1e-12)


def _parallel_form(q, k, v, g, beta, S0):
    """Whole-sequence closed form: with Gamma = exp(cumsum g) from the sequence start,
    K+ = K*Gamma, K- = K/Gamma, Q+ = Q*Gamma,
    (I + StrictLower(diag(beta) K+ K-^T)) U = diag(beta)(V - K+ S0),
    O = Q+ S0 + LowerIncl(Q+ K-^T) U,   S_T = Diag(Gamma_T) S0 + (K*Gamma_T/Gamma)^T U."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    O = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            Gam = np.exp(np.cumsum(g[b, :, h], axis=0))          # [T, dk]
            K, Q, V = k[b, :, h], q[b, :, h], v[b, :, h]
            Kp, Km, Qp = K * Gam, K / Gam, Q * Gam
            S = S0[b, h] if S0 is not None else np.zeros((dk, dv))
            A = np.tril(beta[b, :, h][:, None] * (Kp @ Km.T), -1)
            rhs = beta[b, :, h][:, None] * (V - Kp @ S)
            U = scipy.linalg.solve_triangular(np.eye(T) + A, rhs, lower=True, unit_diagonal=True)
            O[b, :, h] = Qp @ S + np.tril(Qp @ Km.T) @ U
            ST[b, h] = Gam[-1][:, None] * S + (K * (Gam[-1] / Gam)).T @ U
    return O, ST


@pytest.mark.parametrize("s0", [False, True])
def test_parallel_form(oracle_mod, s0):
    rng = np.random.default_rng(8 + s0)
    q, k, v, theta, beta, S0 = _rand_case(rng, 2, 37, 2, 8, 5, s0=s0)
    g = oracle_mod.gate(theta)
    o, S_T = oracle_mod.recurrence(q, k, v, g, beta, S0)
    o_pf, S_pf = _parallel_form(q, k, v, g, beta, S0)
    scale_o, scale_s = np.abs(o_pf).max(), np.abs(S_pf).max()
    assert np.abs(o - o_pf).max() <= 1e-10 * scale_o
    assert np.abs(S_T - S_pf).max() <= 1e-10 * scale_s


# ----------------------------------------------------------------------------- structure
def test_linear_in_state_and_values(oracle_mod):
    rng = np.random.default_rng(10)
    q, k, v, theta, beta, S0 = _rand_case(rng, 1, 20, 2, 8, 6)
    v2 = rng.standard_normal(v.shape)
    S02 = rng.standard_normal(S0.shape)
    a, c = 0.7, -1.3
    o1, s1 = oracle_mod.chunk_fwd(q, k, v, theta, beta, S0)
    o2, s2 = oracle_mod.chunk_fwd(q, k, v2, theta, beta, S02)
    o3, s3 = oracle_mod.chunk_fwd(q, k, a * v + c * v2, theta, beta, a * S0 + c * S02)
    np.testing.assert_allclose(o3, a * o1 + c * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s3, a * s1 + c * s2, rtol=1e-11, atol=1e-12)


def test_column_subset_matches_full(oracle_mod):
    rng = np.random.default_rng(11)
    q, k, v, theta, beta, S0 = _rand_case(rng, 2, 33, 2, 8, 9)
    o, S_T = oracle_mod.chunk_fwd(q, k, v, theta, beta, S0)
    cols = [7, 0, 4]
    oc, Sc = oracle_mod.chunk_fwd(q, k, v, theta, beta, S0, cols=cols)
    np.testing.assert_array_equal(oc, o[..., cols])
    np.testing.assert_array_equal(Sc, S_T[..., cols])


def test_split_and_resume(oracle_mod):
    rng = np.random.default_rng(12)
    q, k, v, theta, beta, S0 = _rand_case(rng, 1, 50, 3, 8, 4)
    o, S_T = oracle_mod.chunk_fwd(q, k, v, theta, beta, S0)
    for T1 in (1, 16, 23):
        o1, S1 = oracle_mod.chunk_fwd(q[:, :T1], k[:, :T1], v[:, :T1], theta[:, :T1], beta[:, :T1], S0)
        o2, S2 = oracle_mod.chunk_fwd(q[:, T1:], k[:, T1:], v[:, T1:], theta[:, T1:], beta[:, T1:], S1)
        np.testing.assert_allclose(np.concatenate([o1, o2], axis=1), o, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(S2, S_T, rtol=1e-13, atol=1e-14)


def test_heads_and_batches_independent(oracle_mod):
    rng = np.random.default_rng(13)
    q, k, v, theta, beta, S0 = _rand_case(rng, 2, 17, 4, 8, 4)
    o, S_T = oracle_mod.chunk_fwd(q, k, v, theta, beta, S0)
    p = [2, 0, 3, 1]
    op, Sp = oracle_mod.chunk_fwd(q[:, :, p], k[:, :, p], v[:, :, p], theta[:, :, p], beta[:, :, p], S0[:, p])
    np.testing.assert_array_equal(op, o[:, :, p])
    np.testing.assert_array_equal(Sp, S_T[:, p])
    ob, Sb = oracle_mod.chunk_fwd(q[1:], k[1:], v[1:], theta[1:], beta[1:], S0[1:])
    np.testing.assert_array_equal(ob, o[1:])


def test_decode_step_is_one_token_of_the_recurrence(oracle_mod):
    rng = np.random.default_rng(14)
    q, k, v, theta, beta, S0 = _rand_case(rng, 3, 1, 2, 8, 6)
    o_d, S_d = oracle_mod.decode_step(q[:, 0], k[:, 0], v[:, 0], theta[:, 0], beta[:, 0], S0)
    o_r, S_r = oracle_mod.chunk_fwd(q, k, v, theta, beta, S0)
    np.testing.assert_array_equal(o_d, o_r[:, 0])
    np.testing.assert_array_equal(S_d, S_r)


# ----------------------------------------------------------------------------- the bound
def test_bf16_bound_on_16_token_inverse_decay():
    """With g >= -5 a 16-token cumulative log-decay is >= -80, and exp(80) fits bf16
    but not fp16 ("Architecture Deep Dive: Kimi K3...", section 3.2)."""
    e80 = math.exp(80.0)
    assert e80 < torch.finfo(torch.bfloat16).max
    assert math.exp(-80.0) > torch.finfo(torch.bfloat16).tiny        # normal, not subnormal
    assert math.exp(-80.0) > torch.finfo(torch.float32).tiny
    assert e80 > torch.finfo(torch.float16).max                      # fp16 inputs are rejected
    assert torch.isfinite(torch.tensor(e80, dtype=torch.float32).to(torch.bfloat16))


@pytest.mark.parametrize("name", ["tiny", "small", "prefill_64k", "decay_stress", "long_memory"])
def test_workload_chunk_decay_within_bound(oracle_mod, name):
    w = kin.scaled(kin.WORKLOADS[name], T=min(kin.WORKLOADS[name].T, 512), B=1)
    th = kin.chunk_inputs(w)["theta"]
    G = oracle_mod.gate_cumsum(oracle_mod.gate(th))
    assert G.min() >= -80.0
    if name == "decay_stress":   # sigma(8 +- 1): most chunks come within 1% of the bound
        assert G.min() < -79.0
    if name == "long_memory":    # most channels keep more than 90% of the state over a chunk
        assert float((G[:, 15::16] > -0.1).mean()) > 0.9


# ----------------------------------------------------------------------------- brute force
def _expanded_products(q, k, v, g, beta, S0):
    """The recurrence written as a sum of products of per-token transition matrices,
    vectorised over a batch of independent sequences ([N, T, d] arrays, S0 [N, d, d]).
    Decay, read and write of one token combine into S_t = M_t S_{t-1} + beta_t k_t v_t^T
    with M_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)), hence
        S_t = P_{t,0} S0 + sum_{s<=t} P_{t,s} beta_s k_s v_s^T,  P_{t,s} = M_t ... M_{s+1},
    and o_t = S_t^T q_t.  Every product P_{t,s} is formed explicitly."""
    N, T, d = q.shape
    eye = np.broadcast_to(np.eye(d), (N, d, d))
    M = [(eye - beta[:, t, None, None] * np.einsum("ni,nj->nij", k[:, t], k[:, t]))
         @ (np.exp(g[:, t])[:, None, :] * eye) for t in range(T)]
    o = np.empty((N, T, d))
    S = None
    for t in range(T):
        P = eye.copy()                      # P_{t,t}
        S = np.zeros((N, d, d))
        for s in range(t, -1, -1):
            S = S + P @ (beta[:, s, None, None] * np.einsum("ni,nj->nij", k[:, s], v[:, s]))
            P = P @ M[s]                    # P_{t,s-1}
        S = S + P @ S0                      # P_{t,0} S0
        o[:, t] = np.einsum("nij,ni->nj", S, q[:, t])
    return o, S


def test_brute_force_grid_against_expanded_products(oracle_mod):
    """Every combination, at each of 4 tokens with d = 2, of the per-channel log-decay
    g in {0, -ln 2, -5} and beta in {0, 1/2, 1} (27^4 = 531,441 sequences), with fixed
    non-orthogonal keys, values, queries and a non-zero start state: the oracle's
    outputs and final state match the expanded-product form to 1e-12."""
    levels_g = [0.0, -math.log(2.0), -5.0]
    levels_b = [0.0, 0.5, 1.0]
    per_tok = [(g0, g1, b) for g0 in levels_g for g1 in levels_g for b in levels_b]   # 27
    T, d = 4, 2
    idx = np.stack(np.meshgrid(*[np.arange(27)] * T, indexing="ij"), -1).reshape(-1, T)
    tab = np.array(per_tok)                                  # [27, 3]
    N = idx.shape[0]
    g = tab[idx][..., :2]                                    # [N, T, 2]
    beta = tab[idx][..., 2]                                  # [N, T]
    keys = np.array([[1.0, 0.0], [0.6, 0.8], [0.0, 1.0], [0.8, -0.6]])
    vals = np.array([[2.0, 3.0], [4.0, -2.0], [1.0, 1.0], [-3.0, 0.5]])
    qs = np.array([[1.0, 1.0], [2.0, 1.0], [1.0, 0.0], [-1.0, 2.0]])
    k = np.broadcast_to(keys, (N, T, d)).copy()
    v = np.broadcast_to(vals, (N, T, d)).copy()
    q = np.broadcast_to(qs, (N, T, d)).copy()
    S0 = np.broadcast_to(np.array([[0.5, -1.0], [2.0, 0.25]]), (N, d, d)).copy()
    o, S_T = oracle_mod.recurrence(q[:, :, None], k[:, :, None], v[:, :, None], g[:, :, None],
                                   beta[:, :, None], S0[:, None])
    o_x, S_x = _expanded_products(q, k, v, g, beta, S0)
    np.testing.assert_allclose(o[:, :, 0], o_x, rtol=0, atol=1e-12 * np.abs(o_x).max())
    np.testing.assert_allclose(S_T[:, 0], S_x, rtol=0, atol=1e-12 * np.abs(S_x).max())
    # the grid reaches the special cases: beta = 0 everywhere leaves only decay
    nowrite = np.all(beta == 0, axis=1)
    decay = np.exp(g.sum(axis=1))                            # [N, 2]
    np.testing.assert_allclose(S_T[nowrite, 0], decay[nowrite][:, :, None] * S0[nowrite], rtol=1e-13)


def test_expanded_products_catch_planted_mistakes(oracle_mod):
    """The brute-force comparison fails for plausible mistakes in a recurrence: the
    decay applied after the write, or the read taken before the decay."""
    rng = np.random.default_rng(21)
    N, T, d = 64, 4, 2
    q, v = rng.standard_normal((N, T, d)), rng.standard_normal((N, T, d))
    k = rng.standard_normal((N, T, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    g = rng.choice([0.0, -math.log(2.0), -5.0], size=(N, T, d))
    beta = rng.choice([0.5, 1.0], size=(N, T))
    S0 = rng.standard_normal((N, d, d))
    o_x, _ = _expanded_products(q, k, v, g, beta, S0)

    def wrong(order):
        S = S0.copy()
        o = np.empty((N, T, d))
        for t in range(T):
            D = np.exp(g[:, t])[:, :, None]
            if order == "decay_after_write":
                u = beta[:, t, None] * (v[:, t] - np.einsum("nij,ni->nj", S, k[:, t]))
                S = D * (S + np.einsum("ni,nj->nij", k[:, t], u))
            else:   # read before decay
                u = beta[:, t, None] * (v[:, t] - np.einsum("nij,ni->nj", S, k[:, t]))
                S = D * S + np.einsum("ni,nj->nij", k[:, t], u)
            o[:, t] = np.einsum("nij,ni->nj", S, q[:, t])
        return o

    for order in ("decay_after_write", "read_before_decay"):
        assert np.abs(wrong(order) - o_x).max() > 1e-3 * np.abs(o_x).max(), order


def test_column_blocks_match_full(oracle_mod):
    """The concurrent column-block evaluation (for few sequences) equals the plain call."""
    rng = np.random.default_rng(22)
    q, k, v, theta, beta, S0 = _rand_case(rng, 1, 45, 2, 8, 12)
    o, S_T = oracle_mod.chunk_fwd(q, k, v, theta, beta, S0)
    ob, Sb = oracle_mod.chunk_fwd_column_blocks(q, k, v, theta, beta, S0, nthreads=8)
    np.testing.assert_array_equal(ob, o)
    np.testing.assert_array_equal(Sb, S_T)
