"""Pins of the oracle's backward pass (CPU only).

The scalar is L = sum_t <do_t, o_t> + <dS_T, S_T>.  Its gradients from
oracle.backward / oracle.chunk_bwd are checked against central finite
differences of L through the forward oracle (an independent computation),
against closed forms derived by hand for one token and for beta = 0, and for
linearity in the incoming gradients (do, dS_T).
"""
import numpy as np
import pytest


def _case(seed, B=1, T=7, H=2, dk=3, dv=4, s0=True):
    rng = np.random.default_rng(seed)
    x = {
        "q": rng.standard_normal((B, T, H, dk)),
        "k": rng.standard_normal((B, T, H, dk)) / np.sqrt(dk),
        "v": rng.standard_normal((B, T, H, dv)),
        "g": -3.0 * rng.random((B, T, H, dk)),
        "beta": rng.random((B, T, H)),
        "S0": rng.standard_normal((B, H, dk, dv)) if s0 else None,
    }
    do = rng.standard_normal((B, T, H, dv))
    dS_T = rng.standard_normal((B, H, dk, dv))
    return x, do, dS_T


def _loss(oracle_mod, x, do, dS_T):
    o, S_T = oracle_mod.recurrence(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"])
    return float((o * do).sum() + (S_T * dS_T).sum())


@pytest.mark.parametrize("seed", [0, 1])
def test_backward_matches_finite_differences(oracle_mod, seed):
    x, do, dS_T = _case(seed)
    grads = oracle_mod.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], do, dS_T)
    h = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"), ("S0", "dS0")):
        base = x[name]
        fd = np.empty_like(base)
        for idx in np.ndindex(base.shape):
            xp = dict(x)
            a = base.copy()
            a[idx] += h
            xp[name] = a
            lp = _loss(oracle_mod, xp, do, dS_T)
            a = base.copy()
            a[idx] -= h
            xp[name] = a
            lm = _loss(oracle_mod, xp, do, dS_T)
            fd[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(grads[gname], fd, rtol=1e-6, atol=1e-7, err_msg=name)


def test_theta_gradient_through_the_gate(oracle_mod):
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 1, 6, 1, 3, 2
    q, k, v = (rng.standard_normal((B, T, H, d)) for d in (dk, dk, dv))
    th = rng.standard_normal((B, T, H, dk)) * 2.0
    beta = rng.random((B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    do, dS_T = rng.standard_normal((B, T, H, dv)), rng.standard_normal((B, H, dk, dv))
    grads = oracle_mod.chunk_bwd(q, k, v, th, beta, S0, do, dS_T)

    def L(t):
        o, S_T = oracle_mod.chunk_fwd(q, k, v, t, beta, S0)
        return float((o * do).sum() + (S_T * dS_T).sum())

    h = 1e-6
    fd = np.empty_like(th)
    for idx in np.ndindex(th.shape):
        a, b = th.copy(), th.copy()
        a[idx] += h
        b[idx] -= h
        fd[idx] = (L(a) - L(b)) / (2 * h)
    np.testing.assert_allclose(grads["dtheta"], fd, rtol=1e-6, atol=1e-8)


def test_one_token_closed_form(oracle_mod):
    # T = 1, S0 = 0: the decayed state is 0, u = beta v, S = beta k v^T, o = beta (k.q) v.
    # With L = <do, o> + <dS_T, S>:
    #   dq = beta (do.v) k;  dv = beta ((k.q) do + dS_T^T k);  dbeta = (k.q)(do.v) + k^T dS_T v;
    #   dk = beta ((do.v) q + dS_T v);  dg = 0;
    #   dS0 = Diag(e^g) (dS - beta k (dS^T k)^T) with dS = q do^T + dS_T.
    rng = np.random.default_rng(9)
    dk, dv = 3, 4
    q, k = rng.standard_normal(dk), rng.standard_normal(dk)
    v, g = rng.standard_normal(dv), -rng.random(dk)
    beta = 0.7
    do, dS_T = rng.standard_normal(dv), rng.standard_normal((dk, dv))
    r = lambda a, d: a.reshape(1, 1, 1, d)
    out = oracle_mod.backward(r(q, dk), r(k, dk), r(v, dv), r(g, dk), np.full((1, 1, 1), beta), None,
                              r(do, dv), dS_T.reshape(1, 1, dk, dv))
    kq, dov = k @ q, do @ v
    np.testing.assert_allclose(out["dq"].ravel(), beta * dov * k, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(out["dv"].ravel(), beta * (kq * do + dS_T.T @ k), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(out["dbeta"].ravel(), [kq * dov + k @ dS_T @ v], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(out["dk"].ravel(), beta * (dov * q + dS_T @ v), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(out["dg"].ravel(), 0.0, atol=0)
    dS = np.outer(q, do) + dS_T
    dS0 = np.exp(g)[:, None] * (dS - beta * np.outer(k, dS.T @ k))
    np.testing.assert_allclose(out["dS0"].reshape(dk, dv), dS0, rtol=1e-13, atol=1e-14)


def test_beta_zero_gradients(oracle_mod):
    # beta = 0: nothing is written, o_t = S0^T (exp(Ghat_t) q_t) with Ghat the running sum of g.
    # So dk = dv = 0 and dS0 = sum_t Diag(exp(Ghat_t)) q_t do_t^T + Diag(exp(Ghat_T)) dS_T.
    x, do, dS_T = _case(3, T=9)
    x["beta"] = np.zeros_like(x["beta"])
    out = oracle_mod.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], do, dS_T)
    assert np.all(out["dk"] == 0.0) and np.all(out["dv"] == 0.0)
    Gh = np.cumsum(x["g"], axis=1)
    ref = np.einsum("bthc,bthj->bhcj", np.exp(Gh) * x["q"], do) + \
        np.exp(Gh[:, -1])[..., None] * dS_T
    np.testing.assert_allclose(out["dS0"], ref, rtol=1e-12, atol=1e-12)
    # dq_t = S_t do_t with S_t = Diag(exp(Ghat_t)) S0
    dq = np.einsum("bthc,bhcj,bthj->bthc", np.exp(Gh), x["S0"], do)
    np.testing.assert_allclose(out["dq"], dq, rtol=1e-12, atol=1e-12)


def test_backward_linear_in_incoming_gradients(oracle_mod):
    x, do1, dS1 = _case(11, B=2, T=20, H=2, dk=4, dv=3)
    _, do2, dS2 = _case(12, B=2, T=20, H=2, dk=4, dv=3)
    f = lambda do, dS: oracle_mod.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["S0"], do, dS)
    a, b, c = f(do1, dS1), f(do2, dS2), f(do1 + 2.0 * do2, dS1 + 2.0 * dS2)
    for key in a:
        np.testing.assert_allclose(c[key], a[key] + 2.0 * b[key], rtol=1e-11, atol=1e-11, err_msg=key)
