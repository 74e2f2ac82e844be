"""Pins of the oracle's gradients (oracle/backward.py) against central finite
differences of the C oracle's forward recurrence (oracle.forward), which
shares no code with it.  The loss is <o, do> + <S_T, ds_final>; every
element of every input is perturbed on a small fp64 case, so a dropped term,
a wrong sign or a transposed operand in any gradient fails here."""
import numpy as np
import pytest

import oracle
from oracle.backward import backward


def _case(seed, B=1, T=6, H=2, dk=3, dv=2):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    z = rng.standard_normal((B, T, H, dk))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    s0 = 0.3 * rng.standard_normal((B, H, dk, dv))
    do = rng.standard_normal((B, T, H, dv))
    dsf = rng.standard_normal((B, H, dk, dv))
    return dict(q=q, k=k, v=v, z=z, beta=beta, s0=s0), do, dsf


def _loss(x, g_min, do, dsf):
    o, s = oracle.forward(x["q"], x["k"], x["v"], x["z"], x["beta"], g_min, x["s0"], nthreads=1)
    return float(np.sum(o * do) + np.sum(s * dsf))


@pytest.mark.parametrize("seed,g_min", [(0, -5.0), (1, -1.5), (2, -0.3)])
def test_gradients_match_finite_differences(seed, g_min):
    x, do, dsf = _case(seed)
    g = backward(x["q"], x["k"], x["v"], x["z"], x["beta"], g_min, x["s0"], do, dsf)
    h = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("z", "dz"), ("beta", "dbeta"), ("s0", "ds0")):
        base = x[name]
        fd = np.empty_like(base)
        for idx in np.ndindex(base.shape):
            xp = dict(x)
            a = base.copy()
            a[idx] += h
            xp[name] = a
            lp = _loss(xp, g_min, do, dsf)
            a = base.copy()
            a[idx] -= h
            xp[name] = a
            lm = _loss(xp, g_min, do, dsf)
            fd[idx] = (lp - lm) / (2 * h)
        err = np.max(np.abs(fd - g[gname])) / max(np.max(np.abs(fd)), 1e-12)
        assert err < 1e-6, (name, err)


def test_no_decay_no_write_passes_gradients_through():
    """With alpha = 1 (z -> -inf) and beta = 0 the state is constant:
    o_t = S0^T q_t, so dq_t = S0 do_t, ds0 = ds_final + sum_t q_t do_t^T,
    dk = dv = dz = 0, and dbeta_t = (D_t^T k_t) . (v_t - S0^T k_t) with
    D_t = ds_final + sum_{tau >= t} q_tau do_tau^T (the write's first-order
    effect)."""
    x, do, dsf = _case(3)
    x["z"] = np.full_like(x["z"], -60.0)
    x["beta"] = np.zeros_like(x["beta"])
    g = backward(x["q"], x["k"], x["v"], x["z"], x["beta"], -5.0, x["s0"], do, dsf)
    S0 = x["s0"][0]
    for t in range(x["q"].shape[1]):
        for h in range(x["q"].shape[2]):
            np.testing.assert_allclose(g["dq"][0, t, h], S0[h] @ do[0, t, h], rtol=1e-12, atol=1e-12)
    expect = dsf[0] + np.einsum("thi,thj->hij", x["q"][0], do[0])
    np.testing.assert_allclose(g["ds0"][0], expect, rtol=1e-12, atol=1e-12)
    for n in ("dk", "dv"):
        assert np.max(np.abs(g[n])) < 1e-12, n
    assert np.max(np.abs(g["dz"])) < 1e-20
    T, H = x["q"].shape[1:3]
    for h in range(H):
        D = dsf[0, h].copy()
        for t in range(T - 1, -1, -1):
            D += np.outer(x["q"][0, t, h], do[0, t, h])
            kt = x["k"][0, t, h]
            w = x["v"][0, t, h] - S0[h].T @ kt
            np.testing.assert_allclose(g["dbeta"][0, t, h], (D.T @ kt) @ w, rtol=1e-12, atol=1e-12)
