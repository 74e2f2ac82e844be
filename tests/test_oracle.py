"""Pins for the fp64 oracle: everything here is checked against something
other than the oracle itself -- the worked example printed on the "KDA
Recurrence" page, closed forms, special cases that reduce to textbook
recurrences, independent formulations of Eq. 1, and brute force.

CPU only; no GPU and no HIP library involved.
"""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import chunked

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kda_recurrence_examples.json")


def rand_inputs(rng, B, T, H, dk, dv, unit_keys=True, beta_range=(0.0, 1.0), z_scale=1.0):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    z = rng.standard_normal((B, T, H, dk)) * z_scale
    beta = rng.uniform(*beta_range, size=(B, T, H))
    return q, k, v, z, beta


def alpha_of(z, g_min):
    return np.exp(g_min / (1.0 + np.exp(-z)))


def rel(a, b):
    return np.linalg.norm(np.ravel(a - b)) / max(np.linalg.norm(np.ravel(b)), 1e-300)


# ---------------------------------------------------------------- P-1, P-2
def test_worked_example_exact():
    """"KDA Recurrence", first worked example: exact printed outputs."""
    ex = json.load(open(GOLDEN))["example_1"]
    f = lambda n: np.array(ex[n], np.float64)
    beta = f("write_strength").reshape(1, 1, 1)
    res = oracle.layer(f("query"), f("key"), f("value"), f("decay_logits"), beta,
                       f("output_gate_logits"), f("output_projection"), f("initial_state"),
                       ex["g_min"], ex["eps"])
    assert res["outputs"].shape == (1, 1, 1)
    assert res["final_state"].shape == (1, 1, 1, 1)
    assert abs(res["outputs"][0, 0, 0] - np.array(ex["outputs"]).item()) <= 1e-15
    assert res["final_state"].item() == np.array(ex["final_state"]).item()


@pytest.mark.parametrize("name", ["example_2", "example_3"])
def test_worked_example_shapes(name):
    ex = json.load(open(GOLDEN))[name]
    B, T, H, dk = ex["query_shape"]
    dv = ex["value_shape"][-1]
    rng = np.random.default_rng(3)
    q, k, v, z, beta = rand_inputs(rng, B, T, H, dk, dv)
    s0 = rng.standard_normal(ex["initial_state_shape"])
    w = rng.standard_normal(ex["output_projection_shape"])
    gate = rng.standard_normal((B, T, H, dv))
    res = oracle.layer(q, k, v, z, beta, gate, w, s0, -5.0, 1e-6)
    assert list(res["outputs"].shape) == ex["outputs_shape"]
    assert list(res["final_state"].shape) == ex["final_state_shape"]


# ---------------------------------------------------------------- P-3, P-4, P-5
def dense_eq1(q, k, v, alpha, beta, s0):
    """Eq. 1 with explicit d_k x d_k transition matrices."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    sf = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = s0[b, h].copy()
            for t in range(T):
                kt = k[b, t, h]
                Mt = (np.eye(dk) - beta[b, t, h] * np.outer(kt, kt)) @ np.diag(alpha[b, t, h])
                S = Mt @ S + beta[b, t, h] * np.outer(kt, v[b, t, h])
                o[b, t, h] = S.T @ q[b, t, h]
            sf[b, h] = S
    return o, sf


def braket(q, k, v, alpha, beta, s0):
    """Transposed (d_v x d_k) bra-ket form of the agentlenshq derivation:
    S~_t = S~_{t-1} D_t + beta_t (|v_t> - S~_{t-1} D_t |k_t>) <k_t|, o = S~ q."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    sf = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            St = s0[b, h].T.copy()
            for t in range(T):
                D = np.diag(alpha[b, t, h])
                SD = St @ D
                St = SD + beta[b, t, h] * np.outer(v[b, t, h] - SD @ k[b, t, h], k[b, t, h])
                o[b, t, h] = St @ q[b, t, h]
            sf[b, h] = St.T
    return o, sf


def dplr_bound(q, k, v, alpha, beta, s0):
    """General DPLR transition (D - a b^T) S + beta k v^T with the variable
    binding a = beta k, b = k * alpha ("Diagonal-Plus-Low-Rank Matrices and
    Kimi Delta Attention", section 3)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    sf = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = s0[b, h].copy()
            for t in range(T):
                a_vec = beta[b, t, h] * k[b, t, h]
                b_vec = k[b, t, h] * alpha[b, t, h]
                S = (np.diag(alpha[b, t, h]) - np.outer(a_vec, b_vec)) @ S \
                    + beta[b, t, h] * np.outer(k[b, t, h], v[b, t, h])
                o[b, t, h] = S.T @ q[b, t, h]
            sf[b, h] = S
    return o, sf


@pytest.mark.parametrize("form", [dense_eq1, braket, dplr_bound])
@pytest.mark.parametrize("dims", [(1, 19, 2, 5, 3), (2, 33, 1, 8, 8), (1, 7, 3, 2, 6)])
def test_independent_formulations(form, dims):
    B, T, H, dk, dv = dims
    rng = np.random.default_rng(11 + dk)
    q, k, v, z, beta = rand_inputs(rng, B, T, H, dk, dv, unit_keys=False, z_scale=2.0)
    s0 = rng.standard_normal((B, H, dk, dv))
    g_min = -3.0
    o, s = oracle.forward(q, k, v, z, beta, g_min, s0)
    o2, s2 = form(q, k, v, alpha_of(z, g_min), beta, s0)
    assert rel(o, o2) < 1e-13
    assert rel(s, s2) < 1e-13


def test_dropped_erase_term_is_caught():
    """A recurrence without the erase term (plain gated linear attention)
    must differ from the oracle: guards P-3 against a vacuous comparison."""
    rng = np.random.default_rng(5)
    q, k, v, z, beta = rand_inputs(rng, 1, 9, 1, 4, 3)
    s0 = rng.standard_normal((1, 1, 4, 3))
    o, s = oracle.forward(q, k, v, z, beta, -5.0, s0)
    S = s0[0, 0].copy()
    for t in range(9):
        S = np.diag(alpha_of(z[0, t, 0], -5.0)) @ S + beta[0, t, 0] * np.outer(k[0, t, 0], v[0, t, 0])
    assert rel(s[0, 0], S) > 1e-3


# ---------------------------------------------------------------- P-6
def test_scalar_closed_form():
    """d_k = d_v = 1: S_T = sum_t [prod_{j>t} (1 - b_j k_j^2) a_j] b_t k_t v_t
    + [prod_j (1 - b_j k_j^2) a_j] S_0."""
    rng = np.random.default_rng(7)
    T = 40
    q, k, v, z, beta = rand_inputs(rng, 1, T, 1, 1, 1, unit_keys=False)
    s0 = np.array([[[[0.7]]]])
    g_min = -2.0
    a = alpha_of(z[0, :, 0, 0], g_min)
    kk, vv, bb = k[0, :, 0, 0], v[0, :, 0, 0], beta[0, :, 0]
    fac = (1 - bb * kk * kk) * a
    expect = np.prod(fac) * 0.7
    for t in range(T):
        expect += np.prod(fac[t + 1:]) * bb[t] * kk[t] * vv[t]
    o, s = oracle.forward(q, k, v, z, beta, g_min, s0)
    assert abs(s.item() - expect) <= 1e-13 * max(1.0, abs(expect))
    # readout of the last token from the updated state
    assert abs(o[0, -1, 0, 0] - s.item() * q[0, -1, 0, 0]) <= 1e-14


# ---------------------------------------------------------------- P-7
def test_beta_zero_pure_decay():
    rng = np.random.default_rng(8)
    B, T, H, dk, dv = 1, 12, 2, 6, 5
    q, k, v, z, _ = rand_inputs(rng, B, T, H, dk, dv)
    beta = np.zeros((B, T, H))
    s0 = rng.standard_normal((B, H, dk, dv))
    o, s = oracle.forward(q, k, v, z, beta, -5.0, s0)
    cum = np.cumprod(alpha_of(z, -5.0), axis=1)          # prod_{j<=t} alpha_j
    for t in range(T):
        St = cum[:, t, :, :, None] * s0                  # Diag(gamma_t) S0
        np.testing.assert_allclose(o[:, t], np.einsum("bhcj,bhc->bhj", St, q[:, t]), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(s, cum[:, -1, :, :, None] * s0, rtol=1e-13, atol=1e-300)
    # alpha == 1 (z -> -inf) and beta == 0: the state never moves
    o1, s1 = oracle.forward(q, k, v, np.full_like(z, -1e4), beta, -5.0, s0)
    assert np.array_equal(s1, s0)


# ---------------------------------------------------------------- P-8
def orthonormal_keys(rng, T, dk):
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    return Qm[:T]


def test_linear_attention_limit_orthonormal_keys():
    """alpha == 1, S0 = 0, orthonormal keys: the delta rule reduces to causal
    linear attention S_t = sum_i beta_i k_i v_i^T."""
    rng = np.random.default_rng(9)
    T, dk, dv = 10, 16, 7
    k = orthonormal_keys(rng, T, dk)[None, :, None, :]
    q = rng.standard_normal((1, T, 1, dk))
    v = rng.standard_normal((1, T, 1, dv))
    beta = rng.uniform(0.1, 1.0, (1, T, 1))
    z = np.full((1, T, 1, dk), -1e4)
    o, s = oracle.forward(q, k, v, z, beta, -5.0, None)
    S = np.zeros((dk, dv))
    for t in range(T):
        S = S + beta[0, t, 0] * np.outer(k[0, t, 0], v[0, t, 0])
        expect_o = sum(beta[0, i, 0] * (q[0, t, 0] @ k[0, i, 0]) * v[0, i, 0] for i in range(t + 1))
        np.testing.assert_allclose(o[0, t, 0], expect_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(s[0, 0], S, rtol=1e-12, atol=1e-13)


def test_linear_attention_small_beta_limit():
    """beta = eps, alpha == 1, general keys: S_t / eps -> sum_i k_i v_i^T
    with an O(eps t) relative deviation."""
    rng = np.random.default_rng(10)
    T, dk, dv = 20, 6, 4
    q, k, v, _, _ = rand_inputs(rng, 1, T, 1, dk, dv)
    z = np.full((1, T, 1, dk), -1e4)
    eps = 1e-7
    _, s = oracle.forward(q, k, v, z, np.full((1, T, 1), eps), -5.0, None)
    la = sum(np.outer(k[0, t, 0], v[0, t, 0]) for t in range(T))
    assert rel(s[0, 0] / eps, la) < 10 * eps * T


# ---------------------------------------------------------------- P-9
def test_uniform_decay_is_gated_deltanet():
    """A decay logit shared by all channels gives a scalar alpha_t: the
    recurrence becomes Gated DeltaNet, S_t = a_t (I - b k k^T) S + b k v^T."""
    rng = np.random.default_rng(12)
    B, T, H, dk, dv = 1, 25, 2, 5, 4
    q, k, v, _, beta = rand_inputs(rng, B, T, H, dk, dv)
    zs = rng.standard_normal((B, T, H, 1))
    z = np.repeat(zs, dk, axis=-1)
    s0 = rng.standard_normal((B, H, dk, dv))
    o, s = oracle.forward(q, k, v, z, beta, -4.0, s0)
    a = alpha_of(zs[..., 0], -4.0)
    for h in range(H):
        S = s0[0, h].copy()
        for t in range(T):
            kt = k[0, t, h]
            S = a[0, t, h] * (np.eye(dk) - beta[0, t, h] * np.outer(kt, kt)) @ S + beta[0, t, h] * np.outer(kt, v[0, t, h])
            np.testing.assert_allclose(o[0, t, h], S.T @ q[0, t, h], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(s[0, h], S, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- P-10
def test_delta_rule_overwrite():
    """beta = 1 and a unit key: after the step, S_t^T k_t = v_t exactly,
    whatever alpha and the previous state are."""
    rng = np.random.default_rng(13)
    dk, dv, T = 8, 5, 6
    q, k, v, z, _ = rand_inputs(rng, 1, T, 1, dk, dv)
    S = rng.standard_normal((1, 1, dk, dv))
    for t in range(T):
        _, S = oracle.forward(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], z[:, t:t + 1],
                              np.ones((1, 1, 1)), -5.0, S)
        np.testing.assert_allclose(S[0, 0].T @ k[0, t, 0], v[0, t, 0], rtol=1e-13, atol=1e-13)
    # alpha == 1, orthonormal keys, beta == 1: every written pair is retrievable
    kk = orthonormal_keys(rng, T, dk)[None, :, None, :]
    _, S = oracle.forward(q, kk, v, np.full_like(z, -1e4), np.ones((1, T, 1)), -5.0, None)
    for i in range(T):
        np.testing.assert_allclose(S[0, 0].T @ kk[0, i, 0], v[0, i, 0], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- P-11
def test_linearity_and_column_independence():
    rng = np.random.default_rng(14)
    B, T, H, dk, dv = 2, 17, 1, 6, 4
    q, k, v, z, beta = rand_inputs(rng, B, T, H, dk, dv)
    v2 = rng.standard_normal(v.shape)
    s0 = rng.standard_normal((B, H, dk, dv))
    s0b = rng.standard_normal((B, H, dk, dv))
    a, b = 0.3, -1.7
    o1, s1 = oracle.forward(q, k, v, z, beta, -5.0, s0)
    o2, s2 = oracle.forward(q, k, v2, z, beta, -5.0, s0b)
    o3, s3 = oracle.forward(q, k, a * v + b * v2, z, beta, -5.0, a * s0 + b * s0b)
    assert rel(o3, a * o1 + b * o2) < 1e-13
    assert rel(s3, a * s1 + b * s2) < 1e-13
    for j in range(dv):
        oj, sj = oracle.forward(q, k, v[..., j:j + 1].copy(), z, beta, -5.0, s0[..., j:j + 1].copy())
        assert np.array_equal(oj[..., 0], o1[..., j])
        assert np.array_equal(sj[..., 0], s1[..., j])


# ---------------------------------------------------------------- P-12
def test_split_resume():
    rng = np.random.default_rng(15)
    B, T, H, dk, dv = 1, 50, 2, 8, 8
    q, k, v, z, beta = rand_inputs(rng, B, T, H, dk, dv)
    s0 = rng.standard_normal((B, H, dk, dv))
    o, s = oracle.forward(q, k, v, z, beta, -5.0, s0)
    t1 = 23
    oa, sa = oracle.forward(q[:, :t1], k[:, :t1], v[:, :t1], z[:, :t1], beta[:, :t1], -5.0, s0)
    ob, sb = oracle.forward(q[:, t1:], k[:, t1:], v[:, t1:], z[:, t1:], beta[:, t1:], -5.0, sa)
    assert np.array_equal(np.concatenate([oa, ob], axis=1), o)
    assert np.array_equal(sb, s)


# ---------------------------------------------------------------- P-13
@pytest.mark.parametrize("chunk", [1, 2, 16, 64])
def test_chunk_form_matches_sequential(chunk):
    """Propositions 1-2 (Eqs. 16-19) evaluated chunk by chunk reproduce the
    sequential recurrence, including a ragged last chunk."""
    rng = np.random.default_rng(16)
    B, T, H, dk, dv = 1, 100, 1, 6, 5
    q, k, v, z, beta = rand_inputs(rng, B, T, H, dk, dv)
    s0 = rng.standard_normal((B, H, dk, dv))
    o, s = oracle.forward(q, k, v, z, beta, -1.0, s0)
    oc, sc = chunked.forward(q, k, v, z, beta, -1.0, s0, chunk=chunk)
    assert rel(oc, o) < 1e-12
    assert rel(sc, s) < 1e-12


def test_chunk_form_beta_placement():
    """The reading that beta_r multiplies the whole bracket of Eqs. 17/19 is
    the one consistent with Eq. 1; beta applied to the first term only is
    not (this is what the garbled render would say)."""
    rng = np.random.default_rng(17)
    C, dk, dv = 8, 4, 3
    q, k, v, z, beta = [x[0, :, 0] for x in rand_inputs(rng, 1, C, 1, dk, dv)]
    alpha = alpha_of(z, -1.0)
    S0 = rng.standard_normal((dk, dv))
    _, S_C, w, u = chunked.chunk_step(S0, q, k, v, alpha, beta)
    _, s_seq = oracle.forward(q[None, :, None], k[None, :, None], v[None, :, None],
                              z[None, :, None], beta[None, :, None], -1.0, S0[None, None])
    assert rel(S_C, s_seq[0, 0]) < 1e-13
    # literal render: w_r = beta_r gamma_r k_r - sum w_i (...), u_r likewise
    gamma = np.cumprod(alpha, axis=0)
    w2 = np.zeros_like(w)
    u2 = np.zeros_like(u)
    for r in range(C):
        w2[r] = beta[r] * gamma[r] * k[r]
        u2[r] = beta[r] * v[r]
        for i in range(r):
            coef = k[i] @ (np.prod(alpha[i + 1:r + 1], axis=0) * k[r])
            w2[r] -= w2[i] * coef
            u2[r] -= u2[i] * coef
    assert rel(w2, w) > 1e-3 and rel(u2, u) > 1e-3


# ---------------------------------------------------------------- P-14
def test_contraction_bound():
    rng = np.random.default_rng(18)
    dk, dv, T = 8, 8, 30
    q, k, v, z, beta = rand_inputs(rng, 1, T, 1, dk, dv)
    S = rng.standard_normal((1, 1, dk, dv))
    for t in range(T):
        prev = np.linalg.norm(S)
        _, S = oracle.forward(q[:, t:t + 1], k[:, t:t + 1], v[:, t:t + 1], z[:, t:t + 1],
                              beta[:, t:t + 1], -5.0, S)
        assert np.linalg.norm(S) <= prev + beta[0, t, 0] * np.linalg.norm(v[0, t, 0]) + 1e-12


# ---------------------------------------------------------------- P-15
@pytest.mark.parametrize("zval,expect", [(0.0, np.exp(-2.5)), (-1e4, 1.0), (1e4, np.exp(-5.0))])
def test_gate_values(zval, expect):
    dk, dv = 3, 2
    s0 = np.arange(1, dk * dv + 1, dtype=np.float64).reshape(1, 1, dk, dv)
    z = np.full((1, 1, 1, dk), zval)
    zero = np.zeros((1, 1, 1, dk))
    _, s = oracle.forward(zero, zero, np.zeros((1, 1, 1, dv)), z, np.zeros((1, 1, 1)), -5.0, s0)
    np.testing.assert_allclose(s, expect * s0, rtol=1e-15)


# ---------------------------------------------------------------- P-16
def test_rmsnorm_constant_and_projection():
    B, T, H, dv = 2, 3, 2, 4
    c = 0.37
    o = np.full((B, T, H, dv), c)
    gate = np.zeros((B, T, H, dv))
    y = oracle.out_gate(o, gate, 1e-6)
    np.testing.assert_allclose(y, np.full((B, T, H * dv), 0.5 * c / np.sqrt(c * c + 1e-6)), rtol=1e-15)
    rng = np.random.default_rng(19)
    o = rng.standard_normal((B, T, H, dv))
    gate = rng.standard_normal((B, T, H, dv))
    w = rng.standard_normal((5, H * dv))
    y = oracle.out_gate(o, gate, 1e-6)
    out = oracle.out_gate(o, gate, 1e-6, w)
    np.testing.assert_allclose(out, y @ w.T, rtol=1e-12, atol=1e-13)
    # per-head normalisation: scaling one head's values leaves y unchanged (eps aside)
    o2 = o.copy()
    o2[:, :, 1] *= 1000.0
    y2 = oracle.out_gate(o2, gate, 0.0)
    np.testing.assert_allclose(y2, oracle.out_gate(o, gate, 0.0), rtol=1e-12)
    # the head's mean square, not the concatenated row's, sets the scale
    yh = y.reshape(B, T, H, dv)
    sig = 1 / (1 + np.exp(-gate))
    ms = np.mean(o * o, axis=-1, keepdims=True)
    np.testing.assert_allclose(yh, o / np.sqrt(ms + 1e-6) * sig, rtol=1e-13)


# ---------------------------------------------------------------- dtype widening
def test_bf16_and_f32_inputs_widen_exactly():
    import torch
    rng = np.random.default_rng(20)
    q, k, v, z, beta = rand_inputs(rng, 1, 9, 2, 8, 4)
    bf = [torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v, z, beta)]
    bits = [t.view(torch.int16).numpy().view(np.uint16) for t in bf]
    wide = [t.to(torch.float64).numpy() for t in bf]
    assert np.array_equal(oracle.bf16_to_f64(bits[0]), wide[0])
    o1, s1 = oracle.forward(*bits, -5.0)
    o2, s2 = oracle.forward(*wide, -5.0)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    f32 = [x.astype(np.float32) for x in (q, k, v, z, beta)]
    o3, s3 = oracle.forward(*f32, -5.0)
    o4, s4 = oracle.forward(*[x.astype(np.float64) for x in f32], -5.0)
    assert np.array_equal(o3, o4) and np.array_equal(s3, s4)


def test_thread_count_does_not_change_bits():
    rng = np.random.default_rng(21)
    q, k, v, z, beta = rand_inputs(rng, 2, 30, 3, 16, 32)
    s0 = rng.standard_normal((2, 3, 16, 32))
    o1, s1 = oracle.forward(q, k, v, z, beta, -5.0, s0, nthreads=1)
    o2, s2 = oracle.forward(q, k, v, z, beta, -5.0, s0, nthreads=7)
    assert np.array_equal(o1, o2) and np.array_equal(s1, s2)


def test_bad_arguments_rejected():
    z1 = np.zeros((1, 2, 1, 4))
    with pytest.raises(TypeError):
        oracle.forward(z1, z1, z1, z1.astype(np.float32), np.zeros((1, 2, 1)), -5.0)
