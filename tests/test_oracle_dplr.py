"""Pins of the DPLR oracle (oracle/dplr.py), CPU only.

"Diagonal-Plus-Low-Rank Matrices and Kimi Delta Attention", sections 1 and 3:
S_t = (Diag(alpha_t) - a_t b_t^T) S_{t-1} + k_t v_t^T, o_t = S_t^T q_t.  Each
pin is computed another way than the oracle's token loop: the KDA oracle (C,
its own rearranged step) under the page's variable binding, closed forms, and
the chunked WY/UT form.
"""
import numpy as np
import pytest

import oracle
from oracle import dplr


def rand(rng, B, T, H, dk, dv, z_shift=0.0):
    q = rng.standard_normal((B, T, H, dk)) / np.sqrt(dk)
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    z = rng.standard_normal((B, T, H, dk)) + z_shift
    a = rng.standard_normal((B, T, H, dk)) * 0.3
    b = rng.standard_normal((B, T, H, dk)) * 0.3
    s0 = rng.standard_normal((B, H, dk, dv)) * 0.1
    return q, k, v, z, a, b, s0


@pytest.mark.parametrize("dims", [(1, 40, 2, 8, 5), (2, 17, 1, 16, 16), (1, 70, 3, 4, 2)])
def test_binding_reduces_to_kda(dims):
    """Section 3: a = beta k, b = k * alpha and the write key beta k give KDA's
    Eq. 1, which the C oracle computes in its own step order."""
    B, T, H, dk, dv = dims
    rng = np.random.default_rng(dk * 7 + T)
    q, k, v, z, _, _, s0 = rand(rng, B, T, H, dk, dv)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    g_min = -3.0
    alpha = dplr.alpha_of(z, g_min)
    bk = beta[..., None] * k
    o, s = dplr.forward(q, bk, v, z, bk, k * alpha, g_min, s0)
    ro, rs = oracle.forward(q, k, v, z, beta, g_min, s0)
    assert np.abs(o - ro).max() < 1e-12 and np.abs(s - rs).max() < 1e-12


def test_binding_mistake_is_caught():
    """A planted mistake (b read against the updated state) must break the
    binding pin."""
    rng = np.random.default_rng(3)
    q, k, v, z, _, _, s0 = rand(rng, 1, 30, 1, 8, 4)
    beta = np.full((1, 30, 1), 0.7)
    g_min = -2.0
    alpha = dplr.alpha_of(z, g_min)
    bk = beta[..., None] * k
    ro, _ = oracle.forward(q, k, v, z, beta, g_min, s0)
    # the wrong order: decay and write first, then erase with b^T of the new state
    S = s0[0, 0].copy()
    out = np.zeros((30, 4))
    for t in range(30):
        S = alpha[0, t, 0][:, None] * S + np.outer(bk[0, t, 0], v[0, t, 0])
        S = S - np.outer(bk[0, t, 0], (k[0, t, 0] * alpha[0, t, 0]) @ S)
        out[t] = S.T @ q[0, t, 0]
    assert np.abs(out - ro[0, :, 0]).max() > 1e-3


def test_no_erase_is_decayed_linear_attention():
    """a = 0: S_t = Diag(gamma_t) S_0 + sum_{i<=t} Diag(gamma_{i->t}) k_i v_i^T,
    evaluated as explicit sums over cumulative log-decays."""
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 1, 25, 2, 6, 3
    q, k, v, z, _, b, s0 = rand(rng, B, T, H, dk, dv)
    g_min = -1.5
    o, s = dplr.forward(q, k, v, z, np.zeros_like(k), b, g_min, s0)
    G = np.cumsum(g_min / (1 + np.exp(-z)), axis=1)           # (B, T, H, dk)
    for h in range(H):
        for t in range(T):
            St = np.exp(G[0, t, h])[:, None] * s0[0, h]
            for i in range(t + 1):
                St = St + np.exp(G[0, t, h] - G[0, i, h])[:, None] * np.outer(k[0, i, h], v[0, i, h])
            assert np.abs(o[0, t, h] - St.T @ q[0, t, h]).max() < 1e-12
        assert np.abs(s[0, h] - St).max() < 1e-12


def test_scalar_case_closed_form():
    """d_k = d_v = 1: S_T = sum_t [prod_{j>t} (alpha_j - a_j b_j)] k_t v_t
    + [prod_j (alpha_j - a_j b_j)] S_0."""
    rng = np.random.default_rng(9)
    T = 30
    q, k, v, z, a, b, s0 = rand(rng, 1, T, 1, 1, 1)
    g_min = -0.7
    _, s = dplr.forward(q, k, v, z, a, b, g_min, s0)
    alpha = dplr.alpha_of(z, g_min)[0, :, 0, 0]
    m = alpha - a[0, :, 0, 0] * b[0, :, 0, 0]
    expect = np.prod(m) * s0[0, 0, 0, 0]
    for t in range(T):
        expect += np.prod(m[t + 1:]) * k[0, t, 0, 0] * v[0, t, 0, 0]
    assert abs(s[0, 0, 0, 0] - expect) < 1e-12


@pytest.mark.parametrize("C", [1, 2, 16, 64])
def test_chunk_form_matches_token_loop(C):
    """The chunked WY/UT form (oracle/dplr.py chunk_forward) equals the token
    loop for several chunk sizes and a ragged tail."""
    rng = np.random.default_rng(C)
    q, k, v, z, a, b, s0 = rand(rng, 2, 100, 2, 8, 5)
    g_min = -2.5
    o, s = dplr.forward(q, k, v, z, a, b, g_min, s0)
    oc, sc = dplr.chunk_forward(q, k, v, z, a, b, g_min, s0, C=C)
    assert np.abs(o - oc).max() < 1e-12 and np.abs(s - sc).max() < 1e-12


def test_linear_in_initial_state_and_values():
    rng = np.random.default_rng(12)
    q, k, v, z, a, b, s0 = rand(rng, 1, 20, 1, 5, 4)
    g_min = -2.0
    o1, s1 = dplr.forward(q, k, v, z, a, b, g_min, s0)
    o2, s2 = dplr.forward(q, k, 2 * v, z, a, b, g_min, 2 * s0)
    assert np.abs(o2 - 2 * o1).max() < 1e-12 and np.abs(s2 - 2 * s1).max() < 1e-12
    # the d_v columns evolve independently
    o3, s3 = dplr.forward(q, k, v[..., :2], z, a, b, g_min, s0[..., :2])
    assert np.abs(o3 - o1[..., :2]).max() < 1e-13 and np.abs(s3 - s1[..., :2]).max() < 1e-13


def test_bf16_bits_are_widened_exactly():
    rng = np.random.default_rng(14)
    q, k, v, z, a, b, s0 = rand(rng, 1, 9, 1, 4, 4)
    to_bits = lambda x: (x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    from_bits = lambda u: (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    args = [to_bits(x) for x in (q, k, v, z, a, b)]
    o, s = dplr.forward(*args, -2.0, s0)
    o2, s2 = dplr.forward(*[from_bits(x) for x in args], -2.0, s0)
    assert np.array_equal(o, o2) and np.array_equal(s, s2)
