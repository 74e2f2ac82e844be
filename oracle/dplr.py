"""fp64 CPU oracle of the general diagonal-plus-low-rank (DPLR) recurrence.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may use it; the product path never imports it.

"Diagonal-Plus-Low-Rank Matrices and Kimi Delta Attention", sections 1 and 3:

    S_t = (D_t - a_t b_t^T) S_{t-1} + k_t v_t^T,        S_t in R^{d_k x d_v}

with a diagonal decay D_t = Diag(alpha_t) and two independent directions a_t,
b_t (section 3: a_t = W_a x_t, b_t = W_b x_t).  Readings taken here (the page
gives the state update only):
  * alpha_t = exp(g_min * sigmoid(z_t)) per key channel, the decay of the
    "KDA Recurrence" problem statement, so that KDA is the special case;
  * the output reads the updated state, o_t = S_t^T q_t, as KDA's Eq. 1 does;
  * there is no separate write strength: k_t v_t^T is written as given.
Section 3's variable binding a_t = beta_t k_t, b_t = k_t * alpha_t with the
write key beta_t k_t turns this into KDA's Eq. 1.

The recurrence is evaluated token by token, all (batch, head) chains at once,
in float64.  Inputs may be float64, float32, or uint16 arrays holding
bfloat16 bit patterns (widened exactly).
"""
import numpy as np


def _f64(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def alpha_of(z, g_min):
    """alpha = exp(g_min * sigmoid(z)) ("KDA Recurrence" decay)."""
    return np.exp(g_min / (1.0 + np.exp(-_f64(z))))


def forward(q, k, v, z, a, b, g_min, s0=None):
    """q, k, z, a, b: (B, T, H, d_k); v: (B, T, H, d_v); s0: (B, H, d_k, d_v)
    or None (zeros).  Returns (o (B, T, H, d_v), s_final (B, H, d_k, d_v)),
    float64."""
    q, k, v, a, b = (_f64(x) for x in (q, k, v, a, b))
    alpha = alpha_of(z, g_min)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if s0 is None else _f64(s0).copy()
    o = np.zeros((B, T, H, dv))
    for t in range(T):
        # (b_t^T S_{t-1}): one row of d_v values per chain, from the state before the update
        bS = np.einsum("bhi,bhij->bhj", b[:, t], S)
        S = alpha[:, t, :, :, None] * S - a[:, t, :, :, None] * bS[:, :, None, :] \
            + k[:, t, :, :, None] * v[:, t, :, None, :]
        o[:, t] = np.einsum("bhi,bhij->bhj", q[:, t], S)
    return o, S


def chunk_forward(q, k, v, z, a, b, g_min, s0=None, C=64):
    """The same recurrence by chunks of C tokens (the last one ragged), in the
    WY/UT form that a chunkwise kernel uses; for pinning that algebra against
    the token loop.  Inside a chunk with entry state S_0, with G_r the
    cumulative log-decay through token r and G_{r-1} the one before it:
        x_r^T = b_r^T S_{r-1}   (the erased row read from the old state)
        (I + L) X = B_g S_0 + M_bk V,   L_ri = b_r^T Diag(e^{G_{r-1} - G_i}) a_i,
                                        M_bk,ri = b_r^T Diag(e^{G_{r-1} - G_i}) k_i   (i < r),
                                        B_g rows b_r * e^{G_{r-1}}
        O = (Q * e^G) S_0 + M_qk V - M_qa X   (i <= r, decay e^{G_r - G_i})
        S_C = e^{G_C} * S_0 + sum_i e^{G_C - G_i} * (k_i v_i^T - a_i x_i^T).
    Derived from section 1's update by unrolling it through the chunk."""
    q, k, v, a, b = (_f64(x) for x in (q, k, v, a, b))
    g = g_min / (1.0 + np.exp(-_f64(z)))           # log alpha
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dk, dv)) if s0 is None else _f64(s0).copy()
    o = np.zeros((B, T, H, dv))
    for bb in range(B):
        for hh in range(H):
            St = S[bb, hh]
            for t0 in range(0, T, C):
                n = min(C, T - t0)
                sl = slice(t0, t0 + n)
                Q, K, V, A, Bv = q[bb, sl, hh], k[bb, sl, hh], v[bb, sl, hh], a[bb, sl, hh], b[bb, sl, hh]
                Gi = np.cumsum(g[bb, sl, hh], axis=0)        # G_r, inclusive
                Ge = Gi - g[bb, sl, hh]                        # G_{r-1}
                # decay between token i and token r (before r for the b side)
                dex = np.exp(Ge[:, None, :] - Gi[None, :, :])  # [r, i, c]
                din = np.exp(Gi[:, None, :] - Gi[None, :, :])
                strict = np.tril(np.ones((n, n)), -1)
                incl = np.tril(np.ones((n, n)))
                L = np.einsum("rc,ic,ric->ri", Bv, A, dex) * strict
                Mbk = np.einsum("rc,ic,ric->ri", Bv, K, dex) * strict
                Mqk = np.einsum("rc,ic,ric->ri", Q, K, din) * incl
                Mqa = np.einsum("rc,ic,ric->ri", Q, A, din) * incl
                X = np.linalg.solve(np.eye(n) + L, (Bv * np.exp(Ge)) @ St + Mbk @ V)
                o[bb, sl, hh] = (Q * np.exp(Gi)) @ St + Mqk @ V - Mqa @ X
                dC = np.exp(Gi[-1][None, :] - Gi)              # e^{G_C - G_i}, [i, c]
                St = np.exp(Gi[-1])[:, None] * St + (K * dC).T @ V - (A * dC).T @ X
            S[bb, hh] = St
    return o, S
