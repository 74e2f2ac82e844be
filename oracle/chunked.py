"""Chunk form of the KDA recurrence in fp64 numpy (test infrastructure).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

This evaluates the same function as the sequential oracle, but through the
chunkwise expansion of the Kimi Linear tech report, appendix B:

* S_r = P_r S_0 + H_r inside a chunk (the partial expansion of Eq. 1 that
  opens section 3.1 and appendix B);
* Proposition 1, Eq. 16:  P_r = Diag(gamma_r) - sum_{i<=r} Diag(gamma_{i->r}) k_i w_i^T,
  with the w-recurrence of Eq. 17;
* Proposition 2, Eq. 18:  H_r = sum_{i<=r} Diag(gamma_{i->r}) k_i u_i^T,
  with the u-recurrence of Eq. 19;
* o_r = S_r^T q_r (readout from the updated state, "KDA Recurrence").

Notation: gamma_r = prod_{j<=r} alpha_j (it includes alpha_r) and
gamma_{i->r} = prod_{j=i+1..r} alpha_j (it excludes alpha_i, so
gamma_{r->r} = 1).  The extracted renders of Eqs. 17 and 19 lose a bracket;
the reading taken here is that beta_r scales the whole right-hand side,
w_r = beta_r (gamma_r * k_r - sum_{i<r} w_i (k_i^T Diag(gamma_{i->r}) k_r)),
which is what the induction from Eq. 1 in the Proposition 2 proof fragment
gives.

Every chunk is evaluated with dense d_k x d_k matrices P_r, so this is for
small shapes only.
"""
import numpy as np


def _alpha(z, g_min):
    return np.exp(g_min / (1.0 + np.exp(-z)))


def chunk_step(S0, q, k, v, alpha, beta):
    """One chunk: positions r = 0..C-1 of one (batch, head).

    S0 (dk, dv); q, k, alpha (C, dk); v (C, dv); beta (C,).
    Returns (o (C, dv), S_C (dk, dv), w (C, dk), u (C, dv)).
    """
    C, dk = k.shape
    dv = v.shape[1]
    # gamma[r] = prod_{j<=r} alpha_j ; gamma_between(i, r) = prod_{j=i+1..r} alpha_j
    gamma = np.cumprod(alpha, axis=0)

    def gamma_between(i, r):
        if i == r:
            return np.ones(dk)
        return np.prod(alpha[i + 1:r + 1], axis=0)

    w = np.zeros((C, dk))
    u = np.zeros((C, dv))
    for r in range(C):
        acc_w = gamma[r] * k[r]
        acc_u = v[r].copy()
        for i in range(r):
            coef = k[i] @ (gamma_between(i, r) * k[r])   # k_i^T Diag(gamma_{i->r}) k_r
            acc_w = acc_w - w[i] * coef
            acc_u = acc_u - u[i] * coef
        w[r] = beta[r] * acc_w                           # Eq. 17
        u[r] = beta[r] * acc_u                           # Eq. 19

    o = np.zeros((C, dv))
    S_r = None
    for r in range(C):
        P = np.diag(gamma[r])                            # Eq. 16
        Hm = np.zeros((dk, dv))                          # Eq. 18
        for i in range(r + 1):
            dg = gamma_between(i, r)
            P = P - np.outer(dg * k[i], w[i])
            Hm = Hm + np.outer(dg * k[i], u[i])
        S_r = P @ S0 + Hm
        o[r] = S_r.T @ q[r]
    return o, S_r, w, u


def forward(q, k, v, z, beta, g_min, s0=None, chunk=64):
    """Chunked fp64 forward over (B, T, H, .) arrays; T need not divide chunk.

    Returns (o (B, T, H, dv), s_final (B, H, dk, dv)).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    z = np.asarray(z, np.float64)
    beta = np.asarray(beta, np.float64)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    alpha = _alpha(z, g_min)
    o = np.zeros((B, T, H, dv))
    s_fin = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if s0 is None else np.asarray(s0[b, h], np.float64).copy()
            for t0 in range(0, T, chunk):
                t1 = min(T, t0 + chunk)
                oc, S, _, _ = chunk_step(S, q[b, t0:t1, h], k[b, t0:t1, h], v[b, t0:t1, h],
                                         alpha[b, t0:t1, h], beta[b, t0:t1, h])
                o[b, t0:t1, h] = oc
            s_fin[b, h] = S
    return o, s_fin
