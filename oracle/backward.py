"""fp64 gradients of the KDA recurrence (test infrastructure, like the rest of
this package: never imported by the product path).

The pages give the forward operator only (Kimi Linear tech report, section 3,
Eq. 1; "KDA Recurrence" problem statement for the decay and the readout):

    alpha_t = exp(g_min * sigmoid(z_t))                (per key channel)
    S'      = Diag(alpha_t) S_{t-1}
    w_t     = v_t - S'^T k_t
    S_t     = S' + beta_t k_t w_t^T                    (= (I - b k k^T) Diag(a) S + b k v^T)
    o_t     = S_t^T q_t

and no gradient formulas.  ``backward`` is the chain rule through that
recurrence, written out here token by token in reverse, for a loss whose
gradients with respect to the outputs and the final state are given (do,
ds_final).  With dS the gradient with respect to S_t:

    dq_t = S_t do_t,                 dS += q_t do_t^T
    u    = dS^T k_t,                 dbeta_t = u . w_t,       dw = beta_t u
    dv_t = dw,                       dk_t = beta_t dS w_t - S' dw
    dS'  = dS - k_t dw^T,            dalpha = rowsum(S_{t-1} * dS')
    dz_t = dalpha * alpha_t * g_min * sigmoid(z_t) (1 - sigmoid(z_t))
    dS   <- Diag(alpha_t) dS'        (the gradient with respect to S_{t-1})

and ds0 is the final dS.  The states S_{t-1} come from a forward sweep kept in
memory (small cases only).  It is pinned against central finite differences
of the C oracle's forward (``oracle.forward``), which shares no code with it.
"""
import numpy as np


def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        from . import bf16_to_f64
        return bf16_to_f64(a)
    return a.astype(np.float64)


def backward(q, k, v, z, beta, g_min, s0, do, ds_final=None):
    """Gradients of <o, do> + <S_T, ds_final> for the recurrence above.

    q, k, z: (B, T, H, dk); v, do: (B, T, H, dv); beta: (B, T, H);
    s0, ds_final: (B, H, dk, dv) or None (zeros).  Token arrays may be
    float64, float32 or uint16 bfloat16 bit patterns (taken exactly).
    Returns a dict of float64 arrays dq, dk, dv, dz, dbeta (the shapes of
    the inputs) and ds0 (B, H, dk, dv).
    """
    q, k, v, z, beta, do = (_f64(a) for a in (q, k, v, z, beta, do))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    S0 = np.zeros((B, H, dk, dv)) if s0 is None else _f64(s0)
    dSf = np.zeros((B, H, dk, dv)) if ds_final is None else _f64(ds_final)
    out = {n: np.zeros_like(a) for n, a in (("dq", q), ("dk", k), ("dv", v), ("dz", z), ("dbeta", beta))}
    out["ds0"] = np.zeros((B, H, dk, dv))
    sig = 1.0 / (1.0 + np.exp(-z))
    alpha = np.exp(g_min * sig)
    for b in range(B):
        for h in range(H):
            # forward sweep: the state before each token, and w
            pre = np.empty((T, dk, dv))
            ws = np.empty((T, dv))
            S = S0[b, h].copy()
            for t in range(T):
                pre[t] = S
                Sp = alpha[b, t, h][:, None] * S
                w = v[b, t, h] - Sp.T @ k[b, t, h]
                S = Sp + beta[b, t, h] * np.outer(k[b, t, h], w)
                ws[t] = w
            # reverse sweep; S is S_t on entry to each step
            dS = dSf[b, h].copy()
            for t in range(T - 1, -1, -1):
                a, kt, qt, bt, w = alpha[b, t, h], k[b, t, h], q[b, t, h], beta[b, t, h], ws[t]
                out["dq"][b, t, h] = S @ do[b, t, h]
                dS += np.outer(qt, do[b, t, h])
                Sprev = pre[t]
                Sp = a[:, None] * Sprev
                u = dS.T @ kt
                out["dbeta"][b, t, h] = u @ w
                dw = bt * u
                out["dv"][b, t, h] = dw
                out["dk"][b, t, h] = bt * (dS @ w) - Sp @ dw
                dSp = dS - np.outer(kt, dw)
                dalpha = np.sum(Sprev * dSp, axis=1)
                s = sig[b, t, h]
                out["dz"][b, t, h] = dalpha * a * g_min * s * (1.0 - s)
                dS = a[:, None] * dSp
                S = Sprev
            out["ds0"][b, h] = dS
    return out
