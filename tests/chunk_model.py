"""fp64 CPU model of the chunked form of the gated delta rule (test infrastructure).

The pages give the rule only token by token (page "linear_attention.rs", step 7,
gated_delta_rule_decode): per v-head, with unit-norm k_t and q_t, gates alpha_t and
beta_t, and the state stored as H[i][j] (S = H^T),
    delta_t = beta_t (v_t - alpha_t H_{t-1}^T k_t),   H_t = alpha_t H_{t-1} + k_t delta_t^T,
    o_t = H_t^T q_t / sqrt(d_k).
The chunked form regroups C consecutive tokens. With H0 the state before a chunk,
g_t = sum_{s<=t} log alpha_s (inside the chunk) and gamma_t = exp(g_t):
    A[t][s] = beta_t exp(g_t - g_s) (k_t . k_s) for s < t, else 0
    (I + A) Delta = R,  R = diag(beta) (V - diag(gamma) K H0)          (rows delta_t)
    O = diag(gamma) Q H0 + P Delta,  P[t][s] = exp(g_t - g_s) (q_t . k_s) for s <= t
    H_C = gamma_C H0 + K^T diag(exp(g_C - g)) Delta
Unrolling the token recurrence inside the chunk gives these identities (delta_t only
reads H_{t-1}, which is gamma_{t-1} H0 plus the decayed rank-one updates of the earlier
tokens of the chunk). Three ways of solving for Delta are modelled:
    "solve"   forward substitution on (I + A) Delta = R
    "wy"      the WY form: T = (I + A)^-1, W = T diag(beta gamma) K, U = T diag(beta) V,
              Delta = U - W H0 (W and U do not depend on the state)
    "inverse" Delta = T R with T built from 2 x 2 blocks of (I + A): T11 = (I + A11)^-1,
              T22 = (I + A22)^-1 (forward substitution), T21 = -T22 A21 T11
Gate differences are formed in log space before the exponential, so a chunk whose
running sum falls below the fp64 range (exp(-745) = 0) stays finite.

This module shares no code with the HIP path or the oracle; numpy float64 only.
"""

from __future__ import annotations

import numpy as np


def softplus(x):
    """log(1 + e^x) in the overflow-free form."""
    return np.logaddexp(0.0, x)


def log_alpha(dt, dt_bias, A_log):
    """log alpha = -exp(A_log) softplus(dt + dt_bias) (page "linear_attention.rs",
    steps 4-5, gdn_gate), without forming alpha itself."""
    return -np.exp(A_log) * softplus(dt + dt_bias)


def sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def unit_lower_inverse(A):
    """(I + A)^-1 for strictly lower-triangular A, by forward substitution on the
    columns of the identity."""
    n = A.shape[0]
    X = np.eye(n)
    for t in range(1, n):
        X[t] -= A[t, :t] @ X[:t]
    return X


def blocked_inverse(A):
    """(I + A)^-1 from 2 x 2 blocks (halves of the rows): the two diagonal blocks by
    substitution, the off-diagonal block as -T22 A21 T11."""
    n = A.shape[0]
    if n < 2:
        return unit_lower_inverse(A)
    h = n // 2
    T11 = unit_lower_inverse(A[:h, :h])
    T22 = unit_lower_inverse(A[h:, h:])
    T = np.zeros((n, n))
    T[:h, :h] = T11
    T[h:, h:] = T22
    T[h:, :h] = -T22 @ (A[h:, :h] @ T11)
    return T


def chunk_step(H0, Q, K, V, la, beta, form="solve"):
    """One chunk of c tokens of one head: H0 [d_k][d_v]; Q, K [c][d_k] (unit rows);
    V [c][d_v]; la [c] log alpha; beta [c]. Returns (O [c][d_v] before the 1/sqrt(d_k)
    scale, H_C)."""
    c = Q.shape[0]
    g = np.cumsum(la)
    diff = g[:, None] - g[None, :]                      # g_t - g_s
    low = np.tril(np.ones((c, c)), -1).astype(bool)     # s < t
    lowe = np.tril(np.ones((c, c))).astype(bool)        # s <= t
    decay = np.where(lowe, np.exp(np.where(lowe, diff, 0.0)), 0.0)
    gamma = np.exp(g)
    A = np.where(low, beta[:, None] * decay * (K @ K.T), 0.0)
    P = np.where(lowe, decay * (Q @ K.T), 0.0)
    R = beta[:, None] * (V - gamma[:, None] * (K @ H0))
    if form == "solve":
        D = np.zeros_like(R)
        for t in range(c):
            D[t] = R[t] - A[t, :t] @ D[:t]
    elif form == "wy":
        Tm = unit_lower_inverse(A)
        W = Tm @ ((beta * gamma)[:, None] * K)
        U = Tm @ (beta[:, None] * V)
        D = U - W @ H0
    elif form == "inverse":
        D = blocked_inverse(A) @ R
    else:
        raise ValueError(form)
    O = gamma[:, None] * (Q @ H0) + P @ D
    tail = np.exp(g[-1] - g)                            # exp(g_C - g_t) <= 1
    H = np.exp(g[-1]) * H0 + K.T @ (tail[:, None] * D)
    return O, H


def sequence(H0, Q, K, V, la, beta, chunk, form="solve"):
    """T tokens of one head in chunks of `chunk` (the last one ragged). Returns
    (o [T][d_v] = O / sqrt(d_k), final H)."""
    T, dk = Q.shape
    H = np.array(H0, dtype=np.float64, copy=True)
    out = np.zeros((T, V.shape[1]))
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        O, H = chunk_step(H, Q[t0:t1], K[t0:t1], V[t0:t1], la[t0:t1], beta[t0:t1], form)
        out[t0:t1] = O
    return out / np.sqrt(dk), H


def decay_product(alpha, i, j):
    """G(i, j) = alpha_i ... alpha_j, 1 when i > j."""
    return float(np.prod(alpha[i:j + 1])) if i <= j else 1.0


def draft_unrolled(H0, Q, K, V, alpha, beta, shift=1):
    """T draft tokens of one head evaluated from the state before them, H0, without
    forming any later state (the speculative verification's form). Unrolling
    H_t = alpha_t H_{t-1} + k_t delta_t^T gives, with G the decay products,
        m_t = H_{t-1}^T k_t = G(0, t-1) H0^T k_t + sum_{s<t} G(s+1, t-1) (k_s . k_t) delta_s
        delta_t = beta_t (v_t - alpha_t m_t)
        o_t = H_t^T q_t = G(0, t) H0^T q_t + sum_{s<=t} G(s+1, t) (k_s . q_t) delta_s.
    alpha are the gates themselves (not their logs). `shift` is the first factor's
    offset from s (1 is the rule; tests plant 0). Returns (delta [T][d_v],
    o [T][d_v] / sqrt(d_k))."""
    T, dk = Q.shape
    a = K @ H0          # row t: H0^T k_t
    b = Q @ H0          # row t: H0^T q_t
    KK = K @ K.T        # [s][t] = k_s . k_t
    KQ = K @ Q.T        # [s][t] = k_s . q_t
    D = np.zeros((T, V.shape[1]))
    O_ = np.zeros_like(D)
    for t in range(T):
        m = decay_product(alpha, 0, t - 1) * a[t]
        for s in range(t):
            m = m + decay_product(alpha, s + shift, t - 1) * KK[s, t] * D[s]
        D[t] = beta[t] * (V[t] - alpha[t] * m)
        o = decay_product(alpha, 0, t) * b[t]
        for s in range(t + 1):
            o = o + decay_product(alpha, s + shift, t) * KQ[s, t] * D[s]
        O_[t] = o / np.sqrt(dk)
    return D, O_


def replay(H0, K, D, alpha, n):
    """The state after the first n of the recorded updates H <- alpha_t H + k_t delta_t^T."""
    H = np.array(H0, dtype=np.float64, copy=True)
    for t in range(n):
        H = alpha[t] * H + np.outer(K[t], D[t])
    return H

