"""Two other fp64 evaluations of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

They exist to pin the sequential oracle (``oracle.prefill``), not to be fast.
Both take already-normalised fp64 keys/queries for one (sequence, head) chain:
q, k [T, dk], v [T, dv], g, beta [T], S0 [dv, dk].

``unrolled_product``
    Written from the matrix form of the update, S_t = S_{t-1} A_t + beta_t v_t k_t^T
    with A_t = e^{g_t} (I - beta_t k_t k_t^T), which is Eqs. 16-18 of
    "Long-Context Aware Upcycling: A New Frontier for Hybrid LLM Scaling"
    (App. A.3) with the decay and the delta correction multiplied out.  Unrolled:
        o_t = scale * [ S_0 A_1...A_t q_t + sum_{j<=t} beta_j v_j k_j^T A_{j+1}...A_t q_t ].
    Each o_t is evaluated right-to-left with a vector, O(T^2 d) per chain, and
    never forms a state matrix.

``chunked_wy``
    The chunked evaluation the same appendix names (chunks of C tokens, delta
    corrections inside a chunk batched into one matrix operation via the WY
    representation, state carried sequentially from chunk to chunk), derived
    here in fp64 with chunk-local cumulative log-decay gamma:
        A_rj  = beta_r (k_r . k_j) e^{gamma_r - gamma_j}    (j < r)
        T     = (I + A)^{-1}
        W     = T diag(beta e^{gamma}) K,   U = T diag(beta) V
        Delta = U - W S0^T                   (rows = beta_r v'_r of Eq. 17-18)
        P_rj  = (q_r . k_j) e^{gamma_r - gamma_j}             (j <= r)
        O     = scale [ diag(e^{gamma}) Q S0^T + P Delta ]
        S_end = e^{gamma_L} S0 + Delta^T diag(e^{gamma_L - gamma}) K
    Exponents are formed only for j <= r, where they are <= 0 for g <= 0.
    Returns per-chunk intermediates too, for unit checks of a chunked kernel.
"""
from __future__ import annotations

import numpy as np


def l2_normalise(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def unrolled_product(q, k, v, g, beta, S0, scale):
    T, dk = q.shape
    dv = v.shape[1]
    alpha = np.exp(g)
    o = np.zeros((T, dv))
    for t in range(T):
        z = q[t].copy()
        acc = np.zeros(dv)
        for j in range(t, -1, -1):
            # term j: beta_j v_j k_j^T (A_{j+1} ... A_t) q_t, z holds (A_{j+1}...A_t) q_t
            acc += beta[j] * v[j] * np.dot(k[j], z)
            # z <- A_j z with A_j = alpha_j (I - beta_j k_j k_j^T)
            z = alpha[j] * (z - beta[j] * k[j] * np.dot(k[j], z))
        acc += S0 @ z
        o[t] = scale * acc
    return o


def chunked_wy(q, k, v, g, beta, S0, scale, C):
    T, dk = q.shape
    dv = v.shape[1]
    S = np.array(S0, dtype=np.float64, copy=True)
    o = np.zeros((T, dv))
    chunks = []
    for c0 in range(0, T, C):
        L = min(C, T - c0)
        Q, K, V = q[c0:c0 + L], k[c0:c0 + L], v[c0:c0 + L]
        b = beta[c0:c0 + L]
        gam = np.cumsum(g[c0:c0 + L])
        diff = gam[:, None] - gam[None, :]
        lower = np.tril(np.ones((L, L), dtype=bool), -1)
        incl = np.tril(np.ones((L, L), dtype=bool), 0)
        dec = np.zeros((L, L))
        dec[incl] = np.exp(diff[incl])  # only j <= r
        A = np.where(lower, b[:, None] * (K @ K.T) * dec, 0.0)
        Tm = np.linalg.inv(np.eye(L) + A)
        W = Tm @ (b[:, None] * np.exp(gam)[:, None] * K)
        U = Tm @ (b[:, None] * V)
        Delta = U - W @ S.T
        P = np.where(incl, (Q @ K.T) * dec, 0.0)
        O = scale * (np.exp(gam)[:, None] * (Q @ S.T) + P @ Delta)
        o[c0:c0 + L] = O
        chunks.append(dict(gamma=gam, A=A, T=Tm, W=W, U=U, Delta=Delta, P=P, S_start=S.copy()))
        S = np.exp(gam[-1]) * S + Delta.T @ (np.exp(gam[-1] - gam)[:, None] * K)
    return o, S, chunks
