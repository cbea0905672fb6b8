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


def chunked_wy_vjp(q, k, v, g, beta, S0, scale, C, dO, dS_end, chunk_grads=None):
    """Gradients of <dO, o> + <dS_end, S_end> for ``chunked_wy`` on one chain,
    by reverse-mode differentiation of the chunked WY form itself (the form a
    chunked backward kernel evaluates).  q, k are used as given (normalise them
    beforehand and apply the normalisation's own gradient after).  Per chunk,
    in reverse order, with dS the gradient of the state after the chunk and
    D = diag(e^{gamma_L - gamma}):

        from S_end = e^{gamma_L} S + Delta^T D K:  dS_in  = e^{gamma_L} dS
                                                  dDelta = D K dS^T,  dK = D Delta dS
        from O = scale [diag(e^gamma) Q S^T + P Delta]:
            dQ += diag(e^gamma) dO' S,  dS_in += dO'^T diag(e^gamma) Q,
            dP = tril(dO' Delta^T),     dDelta += P^T dO'          (dO' = scale dO)
        from P_rj = (q_r . k_j) e^{gamma_r - gamma_j}:  dQ += (dP o Gamma) K, dK += (dP o Gamma)^T Q
        from Delta = U - W S^T:  dU = dDelta, dW = -dDelta S, dS_in -= dDelta^T W
        from U = T diag(b) V, W = T diag(b e^gamma) K:
            dT = dU (diag(b) V)^T + dW (diag(b e^gamma) K)^T
            dV = diag(b) T^T dU,  dK += diag(b e^gamma) T^T dW
        from T = (I + A)^{-1}:  dA = -T^T dT T^T (strictly lower part)
        from A_rj = b_r (k_r . k_j) e^{gamma_r - gamma_j}:  dK += diag(b)(dA o Gamma) K + (diag(b)(dA o Gamma))^T K
    and the beta and gamma terms of each product; dg is the reverse cumulative
    sum of dgamma within the chunk.  Returns dq, dk, dv, dg, dbeta, dS0.  If
    ``chunk_grads`` is a list, it receives, per chunk in chunk order, a dict with
    dDelta (the chunk's total Delta gradient) and dS_after (the gradient of the
    state after the chunk): the outputs of a reverse state-gradient chain.
    """
    T_, dk = q.shape
    dv = v.shape[1]
    _, _, chunks = chunked_wy(q, k, v, g, beta, S0, scale, C)
    dq = np.zeros_like(q, dtype=np.float64)
    dkk = np.zeros_like(k, dtype=np.float64)
    dvv = np.zeros_like(v, dtype=np.float64)
    dg = np.zeros(T_)
    db = np.zeros(T_)
    dS = np.array(dS_end, dtype=np.float64, copy=True)
    for ci in range(len(chunks) - 1, -1, -1):
        ch = chunks[ci]
        c0 = ci * C
        L = ch["gamma"].shape[0]
        Q, K, V = q[c0:c0 + L], k[c0:c0 + L], v[c0:c0 + L]
        b = beta[c0:c0 + L]
        gam, Tm, W, Delta, P, A, S = ch["gamma"], ch["T"], ch["W"], ch["Delta"], ch["P"], ch["A"], ch["S_start"]
        eg = np.exp(gam)
        gL = gam[-1]
        dd = np.exp(gL - gam)
        incl = np.tril(np.ones((L, L), dtype=bool), 0)
        lower = np.tril(np.ones((L, L), dtype=bool), -1)
        Gam = np.zeros((L, L))
        Gam[incl] = np.exp((gam[:, None] - gam[None, :])[incl])
        dgam = np.zeros(L)
        dQ = np.zeros((L, dk))
        dK = np.zeros((L, dk))
        # S_end = e^{gL} S + Delta^T D K
        dS_in = np.exp(gL) * dS
        dgL = np.exp(gL) * np.sum(dS * S)
        dDelta = dd[:, None] * (K @ dS.T)
        dK += dd[:, None] * (Delta @ dS)
        d_dd = np.sum(Delta * (K @ dS.T), axis=1)
        dgL += np.sum(d_dd * dd)
        dgam -= d_dd * dd
        # O = scale [diag(e^gam) Q S^T + P Delta]
        dOs = scale * dO[c0:c0 + L]
        QS = Q @ S.T
        dQ += eg[:, None] * (dOs @ S)
        dS_in += dOs.T @ (eg[:, None] * Q)
        dgam += eg * np.sum(dOs * QS, axis=1)
        dP = np.where(incl, dOs @ Delta.T, 0.0)
        dDelta += P.T @ dOs
        # P = tril_incl((Q K^T) o Gamma)
        dPG = dP * Gam
        dQ += dPG @ K
        dK += dPG.T @ Q
        dgam += np.sum(dP * P, axis=1)
        dgam -= np.sum(dP * P, axis=0)
        # Delta = U - W S^T
        dU = dDelta
        dW = -dDelta @ S
        dS_in -= dDelta.T @ W
        # U = T diag(b) V, W = T diag(b e^gam) K
        Vb = b[:, None] * V
        Kb = (b * eg)[:, None] * K
        dT = dU @ Vb.T + dW @ Kb.T
        dVb = Tm.T @ dU
        dKb = Tm.T @ dW
        dV = b[:, None] * dVb
        db_c = np.sum(dVb * V, axis=1)
        dK += (b * eg)[:, None] * dKb
        db_c += eg * np.sum(dKb * K, axis=1)
        dgam += b * eg * np.sum(dKb * K, axis=1)
        # T = (I + A)^{-1}
        dA = np.where(lower, -Tm.T @ dT @ Tm.T, 0.0)
        # A = tril_strict(diag(b) (K K^T) o Gamma)
        dAG = dA * Gam
        dK += (b[:, None] * dAG) @ K
        dK += (b[:, None] * dAG).T @ K
        db_c += np.sum(dA * (K @ K.T) * Gam, axis=1)
        dgam += np.sum(dA * A, axis=1)
        dgam -= np.sum(dA * A, axis=0)
        # gamma = cumsum(g) within the chunk (gamma_L is gamma[-1])
        dgam[-1] += dgL
        dg[c0:c0 + L] = np.cumsum(dgam[::-1])[::-1]
        db[c0:c0 + L] = db_c
        dq[c0:c0 + L] = dQ
        dkk[c0:c0 + L] = dK
        dvv[c0:c0 + L] = dV
        if chunk_grads is not None:
            chunk_grads.insert(0, dict(dDelta=dDelta.copy(), dS_after=dS.copy()))
        dS = dS_in
    return dq, dkk, dvv, dg, db, dS
