"""fp64 oracle of the gradients of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module; the product library never does.

Training differentiates the mixer ("Long-Context Aware Upcycling: A New
Frontier for Hybrid LLM Scaling", arXiv:2604.24715, App. A.3, the paragraph
after Eq. 21: the recurrence is evaluated in chunks during training).  This
module gives the vector-Jacobian product of the plain token recurrence of
Eqs. 16-19 -- the same map the forward oracle evaluates -- in fp64:

    given cotangents do [T, H, dv] of the outputs and dS_N [N, H, dv, dk] of the
    final states, it returns the gradients of
        L = sum_t <do_t, o_t> + sum_n <dS_N[n], S_final[n]>
    with respect to q, k, v, g, beta and the initial state.

The reverse sweep is derived from the recurrence (state S, rows = value
index, q^ and k^ the L2-normalised q and k, alpha = e^g):

    forward   S~ = alpha S_{t-1};  S_t = S~ + beta (v - S~ k^) k^T;  o_t = scale S_t q^
    backward  G  <- G + scale do_t q^T                       (G = dL/dS_t)
              dq^_t = scale S_t^T do_t
              dv_t  = beta G k^
              dbeta = (v - S~ k^)^T G k^
              dk^_t = beta (G^T (v - S~ k^) - S~^T G k^)
              dS~   = G - beta (G k^) k^T
              dg_t  = alpha <dS~, S_{t-1}>
              G     <- alpha dS~                              (now dL/dS_{t-1})
    and through x^ = x (|x|^2 + eps)^{-1/2}:  dx = r dx^ - r^3 x (x . dx^).

It stores every state of a chain, so it is meant for small and medium sizes.
Pinned in ``tests/test_backward_pins.py`` by central finite differences of
the forward oracle (``gdn_oracle.c``, which shares no code with this module)
and by closed forms; planted mistakes (``BWD_MUTATIONS``) each fail a pin.
"""
from __future__ import annotations

import numpy as np

BWD_MUTATIONS = {
    "no_alpha_carry": 1,       # G <- dS~ instead of alpha dS~
    "dk_one_term": 2,          # dk^ keeps only the beta G^T (v - S~ k^) term
    "dbeta_undecayed": 3,      # dbeta retrieves with S_{t-1} instead of S~
    "read_before_write": 4,    # dq^ and the do term use S_{t-1} instead of S_t
    "norm_grad_naive": 5,      # dx = r dx^ (drops the projection of the norm)
}


def _widen(a, bf16):
    a = np.asarray(a)
    if bf16:
        if a.dtype != np.uint16:
            raise ValueError("bf16 data must be passed as raw uint16 bit patterns")
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def prefill_vjp(q, k, v, g, beta, do, dstate=None, init_state=None, cu_seqlens=None, scale=None,
                qk_l2norm=True, eps=1e-6, bf16=False, mutation=0):
    """Gradients of L = <do, o> + <dstate, final_state> for the packed prefill.

    q, k [T, H, dk]; v [T, H, dv] (raw bf16 bits when ``bf16``); g, beta [T, H];
    do [T, H, dv]; dstate [N, H, dv, dk] or None (zero); init_state [N, H, dv, dk]
    or None (zeros); cu_seqlens as for the forward oracle.
    Returns a dict of fp64 arrays: dq, dk, dv, dg, dbeta (input shapes) and
    dinit [N, H, dv, dk].
    """
    qq, kk, vv = _widen(q, bf16), _widen(k, bf16), _widen(v, bf16)
    gg = np.asarray(g, dtype=np.float64)
    bb = np.asarray(beta, dtype=np.float64)
    dO = np.asarray(do, dtype=np.float64)
    T, H, dk = qq.shape
    dv = vv.shape[2]
    cu = np.array([0, T], dtype=np.int64) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    S0 = np.zeros((N, H, dv, dk)) if init_state is None else np.asarray(init_state, dtype=np.float64)
    dSN = np.zeros((N, H, dv, dk)) if dstate is None else np.asarray(dstate, dtype=np.float64)

    # normalisation (per token and head)
    def unit(x):
        if not qk_l2norm:
            return x, np.ones(x.shape[:-1])
        r = 1.0 / np.sqrt(np.sum(x * x, axis=-1) + eps)
        return x * r[..., None], r

    qh, rq = unit(qq)
    kh, rk = unit(kk)
    dqh = np.zeros_like(qq)
    dkh = np.zeros_like(kk)
    dV = np.zeros_like(vv)
    dG = np.zeros((T, H))
    dB = np.zeros((T, H))
    dinit = np.zeros((N, H, dv, dk))

    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        for h in range(H):
            # forward, keeping S_{t-1} for every token of the chain
            S = S0[n, h].copy()
            prev = []
            for t in range(s, e):
                prev.append(S.copy())
                a = np.exp(gg[t, h])
                St = a * S
                S = St + bb[t, h] * np.outer(vv[t, h] - St @ kh[t, h], kh[t, h])
            G = dSN[n, h].copy()
            S_t = S  # state after the last token
            for t in range(e - 1, s - 1, -1):
                Sp = prev[t - s]
                a = np.exp(gg[t, h])
                b = bb[t, h]
                St = a * Sp
                k_ = kh[t, h]
                read = Sp if mutation == 4 else S_t
                G = G + scale * np.outer(dO[t, h], qh[t, h])
                dqh[t, h] = scale * read.T @ dO[t, h]
                Gk = G @ k_
                resid = vv[t, h] - St @ k_
                dV[t, h] = b * Gk
                dB[t, h] = ((vv[t, h] - Sp @ k_) if mutation == 3 else resid) @ Gk
                dkh[t, h] = b * (G.T @ resid) if mutation == 2 else b * (G.T @ resid - St.T @ Gk)
                dSt = G - b * np.outer(Gk, k_)
                dG[t, h] = a * np.sum(dSt * Sp)
                G = dSt if mutation == 1 else a * dSt
                S_t = Sp
            dinit[n, h] = G

    def through_norm(x, r, dxh):
        if not qk_l2norm:
            return dxh
        if mutation == 5:
            return dxh * r[..., None]
        return dxh * r[..., None] - x * (r ** 3)[..., None] * np.sum(x * dxh, axis=-1, keepdims=True)

    return {"dq": through_norm(qq, rq, dqh), "dk": through_norm(kk, rk, dkh), "dv": dV, "dg": dG,
            "dbeta": dB, "dinit": dinit}
