"""fp64 oracle of the mixer's front end -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module; the product library never does.

"Long-Context Aware Upcycling: A New Frontier for Hybrid LLM Scaling"
(arXiv:2604.24715), App. A.3:

* the paragraph under Table 8: each of Q, K and V passes through a short 1-D
  convolution with kernel size 4, followed by SiLU, before the recurrence;
* the paragraph after Eqs. 16-21: the forget gate is
  g_t = -exp(A_log) * softplus(W_alpha x_t + Delta_bias) and the write strength
  beta_t = sigmoid(W_beta x_t), with A_log and Delta_bias one scalar per head.

Readings where the pages leave a step open (each is the plainest one the rest
supports):

* The convolution is causal and depthwise: channel c of token t mixes only
  channel c of tokens t-3 .. t, y_t[c] = sum_j w[c, j] x_{t-3+j}[c], with
  tap j = 3 on the current token.  No bias (Table 8 lists no conv bias).
* Each sequence of a packed batch starts from its own three preceding inputs
  (``conv_state``; zeros when none are given), so nothing leaks across
  sequence boundaries; the state after a call is the last three inputs.
* The projections W_Q x, W_K x, W_V x, W_alpha x and W_beta x are inputs
  here (the projections themselves are out of scope).
* softplus(u) = log(1 + e^u), sigmoid(u) = 1 / (1 + e^{-u}),
  silu(u) = u * sigmoid(u).

Every function is pinned in ``tests/test_frontend_pins.py`` (a library
convolution, impulse responses, continuation and packing laws, and closed
forms of the gate math); planted misreadings (``CONV_MUTATIONS``,
``GATE_MUTATIONS``) each fail at least one pin.
"""
from __future__ import annotations

import numpy as np

# Planted mistakes, used only by the pin-strength tests.
CONV_MUTATIONS = {
    "taps_reversed": 1,          # tap 0 applied to the current token
    "no_silu": 2,                # convolution output returned without SiLU
    "silu_before_conv": 3,       # SiLU applied to the inputs, then the convolution
    "state_ignored": 4,          # zero history even when a conv state is given
    "leak_across_sequences": 5,  # a packed batch convolved as one sequence
}
GATE_MUTATIONS = {
    "no_dt_bias": 1,      # softplus(a) instead of softplus(a + Delta_bias)
    "A_log_not_exp": 2,   # -A_log * softplus(...) instead of -exp(A_log) * softplus(...)
    "g_positive": 3,      # the minus sign dropped
    "beta_tanh": 4,       # tanh instead of the logistic sigmoid
}


def _widen(a, bf16):
    a = np.asarray(a)
    if bf16:
        if a.dtype != np.uint16:
            raise ValueError("bf16 data must be passed as raw uint16 bit patterns")
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _sigmoid(u):
    with np.errstate(over="ignore"):  # e^{-u} = inf gives the exact limit 0
        return 1.0 / (1.0 + np.exp(-u))


def short_conv_silu(x, weight, cu_seqlens=None, conv_state=None, bf16=False, mutation=0):
    """Causal depthwise convolution of kernel size 4 followed by SiLU (App. A.3,
    the paragraph under Table 8), over packed sequences.

    x:          [T, C] stored inputs (raw bf16 bits as uint16 when ``bf16``);
                C is the flattened (head, channel) axis, H * d.
    weight:     [C, 4] taps, oldest first: tap 3 multiplies the current token,
                tap 0 the token three back.
    cu_seqlens: int [N + 1] or None (one sequence).
    conv_state: [N, 3, C] the three inputs before each sequence, oldest first,
                in the storage type of x; None means zeros.
    Returns (y [T, C] fp64, state_out [N, 3, C] fp64): state_out holds the last
    three inputs of each sequence (reaching into conv_state when the sequence
    has fewer than three tokens).
    """
    xx = _widen(x, bf16)
    if xx.ndim != 2:
        raise ValueError("x must be [T, C]")
    T, C = xx.shape
    w = np.asarray(weight, dtype=np.float64)
    if w.shape != (C, 4):
        raise ValueError("weight must be [C, 4]")
    if mutation == 1:
        w = w[:, ::-1]
    cu = np.array([0, T], dtype=np.int64) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    N = cu.shape[0] - 1
    if cu[0] != 0 or cu[-1] != T or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must rise from 0 to T")
    if conv_state is None or mutation == 4:
        st = np.zeros((N, 3, C))
    else:
        st = _widen(conv_state, bf16)
        if st.shape != (N, 3, C):
            raise ValueError("conv_state must be [N, 3, C]")
    src = _sigmoid(xx) * xx if mutation == 3 else xx
    y = np.empty((T, C))
    st_out = np.empty((N, 3, C))
    prev_tail = st[0] if N > 0 else None
    for n in range(N):
        s, e = int(cu[n]), int(cu[n + 1])
        L = e - s
        before = prev_tail if mutation == 5 else st[n]
        # hist row i holds the input at position i - 3 of this sequence
        hist = np.concatenate([before, src[s:e]], axis=0)
        acc = np.zeros((L, C))
        for j in range(4):  # tap j multiplies the input 3 - j tokens back
            acc += w[:, j] * hist[j:j + L]
        y[s:e] = acc if mutation in (2, 3) else acc * _sigmoid(acc)
        st_out[n] = hist[L:L + 3]
        prev_tail = hist[L:L + 3]
    return y, st_out


def gates(a, b, A_log, dt_bias, mutation=0):
    """Forget gate and write strength of App. A.3 (the paragraph after Eq. 21):

        g_t    = -exp(A_log[h]) * softplus(a[t, h] + dt_bias[h])   (log of alpha_t, <= 0)
        beta_t = sigmoid(b[t, h])

    a = W_alpha x_t and b = W_beta x_t are [T, H] (any float dtype); A_log and
    dt_bias are [H].  Returns (g, beta), fp64 [T, H].
    """
    aa = np.asarray(a, dtype=np.float64)
    bb = np.asarray(b, dtype=np.float64)
    al = np.asarray(A_log, dtype=np.float64)
    db = np.asarray(dt_bias, dtype=np.float64)
    u = aa if mutation == 1 else aa + db
    sp = np.logaddexp(0.0, u)  # log(1 + e^u) without overflow
    scale = al if mutation == 2 else np.exp(al)
    g = scale * sp if mutation == 3 else -scale * sp
    beta = np.tanh(bb) if mutation == 4 else _sigmoid(bb)
    return g, beta
