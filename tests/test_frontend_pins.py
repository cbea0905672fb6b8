"""Pins of the front-end oracle (``oracle/frontend.py``): the short causal
convolution with SiLU and the gate math of "Long-Context Aware Upcycling"
(arXiv:2604.24715), App. A.3 (the paragraph under Table 8, and the paragraph
after Eq. 21).  Each check ties the oracle to something other than itself: a
library convolution and logistic function, impulse responses, composition
laws, and closed forms of softplus and the logistic function.  Each planted
misreading must fail at least one check."""
import math

import numpy as np
import pytest
from scipy.special import expit

import oracle


def _silu(u):
    return u * expit(u)  # scipy's logistic function: an independent evaluation


def _rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------- convolution

def check_conv_matches_numpy_convolve(mutation=0):
    """One sequence from zero history: channel c is silu(np.convolve(x_c, taps_c reversed))
    truncated to the first T outputs (numpy's full convolution pads with zeros)."""
    r = _rng(11)
    T, C = 37, 5
    x = r.standard_normal((T, C))
    w = r.standard_normal((C, 4))
    y, _ = oracle.short_conv_silu(x, w, mutation=mutation)
    ref = np.stack([np.convolve(x[:, c], w[c, ::-1])[:T] for c in range(C)], axis=1)
    return bool(np.allclose(y, _silu(ref), rtol=1e-13, atol=1e-14))


def check_conv_impulse_response(mutation=0):
    """A unit impulse at token 5 of channel 2 gives silu(tap 3), silu(tap 2), silu(tap 1),
    silu(tap 0) at tokens 5..8 of that channel and exactly 0 everywhere else."""
    T, C = 12, 4
    x = np.zeros((T, C))
    x[5, 2] = 1.0
    w = np.arange(1.0, 1.0 + 4 * C).reshape(C, 4) / 7.0
    y, _ = oracle.short_conv_silu(x, w, mutation=mutation)
    ref = np.zeros((T, C))
    for m in range(4):
        ref[5 + m, 2] = _silu(w[2, 3 - m])
    return bool(np.array_equal(y == 0.0, ref == 0.0) and np.allclose(y, ref, rtol=1e-14, atol=0))


def check_conv_continuation(mutation=0):
    """Convolving [0, T) equals convolving [0, T1) and then [T1, T) from the returned
    state, for split points shorter and longer than the kernel."""
    r = _rng(12)
    T, C = 20, 3
    x = r.standard_normal((T, C))
    w = r.standard_normal((C, 4))
    st0 = r.standard_normal((1, 3, C))
    y, s = oracle.short_conv_silu(x, w, conv_state=st0, mutation=mutation)
    ok = True
    for T1 in (1, 2, 3, 11):
        y1, s1 = oracle.short_conv_silu(x[:T1], w, conv_state=st0, mutation=mutation)
        y2, s2 = oracle.short_conv_silu(x[T1:], w, conv_state=s1, mutation=mutation)
        ok &= np.allclose(np.concatenate([y1, y2]), y, rtol=1e-14, atol=1e-15)
        ok &= np.allclose(s2, s, rtol=0, atol=0)
    # two one-token steps from the state equal a two-token call
    ya, sa = oracle.short_conv_silu(x[:1], w, conv_state=st0, mutation=mutation)
    yb, sb = oracle.short_conv_silu(x[1:2], w, conv_state=sa, mutation=mutation)
    yab, sab = oracle.short_conv_silu(x[:2], w, conv_state=st0, mutation=mutation)
    ok &= np.allclose(np.concatenate([ya, yb]), yab, rtol=1e-14, atol=0) and np.array_equal(sb, sab)
    return bool(ok)


def check_conv_packing(mutation=0):
    """A packed batch (lengths 6, 0, 2, 9) equals four separate calls, each from its own
    state; the returned state of a 2-token sequence reaches into the given state."""
    r = _rng(13)
    lens = [6, 0, 2, 9]
    cu = np.concatenate([[0], np.cumsum(lens)])
    C = 4
    x = r.standard_normal((int(cu[-1]), C))
    w = r.standard_normal((C, 4))
    st = r.standard_normal((len(lens), 3, C))
    y, s = oracle.short_conv_silu(x, w, cu_seqlens=cu, conv_state=st, mutation=mutation)
    ok = True
    for n in range(len(lens)):
        yn, sn = oracle.short_conv_silu(x[cu[n]:cu[n + 1]], w, conv_state=st[n:n + 1], mutation=mutation)
        ok &= np.allclose(y[cu[n]:cu[n + 1]], yn, rtol=0, atol=0) and np.array_equal(s[n], sn[0])
    # the state is the last three inputs of the sequence, in order
    ok &= np.array_equal(s[0], x[3:6]) and np.array_equal(s[1], st[1])
    ok &= np.array_equal(s[2], np.concatenate([st[2][2:], x[6:8]]))
    return bool(ok)


def check_conv_silu_identities(mutation=0):
    """With only the current-token tap set to 1 the output is silu(x): silu(0) = 0,
    silu(u) - silu(-u) = u, and silu(u) -> u for large u."""
    u = np.array([[0.0, 0.5, -0.5, 3.0, -3.0, 40.0]])
    x = np.concatenate([u, -u])
    w = np.tile([0.0, 0.0, 0.0, 1.0], (u.shape[1], 1))
    y, _ = oracle.short_conv_silu(x, w, mutation=mutation)
    ok = y[0, 0] == 0.0
    ok &= np.allclose(y[0] - y[1], u[0], rtol=1e-15, atol=1e-15)
    ok &= abs(y[0, 5] - 40.0) < 1e-15 * 40 + 40.0 * math.exp(-40.0) * 1.01
    return bool(ok)


CONV_CHECKS = [check_conv_matches_numpy_convolve, check_conv_impulse_response, check_conv_continuation,
               check_conv_packing, check_conv_silu_identities]


@pytest.mark.parametrize("check", CONV_CHECKS, ids=lambda c: c.__name__)
def test_conv_pin(check):
    assert check()


@pytest.mark.parametrize("name", sorted(oracle.CONV_MUTATIONS))
def test_conv_planted_mistakes_are_caught(name):
    m = oracle.CONV_MUTATIONS[name]
    assert not all(check(mutation=m) for check in CONV_CHECKS), name


def test_conv_bf16_inputs_are_widened_exactly():
    """bf16 inputs are the stored bit patterns: 0x3F80 is 1.0, 0xC000 is -2.0."""
    x = np.array([[0x3F80], [0xC000]], dtype=np.uint16)
    w = np.array([[0.0, 0.0, 0.5, 1.0]])
    y, s = oracle.short_conv_silu(x, w, bf16=True)
    assert np.allclose(y[:, 0], _silu(np.array([1.0, -2.0 + 0.5])), rtol=1e-15, atol=0)
    assert np.array_equal(s[0, :, 0], [0.0, 1.0, -2.0])


# ----------------------------------------------------------------- gates

def check_gate_half(mutation=0):
    """A_log = 0 and a = -dt_bias give softplus(0) = ln 2, so alpha = e^g = 1/2; the
    logistic function gives beta = 1/2 at 0 and 3/4 at ln 3."""
    H = 3
    db = np.array([0.7, -1.2, 2.0])
    g, beta = oracle.gates(-db[None, :], np.array([[0.0, math.log(3.0), 0.0]]), np.zeros(H), db,
                           mutation=mutation)
    return bool(np.allclose(np.exp(g), 0.5, rtol=1e-15, atol=0)
                and np.allclose(beta, [[0.5, 0.75, 0.5]], rtol=1e-15, atol=0))


def check_gate_softplus_difference(mutation=0):
    """A_log = 0: softplus(u) - softplus(-u) = u, so g at a and at a' = -a - 2 dt_bias
    differ by exactly -(a + dt_bias); every g is < 0."""
    r = _rng(14)
    T, H = 7, 4
    a = r.standard_normal((T, H)) * 3
    db = r.standard_normal(H)
    b = r.standard_normal((T, H))
    g1, _ = oracle.gates(a, b, np.zeros(H), db, mutation=mutation)
    g2, _ = oracle.gates(-a - 2 * db, b, np.zeros(H), db, mutation=mutation)
    return bool(np.allclose(g1 - g2, -(a + db), rtol=1e-13, atol=1e-13) and np.all(g1 < 0))


def check_gate_A_log_scaling(mutation=0):
    """g is linear in exp(A_log): A_log = ln 3 triples g; beta does not depend on it."""
    r = _rng(15)
    T, H = 5, 2
    a, b, db = r.standard_normal((T, H)), r.standard_normal((T, H)), r.standard_normal(H)
    g0, b0 = oracle.gates(a, b, np.zeros(H), db, mutation=mutation)
    g3, b3 = oracle.gates(a, b, np.full(H, math.log(3.0)), db, mutation=mutation)
    return bool(np.allclose(g3, 3.0 * g0, rtol=1e-14, atol=0) and np.array_equal(b0, b3))


def check_gate_library_logistic(mutation=0):
    """beta equals scipy's logistic function; 1 - beta(b) = beta(-b)."""
    r = _rng(16)
    b = r.standard_normal((9, 3)) * 4
    _, beta = oracle.gates(np.zeros((9, 3)), b, np.zeros(3), np.zeros(3), mutation=mutation)
    _, beta_m = oracle.gates(np.zeros((9, 3)), -b, np.zeros(3), np.zeros(3), mutation=mutation)
    return bool(np.allclose(beta, expit(b), rtol=1e-15, atol=0) and np.allclose(beta + beta_m, 1.0, atol=1e-15))


GATE_CHECKS = [check_gate_half, check_gate_softplus_difference, check_gate_A_log_scaling,
               check_gate_library_logistic]


@pytest.mark.parametrize("check", GATE_CHECKS, ids=lambda c: c.__name__)
def test_gate_pin(check):
    assert check()


@pytest.mark.parametrize("name", sorted(oracle.GATE_MUTATIONS))
def test_gate_planted_mistakes_are_caught(name):
    m = oracle.GATE_MUTATIONS[name]
    assert not all(check(mutation=m) for check in GATE_CHECKS), name


def test_gates_do_not_overflow():
    """softplus of large arguments stays finite and equals the argument."""
    g, beta = oracle.gates(np.array([[800.0, -800.0]]), np.array([[800.0, -800.0]]), np.zeros(2), np.zeros(2))
    assert g[0, 0] == -800.0 and -1e-300 < g[0, 1] <= 0.0
    assert beta[0, 0] == 1.0 and beta[0, 1] == 0.0
