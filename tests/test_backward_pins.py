"""Pins of the gradient oracle (``oracle/backward.py``): the vector-Jacobian
product of the gated delta rule ("Long-Context Aware Upcycling", App. A.3,
Eqs. 16-19).  It is tied to the forward oracle (the C recurrence, which shares
no code with it) by central finite differences, and to closed forms.  Each
planted mistake must fail a pin."""
import numpy as np
import pytest

import oracle


def _case(seed, l2=True):
    rng = np.random.default_rng(seed)
    cu = np.array([0, 4, 7], dtype=np.int64)
    T, H, dk, dv = 7, 2, 3, 2
    x = dict(q=rng.standard_normal((T, H, dk)), k=rng.standard_normal((T, H, dk)),
             v=rng.standard_normal((T, H, dv)), g=-rng.uniform(0.1, 1.0, (T, H)),
             beta=rng.uniform(0.2, 0.9, (T, H)), init=rng.standard_normal((2, H, dv, dk)) * 0.5)
    do = rng.standard_normal((T, H, dv))
    ds = rng.standard_normal((2, H, dv, dk))
    return x, do, ds, cu


def _loss(x, do, ds, cu, l2):
    o, fs = oracle.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], x["init"], cu_seqlens=cu, qk_l2norm=l2,
                           n_threads=1)
    return float(np.sum(do * o) + np.sum(ds * fs))


def check_finite_differences(mutation=0, l2=True):
    """Central differences (h = 1e-5) of L = <do, o> + <dS, S_final> through the
    forward oracle agree with the gradient oracle for every input element."""
    x, do, ds, cu = _case(3, l2)
    gr = oracle.prefill_vjp(x["q"], x["k"], x["v"], x["g"], x["beta"], do, ds, x["init"], cu_seqlens=cu,
                            qk_l2norm=l2, mutation=mutation)
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "init": "dinit"}
    h = 1e-5
    worst = 0.0
    for key, gkey in names.items():
        a = x[key]
        fd = np.zeros_like(a)
        for idx in np.ndindex(a.shape):
            old = a[idx]
            a[idx] = old + h
            lp = _loss(x, do, ds, cu, l2)
            a[idx] = old - h
            lm = _loss(x, do, ds, cu, l2)
            a[idx] = old
            fd[idx] = (lp - lm) / (2 * h)
        worst = max(worst, float(np.max(np.abs(fd - gr[gkey]))) / max(1.0, float(np.max(np.abs(fd)))))
    return worst < 1e-7


def check_identity_gates_closed_form(mutation=0):
    """alpha = 1, beta = 0, no normalisation: the state never changes, so
    dS_0 = dS_N + scale sum_t do_t q_t^T, dq_t = scale S_0^T do_t, dv = 0."""
    x, do, ds, cu = _case(4, False)
    x["g"][:] = 0.0
    x["beta"][:] = 0.0
    scale = 0.7
    gr = oracle.prefill_vjp(x["q"], x["k"], x["v"], x["g"], x["beta"], do, ds, x["init"], cu_seqlens=cu,
                            scale=scale, qk_l2norm=False, mutation=mutation)
    ok = np.allclose(gr["dv"], 0.0, atol=0)
    for n in range(2):
        s, e = cu[n], cu[n + 1]
        for hh in range(2):
            ref = ds[n, hh] + scale * sum(np.outer(do[t, hh], x["q"][t, hh]) for t in range(s, e))
            ok &= np.allclose(gr["dinit"][n, hh], ref, rtol=1e-13, atol=1e-13)
            for t in range(s, e):
                ok &= np.allclose(gr["dq"][t, hh], scale * x["init"][n, hh].T @ do[t, hh], rtol=1e-13, atol=1e-13)
    return bool(ok)


def check_normalised_grads_are_orthogonal(mutation=0):
    """With eps = 0 the outputs do not change when q_t or k_t is scaled, so each
    dq_t is orthogonal to q_t and each dk_t to k_t."""
    x, do, ds, cu = _case(5)
    gr = oracle.prefill_vjp(x["q"], x["k"], x["v"], x["g"], x["beta"], do, ds, x["init"], cu_seqlens=cu, eps=0.0,
                            mutation=mutation)
    dots = [np.sum(gr["dq"] * x["q"], axis=-1), np.sum(gr["dk"] * x["k"], axis=-1)]
    mags = max(float(np.max(np.abs(gr["dq"]))), float(np.max(np.abs(gr["dk"]))))
    return bool(max(float(np.max(np.abs(d))) for d in dots) < 1e-12 * max(1.0, mags))


BWD_CHECKS = [check_finite_differences, check_identity_gates_closed_form, check_normalised_grads_are_orthogonal]


@pytest.mark.parametrize("check", BWD_CHECKS, ids=lambda c: c.__name__)
def test_backward_pin(check):
    assert check()


def test_finite_differences_without_normalisation():
    assert check_finite_differences(l2=False)


@pytest.mark.parametrize("name", sorted(oracle.BWD_MUTATIONS))
def test_backward_planted_mistakes_are_caught(name):
    m = oracle.BWD_MUTATIONS[name]
    assert not all(check(mutation=m) for check in BWD_CHECKS), name


@pytest.mark.parametrize("C", [1, 3, 16, 64])
def test_chunked_wy_backward_matches_token_gradients(C):
    """Differentiating the chunked WY form (the form a chunked backward kernel
    evaluates) gives the gradients of the token recurrence for any chunk size:
    chunking changes the order of the arithmetic, not the map."""
    from oracle import forms

    rng = np.random.default_rng(40 + C)
    T, dk, dv = 50, 5, 3
    q, k = rng.standard_normal((T, dk)), rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    g, beta = -rng.uniform(0.0, 0.5, T), rng.uniform(0.1, 0.9, T)
    S0 = rng.standard_normal((dv, dk)) * 0.5
    dO, dS = rng.standard_normal((T, dv)), rng.standard_normal((dv, dk))
    scale = 0.6
    got = forms.chunked_wy_vjp(q, k, v, g, beta, S0, scale, C, dO, dS)
    ref = oracle.prefill_vjp(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None], dO[:, None], dS[None, None],
                             S0[None, None], scale=scale, qk_l2norm=False)
    names = ("dq", "dk", "dv", "dg", "dbeta")
    for x, name in zip(got[:5], names):
        r = ref[name][:, 0]
        assert np.allclose(x, r, rtol=1e-10, atol=1e-10 * np.max(np.abs(r))), name
    assert np.allclose(got[5], ref["dinit"][0, 0], rtol=1e-10, atol=1e-10)


def test_chain_fold_identity():
    """The state chain's next product without the next state: with
    Y_{c+1} = W_{c+1} S_c^T and M_{c+1} = W_{c+1} K_c^T diag(e^{gamma_L - gamma}),
    W_{c+1} S_{c+1}^T = e^{gamma_L} Y_{c+1} + M_{c+1} Delta_c (chunked WY form)."""
    from oracle import forms

    rng = np.random.default_rng(9)
    T, dk, dv, C = 200, 8, 6, 32
    q = forms.l2_normalise(rng.standard_normal((T, dk)))
    k = forms.l2_normalise(rng.standard_normal((T, dk)))
    v = rng.standard_normal((T, dv))
    g, beta = -rng.uniform(0.0, 0.3, T), rng.uniform(0.1, 0.9, T)
    _, _, ch = forms.chunked_wy(q, k, v, g, beta, rng.standard_normal((dv, dk)), 0.5, C)
    for c in range(len(ch) - 1):
        a, n = ch[c], ch[c + 1]
        K = k[c * C:(c + 1) * C]
        M = n["W"] @ (np.exp(a["gamma"][-1] - a["gamma"])[:, None] * K).T
        lhs = n["W"] @ n["S_start"].T
        rhs = np.exp(a["gamma"][-1]) * (n["W"] @ a["S_start"].T) + M @ a["Delta"]
        assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12), c


def test_chunk_gradients_chain_recurrence():
    """The per-chunk outputs of the reverse state-gradient chain satisfy its
    recurrence: dS before chunk c = e^{gamma_L} dS_after + dO'^T diag(e^gamma) Q
    - dDelta^T W, and the first one equals the initial-state gradient."""
    from oracle import forms

    rng = np.random.default_rng(10)
    T, dk, dv, C, scale = 100, 5, 4, 16, 0.7
    q, k = rng.standard_normal((T, dk)), rng.standard_normal((T, dk))
    v = rng.standard_normal((T, dv))
    g, beta = -rng.uniform(0.0, 0.5, T), rng.uniform(0.1, 0.9, T)
    S0, dO, dS = rng.standard_normal((dv, dk)), rng.standard_normal((T, dv)), rng.standard_normal((dv, dk))
    cg = []
    out = forms.chunked_wy_vjp(q, k, v, g, beta, S0, scale, C, dO, dS, chunk_grads=cg)
    _, _, ch = forms.chunked_wy(q, k, v, g, beta, S0, scale, C)
    assert len(cg) == len(ch) and np.array_equal(cg[-1]["dS_after"], dS)
    for c in range(len(ch)):
        gam = ch[c]["gamma"]
        Q = q[c * C:c * C + gam.shape[0]]
        dOs = scale * dO[c * C:c * C + gam.shape[0]]
        before = np.exp(gam[-1]) * cg[c]["dS_after"] + dOs.T @ (np.exp(gam)[:, None] * Q) - cg[c]["dDelta"].T @ ch[c]["W"]
        expect = out[5] if c == 0 else cg[c - 1]["dS_after"]
        assert np.allclose(before, expect, rtol=1e-12, atol=1e-12), c
