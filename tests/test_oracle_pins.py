"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Every equation cited is from "Long-Context Aware Upcycling: A New Frontier for
Hybrid LLM Scaling" (arXiv:2604.24715), App. A.3 "GDN Layer Architecture",
Eqs. 16-19 (decay, delta correction, write, read) and the gate domains stated
below them.  No check here re-types the oracle's own loop: each compares it
with a hand-derived example, a closed form, an invariant of the map, or an
independent evaluation (unrolled product form, chunked WY form).

``test_planted_mistakes_are_caught`` runs the same checks against deliberate
misreadings planted in the oracle and asserts each one fails at least one pin.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import forms
from _util import load_golden

pytestmark = pytest.mark.usefixtures("oracle_lib")

RNG = np.random.default_rng(12345)


def _rand_case(T, H, dk, dv, seed, gate="default", init=True, N=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    if gate == "default":
        g = -np.logaddexp(0.0, rng.standard_normal((T, H)) + 2.0)
    else:
        g = -rng.uniform(0.0, 0.05, (T, H))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    Nn = 1 if N is None else N
    S0 = rng.standard_normal((Nn, H, dv, dk)) * 0.3 if init else None
    return q, k, v, g, beta, S0


# ----------------------------------------------------------------------------- checks
# Each returns True when the pin holds; the planted-mistake test reuses them.

def check_hand_examples(mutation=0):
    ok = True
    for ex in load_golden("hand_examples.json")["examples"]:
        T, H, dk, dv = ex["T"], ex["H"], ex["dk"], ex["dv"]
        q = np.array(ex["q"], dtype=np.float64).reshape(T, H, dk)
        k = np.array(ex["k"], dtype=np.float64).reshape(T, H, dk)
        v = np.array(ex["v"], dtype=np.float64).reshape(T, H, dv)
        g = np.log(np.array(ex["alpha"], dtype=np.float64)).reshape(T, H)
        beta = np.array(ex["beta"], dtype=np.float64).reshape(T, H)
        S0 = None if ex["init_state"] is None else np.array(ex["init_state"], dtype=np.float64).reshape(1, H, dv, dk)
        o, fs = oracle.prefill(q, k, v, g, beta, S0, scale=ex["scale"], qk_l2norm=ex["qk_l2norm"],
                               eps=ex["eps"], mutation=mutation)
        ok &= np.allclose(o.reshape(T, dv), np.array(ex["o"]), rtol=0, atol=1e-12)
        ok &= np.allclose(fs.reshape(dv, dk), np.array(ex["final_state"]), rtol=0, atol=1e-12)
    return bool(ok)


def check_identity_gates(mutation=0):
    """alpha=1, beta=0: nothing is written or forgotten, S_t = S_0, o_t = scale S_0 qhat_t."""
    q, k, v, _, _, S0 = _rand_case(40, 2, 7, 5, 1)
    g = np.zeros((40, 2))
    beta = np.zeros((40, 2))
    o, fs = oracle.prefill(q, k, v, g, beta, S0, scale=0.7, mutation=mutation)
    qh = forms.l2_normalise(q)
    ref = 0.7 * np.einsum("hij,thj->thi", S0[0], qh)
    return bool(np.allclose(fs, S0, rtol=0, atol=1e-14) and np.allclose(o, ref, rtol=0, atol=1e-13))


def check_exact_recall(mutation=0):
    """alpha=1, beta=1, unit k: after the write, S_t k_t = v_t exactly (the delta rule
    replaces the value stored under k_t)."""
    ok = True
    q, k, v, _, _, S0 = _rand_case(12, 1, 6, 4, 2)
    kh = forms.l2_normalise(k, eps=0.0)
    g = np.zeros((12, 1))
    beta = np.ones((12, 1))
    for T in (1, 5, 12):
        _, fs = oracle.prefill(q[:T], kh[:T], v[:T], g[:T], beta[:T], S0, qk_l2norm=False, mutation=mutation)
        ok &= np.allclose(fs[0, 0] @ kh[T - 1, 0], v[T - 1, 0], rtol=0, atol=1e-13)
    return bool(ok)


def check_unrolled_product(mutation=0):
    """Sequential recurrence == unrolled product form (independent evaluation, O(T^2 d))."""
    ok = True
    for seed, (T, dk, dv, l2, gate) in enumerate([(33, 5, 7, True, "default"), (48, 8, 3, False, "slow"),
                                                   (20, 16, 16, True, "slow")]):
        q, k, v, g, beta, S0 = _rand_case(T, 2, dk, dv, 10 + seed, gate=gate)
        o, _ = oracle.prefill(q, k, v, g, beta, S0, scale=0.37, qk_l2norm=l2, eps=1e-6, mutation=mutation)
        for h in range(2):
            qq = forms.l2_normalise(q[:, h]) if l2 else q[:, h]
            kk = forms.l2_normalise(k[:, h]) if l2 else k[:, h]
            ref = forms.unrolled_product(qq, kk, v[:, h], g[:, h], beta[:, h], S0[0, h], 0.37)
            ok &= np.max(np.abs(o[:, h] - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
    return bool(ok)


def check_reset(mutation=0):
    """g = -1e3 makes alpha = 0 exactly in fp64: S_t = beta_t v_t khat_t^T, o_t = scale beta_t (khat.qhat) v_t."""
    q, k, v, _, beta, S0 = _rand_case(9, 2, 4, 6, 3)
    g = np.full((9, 2), -1e3)
    o, fs = oracle.prefill(q, k, v, g, beta, S0, scale=1.3, mutation=mutation)
    qh, kh = forms.l2_normalise(q), forms.l2_normalise(k)
    ref_o = 1.3 * beta[..., None] * np.sum(qh * kh, -1)[..., None] * v
    ref_s = beta[-1][:, None, None] * v[-1][:, :, None] * kh[-1][:, None, :]
    return bool(np.allclose(o, ref_o, rtol=0, atol=1e-13) and np.allclose(fs[0], ref_s, rtol=0, atol=1e-13))


def check_associative_memory(mutation=0):
    """Orthonormal keys, alpha=1, beta=1, S_0=0: S_T k_j = v_j for every j <= T <= d_k."""
    rng = np.random.default_rng(4)
    dk, dv, T = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:, :T].T.reshape(T, 1, dk)
    v = rng.standard_normal((T, 1, dv))
    q = rng.standard_normal((T, 1, dk))
    _, fs = oracle.prefill(q, k, v, np.zeros((T, 1)), np.ones((T, 1)), None, qk_l2norm=False, mutation=mutation)
    return bool(np.allclose(fs[0, 0] @ k[:, 0].T, v[:, 0].T, rtol=0, atol=1e-13))


def check_ema_closed_form(mutation=0):
    """d_k = 1 with k = +-1: the state is an exponential moving average,
    s_t = alpha_t (1 - beta_t) s_{t-1} + beta_t k_t v_t, closed form by product of factors."""
    rng = np.random.default_rng(5)
    T, dv = 25, 3
    k = np.where(rng.random((T, 1, 1)) < 0.5, -1.0, 1.0)
    q = np.where(rng.random((T, 1, 1)) < 0.5, -2.0, 2.0)
    v = rng.standard_normal((T, 1, dv))
    g = -rng.uniform(0, 1, (T, 1))
    beta = rng.uniform(0, 1, (T, 1))
    s0 = rng.standard_normal((1, 1, dv, 1))
    o, fs = oracle.prefill(q, k, v, g, beta, s0, scale=1.0, qk_l2norm=False, mutation=mutation)
    ok = True
    for t in range(T):
        # s_t = s0 prod_{m<=t} f_m + sum_{j<=t} beta_j k_j v_j prod_{j<m<=t} f_m, f_m = alpha_m (1 - beta_m)
        f = np.exp(g[:, 0]) * (1.0 - beta[:, 0])
        s = s0[0, 0, :, 0] * np.prod(f[:t + 1])
        for j in range(t + 1):
            s = s + beta[j, 0] * k[j, 0, 0] * v[j, 0] * np.prod(f[j + 1:t + 1])
        ok &= np.allclose(o[t, 0], s * q[t, 0, 0], rtol=0, atol=1e-12)
        if t == T - 1:
            ok &= np.allclose(fs[0, 0, :, 0], s, rtol=0, atol=1e-12)
    return bool(ok)


def check_normalisation_invariance(mutation=0):
    """With eps = 0, scaling q_t and k_t by positive constants leaves o unchanged."""
    q, k, v, g, beta, S0 = _rand_case(16, 1, 6, 4, 6)
    rng = np.random.default_rng(60)
    cq = rng.uniform(0.1, 10, (16, 1, 1))
    ck = rng.uniform(0.1, 10, (16, 1, 1))
    o1, f1 = oracle.prefill(q, k, v, g, beta, S0, qk_l2norm=True, eps=0.0, mutation=mutation)
    o2, f2 = oracle.prefill(q * cq, k * ck, v, g, beta, S0, qk_l2norm=True, eps=0.0, mutation=mutation)
    return bool(np.allclose(o1, o2, rtol=0, atol=1e-13) and np.allclose(f1, f2, rtol=0, atol=1e-13))


ALL_CHECKS = [check_hand_examples, check_identity_gates, check_exact_recall, check_unrolled_product,
              check_reset, check_associative_memory, check_ema_closed_form, check_normalisation_invariance]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    assert check()


@pytest.mark.parametrize("name", sorted(oracle.MUTATIONS))
def test_planted_mistakes_are_caught(name):
    m = oracle.MUTATIONS[name]
    failed = [c.__name__ for c in ALL_CHECKS if not c(mutation=m)]
    assert failed, f"planted mistake {name!r} passed every pin"


# ----------------------------------------------------------------------------- structure

@pytest.mark.parametrize("C", [1, 2, 4, 16, 64])
def test_chunked_wy_matches_sequential(C):
    """The chunked WY evaluation (App. A.3, last paragraph) reaches the sequential result
    for any chunk size, including ragged last chunks; at C=1 it is the recurrence itself."""
    T, dk, dv = 150, 16, 12
    for gate in ("default", "slow"):
        q, k, v, g, beta, S0 = _rand_case(T, 1, dk, dv, 20 + C, gate=gate)
        o, fs = oracle.prefill(q, k, v, g, beta, S0, scale=0.25)
        qh, kh = forms.l2_normalise(q[:, 0]), forms.l2_normalise(k[:, 0])
        oc, sc, chunks = forms.chunked_wy(qh, kh, v[:, 0], g[:, 0], beta[:, 0], S0[0, 0], 0.25, C)
        scale_o = max(1.0, np.max(np.abs(o)))
        assert np.max(np.abs(oc - o[:, 0])) <= 1e-11 * scale_o
        assert np.max(np.abs(sc - fs[0, 0])) <= 1e-11 * max(1.0, np.max(np.abs(fs)))
        for ch in chunks:  # (I + A) T = I, textbook residual of the triangular inverse
            L = ch["A"].shape[0]
            assert np.max(np.abs((np.eye(L) + ch["A"]) @ ch["T"] - np.eye(L))) <= 1e-13


def test_continuation():
    """prefill [0,T) == prefill [0,T1) then [T1,T) from the carried state."""
    q, k, v, g, beta, S0 = _rand_case(90, 3, 8, 5, 7, gate="slow")
    o, fs = oracle.prefill(q, k, v, g, beta, S0)
    for T1 in (1, 37, 89):
        o1, f1 = oracle.prefill(q[:T1], k[:T1], v[:T1], g[:T1], beta[:T1], S0)
        o2, f2 = oracle.prefill(q[T1:], k[T1:], v[T1:], g[T1:], beta[T1:], f1)
        assert np.array_equal(np.concatenate([o1, o2]), o)
        assert np.array_equal(f2, fs)


def test_varlen_packing_has_no_leak():
    """A packed run equals separate per-sequence calls."""
    lens = [5, 1, 30, 17]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v, g, beta, S0 = _rand_case(T, 2, 6, 4, 8, gate="slow", N=len(lens))
    o, fs = oracle.prefill(q, k, v, g, beta, S0, cu_seqlens=cu)
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        on, fn = oracle.prefill(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], S0[n:n + 1])
        assert np.array_equal(o[a:b], on)
        assert np.array_equal(fs[n:n + 1], fn)


def test_decode_after_prefill_equals_longer_prefill():
    q, k, v, g, beta, S0 = _rand_case(40, 2, 8, 6, 9, gate="slow")
    o, fs = oracle.prefill(q, k, v, g, beta, S0, scale=0.5)
    _, st = oracle.prefill(q[:33], k[:33], v[:33], g[:33], beta[:33], S0, scale=0.5)
    st = np.ascontiguousarray(st)
    for t in range(33, 40):
        od = oracle.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1], st, scale=0.5)
        assert np.array_equal(od[0], o[t])
    assert np.array_equal(st, fs)


def test_linearity_in_values_and_state():
    """o and S_T are linear in (V, S_0) jointly; o scales with the read scale."""
    q, k, v, g, beta, S0 = _rand_case(30, 1, 5, 4, 11)
    _, _, v2, _, _, S02 = _rand_case(30, 1, 5, 4, 12)
    a, b = 0.7, -1.9
    o1, f1 = oracle.prefill(q, k, v, g, beta, S0, scale=1.0)
    o2, f2 = oracle.prefill(q, k, v2, g, beta, S02, scale=1.0)
    o3, f3 = oracle.prefill(q, k, a * v + b * v2, g, beta, a * S0 + b * S02, scale=1.0)
    assert np.allclose(o3, a * o1 + b * o2, rtol=0, atol=1e-12)
    assert np.allclose(f3, a * f1 + b * f2, rtol=0, atol=1e-12)
    o4, _ = oracle.prefill(q, k, v, g, beta, S0, scale=0.125)
    assert np.allclose(o4, 0.125 * o1, rtol=0, atol=1e-14)


def test_row_subset_and_threads_agree():
    q, k, v, g, beta, S0 = _rand_case(64, 4, 8, 12, 13)
    o, fs = oracle.prefill(q, k, v, g, beta, S0, n_threads=1)
    o8, fs8 = oracle.prefill(q, k, v, g, beta, S0, n_threads=8)
    assert np.array_equal(o, o8) and np.array_equal(fs, fs8)
    rows = [0, 5, 11]
    osub, fsub = oracle.prefill(q, k, v, g, beta, S0, rows=rows)
    assert np.array_equal(osub[:, :, rows], o[:, :, rows])
    assert np.array_equal(fsub[:, :, rows], fs[:, :, rows])
    assert np.all(np.isnan(np.delete(osub, rows, axis=2)))


def test_bf16_inputs_are_widened_exactly():
    from hybrid_linear_attention_delta_amd import synth

    inp = synth.prefill_inputs(20, 2, 8, 8, "bf16", seed=5)
    o1, f1 = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, bf16=True)
    wid = [synth.bf16_to_f32(x).astype(np.float64) for x in (inp.q, inp.k, inp.v)]
    o2, f2 = oracle.prefill(*wid, inp.g, inp.beta)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


def test_bf16_rounding_is_nearest_even():
    from hybrid_linear_attention_delta_amd import synth

    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa -> 1.0
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: even -> 1 + 2^-6
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -30, -2.5, 0.0])
    got = synth.bf16_to_f32(synth.f64_to_bf16_bits(x)).astype(np.float64)
    want = np.array([1.0, 1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -2.5, 0.0])
    assert np.array_equal(got, want)


def test_bad_arguments_are_rejected():
    q, k, v, g, beta, S0 = _rand_case(8, 1, 4, 4, 14)
    with pytest.raises(ValueError):
        oracle.prefill(q, k, v, g, beta, S0, cu_seqlens=[0, 5, 7])
    with pytest.raises(RuntimeError):
        oracle.prefill(q, k, v, g, beta, S0, rows=[4])
    assert math.isclose(1.0 / math.sqrt(4), 0.5)


# ----------------------------------------------------------------- gated RMSNorm read-out (Eq. 20)

def check_norm_constant_rows(mutation=0):
    """A row of equal values c with weight w and gate z: y = c / sqrt(c^2 + eps) * w * silu(z),
    with silu(z) = z / (1 + e^{-z}) written out by hand for z = 0 (0), z = ln 3 (0.75 ln 3)
    and z = -ln 3 (-0.25 ln 3)."""
    eps = 1e-3
    c = np.array([0.02, -0.5, 3.0])[:, None, None] * np.ones((3, 2, 8))  # [token, head, d_v]
    w = np.linspace(0.5, 2.0, 8)
    z = np.zeros((3, 2, 8))
    z[:, 0, :4] = math.log(3.0)
    z[:, 1, 4:] = -math.log(3.0)
    y = oracle.gated_rmsnorm(c, z, w, eps=eps, mutation=mutation)
    gate = np.zeros((3, 2, 8))
    gate[:, 0, :4] = 0.75 * math.log(3.0)
    gate[:, 1, 4:] = -0.25 * math.log(3.0)
    ref = c / np.sqrt(c * c + eps) * w * gate
    return bool(np.allclose(y, ref, rtol=1e-14, atol=1e-15))


def check_norm_unit_rms_per_head(mutation=0):
    """eps = 0: silu(z) - silu(-z) = z, so y(z) - y(-z) = (o / rms_head(o)) w z, and o / rms
    has mean square exactly 1 within every (token, head), whatever the scale of each head."""
    rng = np.random.default_rng(70)
    o = rng.standard_normal((5, 3, 16)) * np.array([1e-3, 1.0, 40.0])[None, :, None]
    z = rng.standard_normal((5, 3, 16))
    w = rng.uniform(0.5, 1.5, 16)
    d = oracle.gated_rmsnorm(o, z, w, eps=0.0, mutation=mutation) - oracle.gated_rmsnorm(o, -z, w, eps=0.0,
                                                                                      mutation=mutation)
    n = d / (w * z)
    return bool(np.allclose(np.mean(n * n, axis=-1), 1.0, rtol=0, atol=1e-12) and np.all(n * o > 0))


def check_norm_scale_invariance(mutation=0):
    """eps = 0: y(c o) = y(o) for any c > 0 per (token, head), and y = 0 where z = 0."""
    rng = np.random.default_rng(71)
    o = rng.standard_normal((4, 2, 12))
    z = rng.standard_normal((4, 2, 12))
    z[0, 0, 3] = 0.0
    c = rng.uniform(0.01, 100.0, (4, 2, 1))
    y1 = oracle.gated_rmsnorm(o, z, eps=0.0, mutation=mutation)
    y2 = oracle.gated_rmsnorm(o * c, z, eps=0.0, mutation=mutation)
    return bool(np.allclose(y1, y2, rtol=1e-13, atol=0) and y1[0, 0, 3] == 0.0)


NORM_CHECKS = [check_norm_constant_rows, check_norm_unit_rms_per_head, check_norm_scale_invariance]


@pytest.mark.parametrize("check", NORM_CHECKS, ids=lambda c: c.__name__)
def test_norm_pin(check):
    assert check()


@pytest.mark.parametrize("name", sorted(oracle.NORM_MUTATIONS))
def test_norm_planted_mistakes_are_caught(name):
    m = oracle.NORM_MUTATIONS[name]
    assert not all(check(mutation=m) for check in NORM_CHECKS), name


def test_norm_bf16_gate_is_widened_exactly():
    """bf16 gate inputs are the stored bit patterns: 0x3F80 is 1.0, 0xC000 is -2.0."""
    z = np.array([[[0x3F80, 0xC000]]], dtype=np.uint16)
    o = np.array([[[1.0, -1.0]]])
    y = oracle.gated_rmsnorm(o, z, eps=0.0, bf16=True)
    ref = np.array([[[1.0 / (1.0 + math.exp(-1.0)), -1.0 * -2.0 / (1.0 + math.exp(2.0))]]])
    return_ok = np.allclose(y, ref, rtol=1e-15, atol=0)
    assert return_ok
