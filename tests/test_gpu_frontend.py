"""GPU parity of the front end ("Long-Context Aware Upcycling", App. A.3: the
4-tap causal convolution with SiLU under Table 8, and the gates after Eq. 21)
against the fp64 oracle (``oracle.short_conv_silu``, ``oracle.gates``), through
the C ABI (``gdn_frontend_prefill`` / ``gdn_frontend_decode``).

Tolerances: the front end computes in fp32, so q, k, v, g, beta must be within
1e-4 of the output RMS (the fp32 bound), plus the bf16 storage rounding
(2^-8 |ref|) where q, k, v are stored in bf16.  The conv state is a copy of
stored inputs and must match bit for bit.  End to end (front end, then the
mixer) the mixer's own bounds apply: 2e-2 for bf16, 1e-4 for fp32."""
import numpy as np
import pytest

from _util import TOL_BF16, TOL_F32, bound_ratio, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from hybrid_linear_attention_delta_amd import gdn, synth  # noqa: E402

DEV = "cuda:0"


def _t(a, bf16=False):
    return synth.to_torch(a, DEV, bf16=bf16)


def _widen(a, bf16):
    return synth.bf16_to_f32(a).astype(np.float64) if bf16 else np.asarray(a, dtype=np.float64)


def _gpu_frontend(f, T, H, dk, dv, cu, state, out_state=None):
    bf = f.bf16
    xq = _t(f.xq, bf).view(T, H, dk)
    xk = _t(f.xk, bf).view(T, H, dk)
    xv = _t(f.xv, bf).view(T, H, dv)
    cu_t = None if cu is None else torch.from_numpy(np.asarray(cu, dtype=np.int32))
    return gdn.frontend_prefill(xq, xk, xv, _t(f.conv_weight), _t(f.a), _t(f.b), _t(f.A_log), _t(f.dt_bias),
                                conv_state=state, cu_seqlens=cu_t, conv_state_out=out_state)


def _oracle_frontend(f, H, dk, dv, cu, state_np):
    """Oracle of the whole front end on the concatenated channel axis."""
    x = np.concatenate([f.xq, f.xk, f.xv], axis=1)
    y, st = oracle.short_conv_silu(x, f.conv_weight, cu_seqlens=cu, conv_state=state_np, bf16=f.bf16)
    g, beta = oracle.gates(f.a, f.b, f.A_log, f.dt_bias)
    cq = H * dk
    return y[:, :cq], y[:, cq:2 * cq], y[:, 2 * cq:], g, beta, st


def _check_qkv(gpu, ref, bf):
    tol = TOL_F32
    r = bound_ratio(gpu.float().cpu().numpy().reshape(ref.shape), ref, tol, stored_bf16=bf)
    assert r <= 1.0, r


@pytest.mark.parametrize("dtype,H,dk,dv,lens,with_state", [
    ("bf16", 6, 256, 256, None, False),
    ("bf16", 6, 256, 256, [130, 1, 0, 2, 67, 3, 100], True),
    ("bf16", 2, 64, 128, [5, 40, 0, 17], True),
    ("f32", 2, 64, 128, [33, 2, 90], True),
    ("f32", 3, 16, 32, None, True),
    ("bf16", 1, 8, 16, [1, 1, 1, 1], True),
])
def test_frontend_prefill_matches_oracle(dtype, H, dk, dv, lens, with_state):
    T = 300 if lens is None else int(sum(lens))
    cu = None if lens is None else np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    N = 1 if lens is None else len(lens)
    f = synth.frontend_inputs(T, H, dk, dv, dtype, seed=500 + T + dk, cu_seqlens=cu, with_state=with_state, N=N)
    bf = f.bf16
    st = _t(f.conv_state, bf) if with_state else None
    q, k, v, g, beta, st_out = _gpu_frontend(f, T, H, dk, dv, cu, st)
    torch.cuda.synchronize()
    rq, rk, rv, rg, rb, rst = _oracle_frontend(f, H, dk, dv, cu, f.conv_state if with_state else None)
    for gpu, ref in ((q, rq), (k, rk), (v, rv)):
        _check_qkv(gpu, ref, bf)
    assert rel_err(g.cpu().numpy(), rg) <= TOL_F32
    assert rel_err(beta.cpu().numpy(), rb) <= TOL_F32
    got = _widen(st_out.cpu().view(torch.int16).numpy().view(np.uint16), True) if bf else st_out.cpu().numpy()
    assert np.array_equal(got.astype(np.float64), rst), "conv state must be an exact copy of the inputs"


def test_frontend_prefill_state_in_place_and_continuation():
    """Two calls carrying the conv state in place equal one call over the whole
    sequences (split inside the first three tokens of one sequence)."""
    H, dk, dv, dtype = 2, 64, 64, "bf16"
    lens_a, lens_b = [10, 2, 50], [7, 1, 30]
    f = synth.frontend_inputs(sum(lens_a) + sum(lens_b), H, dk, dv, dtype, seed=77, with_state=True, N=3)
    ctot = H * (2 * dk + dv)
    # token ranges: sequence n = part a of length lens_a[n], then part b of length lens_b[n]
    whole = []
    for n in range(3):
        oa = sum(lens_a[:n]) + sum(lens_b[:n])
        whole.append(np.arange(oa, oa + lens_a[n] + lens_b[n]))
    pa = np.concatenate([w[:lens_a[n]] for n, w in enumerate(whole)])
    pb = np.concatenate([w[lens_a[n]:] for n, w in enumerate(whole)])
    cu_a = np.concatenate([[0], np.cumsum(lens_a)]).astype(np.int64)
    cu_b = np.concatenate([[0], np.cumsum(lens_b)]).astype(np.int64)

    def sub(idx):
        return synth.FrontendInputs(f.xq[idx], f.xk[idx], f.xv[idx], f.conv_weight, f.a[idx], f.b[idx], f.A_log,
                                    f.dt_bias, None, dtype, None)

    state = _t(f.conv_state, True)
    qa = _gpu_frontend(sub(pa), len(pa), H, dk, dv, cu_a, state, out_state=state)
    qb = _gpu_frontend(sub(pb), len(pb), H, dk, dv, cu_b, state, out_state=state)
    torch.cuda.synchronize()
    order = np.concatenate(whole)
    cu_w = np.concatenate([[0], np.cumsum(np.array(lens_a) + np.array(lens_b))]).astype(np.int64)
    rq, rk, rv, _, _, rst = _oracle_frontend(sub(order), H, dk, dv, cu_w, f.conv_state)
    pos = {int(t): i for i, t in enumerate(order)}
    ia = [pos[int(t)] for t in pa]
    ib = [pos[int(t)] for t in pb]
    for j, ref in enumerate((rq, rk, rv)):
        _check_qkv(qa[j], ref[ia], True)
        _check_qkv(qb[j], ref[ib], True)
    got = _widen(state.cpu().view(torch.int16).numpy().view(np.uint16), True)
    assert np.array_equal(got.reshape(3, 3, ctot), rst)


def test_frontend_prefill_long_sequence_sampled():
    """1.1 M tokens (more than 65535 tiles of 16 tokens) over few channels:
    checks the tile indexing at long lengths; every output is compared."""
    T, H, dk, dv = 1_100_003, 1, 8, 8
    lens = [600_000, 3, 500_000]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    f = synth.frontend_inputs(T, H, dk, dv, "bf16", seed=31, cu_seqlens=cu, with_state=True)
    q, k, v, g, beta, st_out = _gpu_frontend(f, T, H, dk, dv, cu, _t(f.conv_state, True))
    torch.cuda.synchronize()
    rq, rk, rv, rg, rb, rst = _oracle_frontend(f, H, dk, dv, cu, f.conv_state)
    for gpu, ref in ((q, rq), (k, rk), (v, rv)):
        _check_qkv(gpu, ref, True)
    assert rel_err(g.cpu().numpy(), rg) <= TOL_F32 and rel_err(beta.cpu().numpy(), rb) <= TOL_F32
    got = _widen(st_out.cpu().view(torch.int16).numpy().view(np.uint16), True)
    assert np.array_equal(got, rst)


def test_frontend_prefill_full_size_sampled_channels():
    """The 64K-token workload (H = 6, d = 256, bf16) in the launch the bench times;
    the oracle recomputes 96 sampled channels over every token (channels are
    independent) and all gates."""
    T, H, d = 65536, 6, 256
    f = synth.frontend_inputs(T, H, d, d, "bf16", seed=1002)
    q, k, v, g, beta, _ = _gpu_frontend(f, T, H, d, d, None, None)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    ch = np.sort(rng.choice(H * d, size=32, replace=False))
    x_all = (f.xq, f.xk, f.xv)
    for j, out in enumerate((q, k, v)):
        y, _ = oracle.short_conv_silu(x_all[j][:, ch], f.conv_weight[j * H * d + ch], bf16=True)
        got = out.view(T, H * d)[:, torch.from_numpy(ch).to(DEV)].float().cpu().numpy()
        assert bound_ratio(got, y, TOL_F32, stored_bf16=True) <= 1.0
    rg, rb = oracle.gates(f.a, f.b, f.A_log, f.dt_bias)
    assert rel_err(g.cpu().numpy(), rg) <= TOL_F32 and rel_err(beta.cpu().numpy(), rb) <= TOL_F32


@pytest.mark.parametrize("dtype,H,dk,dv", [("bf16", 6, 256, 256), ("f32", 2, 64, 128), ("bf16", 3, 16, 8)])
def test_frontend_decode_matches_oracle(dtype, H, dk, dv):
    N, steps = 7, 5
    bf = dtype == "bf16"
    ctot = H * (2 * dk + dv)
    f0 = synth.frontend_inputs(N * steps, H, dk, dv, dtype, seed=61 + dk, with_state=True, N=N)
    state = _t(f0.conv_state, bf)
    ref_state = f0.conv_state
    cu1 = np.arange(N + 1, dtype=np.int64)
    for s in range(steps):
        rows = slice(s * N, (s + 1) * N)
        tq = _t(f0.xq[rows], bf).view(N, H, dk)
        tk = _t(f0.xk[rows], bf).view(N, H, dk)
        tv = _t(f0.xv[rows], bf).view(N, H, dv)
        q, k, v, g, beta = gdn.frontend_decode(tq, tk, tv, _t(f0.conv_weight), _t(f0.a[rows]), _t(f0.b[rows]),
                                               _t(f0.A_log), _t(f0.dt_bias), state)
        torch.cuda.synchronize()
        x = np.concatenate([f0.xq[rows], f0.xk[rows], f0.xv[rows]], axis=1)
        y, st = oracle.short_conv_silu(x, f0.conv_weight, cu_seqlens=cu1, conv_state=ref_state, bf16=bf)
        rg, rb = oracle.gates(f0.a[rows], f0.b[rows], f0.A_log, f0.dt_bias)
        cq = H * dk
        for gpu, ref in ((q, y[:, :cq]), (k, y[:, cq:2 * cq]), (v, y[:, 2 * cq:])):
            _check_qkv(gpu, ref, bf)
        assert rel_err(g.cpu().numpy(), rg) <= TOL_F32 and rel_err(beta.cpu().numpy(), rb) <= TOL_F32
        got = _widen(state.cpu().view(torch.int16).numpy().view(np.uint16), True) if bf else state.cpu().numpy()
        assert np.array_equal(got.astype(np.float64).reshape(N, 3, ctot), st), s
        ref_state = synth._store(st, dtype)  # exact: st holds stored inputs


def test_frontend_then_prefill_end_to_end():
    """Front end, then the chunked prefill, against the oracle's front end (rounded
    to the storage type, as the GPU stores it) followed by the oracle recurrence."""
    H, d, lens = 2, 256, [150, 3, 90]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    f = synth.frontend_inputs(T, H, d, d, "bf16", seed=88, cu_seqlens=cu, with_state=True)
    q, k, v, g, beta, _ = _gpu_frontend(f, T, H, d, d, cu, _t(f.conv_state, True))
    o, fs = gdn.chunk_prefill(q, k, v, g, beta, cu_seqlens=cu.astype(np.int32))
    torch.cuda.synchronize()
    rq, rk, rv, rg, rb, _ = _oracle_frontend(f, H, d, d, cu, f.conv_state)
    st = lambda y: synth._store(y, "bf16").reshape(T, H, d)
    o_ref, fs_ref = oracle.prefill(st(rq), st(rk), st(rv), rg.astype(np.float32), rb.astype(np.float32),
                                   cu_seqlens=cu, bf16=True)
    assert bound_ratio(o.float().cpu().numpy(), o_ref, TOL_BF16, stored_bf16=True) <= 1.0
    assert rel_err(fs.cpu().numpy(), fs_ref) <= TOL_BF16


def test_frontend_rejects_bad_arguments():
    H, dk, dv = 2, 12, 16  # dk not a multiple of 8
    xq = torch.zeros((4, H, dk), dtype=torch.bfloat16, device=DEV)
    xv = torch.zeros((4, H, dv), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((H * (2 * dk + dv), 4), device=DEV)
    ab = torch.zeros((4, H), device=DEV)
    hh = torch.zeros(H, device=DEV)
    with pytest.raises(gdn.GdnError):
        gdn.frontend_prefill(xq, xq, xv, w, ab, ab, hh, hh)


def test_frontend_then_pipelined_prefill_sampled_rows():
    """37K tokens (past the prefill's pipelining threshold) through the front end
    and the pipelined prefill, against the oracle's front end (rounded to bf16)
    and the oracle recurrence on sampled state rows."""
    T, H, d = 37000, 2, 256
    f = synth.frontend_inputs(T, H, d, d, "bf16", seed=99)
    q, k, v, g, beta, _ = _gpu_frontend(f, T, H, d, d, None, None)
    o, fs = gdn.chunk_prefill(q, k, v, g, beta)
    torch.cuda.synchronize()
    rq, rk, rv, rg, rb, _ = _oracle_frontend(f, H, d, d, None, None)
    st = lambda y: synth._store(y, "bf16").reshape(T, H, d)
    rows = [0, 101, 255]
    o_ref, fs_ref = oracle.prefill(st(rq), st(rk), st(rv), rg.astype(np.float32), rb.astype(np.float32), bf16=True,
                                   rows=rows)
    assert bound_ratio(o.float().cpu().numpy()[:, :, rows], o_ref[:, :, rows], TOL_BF16, stored_bf16=True) <= 1.0
    assert rel_err(fs.cpu().numpy()[:, :, rows], fs_ref[:, :, rows]) <= TOL_BF16


def test_frontend_prefill_non_square_heads():
    """H = 6, d_k = 128, d_v = 256 (q and k channel blocks narrower than v's)."""
    H, dk, dv, lens = 6, 128, 256, [90, 3, 160]
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    f = synth.frontend_inputs(T, H, dk, dv, "bf16", seed=1282, cu_seqlens=cu, with_state=True)
    q, k, v, g, beta, st_out = _gpu_frontend(f, T, H, dk, dv, cu, _t(f.conv_state, True))
    torch.cuda.synchronize()
    rq, rk, rv, rg, rb, rst = _oracle_frontend(f, H, dk, dv, cu, f.conv_state)
    for gpu, ref in ((q, rq), (k, rk), (v, rv)):
        _check_qkv(gpu, ref, True)
    assert rel_err(g.cpu().numpy(), rg) <= TOL_F32 and rel_err(beta.cpu().numpy(), rb) <= TOL_F32
    got = _widen(st_out.cpu().view(torch.int16).numpy().view(np.uint16), True)
    assert np.array_equal(got, rst)
