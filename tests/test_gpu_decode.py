"""GPU parity of gdn_decode_step against the fp64 oracle (same seeded inputs).

Tolerance on max|gpu - oracle| / rms(oracle): 2e-2 for bf16 q/k/v (fp32 math
and state), 1e-4 for the all-fp32 path.  At the full decode workload (256
sequences x 6 heads, d = 256, 128 steps) the GPU runs every chain and the
oracle recomputes a sample of (sequence, head) chains end to end."""
import numpy as np
import pytest

from _util import TOL_BF16, TOL_F32, bound_ratio, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from hybrid_linear_attention_delta_amd import gdn, synth  # noqa: E402

DEV = "cuda:0"


def _tt(a, bf16):
    return synth.to_torch(a, DEV, bf16=bf16)


def _run_decode(N, H, dk, dv, dtype, steps, seed, sample=None, gate="default", l2=True, scale=None):
    bf16 = dtype == "bf16"
    st0 = synth.decode_state(N, H, dk, dv, seed)
    state = torch.from_numpy(st0).to(DEV)
    chains = sample if sample is not None else [(n, h) for n in range(N) for h in range(H)]
    ns = sorted({n for n, _ in chains})
    ref_state = np.ascontiguousarray(st0[ns].astype(np.float64))
    idx = {n: i for i, n in enumerate(ns)}
    worst_o = 0.0
    for s in range(steps):
        q, k, v, g, beta = synth.decode_step_inputs(N, H, dk, dv, dtype, seed, s, gate=gate)
        o = gdn.decode_step(_tt(q, bf16), _tt(k, bf16), _tt(v, bf16), _tt(g, False), _tt(beta, False), state,
                            scale=scale, qk_l2norm=l2)
        o_ref = oracle.decode_step(q[ns], k[ns], v[ns], g[ns], beta[ns], ref_state, scale=scale, qk_l2norm=l2,
                                   bf16=bf16)
        o_gpu = o.float().cpu().numpy()
        got = np.stack([o_gpu[n, h] for n, h in chains])
        want = np.stack([o_ref[idx[n], h] for n, h in chains])
        tol = TOL_BF16 if bf16 else TOL_F32
        worst_o = max(worst_o, bound_ratio(got, want, tol, stored_bf16=bf16) * tol)
    s_gpu = state.cpu().numpy()
    got = np.stack([s_gpu[n, h] for n, h in chains])
    want = np.stack([ref_state[idx[n], h] for n, h in chains])
    # worst_o is the bound ratio scaled by tol, so "<= tol" means the bound holds
    return worst_o, rel_err(got, want)


@pytest.mark.parametrize("dk,dv", [(16, 16), (64, 32), (128, 128), (256, 256), (256, 512)])
def test_decode_fp32_small(dk, dv):
    eo, es = _run_decode(3, 2, dk, dv, "f32", steps=5, seed=11 + dk)
    assert eo <= TOL_F32 and es <= TOL_F32, (eo, es)


@pytest.mark.parametrize("dk,dv", [(64, 64), (256, 256), (256, 512)])
def test_decode_bf16_small(dk, dv):
    eo, es = _run_decode(5, 3, dk, dv, "bf16", steps=6, seed=21 + dk)
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)


def test_decode_fp32_no_norm_custom_scale_slow_gates():
    eo, es = _run_decode(4, 2, 64, 64, "f32", steps=8, seed=5, gate="slow", l2=False, scale=0.3)
    assert eo <= TOL_F32 and es <= TOL_F32, (eo, es)


@pytest.mark.slow
def test_decode_full_workload_sampled():
    """256 sequences x 6 heads x d=256, 128 consecutive steps; 24 chains checked end to end."""
    rng = np.random.default_rng(4)
    sample = sorted({(int(n), int(h)) for n, h in zip(rng.integers(0, 256, 24), rng.integers(0, 6, 24))})
    sample += [(0, 0), (255, 5)]
    eo, es = _run_decode(256, 6, 256, 256, "bf16", steps=128, seed=synth.seed_for("decode"), sample=sample)
    print(f"decode full workload: o err {eo:.3e}, state err {es:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)


def test_decode_deterministic():
    N, H, d = 8, 2, 256
    st0 = torch.from_numpy(synth.decode_state(N, H, d, d, 3)).to(DEV)
    q, k, v, g, beta = synth.decode_step_inputs(N, H, d, d, "bf16", 3, 0)
    args = [_tt(q, True), _tt(k, True), _tt(v, True), _tt(g, False), _tt(beta, False)]
    s1, s2 = st0.clone(), st0.clone()
    o1 = gdn.decode_step(*args, s1)
    o2 = gdn.decode_step(*args, s2)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_decode_steps_in_a_hip_graph_match_eager():
    """Consecutive decode steps captured once in a HIP graph: every replay, with
    eager work and synchronisations between replays, equals the same steps run
    eagerly from the same state (bit for bit), and the first replay matches the
    oracle."""
    N, H, dk, dv, steps, seed = 8, 3, 256, 256, 4, 4242
    st0 = torch.from_numpy(synth.decode_state(N, H, dk, dv, seed)).to(DEV)
    ins = [[_tt(x, b) for x, b in zip(synth.decode_step_inputs(N, H, dk, dv, "bf16", seed, s),
                                      (True, True, True, False, False))] for s in range(steps)]
    outs = [torch.empty((N, H, dv), dtype=torch.bfloat16, device=DEV) for _ in range(steps)]
    state = st0.clone()
    # eager reference from st0
    ref_state = st0.clone()
    ref_outs = [gdn.decode_step(*ins[s], ref_state).clone() for s in range(steps)]
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for s in range(steps):
                gdn.decode_step(*ins[s], state, out=outs[s])
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        state.copy_(st0)                       # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(state, ref_state), rep
        for s in range(steps):
            assert torch.equal(outs[s], ref_outs[s]), (rep, s)
    ref = np.ascontiguousarray(st0.cpu().numpy().astype(np.float64))
    for s in range(steps):
        q, k, v, g, beta = synth.decode_step_inputs(N, H, dk, dv, "bf16", seed, s)
        o_ref = oracle.decode_step(q, k, v, g, beta, ref, bf16=True)
        assert bound_ratio(outs[s].float().cpu().numpy(), o_ref, TOL_BF16, stored_bf16=True) <= 1.0
    assert rel_err(state.cpu().numpy(), ref) <= TOL_BF16


@pytest.mark.parametrize("N,dk,dv", [(1, 256, 256), (1000, 128, 256), (3, 64, 512)])
def test_decode_odd_batch_sizes(N, dk, dv):
    """One sequence, a thousand, and a few with d_v = 8 d_k: every state row of
    every (sequence, head) pair is updated and read out, and every output and
    the final state of every pair match the oracle."""
    eo, es = _run_decode(N, 2, dk, dv, "bf16", 3, seed=N + dk + dv)
    print(f"decode N={N} dk={dk} dv={dv}: o err {eo:.3e} (bound {TOL_BF16}), state err {es:.3e}")
    assert eo <= TOL_BF16 and es <= TOL_BF16, (eo, es)
