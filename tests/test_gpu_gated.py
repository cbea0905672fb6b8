"""GPU parity of the gated RMSNorm read-out ("Long-Context Aware Upcycling",
App. A.3 Eq. 20) against the fp64 oracle: the prefill (fused into its output
stage) and the decode step (its second small kernel), each against the
oracle's read-out followed by ``oracle.gated_rmsnorm`` on the same seeded
inputs.  The norm divides each row by its own rms and the gate multiplies
every element by w * silu(z) (up to |6| for N(0, 1) gate inputs), so the
read-out's tolerance (2e-2 bf16, 1e-4 fp32) is carried through per row and
per element: |y - y_ref| <= tol * |w silu(z)| + bf16 storage rounding (see
_util.gated_bound_ratio).  States keep the plain metric."""
import numpy as np
import pytest

from _util import TOL_BF16, TOL_F32, gated_bound_ratio, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from hybrid_linear_attention_delta_amd import gdn, synth  # noqa: E402

DEV = "cuda:0"


def _gate(z, w, bf16):
    """w * silu(z) in fp64 from the stored gate inputs."""
    zz = (z.astype(np.uint32) << 16).view(np.float32).astype(np.float64) if bf16 else z.astype(np.float64)
    ww = 1.0 if w is None else w.astype(np.float64)
    return ww * zz / (1.0 + np.exp(-zz))


@pytest.mark.parametrize("dtype,T,H,dk,dv,C,lens,use_w,eps", [
    ("bf16", 300, 2, 256, 256, 64, [170, 130], True, 1e-6),
    ("bf16", 150, 2, 64, 64, 64, None, False, 1e-6),
    ("bf16", 130, 1, 256, 512, 64, None, True, 1e-3),
    ("bf16", 200, 3, 128, 128, 64, [5, 0, 131, 64], True, 1e-6),
    ("f32", 200, 2, 64, 64, 32, [77, 123], True, 1e-6),
    ("f32", 64, 2, 16, 16, 16, None, True, 1e-5),
    ("f32", 100, 1, 256, 256, 64, None, False, 0.0),
])
def test_prefill_gated_matches_oracle(dtype, T, H, dk, dv, C, lens, use_w, eps):
    cu = None if lens is None else np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    seed = 900 + dk + dv + T
    inp = synth.prefill_inputs(T, H, dk, dv, dtype, seed=seed, gate="slow", cu_seqlens=cu, init_state_std=0.3)
    z, w = synth.norm_inputs((T, H, dv), dtype, seed)
    if not use_w:
        w = None
    bf = inp.bf16
    t = lambda a, b=False: synth.to_torch(a, DEV, bf16=b)
    cu_t = None if cu is None else torch.from_numpy(cu.astype(np.int32))
    o, fs = gdn.chunk_prefill(t(inp.q, bf), t(inp.k, bf), t(inp.v, bf), t(inp.g), t(inp.beta),
                              init_state=t(inp.init_state), cu_seqlens=cu_t, chunk=C, gate=t(z, bf),
                              norm_weight=None if w is None else t(w), norm_eps=eps)
    torch.cuda.synchronize()
    o_ref, fs_ref = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state, cu_seqlens=inp.cu_seqlens,
                                   bf16=bf)
    y_ref = oracle.gated_rmsnorm(o_ref, z, w, eps=eps, bf16=bf)
    tol = TOL_BF16 if bf else TOL_F32
    ro = gated_bound_ratio(o.float().cpu().numpy(), y_ref, _gate(z, w, bf), tol, stored_bf16=bf)
    es = rel_err(fs.cpu().numpy(), fs_ref)
    print(f"  gated o bound ratio {ro:.3f}  state err {es:.3e}")
    assert ro <= 1.0 and es <= tol, (ro, es)


def test_prefill_gated_pipelined_equals_oracle():
    """A long sequence (past the pipeline's 576-chunk threshold) with an
    execution context takes the segmented (pipelined) path; the epilogue runs in
    every segment's output launch.  The same call without a context (one
    stream, stage by stage) gives the same bits."""
    T, H, d = 37000, 2, 256
    inp = synth.prefill_inputs(T, H, d, d, "bf16", seed=977, gate="slow")
    z, w = synth.norm_inputs((T, H, d), "bf16", 977)
    t = lambda a, b=False: synth.to_torch(a, DEV, bf16=b)
    args = (t(inp.q, True), t(inp.k, True), t(inp.v, True), t(inp.g), t(inp.beta))
    with gdn.Context() as c:
        o, _ = gdn.chunk_prefill(*args, gate=t(z, True), norm_weight=t(w), norm_eps=1e-6, ctx=c)
        o1, _ = gdn.chunk_prefill(*args, gate=t(z, True), norm_weight=t(w), norm_eps=1e-6)
        torch.cuda.synchronize()
    assert torch.equal(o, o1)
    rows = [0, 77, 255]
    o_ref, _ = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, bf16=True)
    y_ref = oracle.gated_rmsnorm(o_ref, z, w, eps=1e-6, bf16=True)
    ro = gated_bound_ratio(o.float().cpu().numpy()[:, :, rows], y_ref[:, :, rows], _gate(z, w, True)[:, :, rows],
                           TOL_BF16, stored_bf16=True)
    assert ro <= 1.0, ro


@pytest.mark.parametrize("dtype,dk,dv,use_w", [("f32", 64, 64, True), ("f32", 16, 32, False),
                                               ("bf16", 256, 256, True), ("bf16", 256, 512, True),
                                               ("bf16", 64, 64, False)])
def test_decode_gated_matches_oracle(dtype, dk, dv, use_w):
    N, H, steps, seed = 5, 3, 4, 300 + dk + dv
    bf = dtype == "bf16"
    st0 = synth.decode_state(N, H, dk, dv, seed)
    state = torch.from_numpy(st0).to(DEV)
    ref_state = np.ascontiguousarray(st0.astype(np.float64))
    tol = TOL_BF16 if bf else TOL_F32
    for s in range(steps):
        q, k, v, g, beta = synth.decode_step_inputs(N, H, dk, dv, dtype, seed, s)
        z, w = synth.norm_inputs((N, H, dv), dtype, seed + s)
        if not use_w:
            w = None
        tt = lambda a, b=False: synth.to_torch(a, DEV, bf16=b)
        o = gdn.decode_step(tt(q, bf), tt(k, bf), tt(v, bf), tt(g), tt(beta), state, gate=tt(z, bf),
                            norm_weight=None if w is None else tt(w), norm_eps=1e-6)
        o_ref = oracle.decode_step(q, k, v, g, beta, ref_state, bf16=bf)
        y_ref = oracle.gated_rmsnorm(o_ref, z, w, eps=1e-6, bf16=bf)
        ro = gated_bound_ratio(o.float().cpu().numpy(), y_ref, _gate(z, w, bf), tol, stored_bf16=bf)
        assert ro <= 1.0, (s, ro)
    assert rel_err(state.cpu().numpy(), ref_state) <= tol
