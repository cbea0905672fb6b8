"""GPU tests of the prefill with a workspace below gdn_prefill_workspace_size
(down to gdn_prefill_workspace_min_size): the chunks run window by window,
each sequence's state carried between windows in fp32, and the outputs and
final states must equal those of a full-size workspace bit for bit -- for
packed sequences that cross window boundaries (one empty, ragged tails), with
and without an execution context, with the gated read-out -- and match the
oracle on sampled value rows."""
import numpy as np
import pytest

from _util import TOL_BF16, bound_ratio, rel_err

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import oracle  # noqa: E402
from hybrid_linear_attention_delta_amd import gdn, synth  # noqa: E402

DEV = "cuda:0"


def _inputs(T, H, d, lens, seed):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    inp = synth.prefill_inputs(T, H, d, d, "bf16", seed=seed, gate="slow", cu_seqlens=cu, init_state_std=0.3)
    t = lambda a, b=False: synth.to_torch(a, DEV, bf16=b)
    args = (t(inp.q, True), t(inp.k, True), t(inp.v, True), t(inp.g), t(inp.beta))
    return inp, cu, args, t(inp.init_state)


@pytest.mark.parametrize("frac", [0.3, 0.0])
def test_windowed_workspace_equals_full_workspace(frac):
    T, H, d = 12288, 2, 256
    lens = [5000, 0, 4100, 3188]
    inp, cu, args, init = _inputs(T, H, d, lens, 7301)
    N = len(lens)
    cu_host = torch.from_numpy(cu.astype(np.int32))
    full = gdn.prefill_workspace_size(T, N, H, d, d, 64)
    mn = gdn.prefill_workspace_min_size(T, N, H, d, d, 64)
    small = max(mn, int(full * frac)) // 256 * 256 + (256 if frac == 0.0 else 0)
    small = max(small, mn)
    print(f"  windowed prefill T={T} N={N} H={H} d={d}: workspace {small / 2**20:.1f} of {full / 2**20:.1f} MiB "
          f"(min {mn / 2**20:.2f})", flush=True)
    assert mn <= small < full
    o_ref, fs_ref = gdn.chunk_prefill(*args, init_state=init, cu_seqlens=cu_host)
    ws = torch.empty(small, dtype=torch.uint8, device=DEV)
    o, fs = gdn.chunk_prefill(*args, init_state=init, cu_seqlens=cu_host, workspace=ws)
    with gdn.Context() as ctx:
        o2, fs2 = gdn.chunk_prefill(*args, init_state=init, cu_seqlens=cu_host, workspace=ws, ctx=ctx)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(fs, fs_ref)
    assert torch.equal(o2, o_ref) and torch.equal(fs2, fs_ref)
    rows = [0, 129, 255]
    oo, fo = oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state, cu_seqlens=cu, rows=rows,
                            bf16=True)
    assert bound_ratio(o.float().cpu().numpy()[:, :, rows], oo[:, :, rows], TOL_BF16, stored_bf16=True) <= 1.0
    assert rel_err(fs.cpu().numpy()[:, :, rows], fo[:, :, rows]) <= TOL_BF16


def test_windowed_workspace_gated_readout():
    T, H, d = 9000, 2, 128
    lens = [4500, 4500]
    inp, cu, args, init = _inputs(T, H, d, lens, 7302)
    cu_host = torch.from_numpy(cu.astype(np.int32))
    z, w = synth.norm_inputs((T, H, d), "bf16", 7302)
    zt, wt = synth.to_torch(z, DEV, bf16=True), synth.to_torch(w, DEV)
    full = gdn.prefill_workspace_size(T, 2, H, d, d, 64)
    ws = torch.empty(max(gdn.prefill_workspace_min_size(T, 2, H, d, d, 64), full // 5) // 256 * 256,
                     dtype=torch.uint8, device=DEV)
    assert ws.numel() < full
    o_ref, fs_ref = gdn.chunk_prefill(*args, init_state=init, cu_seqlens=cu_host, gate=zt, norm_weight=wt)
    o, fs = gdn.chunk_prefill(*args, init_state=init, cu_seqlens=cu_host, gate=zt, norm_weight=wt, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(fs, fs_ref)


def test_windowed_workspace_refusals():
    """Below the minimum, and for a stage subset with less than the full size,
    the call raises GDN_ERR_WORKSPACE (nothing runs)."""
    T, H, d = 4096, 2, 64
    inp, cu, args, init = _inputs(T, H, d, [T], 7303)
    mn = gdn.prefill_workspace_min_size(T, 1, H, d, d, 64)
    full = gdn.prefill_workspace_size(T, 1, H, d, d, 64)
    with pytest.raises(gdn.GdnError) as e:
        gdn.chunk_prefill(*args, workspace=torch.empty(mn - 256, dtype=torch.uint8, device=DEV))
    assert e.value.status == 6
    with pytest.raises(gdn.GdnError) as e:
        gdn.chunk_prefill(*args, workspace=torch.empty(full - 256, dtype=torch.uint8, device=DEV),
                          stages=gdn.STAGE_PREPARE)
    assert e.value.status == 6


def test_windowed_workspace_fused_frontend():
    """The front end folded into the preparation, run in windows: equal to the
    same call with a full-size workspace, conv state after the call included."""
    T, H, d = 6000, 2, 256
    lens = [2500, 3, 3497]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    f = synth.frontend_inputs(T, H, d, d, "bf16", seed=7304, cu_seqlens=cu, with_state=True, N=len(lens))
    t = lambda a, b=False: synth.to_torch(a, DEV, bf16=b)
    x = (t(f.xq, True).view(T, H, d), t(f.xk, True).view(T, H, d), t(f.xv, True).view(T, H, d))
    rest = tuple(t(a) for a in (f.conv_weight, f.a, f.b, f.A_log, f.dt_bias))
    st = t(f.conv_state, True)
    cu_t = torch.from_numpy(cu.astype(np.int32))
    full = gdn.prefill_workspace_size(T, len(lens), H, d, d, 64)
    ws = torch.empty(max(gdn.prefill_workspace_min_size(T, len(lens), H, d, d, 64), full // 4) // 256 * 256,
                     dtype=torch.uint8, device=DEV)
    o_ref, fs_ref, st_ref = gdn.chunk_prefill_frontend(*x, *rest, conv_state=st, cu_seqlens=cu_t)
    o, fs, st_out = gdn.chunk_prefill_frontend(*x, *rest, conv_state=st, cu_seqlens=cu_t, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(fs, fs_ref) and torch.equal(st_out, st_ref)
