"""Thin Python binding over the C ABI in include/gdn.h (libgdn_mi355x.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  PyTorch supplies device memory and the current
stream.  There is no CPU or PyTorch fallback: if the library is missing or the
tensors are not on a GPU, the calls raise.

The operation is the gated delta rule of "Long-Context Aware Upcycling: A New
Frontier for Hybrid LLM Scaling" (arXiv:2604.24715), App. A.3, Eqs. 16-19,
with the state stored [.., d_v, d_k] (row i = value index).
"""
from __future__ import annotations

import ctypes
import math
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn_mi355x.so")

GDN_F32, GDN_BF16 = 0, 1
DEFAULT_NORM_EPS = 1e-6
STAGE_PREPARE, STAGE_PROPAGATE, STAGE_OUTPUT, STAGE_ALL = 1, 2, 4, 7
STATUS = {
    0: "GDN_OK", 1: "GDN_ERR_NULL_ARG", 2: "GDN_ERR_BAD_SHAPE", 3: "GDN_ERR_UNSUPPORTED",
    4: "GDN_ERR_BAD_SEQLENS", 5: "GDN_ERR_ALIGNMENT", 6: "GDN_ERR_WORKSPACE", 7: "GDN_ERR_LAUNCH",
    8: "GDN_ERR_CONTEXT",
}

_lock = threading.Lock()
_lib = None


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


def load_library(path: str | None = None):
    """Load (once) and return the ctypes handle of the HIP library."""
    global _lib
    with _lock:
        if _lib is None:
            p = path or LIB_PATH
            if not os.path.exists(p):
                raise RuntimeError(
                    f"HIP library {p} is not built; run __graft_entry__.build() or "
                    "python -m hybrid_linear_attention_delta_amd.csrc.build")
            lib = ctypes.CDLL(p)
            vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
            lib.gdn_prefill_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32, ctypes.c_int]
            lib.gdn_prefill_workspace_size.restype = sz
            lib.gdn_prefill_workspace_min_size.argtypes = [i64, i32, i32, i32, i32, i32, ctypes.c_int]
            lib.gdn_prefill_workspace_min_size.restype = sz
            lib.gdn_chunk_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32,
                                              ctypes.c_int, f32, i32, vp, vp, vp, sz, vp]
            lib.gdn_chunk_prefill.restype = ctypes.c_int
            lib.gdn_chunk_prefill_staged.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32,
                                                     ctypes.c_int, f32, i32, vp, vp, vp, sz, i32, vp]
            lib.gdn_chunk_prefill_staged.restype = ctypes.c_int
            lib.gdn_context_create.argtypes = [i32, ctypes.POINTER(vp)]
            lib.gdn_context_create.restype = ctypes.c_int
            lib.gdn_context_destroy.argtypes = [vp]
            lib.gdn_context_destroy.restype = ctypes.c_int
            lib.gdn_chunk_prefill_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32,
                                                      ctypes.c_int, f32, i32, vp, vp, vp]
            lib.gdn_chunk_prefill_noalloc.restype = ctypes.c_int
            lib.gdn_chunk_prefill_ctx.argtypes = [vp] + lib.gdn_chunk_prefill.argtypes
            lib.gdn_chunk_prefill_ctx.restype = ctypes.c_int
            lib.gdn_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int, f32, i32,
                                            vp, vp]
            lib.gdn_decode_step.restype = ctypes.c_int
            lib.gdn_chunk_prefill_gated.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32,
                                                    ctypes.c_int, f32, i32, vp, vp, f32, vp, vp, vp, sz, vp]
            lib.gdn_chunk_prefill_gated.restype = ctypes.c_int
            lib.gdn_chunk_prefill_gated_ctx.argtypes = [vp] + lib.gdn_chunk_prefill_gated.argtypes
            lib.gdn_chunk_prefill_gated_ctx.restype = ctypes.c_int
            lib.gdn_decode_step_gated.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int, f32,
                                                  i32, vp, vp, f32, vp, vp]
            lib.gdn_decode_step_gated.restype = ctypes.c_int
            lib.gdn_frontend_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32,
                                                 ctypes.c_int, vp, vp, vp, vp, vp, vp, vp]
            lib.gdn_frontend_prefill.restype = ctypes.c_int
            lib.gdn_chunk_prefill_frontend.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i64,
                                                       i32, i32, i32, i32, ctypes.c_int, f32, i32, vp, vp, vp, vp,
                                                       sz, vp]
            lib.gdn_chunk_prefill_frontend.restype = ctypes.c_int
            lib.gdn_frontend_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int,
                                                vp, vp, vp, vp, vp, vp]
            lib.gdn_frontend_decode.restype = ctypes.c_int
            lib.gdn_prefill_backward_workspace_size.argtypes = [i64, i32, i32, i32, i32]
            lib.gdn_prefill_backward_workspace_size.restype = sz
            lib.gdn_chunk_prefill_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32,
                                                       i32, ctypes.c_int, f32, i32, vp, vp, vp, vp, vp, vp, vp, sz,
                                                       vp]
            lib.gdn_chunk_prefill_backward.restype = ctypes.c_int
            lib.gdn_status_string.argtypes = [ctypes.c_int]
            lib.gdn_status_string.restype = ctypes.c_char_p
            lib.gdn_version.argtypes = []
            lib.gdn_version.restype = i32
            _lib = lib
    return _lib


class Context:
    """Execution context of the overlapped prefill (gdn_context_create): the
    streams and events that let one ``chunk_prefill(..., ctx=...)`` call overlap
    its three stages.  Created on the current device; ``close()`` (or leaving a
    ``with`` block) waits for its streams and releases them.  Results with and
    without a context are bit-identical."""

    def __init__(self, chain_cus_per_xcd: int = 0):
        lib = load_library()
        h = ctypes.c_void_p()
        st = lib.gdn_context_create(int(chain_cus_per_xcd), ctypes.byref(h))
        if st != 0:
            raise GdnError(st, "gdn_context_create")
        self._h = h

    @property
    def handle(self):
        if self._h is None:
            raise ValueError("the context is closed")
        return self._h

    def close(self):
        h, self._h = getattr(self, "_h", None), None
        if h is not None and h.value:
            st = load_library().gdn_context_destroy(h)
            if st != 0:
                raise GdnError(st, "gdn_context_destroy")

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return GDN_BF16
    if t.dtype == torch.float32:
        return GDN_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _check(t, name, dtype=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device}); there is no CPU path")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def prefill_workspace_size(total_tokens: int, num_seqs: int, H: int, dk: int, dv: int, chunk: int = 64,
                           dtype=None) -> int:
    torch = _torch()
    code = GDN_BF16 if (dtype is None or dtype == torch.bfloat16) else GDN_F32
    return int(load_library().gdn_prefill_workspace_size(total_tokens, num_seqs, H, dk, dv, chunk, code))


def prefill_workspace_min_size(total_tokens: int, num_seqs: int, H: int, dk: int, dv: int, chunk: int = 64,
                               dtype=None) -> int:
    """Smallest workspace a whole-prefill call accepts (gdn_prefill_workspace_min_size):
    below prefill_workspace_size the chunks run in windows that fit, bit-identically."""
    torch = _torch()
    code = GDN_BF16 if (dtype is None or dtype == torch.bfloat16) else GDN_F32
    return int(load_library().gdn_prefill_workspace_min_size(total_tokens, num_seqs, H, dk, dv, chunk, code))


def _norm_args(gate, norm_weight, shape, dt, dev):
    torch = _torch()
    _check(gate, "gate", dtype=dt, device=dev)
    if tuple(gate.shape) != tuple(shape):
        raise ValueError(f"gate must be {list(shape)}")
    if norm_weight is not None:
        _check(norm_weight, "norm_weight", dtype=torch.float32, device=dev)
        if tuple(norm_weight.shape) != (shape[-1],):
            raise ValueError(f"norm_weight must be [{shape[-1]}]")


def chunk_prefill(q, k, v, g, beta, init_state=None, cu_seqlens=None, scale=None, qk_l2norm=True, chunk=64,
                  out=None, final_state=None, workspace=None, return_final_state=True, stages=STAGE_ALL,
                  gate=None, norm_weight=None, norm_eps=DEFAULT_NORM_EPS, ctx=None):
    """Chunked gated delta-rule prefill over packed sequences.

    q, k [T, H, dk]; v [T, H, dv] (bf16 or fp32, same dtype); g, beta [T, H] fp32;
    init_state [N, H, dv, dk] fp32 or None; cu_seqlens int [N+1] (list, CPU or GPU
    tensor) or None for one sequence.  Returns (o [T, H, dv], final_state [N, H, dv, dk]).
    ``stages`` is a bit set of STAGE_PREPARE / STAGE_PROPAGATE / STAGE_OUTPUT (STAGE_ALL:
    all three; see include/gdn.h); a later stage must get the workspace of the earlier
    ones on the same inputs.  With ``gate`` [T, H, dv] (dtype of q) the outputs get the
    gated RMSNorm read-out of App. A.3 Eq. 20 (``norm_weight`` [dv] fp32 or None,
    ``norm_eps``); it needs all stages in one call.  ``ctx`` (a ``Context``) lets a
    whole-prefill call overlap its stages on the context's streams.
    """
    torch = _torch()
    lib = load_library()
    dev = q.device
    _check(q, "q", device=dev)
    dt = q.dtype
    for name, t in (("k", k), ("v", v)):
        _check(t, name, dtype=dt, device=dev)
    _check(g, "g", dtype=torch.float32, device=dev)
    _check(beta, "beta", dtype=torch.float32, device=dev)
    T, H, dk = q.shape
    dv = v.shape[2]
    if k.shape != (T, H, dk) or v.shape[:2] != (T, H) or g.shape != (T, H) or beta.shape != (T, H):
        raise ValueError("shape mismatch among q, k, v, g, beta")

    cu_dev = None
    cu_host = None
    if cu_seqlens is None:
        N = 1
    else:
        if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.device.type == "cuda":
            cu_dev = cu_seqlens.to(torch.int32).contiguous()
        else:
            cu_host = torch.as_tensor(cu_seqlens, dtype=torch.int32).contiguous().cpu()
            cu_dev = cu_host.to(dev)
        N = cu_dev.shape[0] - 1
        if N < 1:
            raise ValueError("cu_seqlens needs at least two entries")
    if init_state is not None:
        _check(init_state, "init_state", dtype=torch.float32, device=dev)
        if init_state.shape != (N, H, dv, dk):
            raise ValueError(f"init_state must be [{N}, {H}, {dv}, {dk}]")
    if out is None:
        out = torch.empty((T, H, dv), dtype=dt, device=dev)
    else:
        _check(out, "out", dtype=dt, device=dev)
    if final_state is None and return_final_state:
        final_state = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    elif final_state is not None:
        _check(final_state, "final_state", dtype=torch.float32, device=dev)
    code = _dtype_code(q)
    need = int(lib.gdn_prefill_workspace_size(T, N, H, dk, dv, chunk, code))
    if need == 0:
        raise GdnError(3, "gdn_prefill_workspace_size")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    else:  # a smaller buffer (down to prefill_workspace_min_size) runs the chunks in windows
        _check(workspace, "workspace", dtype=torch.uint8, device=dev)
    s = -1.0 if scale is None else float(scale)
    cu_host_ptr = None if cu_host is None else ctypes.c_void_p(cu_host.data_ptr())
    if gate is not None:
        if stages != STAGE_ALL:
            raise ValueError("the gated read-out needs all stages in one call")
        _norm_args(gate, norm_weight, (T, H, dv), dt, dev)
        st = lib.gdn_chunk_prefill_gated_ctx(None if ctx is None else ctx.handle, _ptr(q), _ptr(k), _ptr(v),
                                             _ptr(g), _ptr(beta), _ptr(init_state), _ptr(cu_dev), cu_host_ptr, N, T,
                                             H, dk, dv, chunk, code, s, int(bool(qk_l2norm)), _ptr(gate),
                                             _ptr(norm_weight), float(norm_eps), _ptr(out), _ptr(final_state),
                                             _ptr(workspace), workspace.numel(), _stream(dev))
        if st != 0:
            raise GdnError(st, "gdn_chunk_prefill_gated_ctx")
        return out, final_state
    if stages == STAGE_ALL:
        st = lib.gdn_chunk_prefill_ctx(None if ctx is None else ctx.handle, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                       _ptr(beta), _ptr(init_state), _ptr(cu_dev), cu_host_ptr, N, T, H, dk, dv,
                                       chunk, code, s, int(bool(qk_l2norm)), _ptr(out), _ptr(final_state),
                                       _ptr(workspace), workspace.numel(), _stream(dev))
        if st != 0:
            raise GdnError(st, "gdn_chunk_prefill_ctx")
        return out, final_state
    st = lib.gdn_chunk_prefill_staged(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(init_state),
                                      _ptr(cu_dev), cu_host_ptr, N, T, H, dk, dv, chunk, code, s,
                                      int(bool(qk_l2norm)), _ptr(out), _ptr(final_state), _ptr(workspace),
                                      workspace.numel(), int(stages), _stream(dev))
    if st != 0:
        raise GdnError(st, "gdn_chunk_prefill_staged")
    return out, final_state


def _seqlens(cu_seqlens, dev):
    """(device int32 tensor or None, host int32 tensor or None, N)."""
    torch = _torch()
    if cu_seqlens is None:
        return None, None, 1
    cu_host = None
    if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.device.type == "cuda":
        cu_dev = cu_seqlens.to(torch.int32).contiguous()
    else:
        cu_host = torch.as_tensor(cu_seqlens, dtype=torch.int32).contiguous().cpu()
        cu_dev = cu_host.to(dev)
    N = cu_dev.shape[0] - 1
    if N < 1:
        raise ValueError("cu_seqlens needs at least two entries")
    return cu_dev, cu_host, N


def prefill_backward_workspace_size(total_tokens: int, num_seqs: int, H: int, dk: int, dv: int) -> int:
    return int(load_library().gdn_prefill_backward_workspace_size(total_tokens, num_seqs, H, dk, dv))


def chunk_prefill_backward(q, k, v, g, beta, do, init_state=None, dstate=None, cu_seqlens=None, scale=None,
                           qk_l2norm=True, workspace=None, return_dinit=True):
    """Gradients of L = <do, o> + <dstate, final_state> for ``chunk_prefill``.

    Inputs as for ``chunk_prefill``; do [T, H, dv] in the dtype of q; dstate
    [N, H, dv, dk] fp32 or None (zeros).  Returns a dict of fp32 tensors dq, dk
    [T, H, dk], dv [T, H, dv], dg, dbeta [T, H] and dinit [N, H, dv, dk] (None
    when ``return_dinit`` is false).
    """
    torch = _torch()
    lib = load_library()
    dev = q.device
    _check(q, "q", device=dev)
    dt = q.dtype
    for name, t in (("k", k), ("v", v), ("do", do)):
        _check(t, name, dtype=dt, device=dev)
    _check(g, "g", dtype=torch.float32, device=dev)
    _check(beta, "beta", dtype=torch.float32, device=dev)
    T, H, dk = q.shape
    dv = v.shape[2]
    if (k.shape != (T, H, dk) or v.shape[:2] != (T, H) or do.shape != (T, H, dv) or g.shape != (T, H)
            or beta.shape != (T, H)):
        raise ValueError("shape mismatch among q, k, v, do, g, beta")
    cu_dev, cu_host, N = _seqlens(cu_seqlens, dev)
    for name, t in (("init_state", init_state), ("dstate", dstate)):
        if t is not None:
            _check(t, name, dtype=torch.float32, device=dev)
            if t.shape != (N, H, dv, dk):
                raise ValueError(f"{name} must be [{N}, {H}, {dv}, {dk}]")
    code = _dtype_code(q)
    need = int(lib.gdn_prefill_backward_workspace_size(T, N, H, dk, dv))
    if need == 0:
        raise GdnError(3, "gdn_prefill_backward_workspace_size")
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    f32 = torch.float32
    out = {"dq": torch.empty((T, H, dk), dtype=f32, device=dev), "dk": torch.empty((T, H, dk), dtype=f32, device=dev),
           "dv": torch.empty((T, H, dv), dtype=f32, device=dev), "dg": torch.empty((T, H), dtype=f32, device=dev),
           "dbeta": torch.empty((T, H), dtype=f32, device=dev),
           "dinit": torch.empty((N, H, dv, dk), dtype=f32, device=dev) if return_dinit else None}
    s = -1.0 if scale is None else float(scale)
    cu_host_ptr = None if cu_host is None else ctypes.c_void_p(cu_host.data_ptr())
    st = lib.gdn_chunk_prefill_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(init_state), _ptr(do),
                                        _ptr(dstate), _ptr(cu_dev), cu_host_ptr, N, T, H, dk, dv, code, s,
                                        int(bool(qk_l2norm)), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                                        _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dinit"]), _ptr(workspace),
                                        workspace.numel(), _stream(dev))
    if st != 0:
        raise GdnError(st, "gdn_chunk_prefill_backward")
    return out


def decode_step(q, k, v, g, beta, state, scale=None, qk_l2norm=True, out=None, gate=None, norm_weight=None,
                norm_eps=DEFAULT_NORM_EPS):
    """One recurrent decode step: q, k [N, H, dk]; v [N, H, dv]; g, beta [N, H] fp32;
    state [N, H, dv, dk] fp32 updated in place.  Returns o [N, H, dv].  With ``gate``
    [N, H, dv] the output gets the gated RMSNorm read-out (App. A.3 Eq. 20)."""
    torch = _torch()
    lib = load_library()
    dev = q.device
    _check(q, "q", device=dev)
    dt = q.dtype
    for name, t in (("k", k), ("v", v)):
        _check(t, name, dtype=dt, device=dev)
    _check(g, "g", dtype=torch.float32, device=dev)
    _check(beta, "beta", dtype=torch.float32, device=dev)
    _check(state, "state", dtype=torch.float32, device=dev)
    N, H, dk = q.shape
    dv = v.shape[2]
    if state.shape != (N, H, dv, dk):
        raise ValueError("state must be [N, H, dv, dk]")
    if out is None:
        out = torch.empty((N, H, dv), dtype=dt, device=dev)
    s = -1.0 if scale is None else float(scale)
    if gate is not None:
        _norm_args(gate, norm_weight, (N, H, dv), dt, dev)
        st = lib.gdn_decode_step_gated(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), N, H, dk, dv,
                                       _dtype_code(q), s, int(bool(qk_l2norm)), _ptr(gate), _ptr(norm_weight),
                                       float(norm_eps), _ptr(out), _stream(dev))
        if st != 0:
            raise GdnError(st, "gdn_decode_step_gated")
        return out
    st = lib.gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), N, H, dk, dv,
                             _dtype_code(q), s, int(bool(qk_l2norm)), _ptr(out), _stream(dev))
    if st != 0:
        raise GdnError(st, "gdn_decode_step")
    return out


def _frontend_args(xq, xk, xv, conv_weight, a, b, A_log, dt_bias):
    torch = _torch()
    dev = xq.device
    _check(xq, "xq", device=dev)
    dt = xq.dtype
    _dtype_code(xq)
    for name, t in (("xk", xk), ("xv", xv)):
        _check(t, name, dtype=dt, device=dev)
    for name, t in (("conv_weight", conv_weight), ("a", a), ("b", b), ("A_log", A_log), ("dt_bias", dt_bias)):
        _check(t, name, dtype=torch.float32, device=dev)
    T, H, dk = xq.shape
    dv = xv.shape[2]
    if xk.shape != (T, H, dk) or xv.shape[:2] != (T, H) or a.shape != (T, H) or b.shape != (T, H):
        raise ValueError("shape mismatch among xq, xk, xv, a, b")
    if A_log.shape != (H,) or dt_bias.shape != (H,):
        raise ValueError(f"A_log and dt_bias must be [{H}]")
    ctot = H * (2 * dk + dv)
    if conv_weight.shape != (ctot, 4):
        raise ValueError(f"conv_weight must be [{ctot}, 4] (channels of q, then k, then v)")
    return dev, dt, T, H, dk, dv, ctot


def _frontend_outputs(out, xq, xk, xv, rows, H, dev):
    """The five outputs (q, k, v, g, beta): the caller's, checked, or new tensors."""
    torch = _torch()
    if out is None:
        return (torch.empty_like(xq), torch.empty_like(xk), torch.empty_like(xv),
                torch.empty((rows, H), dtype=torch.float32, device=dev),
                torch.empty((rows, H), dtype=torch.float32, device=dev))
    q, k, v, g, beta = out
    for name, t, ref in (("q", q, xq), ("k", k, xk), ("v", v, xv)):
        _check(t, name, dtype=ref.dtype, device=dev)
        if t.shape != ref.shape:
            raise ValueError(f"{name} must have the shape of x{name}")
    for name, t in (("g", g), ("beta", beta)):
        _check(t, name, dtype=torch.float32, device=dev)
        if t.shape != (rows, H):
            raise ValueError(f"{name} must be [{rows}, {H}]")
    return q, k, v, g, beta


def frontend_prefill(xq, xk, xv, conv_weight, a, b, A_log, dt_bias, conv_state=None, cu_seqlens=None,
                     return_conv_state=True, conv_state_out=None, out=None):
    """Front end of App. A.3 over packed sequences: the 4-tap causal depthwise
    convolution with SiLU on the q, k, v projections and the gates
    g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b).

    xq, xk [T, H, dk]; xv [T, H, dv] (bf16 or fp32); conv_weight [H(2dk+dv), 4] fp32
    (channels of q, then k, then v; taps oldest first); a, b [T, H] fp32; A_log, dt_bias
    [H] fp32; conv_state [N, 3, H(2dk+dv)] (dtype of xq) or None (zeros); cu_seqlens as
    for ``chunk_prefill``.  Returns (q, k, v, g, beta, conv_state_out); conv_state_out
    is None unless asked for (``conv_state_out`` may be the input state: in place).
    ``out`` optionally gives the (q, k, v, g, beta) tensors to write.
    """
    torch = _torch()
    lib = load_library()
    dev, dt, T, H, dk, dv, ctot = _frontend_args(xq, xk, xv, conv_weight, a, b, A_log, dt_bias)
    cu_dev = None
    if cu_seqlens is None:
        N = 1
    else:
        if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.device.type == "cuda":
            cu_dev = cu_seqlens.to(torch.int32).contiguous()
        else:
            cu_dev = torch.as_tensor(cu_seqlens, dtype=torch.int32).contiguous().to(dev)
        N = cu_dev.shape[0] - 1
    if conv_state is not None:
        _check(conv_state, "conv_state", dtype=dt, device=dev)
        if conv_state.shape != (N, 3, ctot):
            raise ValueError(f"conv_state must be [{N}, 3, {ctot}]")
    if conv_state_out is None and return_conv_state:
        conv_state_out = torch.empty((N, 3, ctot), dtype=dt, device=dev)
    elif conv_state_out is not None:
        _check(conv_state_out, "conv_state_out", dtype=dt, device=dev)
        if conv_state_out.shape != (N, 3, ctot):
            raise ValueError(f"conv_state_out must be [{N}, 3, {ctot}]")
    q, k, v, g, beta = _frontend_outputs(out, xq, xk, xv, T, H, dev)
    st = lib.gdn_frontend_prefill(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(conv_weight), _ptr(a), _ptr(b), _ptr(A_log),
                                  _ptr(dt_bias), _ptr(conv_state), _ptr(cu_dev), N, T, H, dk, dv, _dtype_code(xq),
                                  _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(conv_state_out), _stream(dev))
    if st != 0:
        raise GdnError(st, "gdn_frontend_prefill")
    return q, k, v, g, beta, conv_state_out


def chunk_prefill_frontend(xq, xk, xv, conv_weight, a, b, A_log, dt_bias, conv_state=None, init_state=None,
                           cu_seqlens=None, scale=None, qk_l2norm=True, chunk=64, out=None, final_state=None,
                           return_conv_state=True, conv_state_out=None, workspace=None, ctx=None):
    """The front end folded into the chunked prefill (bf16): the result of
    ``frontend_prefill`` followed by ``chunk_prefill``, bit for bit, without the
    q, k, v, g, beta round trip.  Arguments as for those two calls.  Returns
    (o [T, H, dv], final_state [N, H, dv, dk], conv_state_out or None)."""
    torch = _torch()
    lib = load_library()
    dev, dt, T, H, dk, dv, ctot = _frontend_args(xq, xk, xv, conv_weight, a, b, A_log, dt_bias)
    cu_dev, cu_host, N = _seqlens(cu_seqlens, dev)
    if conv_state is not None:
        _check(conv_state, "conv_state", dtype=dt, device=dev)
        if conv_state.shape != (N, 3, ctot):
            raise ValueError(f"conv_state must be [{N}, 3, {ctot}]")
    if conv_state_out is None and return_conv_state:
        conv_state_out = torch.empty((N, 3, ctot), dtype=dt, device=dev)
    elif conv_state_out is not None:
        _check(conv_state_out, "conv_state_out", dtype=dt, device=dev)
        if conv_state_out.shape != (N, 3, ctot):
            raise ValueError(f"conv_state_out must be [{N}, 3, {ctot}]")
    if init_state is not None:
        _check(init_state, "init_state", dtype=torch.float32, device=dev)
        if init_state.shape != (N, H, dv, dk):
            raise ValueError(f"init_state must be [{N}, {H}, {dv}, {dk}]")
    if out is None:
        out = torch.empty((T, H, dv), dtype=dt, device=dev)
    else:
        _check(out, "out", dtype=dt, device=dev)
    if final_state is None:
        final_state = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev)
    else:
        _check(final_state, "final_state", dtype=torch.float32, device=dev)
    code = _dtype_code(xq)
    need = int(lib.gdn_prefill_workspace_size(T, N, H, dk, dv, chunk, code))
    if need == 0:
        raise GdnError(3, "gdn_prefill_workspace_size")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    else:  # a smaller buffer (down to prefill_workspace_min_size) runs the chunks in windows
        _check(workspace, "workspace", dtype=torch.uint8, device=dev)
    s = -1.0 if scale is None else float(scale)
    cu_host_ptr = None if cu_host is None else ctypes.c_void_p(cu_host.data_ptr())
    st = lib.gdn_chunk_prefill_frontend(None if ctx is None else ctx.handle, _ptr(xq), _ptr(xk), _ptr(xv),
                                        _ptr(conv_weight), _ptr(a), _ptr(b), _ptr(A_log), _ptr(dt_bias),
                                        _ptr(conv_state), _ptr(init_state), _ptr(cu_dev), cu_host_ptr, N, T, H, dk,
                                        dv, chunk, code, s, int(bool(qk_l2norm)), _ptr(out), _ptr(final_state),
                                        _ptr(conv_state_out), _ptr(workspace), workspace.numel(), _stream(dev))
    if st != 0:
        raise GdnError(st, "gdn_chunk_prefill_frontend")
    return out, final_state, conv_state_out


def frontend_decode(xq, xk, xv, conv_weight, a, b, A_log, dt_bias, conv_state, out=None):
    """Front end for one decode token per sequence: xq, xk [N, H, dk]; xv [N, H, dv];
    a, b [N, H]; conv_state [N, 3, H(2dk+dv)] updated in place.  Returns (q, k, v, g, beta),
    the inputs of ``decode_step``; ``out`` optionally gives those five tensors."""
    torch = _torch()
    lib = load_library()
    dev, dt, N, H, dk, dv, ctot = _frontend_args(xq, xk, xv, conv_weight, a, b, A_log, dt_bias)
    _check(conv_state, "conv_state", dtype=dt, device=dev)
    if conv_state.shape != (N, 3, ctot):
        raise ValueError(f"conv_state must be [{N}, 3, {ctot}]")
    q, k, v, g, beta = _frontend_outputs(out, xq, xk, xv, N, H, dev)
    st = lib.gdn_frontend_decode(_ptr(xq), _ptr(xk), _ptr(xv), _ptr(conv_weight), _ptr(a), _ptr(b), _ptr(A_log),
                                 _ptr(dt_bias), _ptr(conv_state), N, H, dk, dv, _dtype_code(xq), _ptr(q), _ptr(k),
                                 _ptr(v), _ptr(g), _ptr(beta), _stream(dev))
    if st != 0:
        raise GdnError(st, "gdn_frontend_decode")
    return q, k, v, g, beta


def default_scale(dk: int) -> float:
    return 1.0 / math.sqrt(dk)
