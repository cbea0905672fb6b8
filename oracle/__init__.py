"""fp64 CPU oracle of the gated delta rule -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product library never imports it,
and it imports nothing from the product package.

The oracle follows "Long-Context Aware Upcycling: A New Frontier for Hybrid LLM
Scaling" (arXiv:2604.24715), App. A.3 "GDN Layer Architecture", Eqs. 16-19: a
plain sequential recurrence, one token at a time, in fp64 (``gdn_oracle.c``).
``forms.py`` holds two other fp64 evaluations of the same map (the unrolled
product form and the chunked WY form) that exist to pin the recurrence.

Arrays are numpy.  bf16 data is passed as ``numpy.uint16`` holding the raw
bf16 bit patterns (``dtype_code='bf16'``); the oracle widens each stored value
exactly to fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_BUILD_DIR = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD_DIR, "libgdn_oracle.so")

OR_F64, OR_F32, OR_BF16 = 0, 1, 2

# Planted mistakes, used only by the pin-strength tests (see gdn_oracle.c).
MUTATIONS = {
    "retrieve_undecayed": 1,
    "read_before_write": 2,
    "delta_sign": 3,
    "no_beta_write": 4,
    "decay_after_write": 5,
    "q_unnormalised": 6,
    "output_uses_k": 7,
}

DEFAULT_EPS = 1e-6

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile gdn_oracle.c with gcc into oracle/_build/libgdn_oracle.so."""
    os.makedirs(_BUILD_DIR, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        # -O2 without -ffast-math: fp64 arithmetic in source order (no reassociation,
        # no contraction into FMAs).
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-ffp-contract=off",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build()
            lib = ctypes.CDLL(_LIB_PATH)
            vp, i32, i64p, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_double
            lib.oracle_prefill_f64.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int, vp, ctypes.c_int,
                                               i64p, i32, i32, i32, i32, dbl, i32, dbl, vp, i32, vp, vp, i32, i32]
            lib.oracle_prefill_f64.restype = ctypes.c_int
            lib.oracle_decode_f64.argtypes = [vp, vp, vp, ctypes.c_int, vp, vp, ctypes.c_int, vp,
                                              i32, i32, i32, i32, dbl, i32, dbl, vp, i32]
            lib.oracle_decode_f64.restype = ctypes.c_int
            _lib = lib
    return _lib


def _code(a: np.ndarray, bf16: bool) -> int:
    if bf16:
        if a.dtype != np.uint16:
            raise TypeError("bf16 data must be passed as uint16 bit patterns")
        return OR_BF16
    if a.dtype == np.float64:
        return OR_F64
    if a.dtype == np.float32:
        return OR_F32
    raise TypeError(f"unsupported dtype {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def default_threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(n, 16))


def prefill(q, k, v, g, beta, init_state=None, cu_seqlens=None, scale=None, qk_l2norm=True,
            eps=DEFAULT_EPS, rows=None, bf16=False, n_threads=None, mutation=0, timing=None):
    """Sequential fp64 gated delta rule over packed sequences.

    q, k: [T, H, dk]; v: [T, H, dv]; g, beta: [T, H] (g is the log forget gate,
    alpha = e^g); init_state: [N, H, dv, dk] or None (zeros); cu_seqlens: int
    [N+1] or None (one sequence).  scale None -> 1/sqrt(dk) (Eq. 19).
    rows: optional list of state rows (value indices) to evaluate; other
    entries of the returned o / final_state are NaN.
    Returns (o [T, H, dv] fp64, final_state [N, H, dv, dk] fp64).
    ``timing``: optional dict; its "seconds" is set to the wall time of the
    oracle's own computation (the C call alone: argument checks, allocation of
    the outputs and conversions happen outside the timed region).
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    T, H, dk = q.shape
    dv = v.shape[2]
    if k.shape != (T, H, dk) or v.shape[:2] != (T, H):
        raise ValueError("shape mismatch")
    if g.dtype != beta.dtype:
        raise TypeError("g and beta must share a dtype")
    g = np.ascontiguousarray(g)
    beta = np.ascontiguousarray(beta)
    if g.shape != (T, H) or beta.shape != (T, H):
        raise ValueError("gate shape mismatch")
    if cu_seqlens is None:
        cu = np.array([0, T], dtype=np.int64)
    else:
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
    N = cu.shape[0] - 1
    if cu[0] != 0 or cu[-1] != T:
        raise ValueError("cu_seqlens must start at 0 and end at T")
    if init_state is not None:
        init_state = np.ascontiguousarray(init_state)
        if init_state.shape != (N, H, dv, dk):
            raise ValueError("init_state shape")
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    r = None
    if rows is not None:
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32))
    fill = np.nan if rows is not None else 0.0
    o = np.full((T, H, dv), fill, dtype=np.float64)
    fs = np.full((N, H, dv, dk), fill, dtype=np.float64)
    lib = _load()
    args = (_ptr(q), _ptr(k), _ptr(v), _code(q, bf16),
            _ptr(g), _ptr(beta), _code(g, False),
            _ptr(init_state), _code(init_state, False) if init_state is not None else OR_F64,
            _ptr(cu), N, H, dk, dv, float(scale), int(bool(qk_l2norm)), float(eps),
            _ptr(r), 0 if r is None else int(r.shape[0]),
            _ptr(o), _ptr(fs), int(n_threads or default_threads()), int(mutation))
    t0 = time.perf_counter()
    rc = lib.oracle_prefill_f64(*args)
    if timing is not None:
        timing["seconds"] = time.perf_counter() - t0
    if rc != 0:
        raise RuntimeError("oracle_prefill_f64 rejected its arguments")
    return o, fs


def decode_step(q, k, v, g, beta, state, scale=None, qk_l2norm=True, eps=DEFAULT_EPS, bf16=False,
                n_threads=None):
    """One recurrent step for N sequences; ``state`` [N,H,dv,dk] fp64 is updated in place.

    q, k: [N, H, dk]; v: [N, H, dv]; g, beta: [N, H].  Returns o [N, H, dv] fp64.
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    N, H, dk = q.shape
    dv = v.shape[2]
    if state.dtype != np.float64 or not state.flags.c_contiguous or state.shape != (N, H, dv, dk):
        raise ValueError("state must be a contiguous fp64 [N,H,dv,dk] array")
    g = np.ascontiguousarray(g)
    beta = np.ascontiguousarray(beta)
    if scale is None:
        scale = 1.0 / np.sqrt(dk)
    o = np.zeros((N, H, dv), dtype=np.float64)
    rc = _load().oracle_decode_f64(
        _ptr(q), _ptr(k), _ptr(v), _code(q, bf16), _ptr(g), _ptr(beta), _code(g, False),
        _ptr(state), N, H, dk, dv, float(scale), int(bool(qk_l2norm)), float(eps), _ptr(o),
        int(n_threads or default_threads()))
    if rc != 0:
        raise RuntimeError("oracle_decode_f64 rejected its arguments")
    return o


# ----------------------------------------------------------------- gated RMSNorm read-out

DEFAULT_NORM_EPS = 1e-6

# Planted mistakes of the gated read-out, used only by the pin-strength tests.
NORM_MUTATIONS = {
    "sigmoid_gate": 1,     # sigma(z) instead of z sigma(z)
    "sum_not_mean": 2,     # sum of squares over d_v instead of the mean
    "no_eps": 3,           # eps dropped
    "no_weight": 4,        # per-channel weight ignored
    "norm_over_heads": 5,  # statistics over all heads of a token instead of per head
}


def _widen(a, bf16):
    a = np.asarray(a)
    if bf16:
        if a.dtype != np.uint16:
            raise ValueError("bf16 data must be passed as raw uint16 bit patterns")
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def gated_rmsnorm(o, z, weight=None, eps=DEFAULT_NORM_EPS, bf16=False, mutation=0):
    """Gated RMSNorm read-out of "Long-Context Aware Upcycling: A New Frontier for
    Hybrid LLM Scaling" (arXiv:2604.24715), App. A.3 Eq. 20: the read of the
    updated state (Eq. 19) is normalised by its root mean square and gated by a
    projection of the layer input, before the output projection of Eq. 21.

    Read here, per (token, head), over the d_v values of that head:

        y = o / sqrt(mean_v(o_v^2) + eps) * w * silu(z),   silu(x) = x / (1 + e^{-x})

    ``o`` is the read-out [..., H, d_v] (fp64, e.g. this oracle's prefill or
    decode output, with its 1/sqrt(d_k) scale), ``z`` [..., H, d_v] the gate input
    W_G x_t (raw bf16 bit patterns when ``bf16``), ``weight`` [d_v] the per-channel
    scale shared by the heads (None: ones).  The projection W_G itself is not part
    of this path.  Returns fp64 [..., H, d_v].
    """
    o = np.asarray(o, dtype=np.float64)
    zz = _widen(z, bf16)
    if zz.shape != o.shape:
        raise ValueError("z must have the shape of o")
    w = np.ones(o.shape[-1]) if (weight is None or mutation == 4) else np.asarray(weight, dtype=np.float64)
    if mutation == 5:
        ms = np.mean(o * o, axis=(-2, -1), keepdims=True)
    elif mutation == 2:
        ms = np.sum(o * o, axis=-1, keepdims=True)
    else:
        ms = np.mean(o * o, axis=-1, keepdims=True)
    e = 0.0 if mutation == 3 else float(eps)
    sig = 1.0 / (1.0 + np.exp(-zz))
    gate = sig if mutation == 1 else zz * sig
    return o / np.sqrt(ms + e) * w * gate


# ----------------------------------------------------------------- front end (conv + gates)

from .frontend import CONV_MUTATIONS, GATE_MUTATIONS, gates, short_conv_silu  # noqa: E402,F401
from .backward import BWD_MUTATIONS, prefill_vjp  # noqa: E402,F401
