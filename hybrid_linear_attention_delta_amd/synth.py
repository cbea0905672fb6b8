"""Seeded synthetic inputs for the gated delta-rule workloads.

This module holds the data recipe only: random draws, the input distributions
and dtype rounding.  It contains none of the mixer's arithmetic, and it is the
one module that both the checked path (tests, oracle) and the GPU path read.

Recipe (numpy PCG64):
  * seed = 1000 + workload number; one child stream per tensor, spawned from
    ``SeedSequence(seed)`` in the order q, k, v, g, beta, state, per-step data;
  * q, k ~ N(0, 1), then divided by their L2 norm per (token, head) in fp64,
    then rounded to the storage dtype (bf16: round-to-nearest-even directly
    from fp64);
  * v ~ N(0, 1) rounded to the storage dtype;
  * log forget gate g = -softplus(x + 2), x ~ N(0, 1)  ("default"), or
    g = -U(0, 0.02) ("slow", long memory across chunks); stored fp32;
  * write strength beta = sigmoid(y), y ~ N(0, 1); stored fp32;
  * decode state ~ N(0, 0.02^2) fp32.

The gate domains follow "Long-Context Aware Upcycling: A New Frontier for
Hybrid LLM Scaling", App. A.3 (g in (-inf, 0), beta in (0, 1)); the shapes
follow its Table 8 / the HyLo-Qwen GDN card (6 heads, head dim 256).

bf16 tensors are returned as uint16 numpy arrays of bit patterns; ``bf16_to_f32``
widens them and ``to_torch`` wraps them as torch bfloat16 tensors.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

WORKLOADS = {
    # name: (number, description)
    "tiny": 0,
    "prefill8k": 1,
    "prefill64k": 2,
    "decode": 3,
    "varlen2m": 4,
}


def seed_for(workload: str) -> int:
    return 1000 + WORKLOADS[workload]


# ----------------------------------------------------------------------------- rounding

def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (round-to-nearest-even), returning uint16 bits.

    Values must be finite and inside the normal range of binary32 (the recipe's
    values are); zero is handled.
    """
    x = np.ascontiguousarray(x, dtype=np.float64)
    b = x.view(np.uint64)
    # fp64 keeps 52 mantissa bits, bf16 keeps 7: drop the low 45 with RNE.
    lsb = (b >> np.uint64(45)) & np.uint64(1)
    r = b + (np.uint64((1 << 44) - 1) + lsb)
    r &= ~np.uint64((1 << 45) - 1)
    y = r.view(np.float64).astype(np.float32)  # exact: <= 8 significant bits
    return (y.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_torch(a: np.ndarray, device=None, bf16: bool = False):
    import torch

    if bf16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(device) if device is not None else t


# ----------------------------------------------------------------------------- draws

def _unit_rows(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _store(x64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f64_to_bf16_bits(x64)
    if dtype == "f32":
        return x64.astype(np.float32)
    if dtype == "f64":
        return x64
    raise ValueError(dtype)


def _gates(rng_g, rng_b, shape, gate: str):
    if gate == "default":
        x = rng_g.standard_normal(shape)
        g = -np.logaddexp(0.0, x + 2.0)  # -softplus(x + 2)
    elif gate == "slow":
        g = -rng_g.uniform(0.0, 0.02, size=shape)
    else:
        raise ValueError(gate)
    y = rng_b.standard_normal(shape)
    beta = 1.0 / (1.0 + np.exp(-y))
    return g.astype(np.float32), beta.astype(np.float32)


@dataclass
class PrefillInputs:
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    cu_seqlens: np.ndarray
    dtype: str
    init_state: np.ndarray | None = None
    meta: dict = field(default_factory=dict)

    @property
    def bf16(self) -> bool:
        return self.dtype == "bf16"


def prefill_inputs(T: int, H: int, dk: int, dv: int, dtype: str, seed: int, gate: str = "default",
                   cu_seqlens=None, init_state_std: float | None = None) -> PrefillInputs:
    """Packed prefill inputs: q, k [T,H,dk], v [T,H,dv], g, beta [T,H]."""
    ss = np.random.SeedSequence(seed)
    rq, rk, rv, rg, rb, rs = [np.random.default_rng(s) for s in ss.spawn(6)]
    q = _store(_unit_rows(rq, (T, H, dk)), dtype)
    k = _store(_unit_rows(rk, (T, H, dk)), dtype)
    v = _store(rv.standard_normal((T, H, dv)), dtype)
    g, beta = _gates(rg, rb, (T, H), gate)
    cu = np.array([0, T], dtype=np.int64) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    init = None
    if init_state_std is not None:
        N = cu.shape[0] - 1
        init = (rs.standard_normal((N, H, dv, dk)) * init_state_std).astype(np.float32)
    return PrefillInputs(q, k, v, g, beta, cu, dtype, init, dict(seed=seed, gate=gate))


def backward_cotangents(T: int, H: int, dk: int, dv: int, N: int, dtype: str, seed: int,
                        dstate_std: float | None = 0.1):
    """Cotangents for a prefill backward: do [T,H,dv] ~ N(0,1) stored in ``dtype``
    and dstate [N,H,dv,dk] fp32 ~ N(0, dstate_std^2) (None when dstate_std is None)."""
    ss = np.random.SeedSequence([seed, 7])
    ro, rs = [np.random.default_rng(s) for s in ss.spawn(2)]
    do = _store(ro.standard_normal((T, H, dv)), dtype)
    ds = None if dstate_std is None else (rs.standard_normal((N, H, dv, dk)) * dstate_std).astype(np.float32)
    return do, ds


def decode_state(N: int, H: int, dk: int, dv: int, seed: int, std: float = 0.02) -> np.ndarray:
    ss = np.random.SeedSequence(seed)
    rs = np.random.default_rng(ss.spawn(6)[5])
    return (rs.standard_normal((N, H, dv, dk)) * std).astype(np.float32)


def decode_step_inputs(N: int, H: int, dk: int, dv: int, dtype: str, seed: int, step: int,
                       gate: str = "default"):
    """Per-step decode tensors q, k [N,H,dk], v [N,H,dv], g, beta [N,H]."""
    ss = np.random.SeedSequence([seed, 1 + step])
    rq, rk, rv, rg, rb = [np.random.default_rng(s) for s in ss.spawn(5)]
    q = _store(_unit_rows(rq, (N, H, dk)), dtype)
    k = _store(_unit_rows(rk, (N, H, dk)), dtype)
    v = _store(rv.standard_normal((N, H, dv)), dtype)
    g, beta = _gates(rg, rb, (N, H), gate)
    return q, k, v, g, beta


def norm_inputs(shape, dtype: str, seed: int):
    """Inputs of the gated read-out: the gate input z ~ N(0, 1) of the given shape
    [..., d_v] stored in `dtype`, and a per-channel weight U(0.5, 1.5) [d_v] fp32."""
    ss = np.random.SeedSequence([seed, 7919])
    rz, rw = [np.random.default_rng(s) for s in ss.spawn(2)]
    z = _store(rz.standard_normal(tuple(shape)), dtype)
    w = rw.uniform(0.5, 1.5, size=shape[-1]).astype(np.float32)
    return z, w


def varlen_lengths(seed: int, n_seqs: int = 16, total: int = 2_097_152, lo: int = 4096,
                   hi: int = 524_288) -> np.ndarray:
    """Sequence lengths drawn log-uniform on [lo, hi], redrawn until the sum is
    within 2 % of ``total``, then the residual goes to the sequence with the
    most headroom inside the bounds."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7]))
    while True:
        L = np.exp(rng.uniform(np.log(lo), np.log(hi), size=n_seqs)).astype(np.int64)
        L = np.clip(L, lo, hi)
        if abs(int(L.sum()) - total) <= 0.02 * total:
            break
    resid = total - int(L.sum())
    if resid > 0:
        i = int(np.argmax(hi - L))
        L[i] += resid
    elif resid < 0:
        i = int(np.argmax(L - lo))
        L[i] += resid
    assert L.sum() == total and L.min() >= lo and L.max() <= hi
    return L


def varlen_torch_inputs(lengths, H: int, dk: int, dv: int, seed: int, device):
    """Large packed bf16 inputs drawn on the device with torch's seeded generator
    (one generator per sequence), same distributions as ``prefill_inputs``.

    Used where numpy would take minutes (millions of tokens).  Returns torch
    tensors q, k, v (bf16), g, beta (fp32) and cu_seqlens (int32, device)."""
    import torch

    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    q = torch.empty((T, H, dk), dtype=torch.bfloat16, device=device)
    k = torch.empty((T, H, dk), dtype=torch.bfloat16, device=device)
    v = torch.empty((T, H, dv), dtype=torch.bfloat16, device=device)
    g = torch.empty((T, H), dtype=torch.float32, device=device)
    beta = torch.empty((T, H), dtype=torch.float32, device=device)
    t0 = 0
    for i, L in enumerate(lengths):
        gen = torch.Generator(device=device)
        gen.manual_seed(seed * 1000 + i)
        for dst, d in ((q, dk), (k, dk)):
            x = torch.randn((L, H, d), generator=gen, device=device, dtype=torch.float32)
            x = x / x.norm(dim=-1, keepdim=True)
            dst[t0:t0 + L] = x.to(torch.bfloat16)
            del x
        v[t0:t0 + L] = torch.randn((L, H, dv), generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)
        x = torch.randn((L, H), generator=gen, device=device, dtype=torch.float32)
        g[t0:t0 + L] = -torch.nn.functional.softplus(x + 2.0)
        y = torch.randn((L, H), generator=gen, device=device, dtype=torch.float32)
        beta[t0:t0 + L] = torch.sigmoid(y)
        t0 += L
    cu = torch.tensor([0] + list(np.cumsum(lengths)), dtype=torch.int32, device=device)
    return q, k, v, g, beta, cu


@dataclass
class FrontendInputs:
    """Inputs of the mixer's front end: the projections before the short convolution
    (xq, xk [T, H*dk], xv [T, H*dv] in the storage dtype), the depthwise taps
    [2*H*dk + H*dv, 4] fp32 (oldest first, channels of q, then k, then v), the gate
    projections a = W_alpha x, b = W_beta x [T, H] fp32, A_log and dt_bias [H] fp32,
    and an optional conv state [N, 3, 2*H*dk + H*dv] in the storage dtype."""
    xq: np.ndarray
    xk: np.ndarray
    xv: np.ndarray
    conv_weight: np.ndarray
    a: np.ndarray
    b: np.ndarray
    A_log: np.ndarray
    dt_bias: np.ndarray
    cu_seqlens: np.ndarray
    dtype: str
    conv_state: np.ndarray | None = None

    @property
    def bf16(self) -> bool:
        return self.dtype == "bf16"


def frontend_inputs(T: int, H: int, dk: int, dv: int, dtype: str, seed: int, cu_seqlens=None,
                    with_state: bool = False, N: int | None = None) -> FrontendInputs:
    """Front-end inputs.  Projections ~ N(0, 1); taps ~ U(-1/2, 1/2), the uniform
    default initialisation of a 4-tap depthwise convolution (bound 1/sqrt(4));
    A_log = log U(0.5, 2) and dt_bias = 2 + U(-0.5, 0.5) per head, a, b ~ N(0, 1),
    so that g = -e^{A_log} softplus(a + dt_bias) spreads around the prefill
    workloads' -softplus(N(0, 1) + 2); conv state ~ N(0, 1) when asked for."""
    ss = np.random.SeedSequence([seed, 4242])
    rq, rk, rv, rw, ra, rb, rp, rs = [np.random.default_rng(s) for s in ss.spawn(8)]
    cu = np.array([0, T], dtype=np.int64) if cu_seqlens is None else np.asarray(cu_seqlens, dtype=np.int64)
    n_seqs = cu.shape[0] - 1 if N is None else N
    ctot = 2 * H * dk + H * dv
    xq = _store(rq.standard_normal((T, H * dk)), dtype)
    xk = _store(rk.standard_normal((T, H * dk)), dtype)
    xv = _store(rv.standard_normal((T, H * dv)), dtype)
    w = rw.uniform(-0.5, 0.5, size=(ctot, 4)).astype(np.float32)
    a = ra.standard_normal((T, H)).astype(np.float32)
    b = rb.standard_normal((T, H)).astype(np.float32)
    A_log = np.log(rp.uniform(0.5, 2.0, size=H)).astype(np.float32)
    dt_bias = (2.0 + rp.uniform(-0.5, 0.5, size=H)).astype(np.float32)
    st = _store(rs.standard_normal((n_seqs, 3, ctot)), dtype) if with_state else None
    return FrontendInputs(xq, xk, xv, w, a, b, A_log, dt_bias, cu, dtype, st)
