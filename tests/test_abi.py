"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/gdn.h, and rejects bad arguments on the host before any
launch (every call below returns before touching the device)."""
import ctypes
import os
import re
import subprocess

import pytest

from hybrid_linear_attention_delta_amd import gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(gdn_\w+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIB_PATH):
        pytest.fail("libgdn_mi355x.so is not built (run __graft_entry__.build())")
    return gdn.load_library()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("gdn_chunk_prefill", "gdn_decode_step", "gdn_prefill_workspace_size", "gdn_status_string"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", gdn.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, flags=re.M))
    missing = [n for n in _declared_functions() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    for n in _declared_functions():
        getattr(lib, n)  # resolvable through ctypes


def test_no_unresolved_internal_symbols():
    """Every kernel the host code launches is defined in the library itself (a
    host-side kernel stub that the compiler failed to emit shows up here as an
    undefined gdn:: symbol, which only fails when the library is bound eagerly)."""
    out = subprocess.run(["nm", "-u", gdn.LIB_PATH], capture_output=True, text=True, check=True).stdout
    bad = [l.split()[-1] for l in out.splitlines() if "_ZN3gdn" in l]
    assert not bad, f"undefined internal symbols: {bad[:5]}"
    ctypes.CDLL(gdn.LIB_PATH, mode=os.RTLD_NOW)


def test_status_strings(lib):
    for code, name in gdn.STATUS.items():
        assert lib.gdn_status_string(code).decode().startswith(name)
    assert lib.gdn_version() >= 100


def test_workspace_size_queries(lib):
    ws = lib.gdn_prefill_workspace_size(65536, 1, 6, 256, 256, 64, gdn.GDN_BF16)
    assert ws > 0
    # grows with tokens; unsupported combinations give 0
    assert lib.gdn_prefill_workspace_size(131072, 1, 6, 256, 256, 64, gdn.GDN_BF16) > ws
    assert lib.gdn_prefill_workspace_size(1024, 1, 6, 256, 256, 32, gdn.GDN_BF16) == 0
    assert lib.gdn_prefill_workspace_size(1024, 1, 6, 48, 48, 64, gdn.GDN_F32) == 0
    assert lib.gdn_prefill_workspace_size(64, 1, 2, 16, 16, 16, gdn.GDN_F32) > 0
    assert lib.gdn_prefill_workspace_size(-1, 1, 2, 16, 16, 16, gdn.GDN_F32) == 0


def _fake(addr=0x10000):
    return ctypes.c_void_p(addr)


def _prefill(lib, **kw):
    a = dict(q=_fake(), k=_fake(), v=_fake(), g=_fake(), beta=_fake(), init=None, cu=None, cu_host=None, N=1,
             T=128, H=2, dk=64, dv=64, chunk=64, dt=gdn.GDN_BF16, scale=-1.0, l2=1, o=_fake(), fs=None,
             ws=_fake(0x100000), wsb=1 << 40, stream=None)
    a.update(kw)
    return lib.gdn_chunk_prefill(a["q"], a["k"], a["v"], a["g"], a["beta"], a["init"], a["cu"], a["cu_host"], a["N"],
                                 a["T"], a["H"], a["dk"], a["dv"], a["chunk"], a["dt"], a["scale"], a["l2"], a["o"],
                                 a["fs"], a["ws"], a["wsb"], a["stream"])


def test_prefill_host_validation(lib):
    assert _prefill(lib, dk=48) == 3                       # unsupported
    assert _prefill(lib, chunk=32) == 3                    # bf16 needs chunk 64
    assert _prefill(lib, dt=7) == 3
    assert _prefill(lib, T=-5) == 2
    assert _prefill(lib, H=0) == 2
    assert _prefill(lib, N=2) == 2                         # N > 1 needs cu_seqlens
    assert _prefill(lib, q=None) == 1
    assert _prefill(lib, ws=None) == 6
    assert _prefill(lib, wsb=16) == 6
    assert _prefill(lib, q=_fake(0x10004)) == 5            # misaligned
    assert _prefill(lib, g=_fake(0x10002)) == 5            # gates need 4-byte alignment
    assert _prefill(lib, g=_fake(0x10004)) != 5
    assert _prefill(lib, ws=_fake(0x100010)) == 5          # workspace must be 256-byte aligned
    cu = (ctypes.c_int32 * 3)(0, 100, 90)                  # not monotone
    assert _prefill(lib, cu=_fake(0x20000), cu_host=cu, N=2, T=90) == 4
    cu = (ctypes.c_int32 * 3)(0, 50, 120)                  # last != T
    assert _prefill(lib, cu=_fake(0x20000), cu_host=cu, N=2, T=128) == 4
    cu = (ctypes.c_int32 * 3)(1, 50, 128)                  # first != 0
    assert _prefill(lib, cu=_fake(0x20000), cu_host=cu, N=2, T=128) == 4
    # overlapping but distinct init/final state buffers
    assert _prefill(lib, init=_fake(0x40000), fs=_fake(0x40010)) == 2


def test_decode_host_validation(lib):
    f = _fake()
    call = lambda **kw: lib.gdn_decode_step(kw.get("q", f), f, f, f, f, kw.get("state", f), kw.get("N", 4), 2,
                                            kw.get("dk", 64), kw.get("dv", 64), kw.get("dt", gdn.GDN_BF16), -1.0, 1,
                                            kw.get("o", f), None)
    assert call(dk=48) == 3
    assert call(dv=1024) == 3
    assert call(dt=3) == 3
    assert call(N=-1) == 2
    assert call(N=0) == 0                                  # nothing to do, nothing launched
    assert call(state=None) == 1
    assert call(o=_fake(0x10008)) == 5


def test_context_entry_points_check_arguments(lib):
    """gdn_context_create / gdn_context_destroy check their arguments before any
    HIP call; without a GPU, creation fails cleanly (GDN_ERR_CONTEXT) and leaves
    the handle NULL.  gdn_chunk_prefill_ctx validates like gdn_chunk_prefill."""
    h = ctypes.c_void_p()
    assert lib.gdn_context_create(0, None) == 1                # GDN_ERR_NULL_ARG
    assert lib.gdn_context_create(32, ctypes.byref(h)) == 2    # more CUs than an XCD has
    assert lib.gdn_context_destroy(None) == 1
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        assert lib.gdn_context_create(0, ctypes.byref(h)) == 8  # GDN_ERR_CONTEXT
        assert h.value is None
    f = _fake()
    ctx_call = lambda **kw: lib.gdn_chunk_prefill_ctx(None, f, f, f, f, f, None, None, None, 1, 128, 2,
                                                      kw.get("dk", 64), 64, 64, gdn.GDN_BF16, -1.0, 1, f, None,
                                                      kw.get("ws", _fake(0x100000)), 1 << 40, None)
    assert ctx_call(dk=48) == 3
    assert ctx_call(ws=None) == 6


def test_binding_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    q = torch.zeros(4, 1, 16)
    with pytest.raises(ValueError, match="GPU"):
        gdn.decode_step(q, q, q, torch.zeros(4, 1), torch.zeros(4, 1), torch.zeros(4, 1, 16, 16))
    with pytest.raises(ValueError, match="GPU"):
        gdn.chunk_prefill(q, q, q, torch.zeros(4, 1), torch.zeros(4, 1))


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "hybrid_linear_attention_delta_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".h")):
                txt = open(os.path.join(dirpath, fn)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", txt, flags=re.M), fn
                assert "gdn_oracle" not in txt, fn


def test_gated_entry_points_reject_bad_norm_arguments(lib):
    """The gated read-out checks its own arguments first: a missing gate, a gate
    or weight off alignment, and a negative or non-finite eps return before any
    launch."""
    f = _fake()
    base = [f, f, f, f, f, None, None, None, 1, 128, 2, 64, 64, 64, gdn.GDN_BF16, -1.0, 1]
    tail = [f, None, _fake(0x100000), 1 << 40, None]
    call = lambda gate, w, eps: lib.gdn_chunk_prefill_gated(*base, gate, w, eps, *tail)
    assert call(None, None, 1e-6) == 1           # GDN_ERR_NULL_ARG
    assert call(_fake(0x10008), None, 1e-6) == 5  # GDN_ERR_ALIGNMENT (gate)
    assert call(f, _fake(0x10002), 1e-6) == 5     # GDN_ERR_ALIGNMENT (weight)
    assert call(f, None, -1e-3) == 2              # GDN_ERR_BAD_SHAPE
    assert call(f, None, float("inf")) == 2
    assert call(f, None, float("nan")) == 2
    dec = lambda gate, eps: lib.gdn_decode_step_gated(f, f, f, f, f, f, 4, 2, 64, 64, gdn.GDN_BF16, -1.0, 1, gate,
                                                      None, eps, f, None)
    assert dec(None, 1e-6) == 1
    assert dec(f, -1.0) == 2
    # nothing to do: no tokens / no sequences, no gate needed
    assert lib.gdn_decode_step_gated(f, f, f, f, f, f, 0, 2, 64, 64, gdn.GDN_BF16, -1.0, 1, None, None, 1e-6, f,
                                     None) == 0


def test_frontend_host_validation(lib):
    """The front-end entry points check sizes, pointers, alignment and state
    overlap on the host and return before any launch."""
    f = _fake()

    def pre(**kw):
        return lib.gdn_frontend_prefill(f, f, f, kw.get("w", f), f, f, f, f, kw.get("st_in", None), kw.get("cu", None),
                                        kw.get("N", 1), kw.get("T", 64), 2, kw.get("dk", 64), 64,
                                        kw.get("dt", gdn.GDN_BF16), kw.get("q", f), f, f, f, f,
                                        kw.get("st_out", None), None)

    assert pre(dk=12) == 3                      # d_k not a multiple of 8
    assert pre(dt=5) == 3
    assert pre(T=-1) == 2
    assert pre(N=2) == 2                        # several sequences need cu_seqlens
    assert pre(q=None) == 1
    assert pre(w=_fake(0x10004)) == 5           # taps must be 16-byte aligned
    assert pre(st_in=_fake(0x40000), st_out=_fake(0x40010)) == 2  # partial overlap
    assert pre(T=0) == 0                        # nothing to do

    def dec(**kw):
        return lib.gdn_frontend_decode(f, f, f, f, f, f, f, f, kw.get("st", f), kw.get("N", 4), 2, 64, 64,
                                       gdn.GDN_BF16, f, f, f, f, f, None)

    assert dec(st=None) == 1
    assert dec(N=-1) == 2
    assert dec(N=0) == 0
    assert dec(st=_fake(0x10008)) == 5


@pytest.mark.parametrize("T,N,H,dk,dv", [(128, 1, 2, 64, 64), (1000, 3, 2, 64, 128), (65536, 1, 6, 256, 256),
                                         (2_097_152, 16, 6, 256, 256)])
def test_backward_workspace_size_matches_the_header_formula(lib, T, N, H, dk, dv):
    """gdn_prefill_backward_workspace_size is the size the header documents:
    max_chunks * H * (2 dv dk + 64 (10 dk + 8 dv) + 7 * 64 * 64 + 5 * 64) * 4
    bytes for the per-chunk slots, plus the header words, the chunk table and
    at most 256 bytes of alignment per slot."""
    mc = T // 64 + N
    formula = mc * H * (2 * dv * dk + 64 * (10 * dk + 8 * dv) + 7 * 64 * 64 + 5 * 64) * 4
    size = lib.gdn_prefill_backward_workspace_size(T, N, H, dk, dv)
    extra = size - formula
    assert 0 <= extra - mc * 16 - (N + 1) * 4 - 64 < 40 * 256, (size, formula)


def test_backward_host_validation(lib):
    """The backward entry point checks sizes, support, pointers, alignment,
    sequence bounds and the workspace on the host and returns before any launch."""
    f = _fake()
    need = lib.gdn_prefill_backward_workspace_size(128, 1, 2, 64, 64)
    assert need > 0
    assert lib.gdn_prefill_backward_workspace_size(128, 1, 2, 48, 64) == 0
    assert lib.gdn_prefill_backward_workspace_size(128, 0, 2, 64, 64) == 0

    def bwd(**kw):
        return lib.gdn_chunk_prefill_backward(kw.get("q", f), f, f, f, f, None, f, None, kw.get("cu", None),
                                              kw.get("cu_host", None), kw.get("N", 1), kw.get("T", 128), 2,
                                              kw.get("dk", 64), 64, kw.get("dt", gdn.GDN_BF16), -1.0, 1,
                                              kw.get("gq", f), f, f, f, f, None, kw.get("ws", f),
                                              kw.get("wsb", need), None)

    assert bwd(dk=96) == 3
    assert bwd(dt=7) == 3
    assert bwd(T=-1) == 2
    assert bwd(N=2) == 2                       # several sequences need cu_seqlens
    assert bwd(q=None) == 1
    assert bwd(gq=None) == 1
    assert bwd(gq=_fake(0x10004)) == 5         # gradients must be 16-byte aligned
    assert bwd(ws=None) == 6
    assert bwd(wsb=need - 1) == 6
    assert bwd(ws=_fake(0x10010)) == 5         # workspace 256-byte aligned
    bad = (ctypes.c_int32 * 3)(0, 100, 90)
    assert bwd(N=2, cu=f, cu_host=bad) == 4

    def bwd_states(init, dfinal, dinit):
        return lib.gdn_chunk_prefill_backward(f, f, f, f, f, init, f, dfinal, None, None, 1, 128, 2, 64, 64,
                                              gdn.GDN_BF16, -1.0, 1, f, f, f, f, f, dinit, f, need, None)

    assert bwd_states(_fake(0x40000), None, _fake(0x40000)) == 2   # the initial-state gradient over init_state
    assert bwd_states(None, _fake(0x40000), _fake(0x44000)) == 2   # partly over d_final_state
    assert bwd_states(None, _fake(0x40000), _fake(0x40000)) == 2   # or exactly


def test_workspace_min_size_and_windowed_workspace_checks(lib):
    """gdn_prefill_workspace_min_size: between it and the full size a whole-prefill
    call runs in windows of chunks; below it, or for a subset of the stages with
    less than the full size, the call is refused before any launch."""
    args = (65536, 1, 6, 256, 256, 64, gdn.GDN_BF16)
    full = lib.gdn_prefill_workspace_size(*args)
    mn = lib.gdn_prefill_workspace_min_size(*args)
    assert 0 < mn < full
    assert mn >= 6 * 256 * 256 * 4  # at least the fp32 state carry of the six (sequence, head) pairs
    assert lib.gdn_prefill_workspace_min_size(1024, 1, 6, 256, 256, 32, gdn.GDN_BF16) == 0  # unsupported
    assert lib.gdn_prefill_workspace_min_size(-1, 1, 2, 16, 16, 16, gdn.GDN_F32) == 0
    # the minimum grows with the carried state (sequences), not with the tokens
    assert lib.gdn_prefill_workspace_min_size(8 * 65536, 1, 6, 256, 256, 64, gdn.GDN_BF16) < full
    T = 4096
    mn = lib.gdn_prefill_workspace_min_size(T, 1, 2, 64, 64, 64, gdn.GDN_BF16)
    full = lib.gdn_prefill_workspace_size(T, 1, 2, 64, 64, 64, gdn.GDN_BF16)
    assert _prefill(lib, T=T, wsb=mn - 256) == 6
    f = _fake()
    staged = lambda wsb, stages: lib.gdn_chunk_prefill_staged(f, f, f, f, f, None, None, None, 1, T, 2, 64, 64, 64,
                                                               gdn.GDN_BF16, -1.0, 1, f, None, _fake(0x100000), wsb,
                                                               stages, None)
    assert staged(full - 256, gdn.STAGE_PREPARE) == 6
    assert staged(mn, gdn.STAGE_ALL ^ gdn.STAGE_OUTPUT) == 6
