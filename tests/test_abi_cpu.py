"""The C ABI on the host: the library loads without a GPU, exports every
function include/sana_linattn.h declares, and rejects every invalid call with
the documented status before touching HIP.

Every call below carries at least one argument that the host checks reject,
so no kernel is ever launched (the pointers are placeholders, never
dereferenced)."""
import ctypes
import math
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sana_linattn.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, ALIGNMENT, HIPERR = range(6)
F32, BF16 = 0, 1


@pytest.fixture(scope="module")
def L():
    from relu_linear_attention_attn_amd import binding

    if not os.path.exists(binding.LIB_PATH):
        subprocess.run([sys.executable, os.path.join(ROOT, "relu_linear_attention_attn_amd",
                                                      "csrc", "build.py")], check=True)
    return binding.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sana_linattn_\w+)\s*\(", src)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) >= 9, names
    for n in names:
        assert hasattr(L, n), f"{n} declared in the header but not exported"
    from relu_linear_attention_attn_amd import binding
    assert sorted(binding.EXPORTS) == names


def test_version_and_strerror(L):
    assert L.sana_linattn_version() == 1
    seen = set()
    for code in range(6):
        msg = L.sana_linattn_strerror(code).decode()
        assert msg and msg not in seen
        seen.add(msg)
    assert L.sana_linattn_strerror(99).decode() == "unknown status"


def ws_size(L, B, N, H, d=32, dt=BF16):
    n = ctypes.c_size_t(123)
    st = L.sana_linattn_workspace_size(B, N, H, d, dt, ctypes.byref(n))
    return st, n.value


def test_workspace_size_rules(L):
    assert ws_size(L, 2, 16384, 70) [0] == OK
    assert ws_size(L, 0, 16, 2) == (INVALID, 0)
    assert ws_size(L, 1, 0, 2) == (INVALID, 0)
    assert ws_size(L, 1, 16, -1) == (INVALID, 0)
    assert ws_size(L, 1, 16, 2, d=64) == (UNSUPPORTED, 0)
    assert ws_size(L, 1, 16, 2, dt=7) == (UNSUPPORTED, 0)
    assert L.sana_linattn_workspace_size(1, 16, 2, 32, BF16, None) == INVALID
    # B*N*H*d*2 beyond 2^62 bytes, and int64 overflow of the product
    assert ws_size(L, 1, 1 << 40, 1 << 16)[0] == INVALID   # exactly 2^62 bytes
    assert ws_size(L, 1, 1 << 40, 1 << 15)[0] == OK        # 2^61 bytes is addressable
    assert ws_size(L, 1 << 62, 1 << 62, 1)[0] == INVALID
    # head pairs B*ceil(H/2): at most 2^22 (grids stay within 2^32 work-items)
    assert ws_size(L, 1 << 11, 1, 1 << 12)[0] == OK          # exactly 2^22 pairs
    assert ws_size(L, 1 << 11, 1, (1 << 12) + 1)[0] == INVALID
    assert ws_size(L, 1 << 22, 1, 2)[0] == OK
    assert ws_size(L, (1 << 22) + 1, 1, 1)[0] == INVALID
    # the state does not grow with n: constant once N is large
    sizes = {ws_size(L, 2, n, 70)[1] for n in (1 << 16, 1 << 18, 1 << 20, 1 << 24)}
    assert len(sizes) == 1
    # and every size is a multiple of 256 bytes and covers B*H states
    st, n = ws_size(L, 3, 5000, 7)
    assert st == OK and n % 256 == 0 and n >= 3 * 7 * 32 * 33 * 4
    # dtype does not change the state size
    assert ws_size(L, 2, 4096, 36, dt=F32) == ws_size(L, 2, 4096, 36, dt=BF16)


def test_state_size(L):
    n = ctypes.c_size_t(0)
    assert L.sana_linattn_state_size(2, 70, 32, ctypes.byref(n)) == OK
    assert n.value == 2 * 70 * 32 * 33 * 4
    assert L.sana_linattn_state_size(0, 70, 32, ctypes.byref(n)) == INVALID
    assert L.sana_linattn_state_size(1, 70, 16, ctypes.byref(n)) == UNSUPPORTED


A = 1 << 20       # placeholder device addresses, 256-byte aligned and far apart
P_Q, P_K, P_V, P_O, P_W = (A * i for i in range(1, 6))


def fwd(L, q=P_Q, k=P_K, v=P_V, o=P_O, B=1, N=64, H=2, d=32, eps=1e-6, dt=BF16, var=0,
        ws=P_W, wsb=1 << 30):
    return L.sana_linattn_fwd_variant(q, k, v, o, B, N, H, d, eps, dt, var, ws, wsb, None)


def test_fwd_rejects_invalid_arguments(L):
    assert fwd(L, B=0) == INVALID
    assert fwd(L, N=-5) == INVALID
    assert fwd(L, H=0) == INVALID
    assert fwd(L, d=16) == UNSUPPORTED
    assert fwd(L, dt=2) == UNSUPPORTED
    assert fwd(L, var=9) == UNSUPPORTED
    for name in ("q", "k", "v", "o"):
        assert fwd(L, **{name: None}) == INVALID, name
    for eps in (-1e-6, math.nan, math.inf):
        assert fwd(L, eps=eps) == INVALID, eps
    for name in ("q", "k", "v", "o"):
        assert fwd(L, **{name: A * 7 + 8}) == ALIGNMENT, name
    # out overlapping an input (bf16: 1*64*2*32*2 = 8 KB tensors)
    assert fwd(L, o=P_Q + 4096) == INVALID
    assert fwd(L, o=P_V - 4096) == INVALID
    # workspace missing, too small, misaligned, overlapping out
    need = ws_size(L, 1, 64, 2)[1]
    assert fwd(L, ws=None) == WORKSPACE
    assert fwd(L, wsb=need - 1) == WORKSPACE
    assert fwd(L, ws=P_W + 16, wsb=need) == ALIGNMENT
    assert fwd(L, ws=P_O, wsb=need) == INVALID
    # size overflow
    assert fwd(L, B=1 << 40, N=1 << 40) == INVALID
    # the plain entry point checks the same
    assert L.sana_linattn_fwd(P_Q, P_K, P_V, P_O, 1, 64, 2, 32, -1.0, BF16, P_W, 1 << 30,
                              None) == INVALID


def test_profiled_needs_enough_events(L):
    nk = ctypes.c_int(-1)
    events = (ctypes.c_void_p * 1)(None)
    st = L.sana_linattn_fwd_profiled(P_Q, P_K, P_V, P_O, 1, 64, 2, 32, 1e-6, BF16, 1, P_W,
                                     1 << 30, events, 1, ctypes.byref(nk), None)
    assert st == INVALID and nk.value == 2          # split: reduction + apply
    st = L.sana_linattn_fwd_profiled(P_Q, P_K, P_V, P_O, 1, 64, 2, 32, 1e-6, BF16, 2, P_W,
                                     1 << 30, events, 1, ctypes.byref(nk), None)
    assert st == INVALID and nk.value == 1          # fused: one kernel needs two events
    st = L.sana_linattn_fwd_profiled(P_Q, P_K, P_V, P_O, 1, 64, 2, 32, 1e-6, BF16, 1, P_W,
                                     1 << 30, None, 3, ctypes.byref(nk), None)
    assert st == INVALID


def test_kv_state_and_apply_reject_invalid_arguments(L):
    kv = L.sana_linattn_kv_state
    assert kv(P_K, P_V, None, 1, 64, 2, 32, BF16, P_W, 1 << 30, None) == INVALID
    assert kv(P_K, P_V, P_O, 1, 64, 2, 64, BF16, P_W, 1 << 30, None) == UNSUPPORTED
    assert kv(P_K, P_V, P_O + 4, 1, 64, 2, 32, BF16, P_W, 1 << 30, None) == ALIGNMENT
    assert kv(P_K, P_V, P_O, 1, 64, 2, 32, BF16, P_W, 8, None) == WORKSPACE
    assert kv(P_K, P_V, P_K + 64, 1, 64, 2, 32, BF16, P_W, 1 << 30, None) == INVALID
    ap = L.sana_linattn_apply
    assert ap(P_Q, None, P_O, 1, 64, 2, 32, 1e-6, BF16, None) == INVALID
    assert ap(P_Q, P_K, P_O, 1, 64, 2, 32, -2.0, BF16, None) == INVALID
    assert ap(P_Q, P_K, P_Q, 1, 64, 2, 32, 1e-6, BF16, None) == INVALID
    assert ap(P_Q, P_K, P_O + 2, 1, 64, 2, 32, 1e-6, BF16, None) == ALIGNMENT
    assert ap(P_Q, P_K, P_O, 1, 64, 2, 32, 1e-6, 5, None) == UNSUPPORTED


def test_binding_raises_without_gpu_tensors():
    torch = pytest.importorskip("torch")
    import relu_linear_attention_attn_amd as R

    x = torch.zeros((1, 16, 2, 32), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        R.forward(x, x, x)
    with pytest.raises(TypeError if torch.cuda.is_available() else ValueError):
        R.forward(x.half(), x.half(), x.half())


def bws(L, B, N, H, d=32, dt=BF16):
    n = ctypes.c_size_t(123)
    st = L.sana_linattn_bwd_workspace_size(B, N, H, d, dt, ctypes.byref(n))
    return st, n.value


def test_bwd_workspace_size_rules(L):
    st, n = bws(L, 2, 16384, 70)
    assert st == OK and n % 256 == 0 and n >= 2 * 2 * 70 * 32 * 33 * 4
    assert bws(L, 2, 4096, 36, dt=F32) == (UNSUPPORTED, 0)   # the backward is bf16 only
    assert bws(L, 0, 16, 2) == (INVALID, 0)
    assert bws(L, 1, 16, 2, d=64) == (UNSUPPORTED, 0)
    assert L.sana_linattn_bwd_workspace_size(1, 16, 2, 32, BF16, None) == INVALID
    # constant once N is large, like the forward's
    assert len({bws(L, 2, n, 70)[1] for n in (1 << 16, 1 << 20, 1 << 24)}) == 1


P_G, P_DQ, P_DK, P_DV = (A * i for i in range(6, 10))


def bwd(L, q=P_Q, k=P_K, v=P_V, g=P_G, dq=P_DQ, dk=P_DK, dv=P_DV, B=1, N=64, H=2, d=32,
        eps=1e-6, dt=BF16, ws=P_W, wsb=1 << 30, events=None, n_events=0):
    if events is None:
        return L.sana_linattn_bwd(q, k, v, g, dq, dk, dv, B, N, H, d, eps, dt, ws, wsb, None)
    return L.sana_linattn_bwd_profiled(q, k, v, g, dq, dk, dv, B, N, H, d, eps, dt, ws, wsb,
                                       events, n_events, None)


def test_bwd_rejects_invalid_arguments(L):
    assert bwd(L, B=0) == INVALID
    assert bwd(L, d=16) == UNSUPPORTED
    assert bwd(L, dt=F32) == UNSUPPORTED
    for name in ("q", "k", "v", "g", "dq", "dk", "dv"):
        assert bwd(L, **{name: None}) == INVALID, name
        assert bwd(L, **{name: A * 11 + 8}) == ALIGNMENT, name
    for eps in (-1.0, math.nan, math.inf):
        assert bwd(L, eps=eps) == INVALID
    # outputs overlapping an input, each other, or the workspace (8 KB tensors)
    assert bwd(L, dq=P_Q + 4096) == INVALID
    assert bwd(L, dk=P_G) == INVALID
    assert bwd(L, dv=P_DK + 4096) == INVALID
    need = bws(L, 1, 64, 2)[1]
    assert bwd(L, dq=P_W, wsb=need) == INVALID
    # inputs may alias each other (q used as dout too)
    # (no launch happens here because the workspace below is missing)
    assert bwd(L, g=P_Q, ws=None) == WORKSPACE
    assert bwd(L, wsb=need - 1) == WORKSPACE
    assert bwd(L, ws=P_W + 64, wsb=need) == ALIGNMENT
    # the profiled form needs 4 events
    events = (ctypes.c_void_p * 3)(None, None, None)
    assert bwd(L, events=events, n_events=3) == INVALID
    assert L.sana_linattn_bwd_profiled(P_Q, P_K, P_V, P_G, P_DQ, P_DK, P_DV, 1, 64, 2, 32, 1e-6,
                                       BF16, P_W, 1 << 30, None, 4, None) == INVALID


def bwd_fmap(L, fmap=1, q=P_Q, k=P_K, v=P_V, g=P_G, dq=P_DQ, dk=P_DK, dv=P_DV, B=1, N=64, H=2,
             d=32, eps=1e-6, dt=BF16, ws=P_W, wsb=1 << 30, events=None, n_events=0):
    return L.sana_linattn_bwd_fmap(q, k, v, g, dq, dk, dv, B, N, H, d, eps, dt, fmap, ws, wsb,
                                   events, n_events, None)


def test_bwd_fmap_rejects_invalid_arguments(L):
    """The feature-map backward runs sana_linattn_bwd's checks, plus the map."""
    for fmap in (0, 1, 2):
        assert bwd_fmap(L, fmap, B=0) == INVALID
        assert bwd_fmap(L, fmap, d=16) == UNSUPPORTED
        assert bwd_fmap(L, fmap, dt=F32) == UNSUPPORTED
        assert bwd_fmap(L, fmap, dq=P_Q + 4096) == INVALID
        assert bwd_fmap(L, fmap, ws=None) == WORKSPACE
    for fmap in (-1, 3, 1 << 20):
        assert bwd_fmap(L, fmap) == UNSUPPORTED
    for name in ("q", "k", "v", "g", "dq", "dk", "dv"):
        assert bwd_fmap(L, **{name: None}) == INVALID, name
        assert bwd_fmap(L, **{name: A * 11 + 8}) == ALIGNMENT, name
    for eps in (-1.0, math.nan, math.inf):
        assert bwd_fmap(L, eps=eps) == INVALID
    need = bws(L, 1, 64, 2)[1]
    assert bwd_fmap(L, wsb=need - 1) == WORKSPACE
    events = (ctypes.c_void_p * 3)(None, None, None)
    assert bwd_fmap(L, events=events, n_events=3) == INVALID


def bwd_state(L, state=P_W + (1 << 29), q=P_Q, k=P_K, v=P_V, g=P_G, dq=P_DQ, dk=P_DK, dv=P_DV,
              B=1, N=64, H=2, d=32, eps=1e-6, dt=BF16, fmap=0, ws=P_W, wsb=1 << 20, events=None,
              n_events=0):
    return L.sana_linattn_bwd_state(q, k, v, g, state, dq, dk, dv, B, N, H, d, eps, dt, fmap, ws,
                                    wsb, events, n_events, None)


def test_bwd_state_rejects_invalid_arguments(L):
    """The saved-state backward runs sana_linattn_bwd's checks, plus the
    state's: present, 16-byte aligned, overlapping no output and not the
    workspace (inputs may share memory with it: it is read only)."""
    assert bwd_state(L, B=0) == INVALID
    assert bwd_state(L, d=16) == UNSUPPORTED
    assert bwd_state(L, dt=F32) == UNSUPPORTED
    assert bwd_state(L, state=None) == INVALID
    assert bwd_state(L, state=P_W + (1 << 29) + 8) == ALIGNMENT
    for name in ("q", "k", "v", "g", "dq", "dk", "dv"):
        assert bwd_state(L, **{name: None}) == INVALID, name
    # a state overlapping an output or the workspace (its 8448 B for B = 1, H = 2)
    assert bwd_state(L, state=P_DQ + 64) == INVALID
    assert bwd_state(L, state=P_DV) == INVALID
    assert bwd_state(L, state=P_W + 256) == INVALID
    need = bws(L, 1, 64, 2)[1]
    assert bwd_state(L, wsb=need - 1) == WORKSPACE
    # two kernels: three events
    events = (ctypes.c_void_p * 2)(None, None)
    assert bwd_state(L, events=events, n_events=2) == INVALID
    events3 = (ctypes.c_void_p * 3)(None, None, None)
    assert bwd_state(L, events=events3, n_events=3) == INVALID  # NULL events
    for fmap in (-1, 3):
        assert bwd_state(L, fmap=fmap) == UNSUPPORTED
    for fmap in (1, 2):
        assert bwd_state(L, fmap=fmap, state=None) == INVALID


def test_kv_state_fmap_rejects_invalid_arguments(L):
    kv = L.sana_linattn_kv_state_fmap
    for fmap in (-1, 3):
        assert kv(P_K, P_V, P_O, 1, 64, 2, 32, BF16, fmap, P_W, 1 << 20, None) == UNSUPPORTED
    for fmap in (0, 1, 2):
        assert kv(P_K, P_V, P_O, 0, 64, 2, 32, BF16, fmap, P_W, 1 << 20, None) == INVALID
        assert kv(None, P_V, P_O, 1, 64, 2, 32, BF16, fmap, P_W, 1 << 20, None) == INVALID
        assert kv(P_K, P_V, P_O + 8, 1, 64, 2, 32, BF16, fmap, P_W, 1 << 20, None) == ALIGNMENT
        assert kv(P_K, P_V, P_K, 1, 64, 2, 32, BF16, fmap, P_W, 1 << 20, None) == INVALID
        assert kv(P_K, P_V, P_O, 1, 64, 2, 16, BF16, fmap, P_W, 1 << 20, None) == UNSUPPORTED


def bcws(L, B, N, H, blk, d=32, dt=BF16):
    n = ctypes.c_size_t(123)
    st = L.sana_linattn_block_causal_workspace_size(B, N, H, d, blk, dt, ctypes.byref(n))
    return st, n.value


def test_block_causal_workspace_and_errors(L):
    st, n = bcws(L, 1, 1 << 20, 36, 1 << 16)
    assert st == OK and n % 256 == 0 and n >= 16 * 36 * 32 * 33 * 4   # holds the prefix states
    assert bcws(L, 2, 4096, 36, 1024, dt=F32)[0] == OK                # both dtypes
    assert bcws(L, 1, 1000, 2, 3) == (INVALID, 0)                      # N not a multiple of block
    assert bcws(L, 1, 1000, 2, 0) == (INVALID, 0)
    assert bcws(L, 1, 1000, 2, -8) == (INVALID, 0)
    assert bcws(L, 1, 1000, 2, 1000, d=16) == (UNSUPPORTED, 0)
    # per-block path (fp32, or block lengths other than 1, 2, 4, 8, 16): blocks
    # as batch items, B * (N / L) * ceil(H/2) at most 2^22 head pairs
    assert bcws(L, 1, 1 << 22, 2, 1, dt=F32)[0] == OK
    assert bcws(L, 2, 1 << 22, 2, 1, dt=F32)[0] == INVALID
    # and its prefix scan runs 2304 work-items per (b, head pair): within 2^32
    assert bcws(L, 1 << 20, 16, 2, 16, dt=F32)[0] == OK
    assert bcws(L, 1 << 21, 16, 2, 16, dt=F32)[0] == INVALID
    # bf16 blocks of 1, 2, 4, 8 or 16 tokens run on the token-causal kernels:
    # the token-causal workspace (chunk states), whatever the block count
    for blk in (1, 2, 4, 8, 16):
        assert bcws(L, 2, 16384, 70, blk) == cws(L, 2, 16384, 70)
    assert bcws(L, 2, 1 << 22, 2, 1)[0] == OK
    assert bcws(L, 1, 1000, 2, 16) == (INVALID, 0)                     # 1000 % 16 != 0
    # bf16 blocks of 2..16 whole tiles: chunks of whole blocks (here 64 tiles
    # in chunks of 2 for blocks of 32 tokens), longer blocks one state each
    assert bcws(L, 1, 1024, 2, 32) == (OK, 32 * 2 * 32 * 33 * 4)
    assert bcws(L, 1, 1024, 2, 48) == (INVALID, 0)                     # 1024 % 48 != 0
    assert bcws(L, 1, 4096, 2, 512)[1] != cws(L, 1, 4096, 2)[1]        # per block
    assert L.sana_linattn_block_causal_workspace_size(1, 16, 2, 32, 16, BF16, None) == INVALID
    need = bcws(L, 1, 64, 2, 16)[1]
    f = L.sana_linattn_fwd_block_causal
    assert f(P_Q, P_K, P_V, P_O, 1, 64, 2, 32, 5, 1e-6, BF16, P_W, need, None) == INVALID
    assert f(P_Q, P_K, P_V, None, 1, 64, 2, 32, 16, 1e-6, BF16, P_W, need, None) == INVALID
    assert f(P_Q, P_K, P_V, P_O, 1, 64, 2, 32, 16, -1.0, BF16, P_W, need, None) == INVALID
    assert f(P_Q + 8, P_K, P_V, P_O, 1, 64, 2, 32, 16, 1e-6, BF16, P_W, need, None) == ALIGNMENT
    assert f(P_Q, P_K, P_V, P_Q + 64, 1, 64, 2, 32, 16, 1e-6, BF16, P_W, need, None) == INVALID
    assert f(P_Q, P_K, P_V, P_O, 1, 64, 2, 32, 16, 1e-6, BF16, P_W, need - 1, None) == WORKSPACE
    assert f(P_Q, P_K, P_V, P_O, 1, 64, 2, 32, 16, 1e-6, BF16, P_W + 16, need, None) == ALIGNMENT
    assert f(P_Q, P_K, P_V, P_O, 1, 64, 2, 32, 16, 1e-6, BF16, P_O, need, None) == INVALID
    events = (ctypes.c_void_p * 3)(None, None, None)
    assert L.sana_linattn_fwd_block_causal_profiled(P_Q, P_K, P_V, P_O, 1, 64, 2, 32, 16, 1e-6,
                                                    BF16, P_W, need, events, 3, None) == INVALID


def cws(L, B, N, H, d=32, dt=BF16):
    n = ctypes.c_size_t(123)
    st = L.sana_linattn_causal_workspace_size(B, N, H, d, dt, ctypes.byref(n))
    return st, n.value


def test_causal_workspace_and_errors(L):
    state = 2 * 32 * 33 * 4                                  # one head pair's [2][d][d+1] fp32
    st, n = cws(L, 2, 16384, 70)
    assert st == OK and n % 256 == 0 and n >= 70 * state     # at least one chunk per head pair
    assert n <= 70 * 1024 * state                            # at most 1024 chunks per head pair
    assert cws(L, 1, 1, 2) == (OK, state)                    # one token: one chunk
    assert cws(L, 1, 16, 3)[1] == 2 * state                  # two head pairs, one chunk each
    assert 512 * state <= cws(L, 1, 1 << 20, 2)[1] <= 1024 * state  # long sequence: the cap
    assert cws(L, 1, 1000, 2, dt=F32) == (UNSUPPORTED, 0)    # bf16 only
    assert cws(L, 1, 1000, 2, d=64) == (UNSUPPORTED, 0)
    assert cws(L, 0, 1000, 2) == (INVALID, 0)
    assert cws(L, 1, 0, 2) == (INVALID, 0)
    assert L.sana_linattn_causal_workspace_size(1, 16, 2, 32, BF16, None) == INVALID
    need = cws(L, 1, 64, 2)[1]
    f = L.sana_linattn_fwd_causal

    def call(q=P_Q, k=P_K, v=P_V, o=P_O, eps=1e-6, dt=BF16, ws=P_W, wsb=need, ev=None, nev=0):
        return f(q, k, v, o, 1, 64, 2, 32, eps, dt, ws, wsb, ev, nev, None)
    assert call(o=None) == INVALID
    assert call(eps=-1.0) == INVALID
    assert call(eps=float("nan")) == INVALID
    assert call(dt=F32) == UNSUPPORTED
    assert call(q=P_Q + 8) == ALIGNMENT
    assert call(o=P_Q + 64) == INVALID                       # out overlaps q
    assert call(wsb=need - 1) == WORKSPACE
    assert call(ws=None) == WORKSPACE
    assert call(ws=P_W + 16) == ALIGNMENT
    assert call(ws=P_O) == INVALID                           # workspace overlaps out
    events = (ctypes.c_void_p * 3)(None, None, None)
    assert call(ev=events, nev=3) == INVALID                 # needs 4 events
    events4 = (ctypes.c_void_p * 4)(None, None, None, None)
    assert call(ev=events4, nev=4) == INVALID                # null events


def test_fwd_fmap_rejects_invalid_arguments(L):
    need = ws_size(L, 1, 64, 2)[1]

    def f(fmap=1, B=1, eps=1e-6, q=P_Q, o=P_O, ws=P_W, wsb=None, ev=None, nev=0, dt=BF16):
        return L.sana_linattn_fwd_fmap(q, P_K, P_V, o, B, 64, 2, 32, eps, dt, fmap, ws,
                                       need if wsb is None else wsb, ev, nev, None)

    for fmap in (-1, 3, 99):
        assert f(fmap=fmap) == UNSUPPORTED, fmap
    for fmap in (0, 1, 2):
        assert f(fmap=fmap, B=0) == INVALID
        assert f(fmap=fmap, eps=-1.0) == INVALID
        assert f(fmap=fmap, q=P_Q + 8) == ALIGNMENT
        assert f(fmap=fmap, o=P_Q + 64) == INVALID
        assert f(fmap=fmap, wsb=need - 1) == WORKSPACE
        assert f(fmap=fmap, ws=None) == WORKSPACE
        assert f(fmap=fmap, dt=5) == UNSUPPORTED
    # events: at least 3, none NULL
    two = (ctypes.c_void_p * 2)(1, 2)
    assert f(ev=two, nev=2) == INVALID
    holes = (ctypes.c_void_p * 3)(1, None, 3)
    assert f(ev=holes, nev=3, eps=-1.0) == INVALID
    assert f(ev=holes, nev=3) == INVALID


def qkv_ws(L, B, N, C, H, d=32):
    n = ctypes.c_size_t(12345)
    st = L.sana_linattn_qkv_workspace_size(B, N, C, H, d, ctypes.byref(n))
    return st, n.value


def test_qkv_workspace_and_errors(L):
    st, n = qkv_ws(L, 2, 16384, 2240, 70)
    # one [2][d][d+1] fp32 partial per (b, head pair, 256-token tile)
    assert st == OK and n >= 2 * 35 * 64 * 2 * 32 * 33 * 4 and n % 256 == 0
    assert qkv_ws(L, 1, 1, 8, 1)[0] == OK
    assert qkv_ws(L, 1, 16, 12, 2) == (UNSUPPORTED, 0)     # C % 8 != 0
    assert qkv_ws(L, 1, 16, 16, 2, d=64) == (UNSUPPORTED, 0)
    assert qkv_ws(L, 0, 16, 16, 2) == (INVALID, 0)
    assert qkv_ws(L, 1, 16, 0, 2) == (INVALID, 0)
    assert qkv_ws(L, 1, 16, 1 << 22, 2) == (INVALID, 0)   # 32-bit offsets in a tile
    assert qkv_ws(L, 1, 1 << 40, 1 << 20, 2)[0] == INVALID  # x beyond 2^62 bytes
    assert L.sana_linattn_qkv_workspace_size(1, 16, 16, 2, 32, None) == INVALID
    need = qkv_ws(L, 1, 64, 64, 2)[1]
    P_X, P_WQ = P_Q, P_K   # placeholders: x 1*64*64*2 = 8 KB, w 192*64*2 = 24 KB

    def f(x=P_X, w=P_WQ, q=P_V, o=P_O, C=64, eps=1e-6, ws=P_W, wsb=None, ev=None, nev=0):
        return L.sana_linattn_qkv_fwd(x, w, q, o, 1, 64, C, 2, 32, eps, ws,
                                      need if wsb is None else wsb, ev, nev, None)

    assert f(C=60) == UNSUPPORTED
    for name in ("x", "w", "q", "o"):
        assert f(**{name: None}) == INVALID, name
        assert f(**{name: A * 5 + 8}) == ALIGNMENT, name
    assert f(eps=-1.0) == INVALID
    assert f(o=P_V + 64) == INVALID            # out overlaps q
    assert f(q=P_X + 4096) == INVALID          # q overlaps x
    assert f(wsb=need - 1) == WORKSPACE
    assert f(ws=None) == WORKSPACE
    assert f(ws=P_W + 16) == ALIGNMENT
    assert f(ws=P_O) == INVALID                # workspace overlaps out
    two = (ctypes.c_void_p * 2)(1, 2)
    assert f(ev=two, nev=2) == INVALID
    holes = (ctypes.c_void_p * 3)(1, None, 3)
    assert f(ev=holes, nev=3) == INVALID


def test_fwd_strided_rejects_invalid_arguments(L):
    need = ws_size(L, 1, 64, 2)[1]

    def f(ld=192, fmap=0, eps=1e-6, q=P_Q, k=P_K, o=P_O, dt=BF16, ws=P_W, wsb=None, ev=None,
          nev=0):
        return L.sana_linattn_fwd_strided(q, k, P_V, ld, o, 1, 64, 2, 32, eps, dt, fmap, ws,
                                          need if wsb is None else wsb, ev, nev, None)

    for ld in (0, -1, -192, 63):           # below H d = 64
        assert f(ld=ld) == INVALID, ld
    assert f(ld=1 << 60) == INVALID        # span beyond 2^62 bytes
    assert f(ld=68) == ALIGNMENT           # 136-byte token rows
    assert f(ld=72, eps=-1.0) == INVALID   # 144-byte rows pass; eps fails
    assert f(ld=66, dt=F32) == ALIGNMENT   # 264 bytes
    assert f(ld=68, dt=F32, eps=-1.0) == INVALID
    assert f(fmap=3) == UNSUPPORTED
    assert f(q=P_Q + 8) == ALIGNMENT
    assert f(q=None) == INVALID
    # out inside q's strided span (63 * 192 + 64 elements), past a contiguous tensor
    assert f(o=P_Q + 16384) == INVALID
    assert f(ld=64, o=P_Q + 16384, eps=-1.0) == INVALID
    assert f(o=P_K - 4096) == INVALID      # out's end reaches into k
    assert f(wsb=need - 1) == WORKSPACE
    assert f(ws=P_O) == INVALID
    two = (ctypes.c_void_p * 2)(1, 2)
    assert f(ev=two, nev=2) == INVALID


def test_workspace_may_alias_no_tensor(L):
    """The reduction writes partials while other blocks still read k and v,
    so every entry point with a workspace rejects one that overlaps any of
    its tensors (inputs included) with SANA_ERR_INVALID_ARG."""
    need = ws_size(L, 1, 64, 2)[1]
    for ws in (P_Q, P_K + 256, P_V):
        assert fwd(L, ws=ws, wsb=need) == INVALID, ws
        assert L.sana_linattn_fwd_fmap(P_Q, P_K, P_V, P_O, 1, 64, 2, 32, 1e-6, BF16, 1, ws,
                                       need, None, 0, None) == INVALID, ws
    for ws in (P_K, P_V + 256):
        assert L.sana_linattn_kv_state(P_K, P_V, P_O, 1, 64, 2, 32, BF16, ws, need,
                                       None) == INVALID, ws
    bneed = bws(L, 1, 64, 2)[1]
    for ws in (P_Q, P_K, P_V, P_G):
        assert bwd(L, ws=ws, wsb=bneed) == INVALID, ws
    cneed = bcws(L, 1, 64, 2, 16)[1]
    for ws in (P_Q, P_K, P_V):
        assert L.sana_linattn_fwd_block_causal(P_Q, P_K, P_V, P_O, 1, 64, 2, 32, 16, 1e-6, BF16,
                                               ws, cneed, None) == INVALID, ws
    qneed = qkv_ws(L, 1, 64, 64, 2)[1]
    for ws in (P_Q, P_K + 4096):   # x at P_Q (8 KB), w at P_K (24 KB)
        assert L.sana_linattn_qkv_fwd(P_Q, P_K, P_V, P_O, 1, 64, 64, 2, 32, 1e-6, ws, qneed,
                                      None, 0, None) == INVALID, ws
    # strided inputs: the workspace may not fall inside the span of a strided q
    assert L.sana_linattn_fwd_strided(P_Q, P_K, P_V, 192, P_O, 1, 64, 2, 32, 1e-6, BF16, 0,
                                      P_Q + 8192, need, None, 0, None) == INVALID


def test_library_shares_torchs_hip_runtime():
    """Loading the library through the binding leaves one HIP runtime and one
    HSA runtime in the process (torch's), even when nothing imported torch
    before: two copies cannot share streams or memory, and the library's copy
    fails its first device query."""
    pytest.importorskip("torch")
    code = ("import relu_linear_attention_attn_amd as R; R.lib(); import torch; "
            "m = open('/proc/self/maps').read().splitlines(); "
            "print(sorted({l.split()[-1] for l in m if 'libamdhip64' in l or 'hsa-runtime64' in l}))")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT,
                       timeout=300)
    assert r.returncode == 0, r.stderr
    libs = eval(r.stdout.strip().splitlines()[-1])
    assert sum("libamdhip64" in p for p in libs) == 1, libs
    assert sum("hsa-runtime64" in p for p in libs) == 1, libs


C_PROGRAM = r"""
#include "sana_linattn.h"
#include <stdio.h>
int main(void) {
  size_t n = 0;
  sana_status_t s = sana_linattn_causal_workspace_size(1, 1, 2, 32, SANA_DTYPE_BF16, &n);
  printf("%d %zu\n", (int)s, n);
  s = sana_linattn_workspace_size(1, 16, 2, 64, SANA_DTYPE_BF16, &n);
  printf("%d %s\n", (int)s, sana_linattn_strerror(s));
  s = sana_linattn_fwd(NULL, NULL, NULL, NULL, 1, 16, 2, 32, 1e-6f, SANA_DTYPE_BF16, NULL, 0,
                       NULL);
  printf("%d\n", (int)s);
  return sana_linattn_version() > 0 ? 0 : 1;
}
"""


def test_header_is_c_and_library_links_from_c(tmp_path):
    """The header compiles as C99 and a C program linked against the library
    calls its host-side entry points (no GPU needed for these)."""
    import shutil

    from relu_linear_attention_attn_amd import binding

    gcc = shutil.which("gcc")
    if gcc is None or not os.path.exists(binding.LIB_PATH):
        pytest.skip("needs gcc and the built library")
    src = tmp_path / "abi.c"
    src.write_text(C_PROGRAM)
    exe = tmp_path / "abi"
    libdir = os.path.dirname(binding.LIB_PATH)
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror=implicit-function-declaration",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(src), "-o", str(exe), binding.LIB_PATH,
                    f"-Wl,-rpath,{libdir}"], check=True, capture_output=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    assert out[0] == f"{OK} {2 * 32 * 33 * 4}"             # one chunk state of one head pair
    assert out[1].startswith(f"{UNSUPPORTED} ")            # d = 64
    assert out[2] == f"{INVALID}"                          # null pointers, checked on the host


def test_workspace_sizes_never_misreport(L):
    """Property test over random and extreme shapes (negative, zero, near the
    int64 limits): every size query returns a documented status, leaves 0 on
    error, and on success a 256-byte multiple below 2^62."""
    hyp = pytest.importorskip("hypothesis")
    st = hyp.strategies

    dims = st.one_of(st.integers(-3, 70000), st.sampled_from([0, 1, 2, 15, 16, 17, 32, 33, 64]),
                     st.integers(1 << 20, 1 << 40), st.integers(-(1 << 63), (1 << 63) - 1))
    calls = {
        "fwd": lambda B, N, H, d, dt, x, s: L.sana_linattn_workspace_size(B, N, H, d, dt, s),
        "bwd": lambda B, N, H, d, dt, x, s: L.sana_linattn_bwd_workspace_size(B, N, H, d, dt, s),
        "block_causal": lambda B, N, H, d, dt, x, s: L.sana_linattn_block_causal_workspace_size(
            B, N, H, d, x, dt, s),
        "causal": lambda B, N, H, d, dt, x, s: L.sana_linattn_causal_workspace_size(
            B, N, H, d, dt, s),
        "qkv": lambda B, N, H, d, dt, x, s: L.sana_linattn_qkv_workspace_size(B, N, x, H, d, s),
    }

    @hyp.settings(max_examples=400, deadline=None, derandomize=True)
    @hyp.given(name=st.sampled_from(sorted(calls)), B=dims, N=dims, H=dims,
               d=st.sampled_from([32, 32, 32, 16, 64, 0, -32]), dt=st.sampled_from([0, 1, 2, -1]),
               x=dims)
    def check(name, B, N, H, d, dt, x):
        n = ctypes.c_size_t(12345)
        status = calls[name](B, N, H, d, dt, x, ctypes.byref(n))
        assert status in (OK, INVALID, UNSUPPORTED), (name, status)
        if status != OK:
            assert n.value == 0, (name, status, n.value)
        else:
            assert n.value % 256 == 0 and 0 < n.value < (1 << 62), (name, n.value)

    check()
