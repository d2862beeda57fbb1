"""ctypes binding of libsana_linattn.so (argument marshalling only).

Every step of the computation runs in the HIP kernels behind the C ABI
declared in include/sana_linattn.h. PyTorch supplies device memory and the
current stream. There is no fallback: if the library is not built, every
call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

LIB_NAME = "libsana_linattn.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

DTYPE_F32 = 0
DTYPE_BF16 = 1
VARIANT_AUTO = 0
VARIANT_SPLIT = 1
VARIANT_FUSED = 2
HEAD_DIM = 32

STATUS = {
    0: "SANA_OK",
    1: "SANA_ERR_INVALID_ARG",
    2: "SANA_ERR_UNSUPPORTED",
    3: "SANA_ERR_WORKSPACE",
    4: "SANA_ERR_ALIGNMENT",
    5: "SANA_ERR_HIP",
}
EXPORTS = (
    "sana_linattn_workspace_size",
    "sana_linattn_fwd",
    "sana_linattn_fwd_variant",
    "sana_linattn_fwd_profiled",
    "sana_linattn_kv_state",
    "sana_linattn_kv_state_fmap",
    "sana_linattn_apply",
    "sana_linattn_state_size",
    "sana_linattn_bwd_workspace_size",
    "sana_linattn_bwd",
    "sana_linattn_bwd_profiled",
    "sana_linattn_bwd_fmap",
    "sana_linattn_bwd_state",
    "sana_linattn_block_causal_workspace_size",
    "sana_linattn_fwd_block_causal",
    "sana_linattn_fwd_block_causal_profiled",
    "sana_linattn_causal_workspace_size",
    "sana_linattn_fwd_causal",
    "sana_linattn_fwd_fmap",
    "sana_linattn_fwd_strided",
    "sana_linattn_qkv_workspace_size",
    "sana_linattn_qkv_fwd",
    "sana_linattn_fwd_noalloc",
    "sana_linattn_strerror",
    "sana_linattn_version",
)


class SanaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({strerror(status)})")


_lock = threading.Lock()
_lib: Optional[ctypes.CDLL] = None

_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """Load the HIP library once; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python relu_linear_attention_attn_amd/csrc/build.py` (hipcc, gfx950)")
        # torch first: its HIP runtime is then already in the process when the
        # library asks for libamdhip64.so.7 and the library binds to that one.
        # Loaded the other way round, torch pulls in a second copy of the HIP
        # and HSA runtimes (its libraries name the runtime differently), and the
        # library's runtime neither sees torch's streams and memory nor can
        # use the device reliably (hipGetDevice fails).
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        L.sana_linattn_workspace_size.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int,
                                                  ctypes.POINTER(_sz)]
        L.sana_linattn_state_size.argtypes = [_i64, _i64, _i64, ctypes.POINTER(_sz)]
        L.sana_linattn_fwd.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                       ctypes.c_float, ctypes.c_int, _vp, _sz, _vp]
        L.sana_linattn_fwd_noalloc.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                               ctypes.c_float, ctypes.c_int, _vp]
        L.sana_linattn_fwd_noalloc.restype = ctypes.c_int
        L.sana_linattn_fwd_variant.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                               ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp,
                                               _sz, _vp]
        L.sana_linattn_fwd_profiled.argtypes = [_vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                                ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp,
                                                _sz, ctypes.POINTER(_vp), ctypes.c_int,
                                                ctypes.POINTER(ctypes.c_int), _vp]
        L.sana_linattn_kv_state.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int,
                                            _vp, _sz, _vp]
        L.sana_linattn_apply.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_float,
                                         ctypes.c_int, _vp]
        L.sana_linattn_bwd_workspace_size.argtypes = [_i64, _i64, _i64, _i64, ctypes.c_int,
                                                      ctypes.POINTER(_sz)]
        L.sana_linattn_bwd.argtypes = [_vp] * 7 + [_i64] * 4 + [ctypes.c_float, ctypes.c_int,
                                                                _vp, _sz, _vp]
        L.sana_linattn_bwd_profiled.argtypes = [_vp] * 7 + [_i64] * 4 + [
            ctypes.c_float, ctypes.c_int, _vp, _sz, ctypes.POINTER(_vp), ctypes.c_int, _vp]
        L.sana_linattn_bwd_state.argtypes = [_vp] * 8 + [_i64] * 4 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp, _sz, ctypes.POINTER(_vp),
            ctypes.c_int, _vp]
        L.sana_linattn_kv_state_fmap.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _i64,
                                                 ctypes.c_int, ctypes.c_int, _vp, _sz, _vp]
        L.sana_linattn_bwd_fmap.argtypes = [_vp] * 7 + [_i64] * 4 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp, _sz, ctypes.POINTER(_vp),
            ctypes.c_int, _vp]
        L.sana_linattn_block_causal_workspace_size.argtypes = [_i64] * 5 + [
            ctypes.c_int, ctypes.POINTER(_sz)]
        L.sana_linattn_fwd_block_causal.argtypes = [_vp] * 4 + [_i64] * 5 + [
            ctypes.c_float, ctypes.c_int, _vp, _sz, _vp]
        L.sana_linattn_fwd_block_causal_profiled.argtypes = [_vp] * 4 + [_i64] * 5 + [
            ctypes.c_float, ctypes.c_int, _vp, _sz, ctypes.POINTER(_vp), ctypes.c_int, _vp]
        L.sana_linattn_causal_workspace_size.argtypes = [_i64] * 4 + [ctypes.c_int,
                                                                  ctypes.POINTER(_sz)]
        L.sana_linattn_fwd_causal.argtypes = [_vp] * 4 + [_i64] * 4 + [
            ctypes.c_float, ctypes.c_int, _vp, _sz, ctypes.POINTER(_vp), ctypes.c_int, _vp]
        L.sana_linattn_fwd_fmap.argtypes = [_vp] * 4 + [_i64] * 4 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp, _sz, ctypes.POINTER(_vp),
            ctypes.c_int, _vp]
        L.sana_linattn_fwd_strided.argtypes = [_vp] * 3 + [_i64, _vp] + [_i64] * 4 + [
            ctypes.c_float, ctypes.c_int, ctypes.c_int, _vp, _sz, ctypes.POINTER(_vp),
            ctypes.c_int, _vp]
        L.sana_linattn_qkv_workspace_size.argtypes = [_i64] * 5 + [ctypes.POINTER(_sz)]
        L.sana_linattn_qkv_fwd.argtypes = [_vp] * 4 + [_i64] * 5 + [
            ctypes.c_float, _vp, _sz, ctypes.POINTER(_vp), ctypes.c_int, _vp]
        for name in ("sana_linattn_block_causal_workspace_size", "sana_linattn_fwd_block_causal",
                     "sana_linattn_fwd_block_causal_profiled", "sana_linattn_causal_workspace_size",
                     "sana_linattn_fwd_causal", "sana_linattn_fwd_fmap",
                     "sana_linattn_bwd_fmap", "sana_linattn_bwd_state",
                     "sana_linattn_kv_state_fmap",
                     "sana_linattn_fwd_strided",
                     "sana_linattn_qkv_workspace_size", "sana_linattn_qkv_fwd"):
            getattr(L, name).restype = ctypes.c_int
        for name in ("sana_linattn_workspace_size", "sana_linattn_state_size",
                     "sana_linattn_fwd", "sana_linattn_fwd_variant", "sana_linattn_fwd_profiled",
                     "sana_linattn_kv_state", "sana_linattn_apply",
                     "sana_linattn_bwd_workspace_size", "sana_linattn_bwd",
                     "sana_linattn_bwd_profiled"):
            getattr(L, name).restype = ctypes.c_int
        L.sana_linattn_strerror.argtypes = [ctypes.c_int]
        L.sana_linattn_strerror.restype = ctypes.c_char_p
        L.sana_linattn_version.argtypes = []
        L.sana_linattn_version.restype = ctypes.c_int
        _lib = L
        return L


def strerror(status: int) -> str:
    return lib().sana_linattn_strerror(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise SanaError(status, where)


def workspace_size(B: int, N: int, H: int, d: int = HEAD_DIM, dtype: int = DTYPE_BF16) -> int:
    n = _sz(0)
    _check(lib().sana_linattn_workspace_size(B, N, H, d, dtype, ctypes.byref(n)),
           "sana_linattn_workspace_size")
    return n.value


def state_size(B: int, H: int, d: int = HEAD_DIM) -> int:
    n = _sz(0)
    _check(lib().sana_linattn_state_size(B, H, d, ctypes.byref(n)), "sana_linattn_state_size")
    return n.value


# ------------------------------------------------------------ torch glue


def _torch():
    import torch  # imported lazily: the CPU-only tests never need it here

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected torch.bfloat16 or torch.float32")


def _shape(x, heads: Optional[int]) -> Tuple[int, int, int, int]:
    if x.dim() == 4:
        B, N, H, d = x.shape
        if heads is not None and heads != H:
            raise ValueError("heads does not match the tensor's head axis")
        return B, N, H, d
    if x.dim() == 3:
        if heads is None:
            raise ValueError("a (B, N, D) tensor needs heads=")
        B, N, D = x.shape
        if D % heads:
            raise ValueError("D is not a multiple of heads")
        return B, N, heads, D // heads
    raise ValueError("expected a (B, N, H, d) or (B, N, D) tensor")


def _check_tensor(x, name: str, like=None):
    if not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not x.is_contiguous():
        raise ValueError(f"{name} must be contiguous ([B][N][H][d] row-major)")
    if like is not None and (x.dtype != like.dtype or x.shape != like.shape or
                             x.device != like.device):
        raise ValueError(f"{name} must match q in dtype, shape and device")


def _stream(x) -> int:
    torch = _torch()
    return torch.cuda.current_stream(x.device).cuda_stream


def alloc_workspace(B: int, N: int, H: int, dtype: int, device):
    """A workspace for this shape (torch-owned, 256-byte aligned)."""
    torch = _torch()
    n = workspace_size(B, N, H, HEAD_DIM, dtype)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def forward(q, k, v, eps: float = 1e-6, heads: Optional[int] = None, out=None,
            workspace=None, variant: int = VARIANT_AUTO):
    """out = phi(Q)(phi(K)^T [V|1]) split into numerator and normaliser, per head.

    q, k, v: contiguous GPU tensors (B, N, H, d) or (B, N, D) with heads=, all
    bf16 or all fp32. Enqueued on torch's current stream; no synchronisation."""
    torch = _torch()
    B, N, H, d = _shape(q, heads)
    _check_tensor(q, "q")
    _check_tensor(k, "k", q)
    _check_tensor(v, "v", q)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor(out, "out", q)
    if workspace is None:
        workspace = alloc_workspace(B, N, H, dt, q.device)
    _check(lib().sana_linattn_fwd_variant(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                          out.data_ptr(), B, N, H, d, float(eps), dt,
                                          int(variant), workspace.data_ptr(),
                                          workspace.numel() * workspace.element_size(),
                                          _stream(q)),
           "sana_linattn_fwd_variant")
    return out


SCRATCH_BYTES = 64 << 20   # SANA_LINATTN_SCRATCH_BYTES


def forward_noalloc(q, k, v, out, eps: float = 1e-6, heads: Optional[int] = None):
    """forward() through sana_linattn_fwd_noalloc: the library's static device
    scratch serves as the workspace, so the call allocates nothing (out is the
    caller's). Calls on one GPU share that scratch: order them on one stream."""
    B, N, H, d = _shape(q, heads)
    _check_tensor(q, "q")
    _check_tensor(k, "k", q)
    _check_tensor(v, "v", q)
    _check_tensor(out, "out", q)
    _check(lib().sana_linattn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                          out.data_ptr(), B, N, H, d, float(eps),
                                          _dtype_code(q), _stream(q)),
           "sana_linattn_fwd_noalloc")
    return out


def forward_profiled(q, k, v, events, eps: float = 1e-6, heads: Optional[int] = None,
                     out=None, workspace=None, variant: int = VARIANT_AUTO):
    """forward() that records ``events`` (torch.cuda.Event, enable_timing=True)
    around each kernel it launches: events[0] before the first, events[i]
    after kernel i. Returns (out, number of kernels)."""
    torch = _torch()
    B, N, H, d = _shape(q, heads)
    _check_tensor(q, "q")
    _check_tensor(k, "k", q)
    _check_tensor(v, "v", q)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    if workspace is None:
        workspace = alloc_workspace(B, N, H, dt, q.device)
    for e in events:
        if e.cuda_event == 0:  # torch creates the HIP event on first record
            e.record()
    arr = (_vp * len(events))(*[e.cuda_event for e in events])
    nk = ctypes.c_int(0)
    _check(lib().sana_linattn_fwd_profiled(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                           out.data_ptr(), B, N, H, d, float(eps), dt,
                                           int(variant), workspace.data_ptr(),
                                           workspace.numel() * workspace.element_size(), arr,
                                           len(events), ctypes.byref(nk), _stream(q)),
           "sana_linattn_fwd_profiled")
    return out, nk.value


def kv_state(k, v, heads: Optional[int] = None, state=None, workspace=None, fmap: str = "relu"):
    """The fp32 [B, H, d, d+1] state phi(K)^T [V | 1] of every (b, h), for
    the feature map fmap ("relu", "elu1", "cos")."""
    if fmap not in FMAPS:
        raise ValueError(f"unknown feature map {fmap!r}; one of {sorted(FMAPS)}")
    torch = _torch()
    B, N, H, d = _shape(k, heads)
    _check_tensor(k, "k")
    _check_tensor(v, "v", k)
    dt = _dtype_code(k)
    if state is None:
        state = torch.empty((B, H, d, d + 1), dtype=torch.float32, device=k.device)
    elif state.dtype != torch.float32 or state.numel() != B * H * d * (d + 1) or \
            not state.is_contiguous():
        raise ValueError("state must be a contiguous fp32 tensor of B*H*d*(d+1) elements")
    if workspace is None:
        workspace = alloc_workspace(B, N, H, dt, k.device)
    if fmap == "relu":
        _check(lib().sana_linattn_kv_state(k.data_ptr(), v.data_ptr(), state.data_ptr(), B, N, H,
                                           d, dt, workspace.data_ptr(),
                                           workspace.numel() * workspace.element_size(),
                                           _stream(k)),
               "sana_linattn_kv_state")
    else:
        _check(lib().sana_linattn_kv_state_fmap(k.data_ptr(), v.data_ptr(), state.data_ptr(), B,
                                                N, H, d, dt, FMAPS[fmap], workspace.data_ptr(),
                                                workspace.numel() * workspace.element_size(),
                                                _stream(k)),
               "sana_linattn_kv_state_fmap")
    return state


def apply(q, state, eps: float = 1e-6, heads: Optional[int] = None, out=None):
    """out_i = phi(q_i) KV / (phi(q_i) . ksum + eps) from a [B, H, d, d+1] state."""
    torch = _torch()
    B, N, H, d = _shape(q, heads)
    _check_tensor(q, "q")
    dt = _dtype_code(q)
    if state.dtype != torch.float32 or state.numel() != B * H * d * (d + 1) or \
            not state.is_contiguous() or not state.is_cuda:
        raise ValueError("state must be a contiguous fp32 GPU tensor of B*H*d*(d+1) elements")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor(out, "out", q)
    _check(lib().sana_linattn_apply(q.data_ptr(), state.data_ptr(), out.data_ptr(), B, N, H, d,
                                    float(eps), dt, _stream(q)),
           "sana_linattn_apply")
    return out


def bwd_workspace_size(B: int, N: int, H: int, d: int = HEAD_DIM, dtype: int = DTYPE_BF16) -> int:
    n = _sz(0)
    _check(lib().sana_linattn_bwd_workspace_size(B, N, H, d, dtype, ctypes.byref(n)),
           "sana_linattn_bwd_workspace_size")
    return n.value


def backward(q, k, v, dout, eps: float = 1e-6, heads: Optional[int] = None, grads=None,
             workspace=None, events=None, fmap: str = "relu", state=None):
    """(dq, dk, dv) of the forward pass for the upstream gradient dout (bf16).

    q, k, v, dout: contiguous bf16 GPU tensors of one shape. grads: optional
    preallocated (dq, dk, dv). events: optional list of torch.cuda.Event
    (enable_timing=True) recorded before the first and after each kernel (4
    events; 3 with a state). fmap: the forward's feature map ("relu",
    "elu1", "cos"; anything but "relu" calls sana_linattn_bwd_fmap). state:
    optional saved forward state, the fp32 (B, H, d, d + 1) tensor of
    kv_state(k, v, fmap=fmap) (calls sana_linattn_bwd_state, which skips the
    state reduction). Enqueued on torch's current stream; no
    synchronisation."""
    if fmap not in FMAPS:
        raise ValueError(f"unknown feature map {fmap!r}; one of {sorted(FMAPS)}")
    torch = _torch()
    B, N, H, d = _shape(q, heads)
    _check_tensor(q, "q")
    for name, t in (("k", k), ("v", v), ("dout", dout)):
        _check_tensor(t, name, q)
    dt = _dtype_code(q)
    if grads is None:
        grads = tuple(torch.empty_like(q) for _ in range(3))
    else:
        for name, t in zip(("dq", "dk", "dv"), grads):
            _check_tensor(t, name, q)
    if workspace is None:
        workspace = torch.empty(max(bwd_workspace_size(B, N, H, d, dt), 1), dtype=torch.uint8,
                                device=q.device)
    wb = workspace.numel() * workspace.element_size()
    ptrs = [t.data_ptr() for t in (q, k, v, dout, *grads)]
    if state is not None:
        if (not state.is_cuda or state.dtype != torch.float32 or not state.is_contiguous()
                or state.numel() * 4 != state_size(B, H, d) or state.device != q.device):
            raise ValueError("state must be a contiguous float32 tensor of kv_state's size on "
                             "q's device")
        arr, n = _event_array(events)
        _check(lib().sana_linattn_bwd_state(*ptrs[:4], state.data_ptr(), *ptrs[4:], B, N, H, d,
                                            float(eps), dt, FMAPS[fmap], workspace.data_ptr(), wb,
                                            arr, n, _stream(q)), "sana_linattn_bwd_state")
    elif fmap != "relu":
        arr, n = _event_array(events)
        _check(lib().sana_linattn_bwd_fmap(*ptrs, B, N, H, d, float(eps), dt, FMAPS[fmap],
                                           workspace.data_ptr(), wb, arr, n, _stream(q)),
               "sana_linattn_bwd_fmap")
    elif events is None:
        _check(lib().sana_linattn_bwd(*ptrs, B, N, H, d, float(eps), dt, workspace.data_ptr(),
                                      wb, _stream(q)), "sana_linattn_bwd")
    else:
        for e in events:
            if e.cuda_event == 0:  # torch creates the HIP event on first record
                e.record()
        arr = (_vp * len(events))(*[e.cuda_event for e in events])
        _check(lib().sana_linattn_bwd_profiled(*ptrs, B, N, H, d, float(eps), dt,
                                               workspace.data_ptr(), wb, arr, len(events),
                                               _stream(q)), "sana_linattn_bwd_profiled")
    return grads


def block_causal_workspace_size(B: int, N: int, H: int, block: int, d: int = HEAD_DIM,
                                dtype: int = DTYPE_BF16) -> int:
    n = _sz(0)
    _check(lib().sana_linattn_block_causal_workspace_size(B, N, H, d, block, dtype,
                                                          ctypes.byref(n)),
           "sana_linattn_block_causal_workspace_size")
    return n.value


def forward_block_causal(q, k, v, block: int, eps: float = 1e-6, heads: Optional[int] = None,
                         out=None, workspace=None, events=None):
    """Block-causal forward: a query in block c (of `block` tokens) sees keys
    in blocks 0..c. Same tensors as forward(); events: optional list of 4
    torch.cuda.Event recorded around the three kernels."""
    torch = _torch()
    B, N, H, d = _shape(q, heads)
    _check_tensor(q, "q")
    _check_tensor(k, "k", q)
    _check_tensor(v, "v", q)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor(out, "out", q)
    if workspace is None:
        workspace = torch.empty(max(block_causal_workspace_size(B, N, H, block, d, dt), 1),
                                dtype=torch.uint8, device=q.device)
    wb = workspace.numel() * workspace.element_size()
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, N, H, d, int(block),
            float(eps), dt, workspace.data_ptr(), wb)
    if events is None:
        _check(lib().sana_linattn_fwd_block_causal(*args, _stream(q)),
               "sana_linattn_fwd_block_causal")
    else:
        for e in events:
            if e.cuda_event == 0:  # torch creates the HIP event on first record
                e.record()
        arr = (_vp * len(events))(*[e.cuda_event for e in events])
        _check(lib().sana_linattn_fwd_block_causal_profiled(*args, arr, len(events), _stream(q)),
               "sana_linattn_fwd_block_causal_profiled")
    return out


def causal_workspace_size(B: int, N: int, H: int, d: int = HEAD_DIM,
                          dtype: int = DTYPE_BF16) -> int:
    n = _sz(0)
    _check(lib().sana_linattn_causal_workspace_size(B, N, H, d, dtype, ctypes.byref(n)),
           "sana_linattn_causal_workspace_size")
    return n.value


def forward_causal(q, k, v, eps: float = 1e-6, heads: Optional[int] = None, out=None,
                   workspace=None, events=None):
    """Token-causal forward (bf16): query i sees keys 0..i of its batch item.
    Same tensors as forward(); events: optional list of 4 torch.cuda.Event
    recorded around the three kernels."""
    torch = _torch()
    B, N, H, d = _shape(q, heads)
    _check_tensor(q, "q")
    _check_tensor(k, "k", q)
    _check_tensor(v, "v", q)
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor(out, "out", q)
    if workspace is None:
        workspace = torch.empty(max(causal_workspace_size(B, N, H, d, dt), 1),
                                dtype=torch.uint8, device=q.device)
    wb = workspace.numel() * workspace.element_size()
    arr, n_ev = None, 0
    if events is not None:
        for e in events:
            if e.cuda_event == 0:  # torch creates the HIP event on first record
                e.record()
        arr = (_vp * len(events))(*[e.cuda_event for e in events])
        n_ev = len(events)
    _check(lib().sana_linattn_fwd_causal(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                         B, N, H, d, float(eps), dt, workspace.data_ptr(), wb,
                                         arr, n_ev, _stream(q)),
           "sana_linattn_fwd_causal")
    return out


FMAPS = {"relu": 0, "elu1": 1, "cos": 2}


def forward_fmap(q, k, v, fmap: str = "relu", eps: float = 1e-6, heads: Optional[int] = None,
                 out=None, workspace=None, events=None):
    """Forward pass with feature map fmap ("relu", "elu1" = ELU + 1, "cos")
    in place of ReLU (split kernels). Same tensors as forward(); events:
    optional list of 3 torch.cuda.Event recorded around the two kernels."""
    torch = _torch()
    B, N, H, d = _shape(q, heads)
    _check_tensor(q, "q")
    _check_tensor(k, "k", q)
    _check_tensor(v, "v", q)
    dt = _dtype_code(q)
    if fmap not in FMAPS:
        raise ValueError(f"unknown feature map {fmap!r}; one of {sorted(FMAPS)}")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor(out, "out", q)
    if workspace is None:
        workspace = alloc_workspace(B, N, H, dt, q.device)
    arr, n = None, 0
    if events is not None:
        for e in events:
            if e.cuda_event == 0:  # torch creates the HIP event on first record
                e.record()
        arr, n = (_vp * len(events))(*[e.cuda_event for e in events]), len(events)
    _check(lib().sana_linattn_fwd_fmap(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                       B, N, H, d, float(eps), dt, FMAPS[fmap],
                                       workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size(), arr, n,
                                       _stream(q)),
           "sana_linattn_fwd_fmap")
    return out


def _event_array(events):
    if events is None:
        return None, 0
    for e in events:
        if e.cuda_event == 0:  # torch creates the HIP event on first record
            e.record()
    return (_vp * len(events))(*[e.cuda_event for e in events]), len(events)


def _token_stride(x, name: str, H: int, d: int) -> int:
    """ld of a (B, N, H, d) or (B, N, H d) view with packed heads and channels
    whose tokens are ld elements apart and batch items N ld apart."""
    if not x.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    B, N = int(x.shape[0]), int(x.shape[1])
    sb, sn = x.stride()[:2]
    packed = x.stride()[-1] == 1 and (x.dim() == 3 or H == 1 or x.stride()[2] == d)
    ld = sn if N > 1 else (sb if B > 1 else H * d)
    if not packed or (B > 1 and sb != N * ld):
        raise ValueError(f"{name} must be a (B, N, H, d) view with packed heads and channels and "
                         "batch stride N * (token stride)")
    return int(ld)


def forward_strided(q, k, v, fmap: str = "relu", eps: float = 1e-6, heads: Optional[int] = None,
                    out=None, workspace=None, events=None):
    """Forward pass on q, k, v views whose tokens are ld elements apart (one
    ld for all three), e.g. q, k, v = qkv.view(B, N, 3, H, d).unbind(2) for
    the output qkv of one fused linear layer: read in place, no copies.
    Returns a new contiguous (B, N, H, d) out (or fills ``out``)."""
    torch = _torch()
    B, N, H, d = _shape(q, heads)
    lds = {_token_stride(x, name, H, d) for x, name in ((q, "q"), (k, "k"), (v, "v"))}
    if len(lds) != 1:
        raise ValueError("q, k and v must share one token stride")
    for x, name in ((k, "k"), (v, "v")):
        if x.dtype != q.dtype or x.shape != q.shape or x.device != q.device:
            raise ValueError(f"{name} must match q in dtype, shape and device")
    dt = _dtype_code(q)
    if fmap not in FMAPS:
        raise ValueError(f"unknown feature map {fmap!r}; one of {sorted(FMAPS)}")
    if out is None:
        out = torch.empty((B, N, H, d), dtype=q.dtype, device=q.device)
    else:
        _check_tensor(out, "out")
        if out.dtype != q.dtype or out.numel() != B * N * H * d or out.device != q.device:
            raise ValueError("out must hold B * N * H * d elements of q's dtype on q's device")
    if workspace is None:
        workspace = alloc_workspace(B, N, H, dt, q.device)
    arr, n = _event_array(events)
    _check(lib().sana_linattn_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), lds.pop(),
                                          out.data_ptr(), B, N, H, d, float(eps), dt,
                                          FMAPS[fmap], workspace.data_ptr(),
                                          workspace.numel() * workspace.element_size(), arr, n,
                                          _stream(q)),
           "sana_linattn_fwd_strided")
    return out


def qkv_workspace_size(B: int, N: int, C: int, H: int, d: int = HEAD_DIM) -> int:
    n = _sz(0)
    _check(lib().sana_linattn_qkv_workspace_size(B, N, C, H, d, ctypes.byref(n)),
           "sana_linattn_qkv_workspace_size")
    return n.value


def forward_qkv(x, w_qkv, heads: int, eps: float = 1e-6, q=None, out=None, workspace=None,
                events=None):
    """QKV projection x W^T (bf16) with the attention state formed in the
    projection's epilogue, then the forward pass. x: contiguous bf16 GPU
    tensor (B, N, C); w_qkv: (3 D, C), D = heads * 32. Returns (q, out), both
    (B, N, heads, 32). events: optional list of 3 torch.cuda.Event recorded
    around the projection and the apply."""
    torch = _torch()
    if x.dim() != 3:
        raise ValueError("x must be (B, N, C)")
    B, N, C = (int(s) for s in x.shape)
    H, d = int(heads), HEAD_DIM
    _check_tensor(x, "x")
    _check_tensor(w_qkv, "w_qkv")
    if x.dtype != torch.bfloat16 or w_qkv.dtype != torch.bfloat16 or w_qkv.device != x.device:
        raise ValueError("x and w_qkv must be bf16 tensors on one device")
    if tuple(w_qkv.shape) != (3 * H * d, C):
        raise ValueError(f"w_qkv must be ({3 * H * d}, {C})")
    if q is None:
        q = torch.empty((B, N, H, d), dtype=x.dtype, device=x.device)
    if out is None:
        out = torch.empty((B, N, H, d), dtype=x.dtype, device=x.device)
    if workspace is None:
        workspace = torch.empty(max(qkv_workspace_size(B, N, C, H, d), 1), dtype=torch.uint8,
                                device=x.device)
    arr, n = None, 0
    if events is not None:
        for e in events:
            if e.cuda_event == 0:  # torch creates the HIP event on first record
                e.record()
        arr, n = (_vp * len(events))(*[e.cuda_event for e in events]), len(events)
    _check(lib().sana_linattn_qkv_fwd(x.data_ptr(), w_qkv.data_ptr(), q.data_ptr(),
                                      out.data_ptr(), B, N, C, H, d, float(eps),
                                      workspace.data_ptr(),
                                      workspace.numel() * workspace.element_size(), arr, n,
                                      _stream(x)),
           "sana_linattn_qkv_fwd")
    return q, out
