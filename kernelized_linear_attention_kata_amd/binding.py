"""ctypes binding of libkata (include/kata.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libkata.so.  torch supplies device memory (tensors) and the stream
(the current torch stream unless one is passed).  The library is loaded on
first use; a missing library raises KataError, there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))

KATA_OK, KATA_ERR_NULL, KATA_ERR_SHAPE, KATA_ERR_UNSUPPORTED, KATA_ERR_WORKSPACE, KATA_ERR_LAUNCH, \
    KATA_ERR_SCRATCH = range(7)
NOALLOC_SCRATCH_BYTES = 64 << 20     # KATA_NOALLOC_SCRATCH_BYTES
KATA_F32, KATA_BF16, KATA_BF16_HILO = 0, 1, 2
KATA_SCAN_ASSOC, KATA_SCAN_SEQUENTIAL = 0, 1
FEATURE_LAYOUTS = {"full": 0, "packed_key": 1, "packed_query": 2}
ABI_VERSION = 1
P_DIM = 16
N_PACKED = 9 * P_DIM
PACKED_ROWS = 136      # rows of the packed symmetric state (the first 136 packed feature slots)


class KataError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = f"{what}: " if what else ""
        try:
            s = _lib().kata_status_string(status).decode()
        except Exception:  # library unavailable while formatting
            s = f"status {status}"
        super().__init__(msg + s)


class ForwardDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("T", ctypes.c_int64),
        ("d", ctypes.c_int),
        ("dv", ctypes.c_int),
        ("p", ctypes.c_int),
        ("chunk", ctypes.c_int),
        ("in_dtype", ctypes.c_int),
        ("out_dtype", ctypes.c_int),
        ("scan", ctypes.c_int),
        ("scan_leaf", ctypes.c_int),
    ]


_LIB: Optional[ctypes.CDLL] = None


def library_path() -> str:
    return os.environ.get("KATA_LIBRARY", os.path.join(_PKG_DIR, "libkata.so"))


def load_library() -> ctypes.CDLL:
    """Load libkata.so and declare the C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise KataError(KATA_ERR_LAUNCH, f"libkata.so not found at {path}; build it with "
                                         "`python -m kernelized_linear_attention_kata_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, ci, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.kata_abi_version.restype = ci
    lib.kata_abi_version.argtypes = []
    lib.kata_status_string.restype = ctypes.c_char_p
    lib.kata_status_string.argtypes = [ci]
    lib.kata_forward_workspace_bytes.restype = ci
    lib.kata_forward_workspace_bytes.argtypes = [ctypes.POINTER(ForwardDesc), ctypes.POINTER(sz)]
    lib.kata_forward_delta_chunked_plan.restype = ci
    lib.kata_forward_delta_chunked_plan.argtypes = [ctypes.POINTER(ForwardDesc), ctypes.POINTER(ctypes.c_int64),
                                                    ctypes.POINTER(ctypes.c_int64)]
    lib.kata_forward_plan.restype = ci
    lib.kata_forward_plan.argtypes = [ctypes.POINTER(ForwardDesc), ctypes.POINTER(ctypes.c_int64),
                                      ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ci)]
    lib.kata_forward.restype = ci
    lib.kata_forward.argtypes = [ctypes.POINTER(ForwardDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.kata_forward_timed.restype = ci
    lib.kata_forward_timed.argtypes = [ctypes.POINTER(ForwardDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                       ctypes.POINTER(vp)]
    lib.kata_forward_noalloc.restype = ci
    lib.kata_forward_noalloc.argtypes = [ctypes.POINTER(ForwardDesc)] + [vp] * 10
    lib.kata_flash_workspace_bytes.restype = ci
    lib.kata_flash_workspace_bytes.argtypes = [ctypes.POINTER(ForwardDesc), ctypes.POINTER(sz)]
    lib.kata_flash_forward.restype = ci
    lib.kata_flash_forward.argtypes = [ctypes.POINTER(ForwardDesc), vp, vp, vp, vp, vp, vp, sz, vp,
                                       ctypes.POINTER(vp)]
    lib.kata_backward_workspace_bytes.restype = ci
    lib.kata_backward_workspace_bytes.argtypes = [ctypes.POINTER(ForwardDesc), ctypes.POINTER(sz)]
    lib.kata_backward_timed.restype = ci
    lib.kata_backward_timed.argtypes = [ctypes.POINTER(ForwardDesc)] + [vp] * 16 + [sz, vp, ctypes.POINTER(vp)]
    lib.kata_backward.restype = ci
    lib.kata_backward.argtypes = [ctypes.POINTER(ForwardDesc)] + [vp] * 16 + [sz, vp]
    lib.kata_forward_decay_workspace_bytes.restype = ci
    lib.kata_forward_decay_workspace_bytes.argtypes = [ctypes.POINTER(ForwardDesc), ctypes.POINTER(sz)]
    lib.kata_forward_decay_timed.restype = ci
    lib.kata_forward_decay_timed.argtypes = [ctypes.POINTER(ForwardDesc)] + [vp] * 11 + [sz, vp, ctypes.POINTER(vp)]
    lib.kata_forward_decay.restype = ci
    lib.kata_forward_decay.argtypes = [ctypes.POINTER(ForwardDesc)] + [vp] * 11 + [sz, vp]
    lib.kata_decode_step_packed.restype = ci
    lib.kata_decode_step_packed.argtypes = [i64, i64, ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kata_decode_step_delta_packed.restype = ci
    lib.kata_decode_step_delta_packed.argtypes = [i64, i64, ci, ci, ci, ci, ci] + [vp] * 8
    lib.kata_decode_step_decay_packed.restype = ci
    lib.kata_decode_step_decay_packed.argtypes = [i64, i64, ci, ci, ci, ci, ci] + [vp] * 9
    lib.kata_decode_step_factors_packed.restype = ci
    lib.kata_decode_step_factors_packed.argtypes = [i64, i64, ci, ci, ci, ci, ci, ci, ci] + [vp] * 8
    lib.kata_state_pack.restype = ci
    lib.kata_state_pack.argtypes = [i64, ci, vp, vp, vp, vp, vp]
    lib.kata_state_unpack.restype = ci
    lib.kata_state_unpack.argtypes = [i64, ci, vp, vp, vp, vp, vp]
    lib.kata_decode_step_decay.restype = ci
    lib.kata_decode_step_decay.argtypes = [i64, i64, ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kata_forward_factors_workspace_bytes.restype = ci
    lib.kata_forward_factors_workspace_bytes.argtypes = [ctypes.POINTER(ForwardDesc), ci, ci, ctypes.POINTER(sz)]
    lib.kata_forward_factors_timed.restype = ci
    lib.kata_forward_factors_timed.argtypes = [ctypes.POINTER(ForwardDesc), ci, ci] + [vp] * 10 + [sz, vp, vp]
    lib.kata_forward_factors.restype = ci
    lib.kata_forward_factors.argtypes = [ctypes.POINTER(ForwardDesc), ci, ci] + [vp] * 10 + [sz, vp]
    lib.kata_forward_delta_chunked_workspace_bytes.restype = ci
    lib.kata_forward_delta_chunked_workspace_bytes.argtypes = [ctypes.POINTER(ForwardDesc), ctypes.POINTER(sz)]
    lib.kata_forward_delta_chunked_timed.restype = ci
    lib.kata_forward_delta_chunked_timed.argtypes = [ctypes.POINTER(ForwardDesc)] + [vp] * 9 + [sz, vp, vp]
    lib.kata_forward_delta_chunked.restype = ci
    lib.kata_forward_delta_chunked.argtypes = [ctypes.POINTER(ForwardDesc)] + [vp] * 9 + [sz, vp]
    lib.kata_decode_step_factors.restype = ci
    lib.kata_decode_step_factors.argtypes = [i64, i64, ci, ci, ci, ci, ci, ci, ci] + [vp] * 8
    lib.kata_forward_delta.restype = ci
    lib.kata_forward_delta.argtypes = [ctypes.POINTER(ForwardDesc)] + [vp] * 9
    lib.kata_decode_step_delta.restype = ci
    lib.kata_decode_step_delta.argtypes = [i64, i64, ci, ci, ci, ci, ci] + [vp] * 8
    lib.kata_decode_step.restype = ci
    lib.kata_decode_step.argtypes = [i64, i64, ci, ci, ci, ci, ci, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.kata_feature_map.restype = ci
    lib.kata_feature_map.argtypes = [vp, vp, i64, i64, ci, ci, ci, ci, vp, vp]
    if lib.kata_abi_version() != ABI_VERSION:
        raise KataError(KATA_ERR_UNSUPPORTED, f"libkata ABI {lib.kata_abi_version()} != {ABI_VERSION}")
    _LIB = lib
    return lib


def _lib() -> ctypes.CDLL:
    return load_library()


def abi_version() -> int:
    return _lib().kata_abi_version()


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return KATA_F32
    if t == torch.bfloat16:
        return KATA_BF16
    raise KataError(KATA_ERR_UNSUPPORTED, f"dtype {t}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream, device) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _check(status: int, what: str):
    if status != KATA_OK:
        raise KataError(status, what)


def _need(t: torch.Tensor, name: str, shape, dtype=None, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def make_desc(B, H, T, d, dv, chunk, in_dtype, out_dtype, scan="assoc", scan_leaf=0, p=P_DIM) -> ForwardDesc:
    return ForwardDesc(B=B, H=H, T=T, d=d, dv=dv, p=p, chunk=chunk, in_dtype=in_dtype, out_dtype=out_dtype,
                       scan={"assoc": KATA_SCAN_ASSOC, "sequential": KATA_SCAN_SEQUENTIAL}[scan],
                       scan_leaf=scan_leaf)


def _in_code(dtype: torch.dtype, precise: bool) -> int:
    """in_dtype code of q, k, v; precise (bf16 only) selects KATA_BF16_HILO."""
    code = _dtype_code(dtype)
    if precise:
        if code != KATA_BF16:
            raise KataError(KATA_ERR_UNSUPPORTED, "precise=True applies to bfloat16 inputs")
        return KATA_BF16_HILO
    return code


def forward_workspace_bytes(B, H, T, d, dv, chunk, in_dtype=torch.bfloat16, out_dtype=None,
                            scan="assoc", scan_leaf=0, precise=False) -> int:
    out_dtype = in_dtype if out_dtype is None else out_dtype
    desc = make_desc(B, H, T, d, dv, chunk, _in_code(in_dtype, precise), _dtype_code(out_dtype), scan, scan_leaf)
    n = ctypes.c_size_t(0)
    _check(_lib().kata_forward_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)), "kata_forward_workspace_bytes")
    return int(n.value)



def forward_plan(B, H, T, d, dv, chunk, in_dtype=torch.bfloat16, out_dtype=None, scan="assoc", scan_leaf=0,
                 precise=False) -> dict:
    """The leaf plan of forward(): {"n_leaf", "leaf_chunks", "scanned"} (kata_forward_plan)."""
    out_dtype = in_dtype if out_dtype is None else out_dtype
    desc = make_desc(B, H, T, d, dv, chunk, _in_code(in_dtype, precise), _dtype_code(out_dtype), scan, scan_leaf)
    n, leaf, sc = ctypes.c_int64(0), ctypes.c_int64(0), ctypes.c_int(0)
    _check(_lib().kata_forward_plan(ctypes.byref(desc), ctypes.byref(n), ctypes.byref(leaf), ctypes.byref(sc)),
           "kata_forward_plan")
    return {"n_leaf": int(n.value), "leaf_chunks": int(leaf.value), "scanned": bool(sc.value)}


def _event_array(events, n: int, stream, dev):
    """The C array of hipEvent_t handles for a *_timed entry point, or None.

    events: None, or n torch.cuda.Event(enable_timing=True) objects, any of which may be
    None (that stamp is skipped).  torch creates the HIP event lazily on its first
    record, so an event without one is recorded once first on the launch stream."""
    if events is None:
        return None
    if len(events) != n:
        raise ValueError(f"events: {n} torch.cuda.Event objects (or None)")
    s_obj = stream if stream is not None else torch.cuda.current_stream(dev)
    for e in events:
        if e is not None and e.cuda_event == 0:
            e.record(s_obj)
    return (ctypes.c_void_p * n)(*[ctypes.c_void_p(None if e is None else e.cuda_event) for e in events])

def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: torch.Tensor, chunk: int = 64, *,
            S0: Optional[torch.Tensor] = None, z0: Optional[torch.Tensor] = None,
            out_dtype: Optional[torch.dtype] = None, return_state: bool = False, scan: str = "assoc",
            scan_leaf: int = 0, y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
            ST: Optional[torch.Tensor] = None, zT: Optional[torch.Tensor] = None, stream=None,
            events=None, precise: bool = False):
    """KATA causal forward (kata_forward).  q, k: [B,H,T,d]; v: [B,H,T,dv]; P: [H,16,d] fp32.

    precise (bf16 q, k, v): the KATA_BF16_HILO compute type, hi/lo feature and state
    operands for ill-conditioned output gates (about 1.45x the time).

    Returns y [B,H,T,dv] (out_dtype, default q's dtype), or (y, ST, zT) with the final
    state when return_state.  Outputs and the workspace may be passed in preallocated.
    events: optional four torch.cuda.Event(enable_timing=True), stamped by the launches with
    the start of the chunk-state, scan and intra kernels and the end of the last
    (kata_forward_timed).  An event torch has not created yet is recorded once first.
    """
    B, H, T, d = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(q, "q", (B, H, T, d), device=dev)
    _need(k, "k", (B, H, T, d), q.dtype, dev)
    _need(v, "v", (B, H, T, dv), q.dtype, dev)
    _need(P, "P", (H, P_DIM, d), torch.float32, dev)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    ic, oc = _in_code(q.dtype, precise), _dtype_code(out_dtype)
    if (S0 is None) != (z0 is None):
        raise ValueError("S0 and z0 go together")
    if S0 is not None:
        _need(S0, "S0", (B, H, P_DIM * P_DIM, dv), torch.float32, dev)
        _need(z0, "z0", (B, H, P_DIM * P_DIM), torch.float32, dev)
    desc = make_desc(B, H, T, d, dv, chunk, ic, oc, scan, scan_leaf)
    n = ctypes.c_size_t(0)
    lib = _lib()
    _check(lib.kata_forward_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)), "kata_forward_workspace_bytes")
    if y is None:
        y = torch.empty((B, H, T, dv), dtype=out_dtype, device=dev)
    else:
        _need(y, "y", (B, H, T, dv), out_dtype, dev)
    if workspace is None:
        workspace = torch.empty((max(int(n.value), 1),), dtype=torch.uint8, device=dev)
    elif not workspace.is_cuda or workspace.numel() * workspace.element_size() < n.value:
        raise ValueError("workspace too small")
    if return_state:
        if ST is None:
            ST = torch.empty((B, H, P_DIM * P_DIM, dv), dtype=torch.float32, device=dev)
        if zT is None:
            zT = torch.empty((B, H, P_DIM * P_DIM), dtype=torch.float32, device=dev)
        _need(ST, "ST", (B, H, P_DIM * P_DIM, dv), torch.float32, dev)
        _need(zT, "zT", (B, H, P_DIM * P_DIM), torch.float32, dev)
    else:
        ST = zT = None
    sh = _stream_handle(stream, dev)
    evarr = _event_array(events, 4, stream, dev)
    st = lib.kata_forward_timed(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(P), _ptr(S0), _ptr(z0),
                                _ptr(y), _ptr(ST), _ptr(zT), _ptr(workspace),
                                ctypes.c_size_t(workspace.numel() * workspace.element_size()), sh, evarr)
    _check(st, "kata_forward")
    return (y, ST, zT) if return_state else y


def forward_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: torch.Tensor, chunk: int = 64, *,
                    S0: Optional[torch.Tensor] = None, z0: Optional[torch.Tensor] = None,
                    out_dtype: Optional[torch.dtype] = None, return_state: bool = False, scan: str = "assoc",
                    scan_leaf: int = 0, y: Optional[torch.Tensor] = None, ST: Optional[torch.Tensor] = None,
                    zT: Optional[torch.Tensor] = None, stream=None, precise: bool = False):
    """kata_forward_noalloc: the forward of ``forward`` with the library's fixed scratch
    buffer as workspace (no device memory passed in or allocated by the call).  With y (and
    ST, zT when return_state) passed in, this function allocates nothing either."""
    B, H, T, d = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(q, "q", (B, H, T, d), device=dev)
    _need(k, "k", (B, H, T, d), q.dtype, dev)
    _need(v, "v", (B, H, T, dv), q.dtype, dev)
    _need(P, "P", (H, P_DIM, d), torch.float32, dev)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if (S0 is None) != (z0 is None):
        raise ValueError("S0 and z0 go together")
    if S0 is not None:
        _need(S0, "S0", (B, H, P_DIM * P_DIM, dv), torch.float32, dev)
        _need(z0, "z0", (B, H, P_DIM * P_DIM), torch.float32, dev)
    desc = make_desc(B, H, T, d, dv, chunk, _in_code(q.dtype, precise), _dtype_code(out_dtype), scan, scan_leaf)
    if y is None:
        y = torch.empty((B, H, T, dv), dtype=out_dtype, device=dev)
    else:
        _need(y, "y", (B, H, T, dv), out_dtype, dev)
    if return_state:
        if ST is None:
            ST = torch.empty((B, H, P_DIM * P_DIM, dv), dtype=torch.float32, device=dev)
        if zT is None:
            zT = torch.empty((B, H, P_DIM * P_DIM), dtype=torch.float32, device=dev)
        _need(ST, "ST", (B, H, P_DIM * P_DIM, dv), torch.float32, dev)
        _need(zT, "zT", (B, H, P_DIM * P_DIM), torch.float32, dev)
    else:
        ST = zT = None
    st = _lib().kata_forward_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(P), _ptr(S0), _ptr(z0),
                                     _ptr(y), _ptr(ST), _ptr(zT), _stream_handle(stream, dev))
    _check(st, "kata_forward_noalloc")
    return (y, ST, zT) if return_state else y


def forward_decay_workspace_bytes(B, H, T, d=64, dv=64, chunk=64, in_dtype=torch.bfloat16, out_dtype=None,
                                  scan="assoc", scan_leaf=0) -> int:
    """Workspace bytes of kata_forward_decay for these sizes."""
    out_dtype = in_dtype if out_dtype is None else out_dtype
    desc = make_desc(B, H, T, d, dv, chunk, _dtype_code(in_dtype), _dtype_code(out_dtype), scan, scan_leaf)
    n = ctypes.c_size_t(0)
    _check(_lib().kata_forward_decay_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)),
           "kata_forward_decay_workspace_bytes")
    return int(n.value)


def forward_decay(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: torch.Tensor, lam: torch.Tensor,
                  chunk: int = 64, *, S0: Optional[torch.Tensor] = None, z0: Optional[torch.Tensor] = None,
                  out_dtype: Optional[torch.dtype] = None, return_state: bool = False, scan: str = "assoc",
                  scan_leaf: int = 0, y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                  stream=None, events=None):
    """Decay-gated causal forward (kata_forward_decay): S_t = exp(lam_t) S_{t-1} + phi(k_t) v_t^T
    and z_t likewise.  q, k, v: [B,H,T,64] bf16; P: [H,16,64] fp32; lam: [B,H,T] fp32 (<= 0).
    Returns y, or (y, ST, zT) when return_state.  events: optional four torch.cuda.Event."""
    B, H, T, d = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(q, "q", (B, H, T, d), device=dev)
    _need(k, "k", (B, H, T, d), q.dtype, dev)
    _need(v, "v", (B, H, T, dv), q.dtype, dev)
    _need(P, "P", (H, P_DIM, d), torch.float32, dev)
    _need(lam, "lam", (B, H, T), torch.float32, dev)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if (S0 is None) != (z0 is None):
        raise ValueError("S0 and z0 go together")
    if S0 is not None:
        _need(S0, "S0", (B, H, P_DIM * P_DIM, dv), torch.float32, dev)
        _need(z0, "z0", (B, H, P_DIM * P_DIM), torch.float32, dev)
    desc = make_desc(B, H, T, d, dv, chunk, _dtype_code(q.dtype), _dtype_code(out_dtype), scan, scan_leaf)
    lib = _lib()
    n = ctypes.c_size_t(0)
    _check(lib.kata_forward_decay_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)),
           "kata_forward_decay_workspace_bytes")
    if y is None:
        y = torch.empty((B, H, T, dv), dtype=out_dtype, device=dev)
    else:
        _need(y, "y", (B, H, T, dv), out_dtype, dev)
    if workspace is None:
        workspace = torch.empty((max(int(n.value), 1),), dtype=torch.uint8, device=dev)
    elif not workspace.is_cuda or workspace.numel() * workspace.element_size() < n.value:
        raise ValueError("workspace too small")
    ST = zT = None
    if return_state:
        ST = torch.empty((B, H, P_DIM * P_DIM, dv), dtype=torch.float32, device=dev)
        zT = torch.empty((B, H, P_DIM * P_DIM), dtype=torch.float32, device=dev)
    sh = _stream_handle(stream, dev)
    evarr = _event_array(events, 4, stream, dev)
    st = lib.kata_forward_decay_timed(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(P), _ptr(lam), _ptr(S0),
                                      _ptr(z0), _ptr(y), _ptr(ST), _ptr(zT), _ptr(workspace),
                                      ctypes.c_size_t(workspace.numel() * workspace.element_size()), sh, evarr)
    _check(st, "kata_forward_decay")
    return (y, ST, zT) if return_state else y


def decode_step_decay(S: torch.Tensor, z: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                      P: torch.Tensor, lam: torch.Tensor, *, out_dtype: torch.dtype = torch.float32,
                      y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One decay-gated recurrent step (kata_decode_step_decay): S <- exp(lam) S + phi(k) v^T,
    z likewise, in place; lam [N,H] fp32.  Returns y [N,H,dv]."""
    N, H, d = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(S, "S", (N, H, P_DIM * P_DIM, dv), torch.float32, dev)
    _need(z, "z", (N, H, P_DIM * P_DIM), torch.float32, dev)
    _need(q, "q", (N, H, d), device=dev)
    _need(k, "k", (N, H, d), q.dtype, dev)
    _need(v, "v", (N, H, dv), q.dtype, dev)
    _need(P, "P", (H, P_DIM, d), torch.float32, dev)
    _need(lam, "lam", (N, H), torch.float32, dev)
    if y is None:
        y = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    else:
        _need(y, "y", (N, H, dv), out_dtype, dev)
    st = _lib().kata_decode_step_decay(N, H, d, dv, P_DIM, _dtype_code(q.dtype), _dtype_code(out_dtype), _ptr(S),
                                       _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(P), _ptr(lam), _ptr(y),
                                       _stream_handle(stream, dev))
    _check(st, "kata_decode_step_decay")
    return y


FACTOR_MODES = {"concat": 0, "sum": 1}


def forward_factors_workspace_bytes(B, H, T, g, mode="concat", d=64, dv=64, chunk=64, in_dtype=torch.bfloat16,
                                    out_dtype=None) -> int:
    """Workspace bytes of kata_forward_factors for these sizes."""
    out_dtype = in_dtype if out_dtype is None else out_dtype
    desc = make_desc(B, H, T, d, dv, chunk, _dtype_code(in_dtype), _dtype_code(out_dtype))
    n = ctypes.c_size_t(0)
    _check(_lib().kata_forward_factors_workspace_bytes(ctypes.byref(desc), g, FACTOR_MODES[mode], ctypes.byref(n)),
           "kata_forward_factors_workspace_bytes")
    return int(n.value)


def forward_factors(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: torch.Tensor, mode: str = "concat",
                    chunk: int = 64, *, S0: Optional[torch.Tensor] = None, z0: Optional[torch.Tensor] = None,
                    out_dtype: Optional[torch.dtype] = None, return_state: bool = False,
                    y: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None,
                    events=None):
    """KATA with g PSD factors per head (kata_forward_factors): mode "concat" (KATA-Mg,
    a_ts = sum_i (u_i.w_i)^2, state g*256 x dv) or "sum" (KATA-Sigma-g).  P: [H, g, 16, d]
    fp32.  Returns y, or (y, ST, zT) when return_state (ST [B,H,g*256,dv] for concat)."""
    B, H, T, d = q.shape
    dv = v.shape[-1]
    g = P.shape[1]
    dev = q.device
    _need(q, "q", (B, H, T, d), device=dev)
    _need(k, "k", (B, H, T, d), q.dtype, dev)
    _need(v, "v", (B, H, T, dv), q.dtype, dev)
    _need(P, "P", (H, g, P_DIM, d), torch.float32, dev)
    rows = (g if mode == "concat" else 1) * P_DIM * P_DIM
    if (S0 is None) != (z0 is None):
        raise ValueError("S0 and z0 go together")
    if S0 is not None:
        _need(S0, "S0", (B, H, rows, dv), torch.float32, dev)
        _need(z0, "z0", (B, H, rows), torch.float32, dev)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    desc = make_desc(B, H, T, d, dv, chunk, _dtype_code(q.dtype), _dtype_code(out_dtype))
    lib = _lib()
    n = ctypes.c_size_t(0)
    _check(lib.kata_forward_factors_workspace_bytes(ctypes.byref(desc), g, FACTOR_MODES[mode], ctypes.byref(n)),
           "kata_forward_factors_workspace_bytes")
    if y is None:
        y = torch.empty((B, H, T, dv), dtype=out_dtype, device=dev)
    else:
        _need(y, "y", (B, H, T, dv), out_dtype, dev)
    if workspace is None:
        workspace = torch.empty((max(int(n.value), 1),), dtype=torch.uint8, device=dev)
    elif not workspace.is_cuda or workspace.numel() * workspace.element_size() < n.value:
        raise ValueError("workspace too small")
    ST = zT = None
    if return_state:
        ST = torch.empty((B, H, rows, dv), dtype=torch.float32, device=dev)
        zT = torch.empty((B, H, rows), dtype=torch.float32, device=dev)
    sh = _stream_handle(stream, dev)
    evarr = _event_array(events, 4, stream, dev)
    st = lib.kata_forward_factors_timed(ctypes.byref(desc), g, FACTOR_MODES[mode], _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(P), _ptr(S0), _ptr(z0), _ptr(y), _ptr(ST), _ptr(zT), _ptr(workspace),
                                        ctypes.c_size_t(workspace.numel() * workspace.element_size()), sh, evarr)
    _check(st, "kata_forward_factors")
    return (y, ST, zT) if return_state else y


def decode_step_factors(S: torch.Tensor, z: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        P: torch.Tensor, mode: str = "concat", *, out_dtype: torch.dtype = torch.float32,
                        y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One KATA-Mg ("concat") / KATA-Sigma-g ("sum") decode step (kata_decode_step_factors),
    in place on S [N,H,R,dv], z [N,H,R] (R = g*256 for concat, 256 for sum); P [H,g,16,d]."""
    N, H, d = q.shape
    dv = v.shape[-1]
    g = P.shape[1]
    dev = q.device
    rows = (g if mode == "concat" else 1) * P_DIM * P_DIM
    _need(S, "S", (N, H, rows, dv), torch.float32, dev)
    _need(z, "z", (N, H, rows), torch.float32, dev)
    _need(q, "q", (N, H, d), device=dev)
    _need(k, "k", (N, H, d), q.dtype, dev)
    _need(v, "v", (N, H, dv), q.dtype, dev)
    _need(P, "P", (H, g, P_DIM, d), torch.float32, dev)
    if y is None:
        y = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    else:
        _need(y, "y", (N, H, dv), out_dtype, dev)
    st = _lib().kata_decode_step_factors(N, H, d, dv, P_DIM, g, FACTOR_MODES[mode], _dtype_code(q.dtype),
                                         _dtype_code(out_dtype), _ptr(S), _ptr(z), _ptr(q), _ptr(k), _ptr(v),
                                         _ptr(P), _ptr(y), _stream_handle(stream, dev))
    _check(st, "kata_decode_step_factors")
    return y


def forward_delta(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: torch.Tensor, beta: torch.Tensor, *,
                  S0: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                  return_state: bool = False, y: Optional[torch.Tensor] = None, stream=None):
    """DeltaKATA causal forward (kata_forward_delta), by the token recurrence with the state on
    chip: S_t = S_{t-1} + beta_t phi^(k_t) (v_t - S_{t-1}^T phi^(k_t))^T, y_t = S_t^T phi^(q_t),
    phi^ the unit-normalised feature.  q, k: [B,H,T,d]; v: [B,H,T,dv]; P: [H,16,d] fp32;
    beta: [B,H,T] fp32; S0: [B,H,256,dv] fp32 or None.  Returns y, or (y, ST) when return_state."""
    B, H, T, d = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(q, "q", (B, H, T, d), device=dev)
    _need(k, "k", (B, H, T, d), q.dtype, dev)
    _need(v, "v", (B, H, T, dv), q.dtype, dev)
    _need(P, "P", (H, P_DIM, d), torch.float32, dev)
    _need(beta, "beta", (B, H, T), torch.float32, dev)
    if S0 is not None:
        _need(S0, "S0", (B, H, P_DIM * P_DIM, dv), torch.float32, dev)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if y is None:
        y = torch.empty((B, H, T, dv), dtype=out_dtype, device=dev)
    else:
        _need(y, "y", (B, H, T, dv), out_dtype, dev)
    ST = torch.empty((B, H, P_DIM * P_DIM, dv), dtype=torch.float32, device=dev) if return_state else None
    desc = make_desc(B, H, T, d, dv, 64, _dtype_code(q.dtype), _dtype_code(out_dtype))
    st = _lib().kata_forward_delta(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(P), _ptr(beta), _ptr(S0),
                                   _ptr(y), _ptr(ST), _stream_handle(stream, dev))
    _check(st, "kata_forward_delta")
    return (y, ST) if return_state else y


def forward_delta_chunked_workspace_bytes(B, H, T, d=64, dv=64, in_dtype=torch.bfloat16, out_dtype=None,
                                          scan="assoc", scan_leaf=0) -> int:
    """Workspace bytes of kata_forward_delta_chunked for these sizes (and segment plan)."""
    out_dtype = in_dtype if out_dtype is None else out_dtype
    desc = make_desc(B, H, T, d, dv, 64, _dtype_code(in_dtype), _dtype_code(out_dtype), scan, scan_leaf)
    n = ctypes.c_size_t(0)
    _check(_lib().kata_forward_delta_chunked_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)),
           "kata_forward_delta_chunked_workspace_bytes")
    return int(n.value)


def forward_delta_chunked_plan(B, H, T, d=64, dv=64, in_dtype=torch.bfloat16, out_dtype=None, scan="assoc",
                               scan_leaf=0) -> dict:
    """The walk plan of forward_delta_chunked(): {"segments", "segment_chunks"}
    (kata_forward_delta_chunked_plan)."""
    out_dtype = in_dtype if out_dtype is None else out_dtype
    desc = make_desc(B, H, T, d, dv, 64, _dtype_code(in_dtype), _dtype_code(out_dtype), scan, scan_leaf)
    n, per = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(_lib().kata_forward_delta_chunked_plan(ctypes.byref(desc), ctypes.byref(n), ctypes.byref(per)),
           "kata_forward_delta_chunked_plan")
    return {"segments": int(n.value), "segment_chunks": int(per.value)}


def forward_delta_chunked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: torch.Tensor, beta: torch.Tensor, *,
                          S0: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                          return_state: bool = False, y: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, ST: Optional[torch.Tensor] = None,
                          scan: str = "assoc", scan_leaf: int = 0, stream=None, events=None):
    """DeltaKATA causal forward in the chunked form (kata_forward_delta_chunked); same
    definition and arguments as forward_delta.  ST: optional preallocated final state
    [B,H,256,dv] fp32 (implies return_state; may be S0 itself, updated in place).
    scan_leaf: chunks per walk segment (0 = the library's plan); scan="sequential": one
    walk per sequence.  events: optional three torch.cuda.Event (start of the per-chunk
    pass, start and end of the walk)."""
    B, H, T, d = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(q, "q", (B, H, T, d), device=dev)
    _need(k, "k", (B, H, T, d), q.dtype, dev)
    _need(v, "v", (B, H, T, dv), q.dtype, dev)
    _need(P, "P", (H, P_DIM, d), torch.float32, dev)
    _need(beta, "beta", (B, H, T), torch.float32, dev)
    if S0 is not None:
        _need(S0, "S0", (B, H, P_DIM * P_DIM, dv), torch.float32, dev)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    desc = make_desc(B, H, T, d, dv, 64, _dtype_code(q.dtype), _dtype_code(out_dtype), scan, scan_leaf)
    lib = _lib()
    n = ctypes.c_size_t(0)
    _check(lib.kata_forward_delta_chunked_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)),
           "kata_forward_delta_chunked_workspace_bytes")
    if y is None:
        y = torch.empty((B, H, T, dv), dtype=out_dtype, device=dev)
    else:
        _need(y, "y", (B, H, T, dv), out_dtype, dev)
    if workspace is None:
        workspace = torch.empty((max(int(n.value), 1),), dtype=torch.uint8, device=dev)
    elif not workspace.is_cuda or workspace.numel() * workspace.element_size() < n.value:
        raise ValueError("workspace too small")
    if ST is not None:
        _need(ST, "ST", (B, H, P_DIM * P_DIM, dv), torch.float32, dev)
        return_state = True
    elif return_state:
        ST = torch.empty((B, H, P_DIM * P_DIM, dv), dtype=torch.float32, device=dev)
    evarr = _event_array(events, 3, stream, dev)
    st = lib.kata_forward_delta_chunked_timed(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(P), _ptr(beta),
                                              _ptr(S0), _ptr(y), _ptr(ST), _ptr(workspace),
                                              ctypes.c_size_t(workspace.numel() * workspace.element_size()),
                                              _stream_handle(stream, dev), evarr)
    _check(st, "kata_forward_delta_chunked")
    return (y, ST) if return_state else y


def decode_step_delta(S: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: torch.Tensor,
                      beta: torch.Tensor, *, out_dtype: torch.dtype = torch.float32,
                      y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """One DeltaKATA decode step (kata_decode_step_delta), in place on S [N,H,256,dv] fp32;
    beta [N,H] fp32.  Returns y [N,H,dv]."""
    N, H, d = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(S, "S", (N, H, P_DIM * P_DIM, dv), torch.float32, dev)
    _need(q, "q", (N, H, d), device=dev)
    _need(k, "k", (N, H, d), q.dtype, dev)
    _need(v, "v", (N, H, dv), q.dtype, dev)
    _need(P, "P", (H, P_DIM, d), torch.float32, dev)
    _need(beta, "beta", (N, H), torch.float32, dev)
    if y is None:
        y = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    else:
        _need(y, "y", (N, H, dv), out_dtype, dev)
    st = _lib().kata_decode_step_delta(N, H, d, dv, P_DIM, _dtype_code(q.dtype), _dtype_code(out_dtype), _ptr(S),
                                       _ptr(q), _ptr(k), _ptr(v), _ptr(P), _ptr(beta), _ptr(y),
                                       _stream_handle(stream, dev))
    _check(st, "kata_decode_step_delta")
    return y


def flash_workspace_bytes(B, H, T, d=64, dv=64, in_dtype=torch.bfloat16, out_dtype=None) -> int:
    """Workspace bytes of kata_flash_forward for these sizes."""
    out_dtype = in_dtype if out_dtype is None else out_dtype
    desc = make_desc(B, H, T, d, dv, 64, _dtype_code(in_dtype), _dtype_code(out_dtype))
    n = ctypes.c_size_t(0)
    _check(_lib().kata_flash_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)), "kata_flash_workspace_bytes")
    return int(n.value)


def flash_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: torch.Tensor, *,
                  out_dtype: Optional[torch.dtype] = None, y: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None, events=None) -> torch.Tensor:
    """Flash-style O(T^2) forward (kata_flash_forward): the same y as forward() with no
    initial state, without forming the state.  q, k, v: [B,H,T,64] bf16; P: [H,16,64] fp32.
    events: optional three torch.cuda.Event(enable_timing=True), stamped with the start of
    the projection kernel, the start of the attention kernel and its end."""
    B, H, T, d = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(q, "q", (B, H, T, d), device=dev)
    _need(k, "k", (B, H, T, d), q.dtype, dev)
    _need(v, "v", (B, H, T, dv), q.dtype, dev)
    _need(P, "P", (H, P_DIM, d), torch.float32, dev)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    desc = make_desc(B, H, T, d, dv, 64, _dtype_code(q.dtype), _dtype_code(out_dtype))
    lib = _lib()
    n = ctypes.c_size_t(0)
    _check(lib.kata_flash_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)), "kata_flash_workspace_bytes")
    if y is None:
        y = torch.empty((B, H, T, dv), dtype=out_dtype, device=dev)
    else:
        _need(y, "y", (B, H, T, dv), out_dtype, dev)
    if workspace is None:
        workspace = torch.empty((max(int(n.value), 1),), dtype=torch.uint8, device=dev)
    elif not workspace.is_cuda or workspace.numel() * workspace.element_size() < n.value:
        raise ValueError("workspace too small")
    sh = _stream_handle(stream, dev)
    evarr = _event_array(events, 3, stream, dev)
    st = lib.kata_flash_forward(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(P), _ptr(y), _ptr(workspace),
                                ctypes.c_size_t(workspace.numel() * workspace.element_size()), sh, evarr)
    _check(st, "kata_flash_forward")
    return y


def backward_workspace_bytes(B, H, T, d=64, dv=64, chunk=64, in_dtype=torch.bfloat16, out_dtype=None,
                             scan="assoc", scan_leaf=0) -> int:
    """Workspace bytes of kata_backward for these sizes."""
    out_dtype = in_dtype if out_dtype is None else out_dtype
    desc = make_desc(B, H, T, d, dv, chunk, _dtype_code(in_dtype), _dtype_code(out_dtype), scan, scan_leaf)
    n = ctypes.c_size_t(0)
    _check(_lib().kata_backward_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)),
           "kata_backward_workspace_bytes")
    return int(n.value)


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: torch.Tensor, gy: torch.Tensor,
             chunk: int = 64, *, S0: Optional[torch.Tensor] = None,
             z0: Optional[torch.Tensor] = None, gST: Optional[torch.Tensor] = None,
             gzT: Optional[torch.Tensor] = None, return_state_grad: bool = False, scan: str = "assoc",
             scan_leaf: int = 0, workspace: Optional[torch.Tensor] = None, out=None, stream=None, events=None):
    """Gradients of the KATA causal forward (kata_backward).

    q, k, v: [B,H,T,64] bf16; P: [H,16,64] fp32; gy: the gradient of the loss with respect
    to the forward's output y, [B,H,T,64] bf16 or fp32 (y itself is not needed); S0, z0:
    the forward's initial state (or None); gST, gzT: gradient of the final state (or None).  Returns (dq, dk, dv, dP)
    and, when return_state_grad, (dq, dk, dv, dP, dS0, dz0).  out: optional preallocated
    (dq, dk, dv, dP).  events: optional eight torch.cuda.Event(enable_timing=True).
    """
    B, H, T, d = q.shape
    dv_ = v.shape[-1]
    dev = q.device
    _need(q, "q", (B, H, T, d), device=dev)
    _need(k, "k", (B, H, T, d), q.dtype, dev)
    _need(v, "v", (B, H, T, dv_), q.dtype, dev)
    _need(P, "P", (H, P_DIM, d), torch.float32, dev)
    _need(gy, "gy", (B, H, T, dv_), device=dev)
    pp = P_DIM * P_DIM
    for a, b_, n1, n2 in ((S0, z0, "S0", "z0"), (gST, gzT, "gST", "gzT")):
        if (a is None) != (b_ is None):
            raise ValueError(f"{n1} and {n2} go together")
        if a is not None:
            _need(a, n1, (B, H, pp, dv_), torch.float32, dev)
            _need(b_, n2, (B, H, pp), torch.float32, dev)
    desc = make_desc(B, H, T, d, dv_, chunk, _dtype_code(q.dtype), _dtype_code(gy.dtype), scan, scan_leaf)
    lib = _lib()
    n = ctypes.c_size_t(0)
    _check(lib.kata_backward_workspace_bytes(ctypes.byref(desc), ctypes.byref(n)), "kata_backward_workspace_bytes")
    if out is None:
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dvv = torch.empty_like(v)
        dP = torch.empty((H, P_DIM, d), dtype=torch.float32, device=dev)
    else:
        dq, dk, dvv, dP = out
        _need(dq, "dq", q.shape, q.dtype, dev)
        _need(dk, "dk", k.shape, q.dtype, dev)
        _need(dvv, "dv", v.shape, q.dtype, dev)
        _need(dP, "dP", (H, P_DIM, d), torch.float32, dev)
    dS0 = dz0 = None
    if return_state_grad:
        dS0 = torch.empty((B, H, pp, dv_), dtype=torch.float32, device=dev)
        dz0 = torch.empty((B, H, pp), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty((max(int(n.value), 1),), dtype=torch.uint8, device=dev)
    elif not workspace.is_cuda or workspace.numel() * workspace.element_size() < n.value:
        raise ValueError("workspace too small")
    sh = _stream_handle(stream, dev)
    evarr = _event_array(events, 8, stream, dev)
    st = lib.kata_backward_timed(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(P), _ptr(S0), _ptr(z0),
                                 _ptr(gy), _ptr(gST), _ptr(gzT), _ptr(dq), _ptr(dk), _ptr(dvv), _ptr(dP),
                                 _ptr(dS0), _ptr(dz0), _ptr(workspace),
                                 ctypes.c_size_t(workspace.numel() * workspace.element_size()), sh, evarr)
    _check(st, "kata_backward")
    if return_state_grad:
        return dq, dk, dvv, dP, dS0, dz0
    return dq, dk, dvv, dP


def decode_step(S: torch.Tensor, z: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                P: torch.Tensor, *, out_dtype: torch.dtype = torch.float32, y: Optional[torch.Tensor] = None,
                stream=None) -> torch.Tensor:
    """One recurrent step (kata_decode_step): S, z updated in place; returns y [N,H,dv]."""
    N, H, d = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(S, "S", (N, H, P_DIM * P_DIM, dv), torch.float32, dev)
    _need(z, "z", (N, H, P_DIM * P_DIM), torch.float32, dev)
    _need(q, "q", (N, H, d), device=dev)
    _need(k, "k", (N, H, d), q.dtype, dev)
    _need(v, "v", (N, H, dv), q.dtype, dev)
    _need(P, "P", (H, P_DIM, d), torch.float32, dev)
    if y is None:
        y = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    else:
        _need(y, "y", (N, H, dv), out_dtype, dev)
    st = _lib().kata_decode_step(N, H, d, dv, P_DIM, _dtype_code(q.dtype), _dtype_code(out_dtype), _ptr(S),
                                 _ptr(z), _ptr(q), _ptr(k), _ptr(v), _ptr(P), _ptr(y),
                                 _stream_handle(stream, dev))
    _check(st, "kata_decode_step")
    return y


def state_pack(S: torch.Tensor, z: Optional[torch.Tensor] = None, *, Sp: Optional[torch.Tensor] = None,
               zp: Optional[torch.Tensor] = None, stream=None):
    """Canonical state S [..., 256, dv] (and z [..., 256]) to the packed symmetric layout
    Sp [..., 136, dv] (zp [..., 136]) (kata_state_pack): one row per pair {a, b}, the mean
    of its two mirror rows.  Returns Sp, or (Sp, zp) when z is given."""
    lead, dv = tuple(S.shape[:-2]), S.shape[-1]
    dev = S.device
    _need(S, "S", lead + (P_DIM * P_DIM, dv), torch.float32, dev)
    if z is not None:
        _need(z, "z", lead + (P_DIM * P_DIM,), torch.float32, dev)
    n = 1
    for x in lead:
        n *= x
    if Sp is None:
        Sp = torch.empty(lead + (PACKED_ROWS, dv), dtype=torch.float32, device=dev)
    _need(Sp, "Sp", lead + (PACKED_ROWS, dv), torch.float32, dev)
    if z is not None:
        if zp is None:
            zp = torch.empty(lead + (PACKED_ROWS,), dtype=torch.float32, device=dev)
        _need(zp, "zp", lead + (PACKED_ROWS,), torch.float32, dev)
    _check(_lib().kata_state_pack(n, dv, _ptr(S), _ptr(z), _ptr(Sp), _ptr(zp if z is not None else None),
                                  _stream_handle(stream, dev)), "kata_state_pack")
    return (Sp, zp) if z is not None else Sp


def state_unpack(Sp: torch.Tensor, zp: Optional[torch.Tensor] = None, *, S: Optional[torch.Tensor] = None,
                 z: Optional[torch.Tensor] = None, stream=None):
    """Packed symmetric state Sp [..., 136, dv] (and zp) back to the canonical layout
    (kata_state_unpack): both mirror rows of each pair.  Returns S, or (S, z)."""
    lead, dv = tuple(Sp.shape[:-2]), Sp.shape[-1]
    dev = Sp.device
    _need(Sp, "Sp", lead + (PACKED_ROWS, dv), torch.float32, dev)
    if zp is not None:
        _need(zp, "zp", lead + (PACKED_ROWS,), torch.float32, dev)
    n = 1
    for x in lead:
        n *= x
    if S is None:
        S = torch.empty(lead + (P_DIM * P_DIM, dv), dtype=torch.float32, device=dev)
    _need(S, "S", lead + (P_DIM * P_DIM, dv), torch.float32, dev)
    if zp is not None:
        if z is None:
            z = torch.empty(lead + (P_DIM * P_DIM,), dtype=torch.float32, device=dev)
        _need(z, "z", lead + (P_DIM * P_DIM,), torch.float32, dev)
    _check(_lib().kata_state_unpack(n, dv, _ptr(Sp), _ptr(zp), _ptr(S), _ptr(z if zp is not None else None),
                                    _stream_handle(stream, dev)), "kata_state_unpack")
    return (S, z) if zp is not None else S


def decode_step_packed(Sp: torch.Tensor, zp: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       P: torch.Tensor, *, out_dtype: torch.dtype = torch.float32, y: Optional[torch.Tensor] = None,
                       stream=None) -> torch.Tensor:
    """One recurrent step on the packed state (kata_decode_step_packed): Sp [N,H,136,dv],
    zp [N,H,136] updated in place; returns y [N,H,dv], equal to decode_step's on the
    unpacked state."""
    N, H, d = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(Sp, "Sp", (N, H, PACKED_ROWS, dv), torch.float32, dev)
    _need(zp, "zp", (N, H, PACKED_ROWS), torch.float32, dev)
    _need(q, "q", (N, H, d), device=dev)
    _need(k, "k", (N, H, d), q.dtype, dev)
    _need(v, "v", (N, H, dv), q.dtype, dev)
    _need(P, "P", (H, P_DIM, d), torch.float32, dev)
    if y is None:
        y = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    else:
        _need(y, "y", (N, H, dv), out_dtype, dev)
    st = _lib().kata_decode_step_packed(N, H, d, dv, P_DIM, _dtype_code(q.dtype), _dtype_code(out_dtype), _ptr(Sp),
                                        _ptr(zp), _ptr(q), _ptr(k), _ptr(v), _ptr(P), _ptr(y),
                                        _stream_handle(stream, dev))
    _check(st, "kata_decode_step_packed")
    return y


def decode_step_delta_packed(Sp: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, P: torch.Tensor,
                             beta: torch.Tensor, *, out_dtype: torch.dtype = torch.float32,
                             y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """decode_step_delta on the packed state (kata_decode_step_delta_packed): Sp [N,H,136,dv]
    updated in place; beta [N,H] fp32.  Returns y [N,H,dv]."""
    N, H, d = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(Sp, "Sp", (N, H, PACKED_ROWS, dv), torch.float32, dev)
    _need(q, "q", (N, H, d), device=dev)
    _need(k, "k", (N, H, d), q.dtype, dev)
    _need(v, "v", (N, H, dv), q.dtype, dev)
    _need(P, "P", (H, P_DIM, d), torch.float32, dev)
    _need(beta, "beta", (N, H), torch.float32, dev)
    if y is None:
        y = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    else:
        _need(y, "y", (N, H, dv), out_dtype, dev)
    st = _lib().kata_decode_step_delta_packed(N, H, d, dv, P_DIM, _dtype_code(q.dtype), _dtype_code(out_dtype),
                                              _ptr(Sp), _ptr(q), _ptr(k), _ptr(v), _ptr(P), _ptr(beta), _ptr(y),
                                              _stream_handle(stream, dev))
    _check(st, "kata_decode_step_delta_packed")
    return y


def decode_step_decay_packed(Sp: torch.Tensor, zp: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                             P: torch.Tensor, lam: torch.Tensor, *, out_dtype: torch.dtype = torch.float32,
                             y: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """decode_step_decay on the packed state (kata_decode_step_decay_packed); lam [N,H] fp32."""
    N, H, d = q.shape
    dv = v.shape[-1]
    dev = q.device
    _need(Sp, "Sp", (N, H, PACKED_ROWS, dv), torch.float32, dev)
    _need(zp, "zp", (N, H, PACKED_ROWS), torch.float32, dev)
    _need(q, "q", (N, H, d), device=dev)
    _need(k, "k", (N, H, d), q.dtype, dev)
    _need(v, "v", (N, H, dv), q.dtype, dev)
    _need(P, "P", (H, P_DIM, d), torch.float32, dev)
    _need(lam, "lam", (N, H), torch.float32, dev)
    if y is None:
        y = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    else:
        _need(y, "y", (N, H, dv), out_dtype, dev)
    st = _lib().kata_decode_step_decay_packed(N, H, d, dv, P_DIM, _dtype_code(q.dtype), _dtype_code(out_dtype),
                                              _ptr(Sp), _ptr(zp), _ptr(q), _ptr(k), _ptr(v), _ptr(P), _ptr(lam),
                                              _ptr(y), _stream_handle(stream, dev))
    _check(st, "kata_decode_step_decay_packed")
    return y


def decode_step_factors_packed(Sp: torch.Tensor, zp: torch.Tensor, q: torch.Tensor, k: torch.Tensor,
                               v: torch.Tensor, P: torch.Tensor, mode: str = "concat", *,
                               out_dtype: torch.dtype = torch.float32, y: Optional[torch.Tensor] = None,
                               stream=None) -> torch.Tensor:
    """decode_step_factors on packed states (kata_decode_step_factors_packed): P [H,g,16,d];
    Sp [N,H,g*136,dv], zp [N,H,g*136] ("concat") or [N,H,136,...] ("sum")."""
    N, H, d = q.shape
    dv = v.shape[-1]
    g = P.shape[1]
    dev = q.device
    rows = PACKED_ROWS * (g if mode == "concat" else 1)
    _need(Sp, "Sp", (N, H, rows, dv), torch.float32, dev)
    _need(zp, "zp", (N, H, rows), torch.float32, dev)
    _need(q, "q", (N, H, d), device=dev)
    _need(k, "k", (N, H, d), q.dtype, dev)
    _need(v, "v", (N, H, dv), q.dtype, dev)
    _need(P, "P", (H, g, P_DIM, d), torch.float32, dev)
    if y is None:
        y = torch.empty((N, H, dv), dtype=out_dtype, device=dev)
    else:
        _need(y, "y", (N, H, dv), out_dtype, dev)
    st = _lib().kata_decode_step_factors_packed(N, H, d, dv, P_DIM, g, FACTOR_MODES[mode], _dtype_code(q.dtype),
                                                _dtype_code(out_dtype), _ptr(Sp), _ptr(zp), _ptr(q), _ptr(k), _ptr(v),
                                                _ptr(P), _ptr(y), _stream_handle(stream, dev))
    _check(st, "kata_decode_step_factors_packed")
    return y


def feature_map(x: torch.Tensor, P: torch.Tensor, layout: str = "full", stream=None) -> torch.Tensor:
    """phi for every vector of x [n,H,d] (kata_feature_map): [n,H,256] full or [n,H,144] packed."""
    n, H, d = x.shape
    dev = x.device
    _need(x, "x", (n, H, d), device=dev)
    _need(P, "P", (H, P_DIM, d), torch.float32, dev)
    width = P_DIM * P_DIM if layout == "full" else N_PACKED
    phi = torch.empty((n, H, width), dtype=torch.float32, device=dev)
    st = _lib().kata_feature_map(_ptr(x), _ptr(P), n, H, d, P_DIM, FEATURE_LAYOUTS[layout], _dtype_code(x.dtype),
                                 _ptr(phi), _stream_handle(stream, dev))
    _check(st, "kata_feature_map")
    return phi
