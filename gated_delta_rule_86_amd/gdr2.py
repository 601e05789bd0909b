"""ctypes binding of ``libgdr2.so`` (the C ABI declared in include/gdr2.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  PyTorch supplies device memory (``torch.empty``)
and the current HIP stream.  There is no fallback: if the library is missing
or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdr2.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = range(5)
F32, BF16 = 0, 1
PROLOGUE_NORM_QK, PROLOGUE_GATES = 1, 2
ALGO_AUTO, ALGO_STAGED, ALGO_SEGMENTED, ALGO_FUSED = 0, 1, 2, 3
ALGOS = {"auto": ALGO_AUTO, "staged": ALGO_STAGED, "segmented": ALGO_SEGMENTED, "fused": ALGO_FUSED}
STAGES = {"all": 0, "prep": 1, "state": 2}

_c_i64 = ctypes.c_int64
_c_i32 = ctypes.c_int32
_vp = ctypes.c_void_p


class FwdArgs(ctypes.Structure):
    _fields_ = [("B", _c_i64), ("T", _c_i64), ("H", _c_i64), ("Dk", _c_i64), ("Dv", _c_i64),
                ("chunk", _c_i32), ("dtype", _c_i32), ("algo", _c_i32), ("stage", _c_i32),
                ("b_width", _c_i32), ("w_width", _c_i32), ("g_width", _c_i32), ("prologue", _c_i32),
                ("q", _vp), ("k", _vp), ("v", _vp), ("b", _vp), ("w", _vp),
                ("g", _vp), ("S0", _vp), ("o", _vp), ("S_out", _vp),
                ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t), ("S_chunks", _vp)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("N", _c_i64), ("H", _c_i64), ("Dk", _c_i64), ("Dv", _c_i64),
                ("dtype", _c_i32), ("b_width", _c_i32), ("w_width", _c_i32), ("g_width", _c_i32),
                ("q", _vp), ("k", _vp), ("v", _vp), ("b", _vp), ("w", _vp),
                ("g", _vp), ("state", _vp), ("o", _vp), ("prologue", _c_i32), ("reserved", _c_i32)]


class BwdArgs(ctypes.Structure):
    _fields_ = [("B", _c_i64), ("T", _c_i64), ("H", _c_i64), ("Dk", _c_i64), ("Dv", _c_i64),
                ("chunk", _c_i32), ("dtype", _c_i32),
                ("b_width", _c_i32), ("w_width", _c_i32), ("g_width", _c_i32), ("prologue", _c_i32),
                ("q", _vp), ("k", _vp), ("v", _vp), ("b", _vp), ("w", _vp), ("g", _vp),
                ("S_chunks", _vp), ("dO", _vp), ("dS_final", _vp),
                ("dq", _vp), ("dk", _vp), ("dv", _vp), ("db", _vp), ("dw", _vp), ("dg", _vp),
                ("dS0", _vp), ("workspace", _vp), ("workspace_bytes", ctypes.c_size_t),
                ("algo", _c_i32), ("reserved", _c_i32)]


# Every symbol include/gdr2.h declares (checked by the tests).
EXPORTS = ("gdr2_forward_workspace_size", "gdr2_forward_chunked", "gdr2_decode_step",
           "gdr2_backward_workspace_size", "gdr2_backward_chunked",
           "gdr2_status_string", "gdr2_last_error", "gdr2_abi_version", "gdr2_forward_chunked_noalloc")
ABI_VERSION = 6
NOALLOC_SCRATCH_BYTES = 64 << 20
BWD_CHUNK = 64


class Gdr2Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"gdr2 status {status}: {message}")
        self.status = status


_lock = threading.Lock()
_lib = None


def load_library(path: str = LIB_PATH):
    """Load the built library (no build, no fallback)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run __graft_entry__.build() "
                               "or python gated_delta_rule_86_amd/build.py")
        lib = ctypes.CDLL(path)
        lib.gdr2_forward_workspace_size.restype = ctypes.c_size_t
        lib.gdr2_forward_workspace_size.argtypes = [ctypes.POINTER(FwdArgs)]
        lib.gdr2_forward_chunked.restype = ctypes.c_int
        lib.gdr2_forward_chunked.argtypes = [ctypes.POINTER(FwdArgs), _vp]
        lib.gdr2_forward_chunked_noalloc.restype = ctypes.c_int
        lib.gdr2_forward_chunked_noalloc.argtypes = [ctypes.POINTER(FwdArgs), _vp]
        lib.gdr2_decode_step.restype = ctypes.c_int
        lib.gdr2_decode_step.argtypes = [ctypes.POINTER(DecodeArgs), _vp]
        lib.gdr2_backward_workspace_size.restype = ctypes.c_size_t
        lib.gdr2_backward_workspace_size.argtypes = [ctypes.POINTER(BwdArgs)]
        lib.gdr2_backward_chunked.restype = ctypes.c_int
        lib.gdr2_backward_chunked.argtypes = [ctypes.POINTER(BwdArgs), _vp]
        lib.gdr2_status_string.restype = ctypes.c_char_p
        lib.gdr2_status_string.argtypes = [ctypes.c_int]
        lib.gdr2_last_error.restype = ctypes.c_char_p
        lib.gdr2_last_error.argtypes = []
        lib.gdr2_abi_version.restype = ctypes.c_int
        lib.gdr2_abi_version.argtypes = []
        if lib.gdr2_abi_version() != ABI_VERSION:
            raise RuntimeError("libgdr2.so ABI version mismatch")
        _lib = lib
        return lib


def _check(lib, status: int):
    if status != OK:
        raise Gdr2Error(status, lib.gdr2_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _req(t: torch.Tensor, name: str, dtype=None, shape=None, device=None):
    """Dtype, exact shape (when given), then device and contiguity of one
    tensor argument.  The library takes every size from q (or the state)
    and the chunk, so a tensor of another shape would be read or written out
    of bounds: it is refused here, before any launch."""
    _req_shape(t, name, dtype, shape)
    _req_dev(t, name, device)


def _req_shape(t: torch.Tensor, name: str, dtype=None, shape=None):
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _req_dev(t: torch.Tensor, name: str, device=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _gate_shape(t: torch.Tensor, name: str, lead, full: int):
    """Shape of a gate: lead + (1,) or lead + (full,), by its last dim."""
    if t.dim() != len(lead) + 1 or t.shape[-1] not in (1, full):
        raise ValueError(f"{name} must have shape {tuple(lead) + (1,)} or {tuple(lead) + (full,)}, "
                         f"got {tuple(t.shape)}")
    return tuple(lead) + (t.shape[-1],)


def check_forward_shapes(q, k, v, b, w, g, S0=None):
    """Dtypes and shapes of the forward's (and backward's) inputs against
    q [B,T,H,Dk] and v [B,T,H,Dv]; returns (B, T, H, Dk, Dv).  Raises
    ValueError / TypeError on a mismatch (no device is touched)."""
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError(f"q and v must be [B,T,H,D], got {tuple(q.shape)} and {tuple(v.shape)}")
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"unsupported dtype {q.dtype} (float32 or bfloat16)")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    lead = (B, T, H)
    _req_shape(k, "k", q.dtype, (B, T, H, Dk))
    _req_shape(v, "v", q.dtype, (B, T, H, Dv))
    _req_shape(b, "b", q.dtype, _gate_shape(b, "b", lead, Dk))
    _req_shape(w, "w", q.dtype, _gate_shape(w, "w", lead, Dv))
    _req_shape(g, "g", torch.float32, _gate_shape(g, "g", lead, Dk))
    if S0 is not None:
        _req_shape(S0, "S0", torch.float32, (B, H, Dk, Dv))
    return B, T, H, Dk, Dv


def check_decode_shapes(state, q, k, v, b, w, g):
    """Dtypes and shapes of one decode step's arguments against state
    [N,H,Dk,Dv]; returns (N, H, Dk, Dv)."""
    _req_shape(state, "state", torch.float32)
    if state.dim() != 4:
        raise ValueError(f"state must be [N,H,Dk,Dv], got {tuple(state.shape)}")
    N, H, Dk, Dv = state.shape
    if q.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError(f"unsupported dtype {q.dtype} (float32 or bfloat16)")
    _req_shape(q, "q", None, (N, H, Dk))
    _req_shape(k, "k", q.dtype, (N, H, Dk))
    _req_shape(v, "v", q.dtype, (N, H, Dv))
    _req_shape(b, "b", q.dtype, _gate_shape(b, "b", (N, H), Dk))
    _req_shape(w, "w", q.dtype, _gate_shape(w, "w", (N, H), Dv))
    _req_shape(g, "g", torch.float32, _gate_shape(g, "g", (N, H), Dk))
    return N, H, Dk, Dv


def _on_device(dev, **tensors):
    for n, t in tensors.items():
        if t is not None:
            _req_dev(t, n, dev)


def fwd_args(q, k, v, b, w, g, S0=None, o=None, S_out=None, chunk: int = 64,
             algo: str = "auto", workspace=None, stage: str = "all", S_chunks=None,
             prologue: int = 0) -> FwdArgs:
    B, T, H, Dk = q.shape
    a = FwdArgs()
    a.B, a.T, a.H, a.Dk, a.Dv = B, T, H, Dk, v.shape[-1]
    a.chunk, a.dtype, a.algo, a.stage = chunk, _dtype_code(q), ALGOS[algo], STAGES[stage]
    a.b_width, a.w_width, a.g_width = b.shape[-1], w.shape[-1], g.shape[-1]
    a.q, a.k, a.v, a.b, a.w, a.g = (_ptr(x) for x in (q, k, v, b, w, g))
    a.S0, a.o, a.S_out, a.S_chunks = _ptr(S0), _ptr(o), _ptr(S_out), _ptr(S_chunks)
    a.prologue = prologue
    if workspace is not None:
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return a


def forward(q, k, v, b, w, g, S0=None, chunk: int = 64, algo: str = "auto",
            out=None, S_out=None, workspace=None, final_state: bool = True,
            stage: str = "all", chunk_states=None, prologue: int = 0):
    """Chunked forward.  q,k [B,T,H,Dk]; v [B,T,H,Dv]; b [B,T,H,1|Dk];
    w [B,T,H,1|Dv] (all float32 or bfloat16); g float32 [B,T,H,1|Dk];
    S0 float32 [B,H,Dk,Dv] or None.  Returns (o, S_final), or
    (o, S_final, S_chunks) when chunk_states is True or a float32 tensor
    [B,H,ceil(T/chunk),Dk,Dv]: the state at the start of every chunk.
    stage='prep' / 'state' runs one kernel of the staged algorithm (pass the
    same workspace, out and S_out to both calls).  prologue: PROLOGUE_* bits
    (raw q, k normalised and raw gates activated inside the kernels)."""
    B, T, H, Dk, Dv = check_forward_shapes(q, k, v, b, w, g, S0)
    if chunk <= 0:
        raise ValueError(f"chunk must be positive, got {chunk}")
    if out is not None:
        _req_shape(out, "out", q.dtype, (B, T, H, Dv))
    if S_out is not None:
        _req_shape(S_out, "S_out", torch.float32, (B, H, Dk, Dv))
    ckt = chunk_states if isinstance(chunk_states, torch.Tensor) else None
    if ckt is not None:
        _req_shape(ckt, "chunk_states", torch.float32, (B, H, -(-T // chunk), Dk, Dv))
    _on_device(q.device, q=q, k=k, v=v, b=b, w=w, g=g, S0=S0, out=out, S_out=S_out, chunk_states=ckt,
               workspace=workspace)
    lib = load_library()
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=q.dtype, device=q.device)
    if S_out is None and final_state:
        S_out = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    ck = ckt
    if chunk_states is True:
        ck = torch.empty((B, H, -(-T // chunk), Dk, Dv), dtype=torch.float32, device=q.device)
    a = fwd_args(q, k, v, b, w, g, S0, out, S_out, chunk, algo, stage=stage, S_chunks=ck, prologue=prologue)
    need = lib.gdr2_forward_workspace_size(ctypes.byref(a))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib, lib.gdr2_forward_chunked(ctypes.byref(a), stream))
    return (out, S_out) if ck is None else (out, S_out, ck)


def forward_noalloc(q, k, v, b, w, g, S0=None, out=None, S_out=None, chunk: int = 64, algo: str = "auto",
                    chunk_states=None, prologue: int = 0):
    """The chunked forward through gdr2_forward_chunked_noalloc: the
    workspace is the library's static device scratch (NOALLOC_SCRATCH_BYTES
    per device), so the library allocates nothing.  Pass `out` and `S_out`
    (and chunk_states) preallocated to allocate nothing here either.  Calls
    that overlap in time on one device share that scratch and race."""
    B, T, H, Dk, Dv = check_forward_shapes(q, k, v, b, w, g, S0)
    if out is not None:
        _req_shape(out, "out", q.dtype, (B, T, H, Dv))
    if S_out is not None:
        _req_shape(S_out, "S_out", torch.float32, (B, H, Dk, Dv))
    if chunk_states is not None:
        _req_shape(chunk_states, "chunk_states", torch.float32, (B, H, -(-T // chunk), Dk, Dv))
    _on_device(q.device, q=q, k=k, v=v, b=b, w=w, g=g, S0=S0, out=out, S_out=S_out, chunk_states=chunk_states)
    lib = load_library()
    if out is None:
        out = torch.empty((B, T, H, Dv), dtype=q.dtype, device=q.device)
    if S_out is None:
        S_out = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    a = fwd_args(q, k, v, b, w, g, S0, out, S_out, chunk, algo, S_chunks=chunk_states, prologue=prologue)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib, lib.gdr2_forward_chunked_noalloc(ctypes.byref(a), stream))
    return out, S_out


def workspace_size(q, k, v, b, w, g, chunk: int = 64, algo: str = "auto") -> int:
    lib = load_library()
    return int(lib.gdr2_forward_workspace_size(ctypes.byref(fwd_args(q, k, v, b, w, g, chunk=chunk, algo=algo))))


def decode_args(state, q, k, v, b, w, g, o, prologue: int = 0) -> DecodeArgs:
    N, H, Dk, Dv = state.shape
    a = DecodeArgs()
    a.N, a.H, a.Dk, a.Dv = N, H, Dk, Dv
    a.dtype = _dtype_code(q)
    a.b_width, a.w_width, a.g_width = b.shape[-1], w.shape[-1], g.shape[-1]
    a.q, a.k, a.v, a.b, a.w, a.g = (_ptr(x) for x in (q, k, v, b, w, g))
    a.state, a.o = _ptr(state), _ptr(o)
    a.prologue = prologue
    return a


def decode_step(state, q, k, v, b, w, g, out=None, prologue: int = 0):
    """One decode step, in place on ``state`` float32 [N,H,Dk,Dv].
    q,k [N,H,Dk]; v [N,H,Dv]; b [N,H,1|Dk]; w [N,H,1|Dv]; g float32 [N,H,1|Dk].
    Returns o [N,H,Dv]."""
    N, H, Dk, Dv = check_decode_shapes(state, q, k, v, b, w, g)
    if out is not None:
        _req_shape(out, "out", q.dtype, (N, H, Dv))
    _on_device(state.device, state=state, q=q, k=k, v=v, b=b, w=w, g=g, out=out)
    lib = load_library()
    if out is None:
        out = torch.empty((N, H, Dv), dtype=q.dtype, device=q.device)
    a = decode_args(state, q, k, v, b, w, g, out, prologue)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib, lib.gdr2_decode_step(ctypes.byref(a), stream))
    return out


def bwd_args(q, k, v, b, w, g, S_chunks, dO, dS_final=None, grads=None, dS0=None,
             workspace=None, chunk: int = BWD_CHUNK, prologue: int = 0, algo: str = "auto") -> BwdArgs:
    """grads: (dq, dk, dv, db, dw, dg) or None."""
    B, T, H, Dk = q.shape
    a = BwdArgs()
    a.B, a.T, a.H, a.Dk, a.Dv = B, T, H, Dk, v.shape[-1]
    a.chunk, a.dtype = chunk, _dtype_code(q)
    a.b_width, a.w_width, a.g_width = b.shape[-1], w.shape[-1], g.shape[-1]
    a.q, a.k, a.v, a.b, a.w, a.g = (_ptr(x) for x in (q, k, v, b, w, g))
    a.S_chunks, a.dO, a.dS_final, a.dS0 = _ptr(S_chunks), _ptr(dO), _ptr(dS_final), _ptr(dS0)
    a.prologue = prologue
    a.algo = ALGOS[algo]
    if grads is not None:
        a.dq, a.dk, a.dv, a.db, a.dw, a.dg = (_ptr(x) for x in grads)
    if workspace is not None:
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    return a


def backward_workspace_size(q, k, v, b, w, g, algo: str = "auto") -> int:
    lib = load_library()
    return int(lib.gdr2_backward_workspace_size(ctypes.byref(bwd_args(q, k, v, b, w, g, None, None, algo=algo))))


def backward(q, k, v, b, w, g, S_chunks, dO, dS_final=None, workspace=None, grads=None,
             dS0=None, want_dS0: bool = True, prologue: int = 0, algo: str = "auto"):
    """Chunked backward (chunk 64).  Inputs as for ``forward``; S_chunks is
    the float32 [B,H,ceil(T/64),Dk,Dv] chunk-start states of a chunk-64
    forward; dO [B,T,H,Dv] in the inputs' dtype; dS_final float32
    [B,H,Dk,Dv] or None.  Returns a dict of float32 gradients dq, dk, dv,
    db, dw, dg (shaped like their inputs) and dS0 (None unless want_dS0 or
    given).  algo: 'staged' (one reverse pass over the chunks per (b, h)),
    'segmented' (the two-level scan over chunk segments) or 'auto'."""
    B, T, H, Dk, Dv = check_forward_shapes(q, k, v, b, w, g)
    dev = q.device
    _req_shape(dO, "dO", q.dtype, (B, T, H, Dv))
    _req_shape(S_chunks, "S_chunks", torch.float32, (B, H, -(-T // BWD_CHUNK), Dk, Dv))
    if dS_final is not None:
        _req_shape(dS_final, "dS_final", torch.float32, (B, H, Dk, Dv))
    if grads is not None:
        if len(grads) != 6:
            raise ValueError("grads must be (dq, dk, dv, db, dw, dg)")
        for n, gt, x in zip(("dq", "dk", "dv", "db", "dw", "dg"), grads, (q, k, v, b, w, g)):
            _req_shape(gt, n, torch.float32, tuple(x.shape))
    if dS0 is not None:
        _req_shape(dS0, "dS0", torch.float32, (B, H, Dk, Dv))
    _on_device(dev, q=q, k=k, v=v, b=b, w=w, g=g, dO=dO, S_chunks=S_chunks, dS_final=dS_final, dS0=dS0,
               workspace=workspace, **({} if grads is None else dict(zip(("dq", "dk", "dv", "db", "dw", "dg"), grads))))
    lib = load_library()
    if grads is None:
        grads = tuple(torch.empty(x.shape, dtype=torch.float32, device=q.device) for x in (q, k, v, b, w, g))
    if dS0 is None and want_dS0:
        dS0 = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=q.device)
    a = bwd_args(q, k, v, b, w, g, S_chunks, dO, dS_final, grads, dS0, prologue=prologue, algo=algo)
    need = lib.gdr2_backward_workspace_size(ctypes.byref(a))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        a.workspace, a.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    stream = torch.cuda.current_stream(q.device).cuda_stream
    _check(lib, lib.gdr2_backward_chunked(ctypes.byref(a), stream))
    return dict(zip(("dq", "dk", "dv", "db", "dw", "dg"), grads), dS0=dS0)
