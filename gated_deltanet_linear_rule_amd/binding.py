"""Thin Python binding of libgdn.so (argument marshalling only).

The functions here take torch tensors that live on the GPU, check that their
dtypes/shapes/contiguity match the C ABI (include/gdn.h), and pass raw device
pointers and the current HIP stream to the library.  Every step of the
computation runs in the library's HIP kernels; there is no fallback: if the
library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn.so")
POISON_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn_poison.so")
_lib = None

GDN_SUCCESS = 0
GDN_ERROR_INVALID_VALUE = 1
GDN_ERROR_NOT_SUPPORTED = 2
GDN_ERROR_LAUNCH = 3
GDN_ERROR_OUT_OF_MEMORY = 4
GDN_DTYPE_F32 = 0
GDN_DTYPE_BF16 = 1
GDN_WS_PACKED = 1
GDN_WS_RAW = 2
GDN_WS_AFFINE = 4
GDN_STATIC_SCRATCH_BYTES = 64 << 20


class GdnShape(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_tokens", ctypes.c_int64),
                ("num_qk_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("dtype", ctypes.c_int)]


class GdnError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status} ({status_string(status)}): {detail}")
        self.status = status


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """The loaded libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = open_library(_LIB_PATH)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """Load a build of the library (libgdn.so, or its race-check build libgdn_poison.so)
    and declare the C ABI's argument types on it."""
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m gated_deltanet_linear_rule_amd.build`")
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    L.gdn_prefill.argtypes = [ctypes.POINTER(GdnShape), P, P, P, P, P, P, P, P, P, P]
    L.gdn_prefill.restype = ctypes.c_int
    L.gdn_decode_step.argtypes = [ctypes.POINTER(GdnShape), P, P, P, P, P, P, P, P]
    L.gdn_decode_step.restype = ctypes.c_int
    L.gdn_decode_tokens.argtypes = [ctypes.POINTER(GdnShape), ctypes.c_int32, P, P, P, P, P, P, P, P, P]
    L.gdn_decode_tokens.restype = ctypes.c_int
    L.gdn_decode_slots.argtypes = [ctypes.POINTER(GdnShape), ctypes.c_int32, P, P, P, P, P, P, ctypes.c_int64,
                                   P, P, P, P]
    L.gdn_decode_slots.restype = ctypes.c_int
    L.gdn_prefill_snapshots.argtypes = [ctypes.POINTER(GdnShape), P, P, P, P, P, P, P, P, P, ctypes.c_int32, P, P]
    L.gdn_prefill_snapshots.restype = ctypes.c_int
    L.gdn_prefill_snapshots_ws.argtypes = [ctypes.POINTER(GdnShape), P, P, P, P, P, P, P, P, P, ctypes.c_int32,
                                           P, P, ctypes.c_size_t, P]
    L.gdn_prefill_snapshots_ws.restype = ctypes.c_int
    L.gdn_prefill_workspace_size.argtypes = [ctypes.POINTER(GdnShape), ctypes.c_uint32,
                                             ctypes.POINTER(ctypes.c_size_t)]
    L.gdn_prefill_workspace_size.restype = ctypes.c_int
    L.gdn_prefill_ws.argtypes = [ctypes.POINTER(GdnShape), P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.gdn_prefill_ws.restype = ctypes.c_int
    L.gdn_prefill_static.argtypes = L.gdn_prefill.argtypes
    L.gdn_prefill_static.restype = ctypes.c_int
    L.gdn_prefill_affine.argtypes = [ctypes.POINTER(GdnShape), P, P, P, P, P, P, P, P]
    L.gdn_prefill_affine.restype = ctypes.c_int
    L.gdn_prefill_affine_ws.argtypes = [ctypes.POINTER(GdnShape), P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.gdn_prefill_affine_ws.restype = ctypes.c_int
    L.gdn_prefill_raw.argtypes = L.gdn_prefill.argtypes
    L.gdn_prefill_raw.restype = ctypes.c_int
    L.gdn_prefill_raw_ws.argtypes = L.gdn_prefill_ws.argtypes
    L.gdn_prefill_raw_ws.restype = ctypes.c_int
    L.gdn_decode_tokens_raw.argtypes = L.gdn_decode_tokens.argtypes
    L.gdn_decode_tokens_raw.restype = ctypes.c_int
    L.gdn_status_string.argtypes = [ctypes.c_int]
    L.gdn_status_string.restype = ctypes.c_char_p
    L.gdn_last_error.argtypes = []
    L.gdn_last_error.restype = ctypes.c_char_p
    L.gdn_abi_version.argtypes = []
    L.gdn_abi_version.restype = ctypes.c_int
    return L


def gdn_abi_version() -> int:
    return lib().gdn_abi_version()


def status_string(status: int) -> str:
    return lib().gdn_status_string(status).decode()


gdn_status_string = status_string


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _io_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return GDN_DTYPE_BF16
    if t.dtype == torch.float32:
        return GDN_DTYPE_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _check(t, name, dtype=None, shape=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _raise(rc, where):
    if rc != GDN_SUCCESS:
        raise GdnError(rc, where, lib().gdn_last_error().decode())


def gdn_prefill_workspace_size(q, v, cu_seqlens=None, num_seqs=None, raw=False, affine=False) -> int:
    """Bytes of device workspace a prefill call with these shapes needs on the current device
    (q [T, Hqk, dk] -- for the affine map pass k --, v [T, Hv, dv]; packed if cu_seqlens is given;
    raw / affine for gdn_prefill_raw / gdn_prefill_affine)."""
    T, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    N = cu_seqlens.numel() - 1 if cu_seqlens is not None else (1 if num_seqs is None else int(num_seqs))
    shape = GdnShape(N, T, hqk, hv, dk, dv, _io_dtype(q))
    flags = (GDN_WS_PACKED if cu_seqlens is not None else 0) | (GDN_WS_RAW if raw else 0) | \
        (GDN_WS_AFFINE if affine else 0)
    n = ctypes.c_size_t(0)
    _raise(lib().gdn_prefill_workspace_size(ctypes.byref(shape), flags, ctypes.byref(n)),
           "gdn_prefill_workspace_size")
    return int(n.value)


def _workspace(workspace, use_pool, q, v, cu_seqlens, N, raw=False, affine=False):
    """(pointer, bytes) of the workspace for a *_ws call, or None for the pool form.
    workspace=None allocates one from torch's allocator for this call."""
    if use_pool:
        if workspace is not None:
            raise ValueError("use_pool=True takes no workspace")
        return None
    if workspace is None:
        n = gdn_prefill_workspace_size(q, v, cu_seqlens, N, raw=raw, affine=affine)
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)
    _check(workspace, "workspace")
    return workspace, ctypes.c_size_t(workspace.numel() * workspace.element_size())


def gdn_prefill(q, k, v, g, beta, init_state=None, cu_seqlens=None, out=None, final_state=None,
                stream=None, num_seqs=None, return_final_state=True, raw=False, workspace=None, use_pool=False,
                use_static=False):
    """Chunked GDN prefill over packed sequences.

    q, k [T, Hqk, dk]; v [T, Hv, dv] (bf16 or fp32, same dtype); g, beta [T, Hv]
    fp32; init_state [N, Hv, dv, dk] fp32 or None; cu_seqlens int32 [N+1] on
    the GPU or None (then ``num_seqs`` equal-length sequences, default 1).
    Returns (out, final_state); final_state is None if not requested.
    raw=True calls the raw-projection form: q, k unnormalised, g and beta are the logits a, b.
    workspace: a contiguous GPU tensor of at least gdn_prefill_workspace_size bytes (allocated from
    torch for this call if None); the library's *_ws entry point runs on it.  use_pool=True calls the
    form that takes its workspace from HIP's default stream-ordered pool instead, use_static=True the
    one that runs on the library's static scratch (gdn_prefill_static; not with raw).
    """
    T, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    io = _io_dtype(q)
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", torch.int32)
        N = cu_seqlens.numel() - 1
    else:
        N = 1 if num_seqs is None else int(num_seqs)
    _check(q, "q", q.dtype, (T, hqk, dk))
    _check(k, "k", q.dtype, (T, hqk, dk))
    _check(v, "v", q.dtype, (T, hv, dv))
    _check(g, "g", torch.float32, (T, hv))
    _check(beta, "beta", torch.float32, (T, hv))
    _check(init_state, "init_state", torch.float32, (N, hv, dv, dk))
    if out is None:
        out = torch.empty((T, hv, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", q.dtype, (T, hv, dv))
    if final_state is None and return_final_state:
        final_state = torch.empty((N, hv, dv, dk), dtype=torch.float32, device=q.device)
    _check(final_state, "final_state", torch.float32, (N, hv, dv, dk))
    shape = GdnShape(N, T, hqk, hv, dk, dv, io)
    args = (ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(init_state), _ptr(cu_seqlens),
            _ptr(out), _ptr(final_state))
    if use_static:
        if raw or use_pool or workspace is not None:
            raise ValueError("use_static=True takes no workspace and has no raw-projection form")
        _raise(lib().gdn_prefill_static(*args, _stream(stream)), "gdn_prefill_static")
        return out, final_state
    ws = _workspace(workspace, use_pool, q, v, cu_seqlens, N, raw=raw)
    name = "gdn_prefill" + ("_raw" if raw else "") + ("" if ws is None else "_ws")
    fn = getattr(lib(), name)
    rc = fn(*args, _stream(stream)) if ws is None else fn(*args, _ptr(ws[0]), ws[1], _stream(stream))
    _raise(rc, name)
    return out, final_state


def gdn_prefill_affine(k, v, g, beta, cu_seqlens=None, transition=None, offset=None, stream=None, num_seqs=None,
                       workspace=None, use_pool=False):
    """State map of each whole sequence: S -> S @ transition + offset.

    k [T, Hqk, dk]; v [T, Hv, dv] (bf16 or fp32); g, beta [T, Hv] fp32; cu_seqlens as for gdn_prefill.
    Returns (transition [N, Hv, dk, dk], offset [N, Hv, dv, dk]), fp32 (allocated if None).
    workspace / use_pool as for gdn_prefill."""
    T, hqk, dk = k.shape
    hv, dv = v.shape[1], v.shape[2]
    io = _io_dtype(k)
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", torch.int32)
        N = cu_seqlens.numel() - 1
    else:
        N = 1 if num_seqs is None else int(num_seqs)
    _check(k, "k", k.dtype, (T, hqk, dk))
    _check(v, "v", k.dtype, (T, hv, dv))
    _check(g, "g", torch.float32, (T, hv))
    _check(beta, "beta", torch.float32, (T, hv))
    if transition is None:
        transition = torch.empty((N, hv, dk, dk), dtype=torch.float32, device=k.device)
    if offset is None:
        offset = torch.empty((N, hv, dv, dk), dtype=torch.float32, device=k.device)
    _check(transition, "transition", torch.float32, (N, hv, dk, dk))
    _check(offset, "offset", torch.float32, (N, hv, dv, dk))
    shape = GdnShape(N, T, hqk, hv, dk, dv, io)
    args = (ctypes.byref(shape), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens), _ptr(transition),
            _ptr(offset))
    ws = _workspace(workspace, use_pool, k, v, cu_seqlens, N, affine=True)
    if ws is None:
        _raise(lib().gdn_prefill_affine(*args, _stream(stream)), "gdn_prefill_affine")
    else:
        _raise(lib().gdn_prefill_affine_ws(*args, _ptr(ws[0]), ws[1], _stream(stream)), "gdn_prefill_affine_ws")
    return transition, offset


def gdn_decode_step(q, k, v, g, beta, state, out=None, stream=None):
    """One decode token per sequence; ``state`` [N, Hv, dv, dk] is updated in place.

    q, k [N, Hqk, dk]; v [N, Hv, dv]; g, beta [N, Hv].  Returns out [N, Hv, dv].
    """
    N, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    io = _io_dtype(q)
    _check(q, "q", q.dtype, (N, hqk, dk))
    _check(k, "k", q.dtype, (N, hqk, dk))
    _check(v, "v", q.dtype, (N, hv, dv))
    _check(g, "g", torch.float32, (N, hv))
    _check(beta, "beta", torch.float32, (N, hv))
    _check(state, "state", torch.float32, (N, hv, dv, dk))
    if out is None:
        out = torch.empty((N, hv, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", q.dtype, (N, hv, dv))
    shape = GdnShape(N, N, hqk, hv, dk, dv, io)
    rc = lib().gdn_decode_step(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                               _ptr(state), _ptr(out), _stream(stream))
    _raise(rc, "gdn_decode_step")
    return out


def gdn_decode_tokens(q, k, v, g, beta, state, tokens_per_seq, out=None, token_states=None, stream=None,
                      raw=False):
    """T = ``tokens_per_seq`` tokens per sequence in one pass; ``state`` [N, Hv, dv, dk] is updated in place.

    q, k [N*T, Hqk, dk]; v [N*T, Hv, dv]; g, beta [N*T, Hv] (token t of sequence n at row n*T + t).
    ``token_states``: None, True (allocate) or a float32 tensor [N, T, Hv, dv, dk] that receives the
    state after every token.  Returns (out [N*T, Hv, dv], token_states or None).
    raw=True calls gdn_decode_tokens_raw: q, k unnormalised, g and beta are the logits a, b.
    """
    NT, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    T = int(tokens_per_seq)
    N = state.shape[0]
    io = _io_dtype(q)
    _check(q, "q", q.dtype, (NT, hqk, dk))
    _check(k, "k", q.dtype, (NT, hqk, dk))
    _check(v, "v", q.dtype, (NT, hv, dv))
    _check(g, "g", torch.float32, (NT, hv))
    _check(beta, "beta", torch.float32, (NT, hv))
    _check(state, "state", torch.float32, (N, hv, dv, dk))
    if out is None:
        out = torch.empty((NT, hv, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", q.dtype, (NT, hv, dv))
    if token_states is True:
        token_states = torch.empty((N, T, hv, dv, dk), dtype=torch.float32, device=q.device)
    if token_states is not None:
        _check(token_states, "token_states", torch.float32, (N, T, hv, dv, dk))
    shape = GdnShape(N, NT, hqk, hv, dk, dv, io)
    fn = lib().gdn_decode_tokens_raw if raw else lib().gdn_decode_tokens
    rc = fn(ctypes.byref(shape), T, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
            _ptr(state), _ptr(out), _ptr(token_states), _stream(stream))
    _raise(rc, "gdn_decode_tokens_raw" if raw else "gdn_decode_tokens")
    return out, token_states


def gdn_decode_slots(q, k, v, g, beta, state_pool, slot_idx, tokens_per_seq=1, out=None, token_states=None,
                     stream=None):
    """``gdn_decode_tokens`` over a state pool: sequence n uses ``state_pool[slot_idx[n]]``.

    state_pool float32 [P, Hv, dv, dk]; slot_idx int32 [N] on the GPU (negative = padding, skipped).
    Returns (out [N*T, Hv, dv], token_states or None).
    """
    NT, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    T = int(tokens_per_seq)
    N = slot_idx.shape[0]
    io = _io_dtype(q)
    _check(q, "q", q.dtype, (NT, hqk, dk))
    _check(k, "k", q.dtype, (NT, hqk, dk))
    _check(v, "v", q.dtype, (NT, hv, dv))
    _check(g, "g", torch.float32, (NT, hv))
    _check(beta, "beta", torch.float32, (NT, hv))
    _check(state_pool, "state_pool", torch.float32, (state_pool.shape[0], hv, dv, dk))
    _check(slot_idx, "slot_idx", torch.int32, (N,))
    if out is None:
        out = torch.empty((NT, hv, dv), dtype=q.dtype, device=q.device)
    _check(out, "out", q.dtype, (NT, hv, dv))
    if token_states is True:
        token_states = torch.empty((N, T, hv, dv, dk), dtype=torch.float32, device=q.device)
    if token_states is not None:
        _check(token_states, "token_states", torch.float32, (N, T, hv, dv, dk))
    shape = GdnShape(N, NT, hqk, hv, dk, dv, io)
    rc = lib().gdn_decode_slots(ctypes.byref(shape), T, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(state_pool), int(state_pool.shape[0]), _ptr(slot_idx), _ptr(out),
                                _ptr(token_states), _stream(stream))
    _raise(rc, "gdn_decode_slots")
    return out, token_states


def snapshot_slots(num_tokens, num_seqs, snapshot_chunks):
    """Slots a snapshot buffer needs: floor(num_tokens / P) + num_seqs, P = 64 * snapshot_chunks."""
    return num_tokens // (64 * snapshot_chunks) + num_seqs


def gdn_prefill_snapshots(q, k, v, g, beta, snapshot_chunks, init_state=None, cu_seqlens=None, snapshots=None,
                          out=None, final_state=None, stream=None, num_seqs=None, workspace=None, use_pool=False):
    """``gdn_prefill`` that also writes the state after every 64 * ``snapshot_chunks`` tokens of each
    sequence into ``snapshots`` [slots, Hv, dv, dk] (allocated if None; see ``snapshot_slots``).
    workspace / use_pool as for gdn_prefill.  Returns (out, final_state, snapshots)."""
    T, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    if num_seqs is None:
        num_seqs = (cu_seqlens.shape[0] - 1) if cu_seqlens is not None else 1
    N = int(num_seqs)
    io = _io_dtype(q)
    for t, n, dt, shp in ((q, "q", q.dtype, (T, hqk, dk)), (k, "k", q.dtype, (T, hqk, dk)),
                          (v, "v", q.dtype, (T, hv, dv)), (g, "g", torch.float32, (T, hv)),
                          (beta, "beta", torch.float32, (T, hv))):
        _check(t, n, dt, shp)
    if init_state is not None:
        _check(init_state, "init_state", torch.float32, (N, hv, dv, dk))
    if cu_seqlens is not None:
        _check(cu_seqlens, "cu_seqlens", torch.int32, (N + 1,))
    if out is None:
        out = torch.empty((T, hv, dv), dtype=q.dtype, device=q.device)
    if final_state is None:
        final_state = torch.empty((N, hv, dv, dk), dtype=torch.float32, device=q.device)
    if snapshots is None:
        snapshots = torch.zeros((snapshot_slots(T, N, snapshot_chunks), hv, dv, dk), dtype=torch.float32,
                                device=q.device)
    _check(out, "out", q.dtype, (T, hv, dv))
    _check(final_state, "final_state", torch.float32, (N, hv, dv, dk))
    _check(snapshots, "snapshots", torch.float32, (snapshots.shape[0], hv, dv, dk))
    shape = GdnShape(N, T, hqk, hv, dk, dv, io)
    args = (ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(init_state), _ptr(cu_seqlens),
            _ptr(out), _ptr(final_state), int(snapshot_chunks), _ptr(snapshots))
    ws = _workspace(workspace, use_pool, q, v, cu_seqlens, N)
    if ws is None:
        _raise(lib().gdn_prefill_snapshots(*args, _stream(stream)), "gdn_prefill_snapshots")
    else:
        _raise(lib().gdn_prefill_snapshots_ws(*args, _ptr(ws[0]), ws[1], _stream(stream)), "gdn_prefill_snapshots_ws")
    return out, final_state, snapshots
