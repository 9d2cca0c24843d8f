"""ctypes access to the plain-C fp64 oracle (oracle/gdn_oracle.c).

TEST INFRASTRUCTURE: only tests, the smoke check and the benchmark's CPU
baseline may import this module.  It builds and loads ``libgdn_oracle.so``
with gcc; it has no HIP dependency and shares no code with the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (OpenMP over independent chains)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        lib.gdn_oracle_prefill.argtypes = [ctypes.c_int64, P, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           P, P, P, P, P, P, P, P, ctypes.c_int]
        lib.gdn_oracle_prefill.restype = ctypes.c_int
        lib.gdn_oracle_decode_step.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int,
                                               ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                               P, P, P, P, P, P, P, ctypes.c_int]
        lib.gdn_oracle_decode_step.restype = ctypes.c_int
        lib.gdn_oracle_prefill_raw.argtypes = lib.gdn_oracle_prefill.argtypes
        lib.gdn_oracle_prefill_raw.restype = ctypes.c_int
        lib.gdn_oracle_decode_step_raw.argtypes = lib.gdn_oracle_decode_step.argtypes
        lib.gdn_oracle_decode_step_raw.restype = ctypes.c_int
        lib.gdn_oracle_threads.argtypes = [ctypes.c_int]
        lib.gdn_oracle_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _elem(a):
    if a.dtype == np.uint16:
        return 1
    if a.dtype == np.float32:
        return 0
    raise TypeError(f"oracle inputs are bf16 bits (uint16) or float32, got {a.dtype}")


def threads(nthreads: int = 0) -> int:
    """Number of OpenMP threads a call with ``nthreads`` (0 = default) uses."""
    return _load().gdn_oracle_threads(nthreads)


def prefill(q, k, v, g, beta, init_state=None, cu=None, nthreads=0, final=True, raw=False):
    """fp64 outputs [T, Hv, dv] and final states [N, Hv, dv, dk].

    raw=True: q, k are unnormalised and g, beta hold the gate and write-strength
    logits a, b; the prologue (q, k L2-normalised, g = -softplus(a),
    beta = sigmoid(b)) is applied per token in fp64.
    q, k, v are stored inputs (uint16 bf16 bits or float32); g, beta float32;
    init_state float32 [N, Hv, dv, dk] or None; cu int [N+1] or None.
    """
    T, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    cu64 = np.array([0, T] if cu is None else cu, dtype=np.int64)
    nseq = len(cu64) - 1
    arrs = [np.ascontiguousarray(x) for x in (q, k, v)]
    g = np.ascontiguousarray(g, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    s0 = None if init_state is None else np.ascontiguousarray(init_state, dtype=np.float32)
    out = np.empty((T, hv, dv), dtype=np.float64)
    fin = np.empty((nseq, hv, dv, dk), dtype=np.float64) if final else None
    fn = _load().gdn_oracle_prefill_raw if raw else _load().gdn_oracle_prefill
    rc = fn(nseq, _ptr(cu64), hqk, hv, dk, dv, _elem(arrs[0]),
                                    _ptr(arrs[0]), _ptr(arrs[1]), _ptr(arrs[2]), _ptr(g),
                                    _ptr(beta), _ptr(s0), _ptr(out), _ptr(fin), nthreads)
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_prefill failed ({rc})")
    return out, fin


def decode_step(q, k, v, g, beta, state, nthreads=0, raw=False):
    """Advance the fp64 ``state`` [N, Hv, dv, dk] in place; returns out [N, Hv, dv]."""
    N, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    assert state.dtype == np.float64 and state.flags.c_contiguous
    arrs = [np.ascontiguousarray(x) for x in (q, k, v)]
    g = np.ascontiguousarray(g, dtype=np.float32)
    beta = np.ascontiguousarray(beta, dtype=np.float32)
    out = np.empty((N, hv, dv), dtype=np.float64)
    fn = _load().gdn_oracle_decode_step_raw if raw else _load().gdn_oracle_decode_step
    rc = fn(N, hqk, hv, dk, dv, _elem(arrs[0]), _ptr(arrs[0]),
                                        _ptr(arrs[1]), _ptr(arrs[2]), _ptr(g), _ptr(beta),
                                        _ptr(state), _ptr(out), nthreads)
    if rc != 0:
        raise RuntimeError(f"gdn_oracle_decode_step failed ({rc})")
    return out


def decode_tokens(q, k, v, g, beta, state, tokens_per_seq, nthreads=0, raw=False):
    """T tokens per sequence as T successive C decode steps (fp64).

    Stored inputs as for ``decode_step`` but with N*T token rows (token t of
    sequence n at row n*T + t); ``state`` fp32 or fp64 [N, Hv, dv, dk] (not
    modified).  Returns (out [N*T, Hv, dv], token_states [N, T, Hv, dv, dk],
    final [N, Hv, dv, dk]), all fp64.
    """
    T = int(tokens_per_seq)
    N = state.shape[0]
    hv, dv, dk = state.shape[1], state.shape[2], state.shape[3]
    st = np.array(state, dtype=np.float64, copy=True, order="C")
    out = np.empty((N * T, hv, dv), dtype=np.float64)
    states = np.empty((N, T, hv, dv, dk), dtype=np.float64)
    for t in range(T):
        out[t::T] = decode_step(q[t::T], k[t::T], v[t::T], g[t::T], beta[t::T], st, nthreads=nthreads, raw=raw)
        states[:, t] = st
    return out, states, st
