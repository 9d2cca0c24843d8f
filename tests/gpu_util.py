"""Helpers for GPU parity tests: upload seeded inputs, run the HIP library
through its binding, run the fp64 oracle on the same stored values, and
compare with the relative metric max|gpu - ref| / max|ref|."""
from __future__ import annotations

import sys

import numpy as np
import torch

from gated_deltanet_linear_rule_amd import binding as B
from gated_deltanet_linear_rule_amd import inputs as gi
from oracle import c_oracle

TOL = {"f32": 1e-5, "bf16": 1e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(x, dtype=None):
    """numpy stored input -> GPU tensor (uint16 arrays are bf16 bit patterns)."""
    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref))) / max(den, 1e-30)


def run_prefill(inp, init_mode="given", out_alias=False, num_seqs=None):
    """Run the HIP prefill on a generator Inputs; returns (out, final) as fp64 numpy."""
    wl = inp.wl
    q, k, v, g, beta = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta)
    cu = dev(inp.cu_seqlens) if inp.cu_seqlens is not None else None
    N = wl.num_seqs
    if init_mode == "given":
        s0 = dev(inp.init_state)
    elif init_mode == "zeros":
        s0 = torch.zeros((N, wl.num_v_heads, wl.head_dim_v, wl.head_dim_k), device="cuda")
    else:
        s0 = None
    fin = s0 if (out_alias and s0 is not None) else None
    out, fin = B.gdn_prefill(q, k, v, g, beta, s0, cu, final_state=fin,
                             num_seqs=None if cu is not None else (num_seqs or N))
    torch.cuda.synchronize()
    return host64(out), host64(fin)


def oracle_prefill(inp, nthreads=0):
    return c_oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state,
                            inp.cu_seqlens, nthreads=nthreads)


def check_prefill(inp, tol=None, label="", **kw):
    tol = TOL[inp.wl.dtype] if tol is None else tol
    out, fin = run_prefill(inp, **kw)
    ro, rf = oracle_prefill(inp)
    eo, ef = rel_err(out, ro), rel_err(fin, rf)
    say(f"[parity] {label or inp.wl.name}: out {eo:.3e}  final {ef:.3e}  (tol {tol:g})")
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(fin))
    assert eo <= tol, f"out rel err {eo}"
    assert ef <= tol, f"final-state rel err {ef}"
    return eo, ef


def oracle_affine(inp):
    """(M, B) of every sequence from the oracle: B is the state reached from zero; M is the state
    reached from the identity with v = 0 (so that its rows carry the transition alone)."""
    dk = inp.wl.head_dim_k
    N, hv = inp.wl.num_seqs, inp.wl.num_v_heads
    _, rb = c_oracle.prefill(inp.k, inp.k, inp.v, inp.g, inp.beta, None, inp.cu_seqlens)
    zv = np.zeros((inp.k.shape[0], hv, dk), dtype=inp.v.dtype)
    eye = np.broadcast_to(np.eye(dk, dtype=np.float32), (N, hv, dk, dk)).copy()
    _, rm = c_oracle.prefill(inp.k, inp.k, zv, inp.g, inp.beta, eye, inp.cu_seqlens)
    return rm, rb


def oracle_snapshots(inp, P):
    """fp64 states after every P tokens of each sequence, keyed by snapshot slot
    floor(cu[n] / P) + n + s - 1: the oracle run on each prefix of s * P tokens
    from the sequence's own initial state (no hand-over between runs)."""
    T = inp.q.shape[0]
    cu = inp.cu_seqlens if inp.cu_seqlens is not None else np.array([0, T])
    snaps = {}
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        st = None if inp.init_state is None else inp.init_state[n:n + 1]
        for s in range(1, (b - a) // P + 1):
            t1 = a + s * P
            _, fin = c_oracle.prefill(inp.q[a:t1], inp.k[a:t1], inp.v[a:t1], inp.g[a:t1], inp.beta[a:t1], st, None)
            snaps[a // P + n + s - 1] = fin[0]
    return snaps
