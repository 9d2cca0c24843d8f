"""numpy fp64 forms of the Gated DeltaNet recurrence (tiny sizes).

TEST INFRASTRUCTURE: only tests, the smoke check and the benchmark's CPU
baseline may import this module.  It shares nothing with the HIP library.

The pages (flozi.net, "Qwen3.8-Flash-Next architecture", "Der Weg eines
Tokens durch das Modell", item 1) state that a GDN layer keeps a fixed-size
recurrent state per head in place of a per-token KV cache; they give no
formula.  The recurrence used, per value head, with S of shape (d_v, d_k):

    S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t q_t,   alpha_t = exp(g_t).

Three routes are written out here, each from its own definition:

* ``sequential``  -- the formula above, literally, with the d_k x d_k matrix
  (I - beta k k^T) formed explicitly;
* ``unrolled``    -- the closed form of that linear recurrence,
  S_T = S_0 prod_t A_t + sum_t beta_t v_t k_t^T prod_{s>t} A_s with
  A_t = alpha_t (I - beta_t k_t k_t^T), o_t read from the partial products;
* ``chunked``     -- the chunk-wise WY / UT-transform form over chunks of C
  tokens (the form the GPU kernels use), derived in the module body below.

All arrays are fp64 numpy arrays of the *widened* inputs.  Shapes:
q, k [T, Hqk, dk]; v [T, Hv, dv]; g, beta [T, Hv]; states [N, Hv, dv, dk];
cu [N+1] token offsets.  Value head h uses q/k head h * Hqk // Hv.
"""
from __future__ import annotations

import numpy as np


def _chains(cu, hv, hqk):
    for n in range(len(cu) - 1):
        for h in range(hv):
            yield n, h, (h * hqk) // hv, int(cu[n]), int(cu[n + 1])


def _init(init_state, n, h, dv, dk):
    if init_state is None:
        return np.zeros((dv, dk))
    return np.array(init_state[n, h], dtype=np.float64)


def sequential(q, k, v, g, beta, init_state=None, cu=None):
    """The recurrence exactly as defined, token by token (matrix form)."""
    T, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    cu = np.array([0, T]) if cu is None else np.asarray(cu)
    out = np.zeros((T, hv, dv))
    final = np.zeros((len(cu) - 1, hv, dv, dk))
    eye = np.eye(dk)
    for n, h, hq, t0, t1 in _chains(cu, hv, hqk):
        S = _init(init_state, n, h, dv, dk)
        for t in range(t0, t1):
            kt, qt, vt = k[t, hq], q[t, hq], v[t, h]
            a, b = np.exp(g[t, h]), beta[t, h]
            S = a * S @ (eye - b * np.outer(kt, kt)) + b * np.outer(vt, kt)
            out[t, h] = S @ qt
        final[n, h] = S
    return out, final


def unrolled(q, k, v, g, beta, init_state=None, cu=None):
    """Closed form of the linear recurrence, built from transition products.

    With A_t = alpha_t (I - beta_t k_t k_t^T) and B_t = beta_t v_t k_t^T the
    recurrence is S_t = S_{t-1} A_t + B_t, hence
    S_t = S_0 A_1...A_t + sum_{s<=t} B_s A_{s+1}...A_t.  Each term is formed
    from scratch (quadratic in T): use only for tiny T.
    """
    T, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    cu = np.array([0, T]) if cu is None else np.asarray(cu)
    out = np.zeros((T, hv, dv))
    final = np.zeros((len(cu) - 1, hv, dv, dk))
    eye = np.eye(dk)
    for n, h, hq, t0, t1 in _chains(cu, hv, hqk):
        S0 = _init(init_state, n, h, dv, dk)
        A = [np.exp(g[t, h]) * (eye - beta[t, h] * np.outer(k[t, hq], k[t, hq]))
             for t in range(t0, t1)]
        B = [beta[t, h] * np.outer(v[t, h], k[t, hq]) for t in range(t0, t1)]
        L = t1 - t0
        S = S0
        for t in range(L):
            prod0 = eye
            for j in range(t + 1):
                prod0 = prod0 @ A[j]
            S = S0 @ prod0
            for s in range(t + 1):
                P = eye
                for j in range(s + 1, t + 1):
                    P = P @ A[j]
                S = S + B[s] @ P
            out[t0 + t, h] = S @ q[t0 + t, hq]
        final[n, h] = S
    return out, final


# --------------------------------------------------------------------------
# Chunk-wise form.  Within a chunk starting from state S (tokens 1..n,
# cumulative log-decay G_t = g_1 + ... + g_t, gamma_t = e^{G_t}):
#   write S_t = alpha_t S_{t-1} + u_t k_t^T with u_t = beta_t (v_t - alpha_t S_{t-1} k_t);
#   unrolling, S_t = gamma_t S + sum_{s<=t} e^{G_t - G_s} u_s k_s^T, so
#   u_t + beta_t sum_{s<t} e^{G_t-G_s} (k_t.k_s) u_s = beta_t v_t - beta_t gamma_t S k_t.
#   With A = strict_lower(diag(beta) (Gamma o K K^T)), Gamma_ts = e^{G_t-G_s}:
#       (I + A) U = diag(beta) V - diag(beta gamma) K S^T
#       U = T diag(beta) V - T diag(beta gamma) K S^T,   T = (I + A)^{-1}
#   Outputs  O = diag(gamma) Q S^T + lower_incl(Gamma o Q K^T) U
#   Next     S' = gamma_n S + U^T diag(e^{G_n - G}) K
# --------------------------------------------------------------------------
def chunked(q, k, v, g, beta, init_state=None, cu=None, chunk=64):
    """Chunk-wise WY/UT evaluation of the same recurrence (fp64)."""
    T, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    cu = np.array([0, T]) if cu is None else np.asarray(cu)
    out = np.zeros((T, hv, dv))
    final = np.zeros((len(cu) - 1, hv, dv, dk))
    for n, h, hq, t0, t1 in _chains(cu, hv, hqk):
        S = _init(init_state, n, h, dv, dk)
        for c0 in range(t0, t1, chunk):
            c1 = min(t1, c0 + chunk)
            K, Q, V = k[c0:c1, hq], q[c0:c1, hq], v[c0:c1, h]
            b = beta[c0:c1, h]
            G = np.cumsum(g[c0:c1, h])
            gam = np.exp(G)
            Gam = np.exp(G[:, None] - G[None, :])
            A = np.tril(b[:, None] * Gam * (K @ K.T), -1)
            Tm = np.linalg.inv(np.eye(c1 - c0) + A)
            U = Tm @ (b[:, None] * V) - Tm @ ((b * gam)[:, None] * K) @ S.T
            O = gam[:, None] * (Q @ S.T) + np.tril(Gam * (Q @ K.T)) @ U
            D = np.exp(G[-1] - G)
            S = gam[-1] * S + U.T @ (D[:, None] * K)
            out[c0:c1, h] = O
        final[n, h] = S
    return out, final


def decode_step(q, k, v, g, beta, state):
    """One token per sequence: returns (out [N, Hv, dv], new state).

    q, k [N, Hqk, dk]; v [N, Hv, dv]; g, beta [N, Hv]; state [N, Hv, dv, dk].
    Same recurrence as ``sequential`` with T = 1 per sequence.
    """
    N, hqk, dk = q.shape
    hv, dv = v.shape[1], v.shape[2]
    out = np.zeros((N, hv, dv))
    new = np.array(state, dtype=np.float64, copy=True)
    eye = np.eye(dk)
    for n in range(N):
        for h in range(hv):
            hq = (h * hqk) // hv
            kt, qt, vt = k[n, hq], q[n, hq], v[n, h]
            a, b = np.exp(g[n, h]), beta[n, h]
            S = a * new[n, h] @ (eye - b * np.outer(kt, kt)) + b * np.outer(vt, kt)
            new[n, h] = S
            out[n, h] = S @ qt
    return out, new


def decode_tokens(q, k, v, g, beta, state, tokens_per_seq):
    """T tokens per sequence, applied as T successive decode steps.

    q, k [N*T, Hqk, dk]; v [N*T, Hv, dv]; g, beta [N*T, Hv], token t of
    sequence n at row n*T + t; state [N, Hv, dv, dk].  Returns
    (out [N*T, Hv, dv], token_states [N, T, Hv, dv, dk], final [N, Hv, dv, dk]),
    token_states[n, t] being the state after token t.  (Several tokens per
    sequence per call: the verification step of multi-token-prediction
    drafting, flozi.net, "Qwen3.8-Flash-Next architecture", stack table,
    draft-module row.)
    """
    T = int(tokens_per_seq)
    N = state.shape[0]
    hv, dv, dk = state.shape[1], state.shape[2], state.shape[3]
    out = np.zeros((N * T, hv, dv))
    states = np.zeros((N, T, hv, dv, dk))
    st = np.array(state, dtype=np.float64, copy=True)
    for t in range(T):
        o, st = decode_step(q[t::T], k[t::T], v[t::T], g[t::T], beta[t::T], st)
        out[t::T] = o
        states[:, t] = st
    return out, states, st
