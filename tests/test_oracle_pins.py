"""Pins for the fp64 oracle: closed forms and invariants of the recurrence.

The pages print no worked GDN example, so the oracle is pinned by what the
definition itself fixes (flozi.net, "Qwen3.8-Flash-Next architecture",
"Der Weg eines Tokens durch das Modell", item 1: a fixed-size recurrent state
per head; recurrence S_t = alpha_t S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
o_t = S_t q_t).  Each test below would fail for a plausible slip: a dropped
alpha in the delta term, a sign error, a transposed outer product, reading the
state before instead of after the write, a wrong q/k head for grouped value
heads, or chunking that leaks across sequences.
"""
import math

import numpy as np
import pytest

from oracle import c_oracle, reference as ref

RTOL = 1e-12


def _rel(a, b):
    den = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


def _rand(rng, T, hqk, hv, dk, dv, nseq_init=None):
    q = rng.standard_normal((T, hqk, dk))
    k = rng.standard_normal((T, hqk, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, hv, dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, hv))))
    g = -np.log1p(np.exp(rng.standard_normal((T, hv))))
    s0 = None if nseq_init is None else 0.1 * rng.standard_normal((nseq_init, hv, dv, dk))
    return q, k, v, g, beta, s0


def _f32(*arrs):
    """Store fp64 test arrays as fp32 and widen them back (exact round trip)."""
    outs = []
    for a in arrs:
        outs.append(None if a is None else np.asarray(a, dtype=np.float32))
    return outs


def _c_prefill(q, k, v, g, beta, s0=None, cu=None, **kw):
    q, k, v, g, beta, s0 = _f32(q, k, v, g, beta, s0)
    return c_oracle.prefill(q, k, v, g, beta, s0, cu, **kw)


def _hadamard(n):
    """Normalised Hadamard matrix: orthonormal rows, entries exactly +-1/sqrt(n)."""
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H / math.sqrt(n)


# --------------------------------------------------------------------------
# a worked example, derived by hand from the definition (d_k = d_v = 2)
# --------------------------------------------------------------------------
def test_hand_worked_example():
    # token 1: S0 = 0, k = e1, v = (1, 2), beta = 1/2, alpha = 1
    #   s = 0, u = (1/2)(1, 2) = (0.5, 1), S1 = u e1^T = [[0.5, 0], [1, 0]]
    #   q = e1 -> o1 = (0.5, 1)
    # token 2: k = e2, v = (4, 0), beta = 1, alpha = 1/2
    #   s = S1 e2 = 0, u = (4, 0), S2 = S1/2 + u e2^T = [[0.25, 4], [0.5, 0]]
    #   q = (1, 1) -> o2 = (4.25, 0.5)
    # token 3: k = (0.6, 0.8), v = 0, beta = 1/2, alpha = 1
    #   s = S2 k = (3.35, 0.3), u = -(1/2) s = (-1.675, -0.15)
    #   S3 = S2 + u k^T = [[-0.755, 2.66], [0.41, -0.12]]
    #   q = e2 -> o3 = (2.66, -0.12)
    q = np.array([[[1, 0]], [[1, 1]], [[0, 1]]], dtype=float)
    k = np.array([[[1, 0]], [[0, 1]], [[0.6, 0.8]]])
    v = np.array([[[1, 2]], [[4, 0]], [[0, 0]]], dtype=float)
    beta = np.array([[0.5], [1.0], [0.5]])
    g = np.array([[0.0], [math.log(0.5)], [0.0]])
    o_exp = np.array([[[0.5, 1]], [[4.25, 0.5]], [[2.66, -0.12]]])
    S_exp = np.array([[[[-0.755, 2.66], [0.41, -0.12]]]])
    for fn in (ref.sequential, ref.unrolled, ref.chunked):
        o, S = fn(q, k, v, g, beta)
        assert np.allclose(o, o_exp, atol=1e-13), fn.__name__
        assert np.allclose(S, S_exp, atol=1e-13), fn.__name__
    o, S = _c_prefill(q, k, v, g, beta)
    # fp32 storage of 0.6, 0.8 and log(1/2) perturbs the values by ~1e-8
    assert np.allclose(o, o_exp, atol=1e-6) and np.allclose(S, S_exp, atol=1e-6)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
@pytest.mark.parametrize("route", ["c", "sequential", "chunked", "unrolled"])
def test_beta_zero_is_pure_decay(route):
    """beta = 0: S_t = e^{G_t} S_0 and o_t = e^{G_t} S_0 q_t (G = cumulative g)."""
    rng = np.random.default_rng(1)
    T = 9 if route == "unrolled" else 150
    q, k, v, g, beta, s0 = _rand(rng, T, 2, 2, 8, 6, nseq_init=1)
    beta = np.zeros_like(beta)
    if route == "c":
        q, k, v, g, beta, s0 = [x.astype(np.float64) for x in _f32(q, k, v, g, beta, s0)]
        o, S = c_oracle.prefill(*_f32(q, k, v, g, beta, s0))
    else:
        kw = dict(chunk=16) if route == "chunked" else {}
        o, S = getattr(ref, route)(q, k, v, g, beta, s0, **kw)
    G = np.cumsum(g, axis=0)                                   # [T, H]
    o_exp = np.exp(G)[:, :, None] * np.einsum("hij,thj->thi", s0[0], q)
    S_exp = np.exp(G[-1])[None, :, None, None] * s0
    assert _rel(o, o_exp) < 1e-12 and _rel(S, S_exp) < 1e-12


@pytest.mark.parametrize("route", ["c", "sequential", "chunked"])
def test_exact_recall_with_orthonormal_keys(route):
    """alpha = beta = 1, orthonormal keys: S k_i = v_i for every key written.

    With q_t = k_t the output equals the value just written; after d_k keys
    (a full basis) S = sum_i v_i k_i^T whatever S_0 was.  Hadamard rows are
    exactly representable, so this holds to rounding for every route.
    """
    dk = dv = 16
    H = _hadamard(dk)
    rng = np.random.default_rng(2)
    perm = rng.permutation(dk)
    T = dk
    k = H[perm][:, None, :]                 # [T, 1, dk]
    q = k.copy()
    v = np.round(rng.standard_normal((T, 1, dv)) * 64) / 64
    g = np.zeros((T, 1))
    beta = np.ones((T, 1))
    s0 = np.round(rng.standard_normal((1, 1, dv, dk)) * 64) / 64
    if route == "c":
        o, S = _c_prefill(q, k, v, g, beta, s0)
    else:
        o, S = getattr(ref, route)(q, k, v, g, beta, s0, **({"chunk": 7} if route == "chunked" else {}))
    assert _rel(o, v) < 1e-12
    S_exp = np.einsum("ti,tj->ij", v[:, 0], k[:, 0])
    assert _rel(S[0, 0], S_exp) < 1e-12
    # recall of every key written so far, part way through
    o8, S8 = ref.sequential(q[:8], k[:8], v[:8], g[:8], beta[:8], s0)
    assert _rel(S8[0, 0] @ k[:8, 0].T, v[:8, 0].T) < 1e-12


@pytest.mark.parametrize("route", ["c", "sequential", "chunked"])
def test_read_only_path(route):
    """g = 0, beta = 0: the state never changes and o_t = S_0 q_t."""
    rng = np.random.default_rng(3)
    q, k, v, g, beta, s0 = _rand(rng, 70, 1, 1, 8, 8, nseq_init=1)
    g = np.zeros_like(g)
    beta = np.zeros_like(beta)
    if route == "c":
        q, k, v, g, beta, s0 = [x.astype(np.float64) for x in _f32(q, k, v, g, beta, s0)]
        o, S = c_oracle.prefill(*_f32(q, k, v, g, beta, s0))
    else:
        o, S = getattr(ref, route)(q, k, v, g, beta, s0)
    assert _rel(o[:, 0], q[:, 0] @ s0[0, 0].T) < 1e-13
    assert _rel(S, s0) == 0.0


@pytest.mark.parametrize("route", ["c", "sequential", "chunked"])
def test_scalar_case_is_first_order_linear_recurrence(route):
    """d_k = d_v = 1: s_t = a_t s_{t-1} + b_t with a_t = alpha_t (1 - beta_t k_t^2),
    b_t = beta_t v_t k_t; solution s_T = s_0 prod a + sum_t b_t prod_{j>t} a_j."""
    rng = np.random.default_rng(4)
    T = 40
    q = rng.uniform(-1, 1, (T, 1, 1))
    k = rng.uniform(-1, 1, (T, 1, 1))
    v = rng.standard_normal((T, 1, 1))
    beta = rng.uniform(0, 1, (T, 1))
    g = -rng.uniform(0, 1, (T, 1))
    s0 = np.array([[[[0.7]]]])
    if route == "c":
        q, k, v, g, beta, s0 = [x.astype(np.float64) for x in _f32(q, k, v, g, beta, s0)]
        o, S = c_oracle.prefill(*_f32(q, k, v, g, beta, s0))
    else:
        o, S = getattr(ref, route)(q, k, v, g, beta, s0, **({"chunk": 16} if route == "chunked" else {}))
    a = np.exp(g[:, 0]) * (1 - beta[:, 0] * k[:, 0, 0] ** 2)
    b = beta[:, 0] * v[:, 0, 0] * k[:, 0, 0]
    s_exp = np.empty(T)
    for t in range(T):
        tail = np.array([np.prod(a[j + 1:t + 1]) for j in range(t + 1)])
        s_exp[t] = s0[0, 0, 0, 0] * np.prod(a[:t + 1]) + np.sum(b[:t + 1] * tail)
    assert _rel(S[0, 0, 0, 0], s_exp[-1]) < 1e-12
    assert _rel(o[:, 0, 0], s_exp * q[:, 0, 0]) < 1e-12


def test_householder_preserves_frobenius_norm():
    """beta = 2, alpha = 1, v = 0, unit k: S <- S (I - 2 k k^T) is orthogonal."""
    dk = 16
    H = _hadamard(dk)
    rng = np.random.default_rng(5)
    idx = rng.integers(0, dk, 40)
    k = H[idx][:, None, :]
    q = k.copy()
    v = np.zeros((40, 1, 8))
    s0 = np.round(rng.standard_normal((1, 1, 8, dk)) * 64) / 64
    g = np.zeros((40, 1))
    beta = 2 * np.ones((40, 1))
    for o, S in (ref.sequential(q, k, v, g, beta, s0), _c_prefill(q, k, v, g, beta, s0)):
        assert abs(np.linalg.norm(S) / np.linalg.norm(s0) - 1) < 1e-12


def test_contraction_spectral_norm_nonincreasing():
    """beta in (0, 1], alpha <= 1, v = 0: every step maps S to S A_t with ||A_t||_2 <= 1."""
    rng = np.random.default_rng(6)
    q, k, v, g, beta, s0 = _rand(rng, 60, 1, 1, 8, 8, nseq_init=1)
    v = np.zeros_like(v)
    norms = [np.linalg.norm(s0[0, 0], 2)]
    for t in range(60):
        _, S = ref.sequential(q[:t + 1], k[:t + 1], v[:t + 1], g[:t + 1], beta[:t + 1], s0)
        norms.append(np.linalg.norm(S[0, 0], 2))
    assert all(b <= a * (1 + 1e-12) for a, b in zip(norms, norms[1:]))


def test_transition_of_a_contracting_range_is_bounded_by_its_decay():
    """The bound a part summary's decay horizon rests on: when every token has g_t <= 0 and
    0 <= beta_t |k_t|^2 <= 2, the map of a token range, M (the state reached from the identity with
    v = 0), has spectral norm <= prod alpha_t = exp(sum g_t).  beta up to 1.99 / |k|^2 is included.
    One token with beta |k|^2 = 2.5 (and alpha = 1) breaks it: I - 2.5 k k^T has norm 1.5."""
    rng = np.random.default_rng(16)
    dk = 8
    for trial in range(4):
        q, k, v, g, beta, _ = _rand(rng, 50, 1, 1, dk, dk)
        beta = rng.uniform(0.0, 1.99, size=beta.shape)          # |k| = 1: beta |k|^2 in [0, 1.99]
        g = g * rng.uniform(0.0, 0.2)                           # mild decay: the bound stays far above 0
        eye = np.eye(dk)[None, None]
        _, M = ref.sequential(q, k, np.zeros_like(v), g, beta, eye)
        bound = math.exp(float(g.sum()))
        assert np.linalg.norm(M[0, 0], 2) <= bound * (1 + 1e-12)
    k1 = np.zeros((1, 1, dk))
    k1[0, 0, 0] = 1.0
    _, M1 = ref.sequential(k1, k1, np.zeros((1, 1, dk)), np.zeros((1, 1)), np.full((1, 1), 2.5), np.eye(dk)[None, None])
    assert abs(np.linalg.norm(M1[0, 0], 2) - 1.5) < 1e-12


# --------------------------------------------------------------------------
# structure: linearity, row independence, boundaries
# --------------------------------------------------------------------------
def test_joint_linearity_in_values_and_initial_state():
    rng = np.random.default_rng(7)
    q, k, v1, g, beta, s1 = _rand(rng, 90, 1, 1, 8, 8, nseq_init=1)
    # entries on a 1/64 grid keep v1 + 2 v2 exact in fp32 storage
    v1 = np.round(v1 * 64) / 64
    v2 = np.round(rng.standard_normal(v1.shape) * 64) / 64
    s1 = np.round(s1 * 64) / 64
    s2 = np.round(0.1 * rng.standard_normal(s1.shape) * 64) / 64
    for run in (lambda vv, ss: ref.sequential(q, k, vv, g, beta, ss),
                lambda vv, ss: _c_prefill(q, k, vv, g, beta, ss)):
        o1, f1 = run(v1, s1)
        o2, f2 = run(v2, s2)
        o3, f3 = run(v1 + 2 * v2, s1 + 2 * s2)
        assert _rel(o3, o1 + 2 * o2) < 1e-12 and _rel(f3, f1 + 2 * f2) < 1e-12


def test_value_rows_are_independent():
    """Permuting / slicing d_v permutes / slices outputs and state rows bit for bit."""
    rng = np.random.default_rng(8)
    q, k, v, g, beta, s0 = _rand(rng, 80, 2, 2, 16, 12, nseq_init=1)
    o, S = _c_prefill(q, k, v, g, beta, s0)
    perm = rng.permutation(12)
    op, Sp = _c_prefill(q, k, v[:, :, perm], g, beta, s0[:, :, perm])
    assert np.array_equal(op, o[:, :, perm]) and np.array_equal(Sp, S[:, :, perm])
    os_, Ss = _c_prefill(q, k, v[:, :, 4:8], g, beta, s0[:, :, 4:8])
    assert np.array_equal(os_, o[:, :, 4:8]) and np.array_equal(Ss, S[:, :, 4:8])


def test_split_with_state_handoff_equals_unsplit():
    rng = np.random.default_rng(9)
    q, k, v, g, beta, s0 = _rand(rng, 130, 2, 2, 8, 8, nseq_init=1)
    o, S = ref.sequential(q, k, v, g, beta, s0)
    for cut in (1, 64, 77):
        oa, Sa = ref.sequential(q[:cut], k[:cut], v[:cut], g[:cut], beta[:cut], s0)
        ob, Sb = ref.sequential(q[cut:], k[cut:], v[cut:], g[cut:], beta[cut:], Sa)
        assert _rel(np.concatenate([oa, ob]), o) < 1e-13 and _rel(Sb, S) < 1e-13


def test_prefill_equals_repeated_decode_steps():
    rng = np.random.default_rng(10)
    q, k, v, g, beta, s0 = [None if x is None else x for x in _f32(*_rand(rng, 20, 2, 4, 16, 8, nseq_init=1))]
    o, S = c_oracle.prefill(q, k, v, g, beta, s0)
    state = s0.astype(np.float64).copy()
    for t in range(20):
        ot = c_oracle.decode_step(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1],
                                  beta[t:t + 1], state)
        assert np.array_equal(ot, o[t:t + 1])
    assert np.array_equal(state, S)
    # the numpy decode step agrees with the numpy sequential form
    st = s0.astype(np.float64)
    q64, k64, v64, g64, b64 = [x.astype(np.float64) for x in (q, k, v, g, beta)]
    for t in range(20):
        ot, st = ref.decode_step(q64[t:t + 1], k64[t:t + 1], v64[t:t + 1], g64[t:t + 1], b64[t:t + 1], st)
        assert _rel(ot, o[t:t + 1]) < 1e-12
    assert _rel(st, S) < 1e-12


def test_packed_sequences_equal_separate_runs():
    rng = np.random.default_rng(11)
    lens = [70, 1, 64, 129, 0, 5]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    q, k, v, g, beta, s0 = [x.astype(np.float64) for x in
                            _f32(*_rand(rng, T, 2, 4, 8, 8, nseq_init=len(lens)))]
    o, S = _c_prefill(q, k, v, g, beta, s0, cu)
    oc, Sc = ref.chunked(q, k, v, g, beta, s0, cu, chunk=64)
    assert _rel(o, oc) < 1e-12 and _rel(S, Sc) < 1e-12
    for n, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        on, Sn = _c_prefill(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], s0[n:n + 1])
        assert np.array_equal(on, o[a:b]) and np.array_equal(Sn[0], S[n])
    # an empty sequence hands its initial state through unchanged
    assert np.array_equal(S[4], s0[4].astype(np.float32).astype(np.float64))


def test_grouped_value_heads_equal_repeated_qk_heads():
    """Hv = 2 Hqk: value heads 2i and 2i+1 read q/k head i."""
    rng = np.random.default_rng(12)
    q, k, v, g, beta, s0 = _rand(rng, 50, 3, 6, 8, 8, nseq_init=1)
    o, S = _c_prefill(q, k, v, g, beta, s0)
    qr, kr = np.repeat(q, 2, axis=1), np.repeat(k, 2, axis=1)
    o2, S2 = _c_prefill(qr, kr, v, g, beta, s0)
    assert np.array_equal(o, o2) and np.array_equal(S, S2)
    o3, S3 = ref.sequential(q, k, v, g, beta, s0)
    assert _rel(o3, o) < 1e-6  # fp32 storage of the inputs on the C side


# --------------------------------------------------------------------------
# independent routes agree
# --------------------------------------------------------------------------
@pytest.mark.parametrize("chunk", [64, 16, 5])
def test_chunked_form_equals_sequential(chunk):
    rng = np.random.default_rng(13)
    lens = [200, 64, 1, 90]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta, s0 = _rand(rng, int(cu[-1]), 2, 4, 16, 12, nseq_init=4)
    o, S = ref.sequential(q, k, v, g, beta, s0, cu)
    oc, Sc = ref.chunked(q, k, v, g, beta, s0, cu, chunk=chunk)
    assert _rel(oc, o) < RTOL and _rel(Sc, S) < RTOL


def test_unrolled_closed_form_equals_sequential():
    rng = np.random.default_rng(14)
    q, k, v, g, beta, s0 = _rand(rng, 7, 1, 2, 5, 4, nseq_init=1)
    o, S = ref.sequential(q, k, v, g, beta, s0)
    ou, Su = ref.unrolled(q, k, v, g, beta, s0)
    assert _rel(ou, o) < RTOL and _rel(Su, S) < RTOL


def test_c_oracle_equals_numpy_literal_form():
    rng = np.random.default_rng(15)
    q, k, v, g, beta, s0 = [x for x in _f32(*_rand(rng, 150, 2, 2, 32, 16, nseq_init=1))]
    o, S = c_oracle.prefill(q, k, v, g, beta, s0)
    o2, S2 = ref.sequential(*[x.astype(np.float64) for x in (q, k, v, g, beta, s0)])
    assert _rel(o, o2) < RTOL and _rel(S, S2) < RTOL


def test_c_oracle_threads_do_not_change_results():
    rng = np.random.default_rng(16)
    q, k, v, g, beta, s0 = _f32(*_rand(rng, 100, 2, 4, 16, 16, nseq_init=1))
    a = c_oracle.prefill(q, k, v, g, beta, s0, nthreads=1)
    b = c_oracle.prefill(q, k, v, g, beta, s0, nthreads=4)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_state_size_is_independent_of_length():
    """The pages' fixed-size state: the final state has the same shape for any T."""
    rng = np.random.default_rng(17)
    shapes = set()
    for T in (1, 10, 300):
        q, k, v, g, beta, _ = _rand(rng, T, 1, 1, 8, 4)
        shapes.add(_c_prefill(q, k, v, g, beta)[1].shape)
    assert shapes == {(1, 1, 4, 8)}


# --------------------------------------------------------------------------
# Multi-token decode: T decode steps per sequence.  Pinned against two other
# routes: the literal matrix-form recurrence over packed sequences of T
# tokens, and (per-token states) that recurrence cut after t + 1 tokens.
def test_decode_tokens_equals_packed_sequential_and_truncations():
    rng = np.random.default_rng(41)
    N, T, hqk, hv, dk, dv = 3, 5, 1, 2, 4, 3
    q, k, v, g, beta, s0 = _rand(rng, N * T, hqk, hv, dk, dv, nseq_init=N)
    out, states, fin = ref.decode_tokens(q, k, v, g, beta, s0, T)
    cu = np.arange(0, N * T + 1, T)
    so, sf = ref.sequential(q, k, v, g, beta, s0, cu)
    assert _rel(out, so) <= RTOL and _rel(fin, sf) <= RTOL
    assert _rel(states[:, -1], sf) <= RTOL
    for t in range(T):
        rows = np.concatenate([np.arange(n * T, n * T + t + 1) for n in range(N)])
        cut = np.arange(0, N * (t + 1) + 1, t + 1)
        _, ft = ref.sequential(q[rows], k[rows], v[rows], g[rows], beta[rows], s0, cut)
        assert _rel(states[:, t], ft) <= RTOL, t


def test_c_decode_tokens_equals_c_prefill_and_numpy():
    rng = np.random.default_rng(42)
    N, T, hqk, hv, dk, dv = 4, 3, 2, 4, 8, 6
    q, k, v, g, beta, s0 = _rand(rng, N * T, hqk, hv, dk, dv, nseq_init=N)
    q, k, v, g, beta, s0 = _f32(q, k, v, g, beta, s0)
    out, states, fin = c_oracle.decode_tokens(q, k, v, g, beta, s0, T)
    po, pf = c_oracle.prefill(q, k, v, g, beta, s0, np.arange(0, N * T + 1, T))
    assert _rel(out, po) <= RTOL and _rel(fin, pf) <= RTOL
    ro, rs, rf = ref.decode_tokens(*(x.astype(np.float64) for x in (q, k, v, g, beta, s0)), T)
    assert _rel(out, ro) <= RTOL and _rel(states, rs) <= RTOL and _rel(fin, rf) <= RTOL


# --------------------------------------------------------------------------
# Raw-projection prologue (q, k L2-normalised, g = -softplus(a), beta = sigmoid(b)).
def _raw_inputs(rng, T, hqk, hv, dk, dv):
    q = 3.0 * rng.standard_normal((T, hqk, dk))
    k = 0.7 * rng.standard_normal((T, hqk, dk))
    v = rng.standard_normal((T, hv, dv))
    a = rng.standard_normal((T, hv))
    b = rng.standard_normal((T, hv))
    return _f32(q, k, v, a, b)


def test_raw_prologue_is_invariant_to_the_scale_of_q_and_k():
    rng = np.random.default_rng(60)
    q, k, v, a, b = _raw_inputs(rng, 40, 1, 2, 8, 4)
    o1, f1 = c_oracle.prefill(q, k, v, a, b, raw=True)
    o2, f2 = c_oracle.prefill((q * 0.25).astype(np.float32), (k * 4.0).astype(np.float32), v, a, b, raw=True)
    assert _rel(o2, o1) <= 1e-6 and _rel(f2, f1) <= 1e-6


def test_raw_prologue_at_zero_logits_is_half_decay_and_half_write():
    """a = b = 0: alpha = exp(-ln 2) = 1/2 and beta = 1/2 exactly; unit-norm q, k stay unit up to the
    1e-6 guard, so the result is the plain recurrence with g = -ln 2, beta = 1/2."""
    rng = np.random.default_rng(61)
    q, k, v, g, beta, _ = _rand(rng, 30, 1, 2, 8, 4)
    q, k, v = _f32(q, k, v)
    z = np.zeros((30, 2), dtype=np.float32)
    o1, f1 = c_oracle.prefill(q, k, v, z, z, raw=True)
    o2, f2 = ref.sequential(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                            np.full((30, 2), -math.log(2.0)), np.full((30, 2), 0.5))
    assert _rel(o1, o2) <= 1e-5 and _rel(f1, f2) <= 1e-5


def test_raw_prologue_saturated_logits_give_no_decay_and_full_write():
    """a -> -inf gives alpha -> 1, b -> +inf gives beta -> 1."""
    rng = np.random.default_rng(62)
    q, k, v, _, _, _ = _rand(rng, 20, 1, 1, 8, 3)
    q, k, v = _f32(q, k, v)
    a = np.full((20, 1), -60.0, dtype=np.float32)
    b = np.full((20, 1), 60.0, dtype=np.float32)
    o1, f1 = c_oracle.prefill(q, k, v, a, b, raw=True)
    o2, f2 = ref.sequential(q.astype(np.float64), k.astype(np.float64), v.astype(np.float64),
                            np.zeros((20, 1)), np.ones((20, 1)))
    assert _rel(o1, o2) <= 1e-5 and _rel(f1, f2) <= 1e-5


def test_raw_prologue_guard_halves_rows_of_squared_norm_1e6():
    """Rows with |x|^2 = 1e-6 meet the 1e-6 guard: x / sqrt(|x|^2 + 1e-6) = x_hat / sqrt(2).  With zero
    logits (alpha = beta = 1/2) the raw path must equal the plain recurrence on q_hat / sqrt(2) and
    k_hat / sqrt(2); a guard of any other size (or none) gives a different row scale."""
    rng = np.random.default_rng(64)
    T, H, dk, dv = 24, 2, 8, 5
    qh = rng.standard_normal((T, 1, dk))
    kh = rng.standard_normal((T, 1, dk))
    qh /= np.linalg.norm(qh, axis=-1, keepdims=True)
    kh /= np.linalg.norm(kh, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv)).astype(np.float32)
    q32, k32 = (1e-3 * qh).astype(np.float32), (1e-3 * kh).astype(np.float32)
    z = np.zeros((T, H), dtype=np.float32)
    o1, f1 = c_oracle.prefill(q32, k32, v, z, z, raw=True)
    q64, k64 = q32.astype(np.float64), k32.astype(np.float64)
    qs = q64 / np.linalg.norm(q64, axis=-1, keepdims=True) / math.sqrt(2.0)
    ks = k64 / np.linalg.norm(k64, axis=-1, keepdims=True) / math.sqrt(2.0)
    o2, f2 = ref.sequential(qs, ks, v.astype(np.float64), np.full((T, H), -math.log(2.0)), np.full((T, H), 0.5))
    assert _rel(o1, o2) <= 1e-6 and _rel(f1, f2) <= 1e-6
    # and the guard is what makes the difference: unit rows would give sqrt(2) larger outputs
    o3, _ = ref.sequential(qs * math.sqrt(2.0), ks * math.sqrt(2.0), v.astype(np.float64),
                           np.full((T, H), -math.log(2.0)), np.full((T, H), 0.5))
    assert _rel(o1, o3) > 0.1


def test_raw_decode_tokens_equals_raw_prefill():
    rng = np.random.default_rng(63)
    N, T = 3, 4
    q, k, v, a, b = _raw_inputs(rng, N * T, 2, 4, 8, 6)
    s0 = (0.1 * rng.standard_normal((N, 4, 6, 8))).astype(np.float32)
    o1, _, f1 = c_oracle.decode_tokens(q, k, v, a, b, s0, T, raw=True)
    o2, f2 = c_oracle.prefill(q, k, v, a, b, s0, np.arange(0, N * T + 1, T), raw=True)
    assert _rel(o1, o2) <= RTOL and _rel(f1, f2) <= RTOL
