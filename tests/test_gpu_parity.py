"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Tolerances: max|gpu - ref| / max|ref| <= 1e-5 on the fp32 path and <= 1e-2
on the bf16 path, for outputs and final states separately.  Inputs are the
seeded synthetic workloads (gated_deltanet_linear_rule_amd.inputs); the
oracle sees exactly the stored values the GPU reads.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_rule_amd import binding as B
from gated_deltanet_linear_rule_amd import inputs as gi
from oracle import c_oracle
from tests.gpu_util import (TOL, check_prefill, dev, host64, oracle_affine, oracle_prefill, oracle_snapshots,
                            rel_err, run_prefill, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()   # fails loudly if the HIP library is missing


# ---------------------------------------------------------------- small shapes
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128), (128, 64)])
def test_single_chunk_shapes(dtype, dk, dv):
    inp = gi.make_inputs(gi.custom(dtype=dtype, Hqk=2, Hv=2, dk=dk, dv=dv, seqlens=(64,)), seed=1)
    check_prefill(inp, label=f"one chunk {dtype} dk={dk} dv={dv}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("lens", [(1,), (63,), (65,), (200,), (64, 1, 127, 0, 5), (0, 0), (300, 64)])
def test_ragged_packed_lengths(dtype, lens):
    inp = gi.make_inputs(gi.custom(dtype=dtype, Hqk=2, Hv=4, dk=64, dv=64, seqlens=lens,
                                   init_state="normal"), seed=2)
    check_prefill(inp, label=f"ragged {dtype} {lens}")


@pytest.mark.parametrize("ratio", [1, 2, 4])
def test_grouped_value_heads(ratio):
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=2, Hv=2 * ratio, dk=128, dv=128, seqlens=(150, 77),
                                   init_state="normal"), seed=3)
    check_prefill(inp, label=f"GVA 1:{ratio}")


def test_equal_length_batch_without_offsets():
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=2, Hv=2, dk=128, dv=128, seqlens=(96, 96, 96),
                                   init_state="normal"), seed=4)
    cu = inp.cu_seqlens
    inp.cu_seqlens = None            # equal lengths: the library derives the offsets
    out, fin = run_prefill(inp, num_seqs=3)
    inp.cu_seqlens = cu
    ro, rf = c_oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state, cu)
    assert rel_err(out, ro) <= 1e-2 and rel_err(fin, rf) <= 1e-2


def test_zero_initial_state_null_equals_zeros():
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=2, Hv=2, dk=128, dv=128, seqlens=(130,)), seed=5)
    a = run_prefill(inp, init_mode="null")
    b = run_prefill(inp, init_mode="zeros")
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    check_prefill(inp, init_mode="null", label="NULL init")


def test_init_state_may_alias_final_state():
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=2, Hv=4, dk=128, dv=128, seqlens=(100, 40),
                                   init_state="normal"), seed=6)
    a = run_prefill(inp)
    b = run_prefill(inp, out_alias=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_split_with_state_handoff_matches_unsplit():
    inp = gi.make_inputs(gi.custom(dtype="f32", Hqk=2, Hv=2, dk=64, dv=64, seqlens=(300,),
                                   init_state="normal"), seed=7)
    full_o, full_s = run_prefill(inp)
    for cut in (1, 64, 100):
        a = gi.Inputs(gi.custom(dtype="f32", Hqk=2, Hv=2, dk=64, dv=64, seqlens=(cut,)))
        a.q, a.k, a.v, a.g, a.beta, a.init_state = inp.q[:cut], inp.k[:cut], inp.v[:cut], inp.g[:cut], inp.beta[:cut], inp.init_state
        oa, sa = run_prefill(a)
        b = gi.Inputs(gi.custom(dtype="f32", Hqk=2, Hv=2, dk=64, dv=64, seqlens=(300 - cut,)))
        b.q, b.k, b.v, b.g, b.beta = inp.q[cut:], inp.k[cut:], inp.v[cut:], inp.g[cut:], inp.beta[cut:]
        b.init_state = sa.astype(np.float32)
        ob, sb = run_prefill(b)
        assert rel_err(np.concatenate([oa, ob]), full_o) < 1e-5 and rel_err(sb, full_s) < 1e-5


def test_results_are_bitwise_deterministic():
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=4, Hv=8, dk=128, dv=128, seqlens=(500, 300),
                                   init_state="normal"), seed=8)
    a = run_prefill(inp)
    b = run_prefill(inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_multi_part_results_are_bitwise_deterministic():
    """A 40000-token sequence cut into parts (summary, link and rerun kernels), twice in one process:
    outputs, final states and the affine map are bit-identical."""
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=2, Hv=2, dk=128, dv=128, seqlens=(40000,),
                                   init_state="normal"), seed=21)
    q, k, v, g, beta, s0 = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state))
    runs = [B.gdn_prefill(q, k, v, g, beta, s0) for _ in range(2)]
    maps = [B.gdn_prefill_affine(k, v, g, beta) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])
    assert torch.equal(maps[0][0], maps[1][0]) and torch.equal(maps[0][1], maps[1][1])


def test_long_decay_free_stretch_stays_accurate():
    """g = 0 and small beta: no decay hides accumulated error across many chunks."""
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=1, Hv=1, dk=128, dv=128, seqlens=(2048,)), seed=9)
    inp.g = np.zeros_like(inp.g)
    inp.beta = (inp.beta * 0.1).astype(np.float32)
    check_prefill(inp, label="g=0, beta/10")


# ------------------------------------------------------- sequences cut into parts
# With fewer (sequence, head) chains than compute units, long sequences are cut
# into parts of L chunks (at least 6): every part but the last is summarised
# (transition and offset), the link composes the start states, and every part
# reruns from its true start state.
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_parts_long_sequence(dtype):
    """One 40000-token sequence (625 chunks: 105 parts of 6 on 256 compute units, the last partial), given
    initial state."""
    inp = gi.make_inputs(gi.custom(dtype=dtype, Hqk=2, Hv=2, dk=128, dv=128, seqlens=(40000,),
                                   init_state="normal"), seed=21)
    check_prefill(inp, label=f"parts 40000 {dtype}")


def test_parts_unequal_packed_sequences():
    """Two packed sequences of 33000 and 40000 tokens (516 and 625 chunks): different part counts
    per sequence, a partial last part and a partial last chunk in each."""
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=1, Hv=2, dk=128, dv=64, seqlens=(33000, 40000),
                                   init_state="normal"), seed=22)
    check_prefill(inp, label="parts 33000+40000")


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64)])
def test_parts_decay_free_f32(dk, dv):
    """g = 0 over 64 chunks cut into 8 parts: no decay hides an error in the composed transitions
    (fp32 path, 1e-5)."""
    inp = gi.make_inputs(gi.custom(dtype="f32", Hqk=1, Hv=1, dk=dk, dv=dv, seqlens=(4096,),
                                   init_state="normal"), seed=24)
    inp.g = np.zeros_like(inp.g)
    inp.beta = (inp.beta * 0.25).astype(np.float32)
    check_prefill(inp, label=f"parts g=0 f32 dk={dk} dv={dv}")


def test_parts_equal_length_batch_without_offsets_in_place_state():
    """Two 36864-token sequences without offsets, initial state updated in place."""
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=2, Hv=2, dk=64, dv=128, seqlens=(36864, 36864),
                                   init_state="normal"), seed=23)
    cu = inp.cu_seqlens
    inp.cu_seqlens = None            # equal lengths: the library derives the offsets
    out, fin = run_prefill(inp, out_alias=True, num_seqs=2)
    inp.cu_seqlens = cu
    ro, rf = c_oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state, cu)
    eo, ef = rel_err(out, ro), rel_err(fin, rf)
    say(f"[parity] parts 2x36864 no offsets, in place: out {eo:.3e} final {ef:.3e}")
    assert eo <= 1e-2 and ef <= 1e-2


# ------------------------------------------- the balanced schedule (packed bf16)
# With between one and two (sequence, value head) chains per compute unit on
# packed bf16 input (d_k = d_v), a sequence of more than one share of chunks
# (share = chunk steps per compute unit) keeps a first part of about one share
# and is cut into parts of 0.2 shares (at least 6 chunks) after it.  The first
# parts run from init_state in the launch that also summarises the later
# parts; their end states seed the link, and a second launch runs the later
# parts.
def _balanced_batch(seed, dk=128, raw=False):
    """16 value heads and num_seqs x 16 = compute units: one 15000-token sequence and shorter ones,
    empty and one-token ones among them.  At 256 compute units: share 34.75 chunks, parts of 6, first
    parts of 30 chunks (5 slots); the long sequence has 35 later parts (34 link steps), the 3000- and
    2900-token ones three (two steps), the 2600- and 2500-token ones two (one step)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    hv = 16
    n = max(2, cus // hv)
    tail = [1700, 3000, 0, 2600, 64, 1, 1700, 900, 2000, 130, 2900, 1200, 65, 1800, 2500]
    lens = ([15000] + tail * ((n - 1) // len(tail) + 1))[:n]
    return gi.make_inputs(gi.custom(dtype="bf16", Hqk=hv // 2, Hv=hv, dk=dk, dv=dk, seqlens=lens,
                                    init_state="normal", raw=raw), seed=seed)


@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("decay", [True, False])
def test_balanced_schedule_packed_batch(dk, decay):
    """Decay-free with small beta, the later parts' outputs depend on the linked start states."""
    inp = _balanced_batch(80 + dk, dk=dk)
    if not decay:
        inp.g = np.zeros_like(inp.g)
        inp.beta = (inp.beta * 0.1).astype(np.float32)
    check_prefill(inp, label=f"balanced dk={dk} decay={decay}")


def test_balanced_schedule_in_place_state():
    """init_state and final_state are one buffer: the first parts read it in the first launch, the
    last parts write it in the second."""
    inp = _balanced_batch(82)
    check_prefill(inp, label="balanced in place", out_alias=True)


def test_balanced_schedule_raw_projections():
    inp = _balanced_batch(83, raw=True)
    _check_raw_prefill(inp, TOL["bf16"], "balanced raw")


@pytest.mark.parametrize("i", range(6))
def test_balanced_schedule_seeded_batches(i):
    """Seeded packed batches with one to two (sequence, value head) chains per compute unit: mostly
    short sequences (some empty or one token), one to three long ones, d = 64 or 128, grouped value
    heads, with initial state; every cut falls where the lengths put it."""
    rng = np.random.default_rng(900 + i)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    hv = int(rng.choice([16, 32]))
    hqk = hv // int(rng.choice([1, 2]))
    dk = int(rng.choice([64, 128]))
    n = int(rng.integers(cus // hv, 2 * cus // hv + 1))
    lens = [int(x) for x in rng.integers(0, 1500, size=n)]
    lens[int(rng.integers(0, n))] = int(rng.integers(0, 2))
    for j in rng.choice(n, size=int(rng.integers(1, 4)), replace=False):
        lens[int(j)] = int(rng.integers(4000, 12000))
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=hqk, Hv=hv, dk=dk, dv=dk, seqlens=lens,
                                   init_state="normal"), seed=910 + i)
    check_prefill(inp, label=f"balanced seeded {i}: N={n} Hv={hv} Hqk={hqk} d={dk} longest {max(lens)}")


def test_balanced_schedule_bitwise_deterministic():
    inp = _balanced_batch(84)
    a = run_prefill(inp)
    b = run_prefill(inp)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------- the workloads
def test_tiny_f32_workload():
    """T=256, H=2, d=64, fp32 throughout, zero initial state, seed 0."""
    check_prefill(gi.make_inputs("tiny_f32", seed=0))


def test_prefill_4k_workload():
    """T=4096, H=16, d=128, bf16, zero initial state."""
    check_prefill(gi.make_inputs("prefill_4k", seed=0))


def test_varlen_packed_workload():
    """8 packed sequences (lengths U[1024,16384] from the seed), 32 v-heads on 16 q/k heads."""
    inp = gi.make_inputs("varlen_8x", seed=0)
    say(f"[parity] varlen lengths {inp.wl.seqlens}")
    check_prefill(inp)


def test_prefill_256k_workload_all_heads():
    """T=262144, H=16, d=128: the full call, every head against the oracle (four heads per oracle call
    so that the fp64 reference stays bounded in memory)."""
    inp = gi.make_inputs("prefill_256k", seed=0)
    q, k, v, g, beta = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    out, fin = B.gdn_prefill(q, k, v, g, beta)
    torch.cuda.synchronize()
    del q, k, v, g, beta
    worst_o, worst_f = 0.0, 0.0
    for h0 in range(0, 16, 4):
        hs = list(range(h0, h0 + 4))
        ro, rf = c_oracle.prefill(inp.q[:, hs], inp.k[:, hs], inp.v[:, hs], inp.g[:, hs], inp.beta[:, hs], None, None)
        for j, h in enumerate(hs):
            oh = host64(out[:, h])
            assert np.all(np.isfinite(oh))
            eo, ef = rel_err(oh, ro[:, j]), rel_err(host64(fin[:, h]), rf[:, j])
            say(f"[parity] prefill_256k head {h}: out {eo:.3e} final {ef:.3e}")
            worst_o, worst_f = max(worst_o, eo), max(worst_f, ef)
        del ro, rf
    # the metric over the whole tensor: max|err| over all heads / max|ref| over all heads is at most the
    # worst per-head ratio, so the per-head bound implies it
    say(f"[parity] prefill_256k all 16 heads: worst out {worst_o:.3e} final {worst_f:.3e}")
    assert worst_o <= 1e-2 and worst_f <= 1e-2


# ------------------------------------------------------------------- decode
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64)])
def test_decode_small(dtype, dk, dv):
    wl = gi.custom(dtype=dtype, Hqk=2, Hv=4, dk=dk, dv=dv, seqlens=(1,) * 5, init_state="normal",
                   decode_steps=6)
    inp = gi.make_inputs(wl, seed=10)
    state = dev(inp.init_state)
    ref = inp.init_state.astype(np.float64)
    worst = 0.0
    for st in inp.steps:
        out = B.gdn_decode_step(dev(st["q"]), dev(st["k"]), dev(st["v"]), dev(st["g"]), dev(st["beta"]), state)
        ro = c_oracle.decode_step(st["q"], st["k"], st["v"], st["g"], st["beta"], ref)
        worst = max(worst, rel_err(host64(out), ro))
    es = rel_err(host64(state), ref)
    say(f"[parity] decode {dtype} dk={dk} dv={dv}: out {worst:.3e} state {es:.3e}")
    assert worst <= TOL[dtype] and es <= TOL[dtype]


def test_decode_equals_prefill_token_by_token():
    inp = gi.make_inputs(gi.custom(dtype="f32", Hqk=2, Hv=2, dk=64, dv=64, seqlens=(20,),
                                   init_state="normal"), seed=11)
    po, ps = run_prefill(inp)
    state = dev(inp.init_state)
    for t in range(20):
        out = B.gdn_decode_step(dev(inp.q[t:t + 1]), dev(inp.k[t:t + 1]), dev(inp.v[t:t + 1]),
                                dev(inp.g[t:t + 1]), dev(inp.beta[t:t + 1]), state)
        assert rel_err(host64(out), po[t:t + 1]) < 1e-5
    assert rel_err(host64(state), ps) < 1e-5


def test_decode_256x64_workload():
    """256 sequences x 16 heads, d=128, bf16, fp32 state in place, 64 steps."""
    inp = gi.make_inputs("decode_256x64", seed=0)
    state = dev(inp.init_state)
    ref = inp.init_state.astype(np.float64)
    worst_num, worst_den = 0.0, 0.0
    for st in inp.steps:
        out = B.gdn_decode_step(dev(st["q"]), dev(st["k"]), dev(st["v"]), dev(st["g"]), dev(st["beta"]), state)
        ro = c_oracle.decode_step(st["q"], st["k"], st["v"], st["g"], st["beta"], ref)
        o = host64(out)
        worst_num = max(worst_num, float(np.max(np.abs(o - ro))))
        worst_den = max(worst_den, float(np.max(np.abs(ro))))
    eo = worst_num / worst_den
    es = rel_err(host64(state), ref)
    say(f"[parity] decode_256x64: out {eo:.3e} state {es:.3e}")
    assert eo <= 1e-2 and es <= 1e-2


# ------------------------------------------------------- multi-token decode
def _decode_tokens_check(inp, T, tol, label, with_states=True):
    N = inp.wl.num_seqs
    state = dev(inp.init_state)
    out, ts = B.gdn_decode_tokens(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), state, T,
                                  token_states=True if with_states else None)
    torch.cuda.synchronize()
    ro, rs, rf = c_oracle.decode_tokens(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state, T)
    eo, ef = rel_err(host64(out), ro), rel_err(host64(state), rf)
    et = rel_err(host64(ts), rs) if with_states else 0.0
    say(f"[parity] {label}: out {eo:.3e} final {ef:.3e} token states {et:.3e}")
    assert np.all(np.isfinite(host64(out)))
    assert eo <= tol and ef <= tol and et <= tol
    return out, ts, state


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64), (64, 128)])
@pytest.mark.parametrize("T", [1, 2, 5, 8])
def test_decode_tokens_small(dtype, dk, dv, T):
    """N = 5 sequences x T tokens, grouped value heads, per-token states checked."""
    inp = gi.make_inputs(gi.custom(dtype=dtype, Hqk=2, Hv=4, dk=dk, dv=dv, seqlens=(T,) * 5,
                                   init_state="normal"), seed=30 + T)
    _decode_tokens_check(inp, T, TOL[dtype], f"decode_tokens {dtype} dk={dk} dv={dv} T={T}")


def test_decode_tokens_without_token_states_matches_with():
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=2, Hv=2, dk=128, dv=128, seqlens=(6,) * 3,
                                   init_state="normal"), seed=37)
    o1, _, s1 = _decode_tokens_check(inp, 6, TOL["bf16"], "decode_tokens with states")
    o2, _, s2 = _decode_tokens_check(inp, 6, TOL["bf16"], "decode_tokens without states", with_states=False)
    assert torch.equal(o1, o2) and torch.equal(s1, s2)


def test_decode_tokens_rollback_to_accepted_prefix():
    """Accept the first m of T drafted tokens: restoring token_states[:, m - 1] and decoding the
    corrected token equals the oracle run over the accepted prefix plus that token."""
    T, m = 4, 2
    inp = gi.make_inputs(gi.custom(dtype="f32", Hqk=1, Hv=2, dk=64, dv=64, seqlens=(T,) * 3,
                                   init_state="normal"), seed=38)
    state = dev(inp.init_state)
    _, ts = B.gdn_decode_tokens(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), state, T,
                                token_states=True)
    state = ts[:, m - 1].contiguous()
    fix = gi.make_inputs(gi.custom(dtype="f32", Hqk=1, Hv=2, dk=64, dv=64, seqlens=(1,) * 3), seed=39)
    out = B.gdn_decode_step(dev(fix.q), dev(fix.k), dev(fix.v), dev(fix.g), dev(fix.beta), state)
    torch.cuda.synchronize()
    keep = np.concatenate([np.arange(n * T, n * T + m) for n in range(3)])
    ro, _, rf = c_oracle.decode_tokens(inp.q[keep], inp.k[keep], inp.v[keep], inp.g[keep], inp.beta[keep],
                                       inp.init_state, m)
    r2 = rf.copy()
    ro2 = c_oracle.decode_step(fix.q, fix.k, fix.v, fix.g, fix.beta, r2)
    eo, es = rel_err(host64(out), ro2), rel_err(host64(state), r2)
    say(f"[parity] rollback to {m} of {T}: out {eo:.3e} state {es:.3e}")
    assert eo <= TOL["f32"] and es <= TOL["f32"]


def test_decode_tokens_draft_256x4_workload():
    """256 sequences x 16 heads x 4 tokens, d=128, bf16, fp32 state in place, per-token states."""
    inp = gi.make_inputs("draft_256x4", seed=0)
    _decode_tokens_check(inp, 4, 1e-2, "draft_256x4")


@pytest.mark.parametrize("dtype,T", [("f32", 1), ("bf16", 3)])
def test_decode_slots_over_a_state_pool(dtype, T):
    """5 sequences over a pool of 7 states, one padding row (-1): used slots match the oracle run on
    their own states, other slots and the padding row's outputs and token states stay untouched."""
    N, P = 5, 7
    slots = np.array([4, -1, 0, 6, 2], dtype=np.int32)
    inp = gi.make_inputs(gi.custom(dtype=dtype, Hqk=2, Hv=4, dk=128, dv=64, seqlens=(T,) * N,
                                   init_state="normal"), seed=40 + T)
    pool0 = (0.1 * np.random.default_rng(5).standard_normal((P, 4, 64, 128))).astype(np.float32)
    pool = dev(pool0)
    out = torch.full((N * T, 4, 64), 7.0, dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device="cuda")
    ts = torch.full((N, T, 4, 64, 128), 5.0, dtype=torch.float32, device="cuda")
    B.gdn_decode_slots(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), pool,
                       torch.from_numpy(slots).cuda(), T, out=out, token_states=ts)
    torch.cuda.synchronize()
    po, o, t = host64(pool), host64(out), host64(ts)
    live = [n for n in range(N) if slots[n] >= 0]
    rows = np.concatenate([np.arange(n * T, n * T + T) for n in live])
    sub = lambda a: a[rows]
    ro, rs, rf = c_oracle.decode_tokens(sub(inp.q), sub(inp.k), sub(inp.v), sub(inp.g), sub(inp.beta),
                                        pool0[slots[live]], T)
    eo = rel_err(o[rows], ro)
    es = rel_err(po[slots[live]], rf)
    et = rel_err(t[live], rs)
    say(f"[parity] decode_slots {dtype} T={T}: out {eo:.3e} states {es:.3e} token states {et:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype] and et <= TOL[dtype]
    for s in set(range(P)) - set(int(x) for x in slots if x >= 0):
        assert np.array_equal(po[s], pool0[s].astype(np.float64)), s
    assert np.all(o[T:2 * T] == 7.0) and np.all(t[1] == 5.0)


# ------------------------------------------------------- prefill snapshots
def _check_snapshots(inp, chunks, tol, label, num_seqs=None):
    P = 64 * chunks
    T = inp.q.shape[0]
    N = num_seqs or (len(inp.cu_seqlens) - 1 if inp.cu_seqlens is not None else 1)
    slots = B.snapshot_slots(T, N, chunks)
    snaps = torch.full((slots, inp.v.shape[1], inp.v.shape[2], inp.q.shape[2]), 3.0, dtype=torch.float32,
                       device="cuda")
    cu = None if inp.cu_seqlens is None or num_seqs else dev(inp.cu_seqlens)
    out, fin, snaps = B.gdn_prefill_snapshots(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), chunks,
                                              None if inp.init_state is None else dev(inp.init_state), cu,
                                              snapshots=snaps, num_seqs=num_seqs)
    torch.cuda.synchronize()
    ro, rf = oracle_prefill(inp)
    ref = oracle_snapshots(inp, P)
    got = host64(snaps)
    es = max((rel_err(got[i], r) for i, r in ref.items()), default=0.0)
    eo, ef = rel_err(host64(out), ro), rel_err(host64(fin), rf)
    say(f"[parity] {label}: {len(ref)} snapshots {es:.3e} out {eo:.3e} final {ef:.3e}")
    assert len(ref) > 0 and es <= tol and eo <= tol and ef <= tol
    for i in set(range(slots)) - set(ref):
        assert np.all(got[i] == 3.0), i


def test_prefill_snapshots_packed_varlen():
    """Lengths 300, 64, 1000, 129 with a snapshot every 128 tokens (one sequence shorter than the
    interval, one ending exactly on it), grouped value heads, bf16."""
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=1, Hv=2, dk=128, dv=128, seqlens=(300, 64, 1000, 128),
                                   init_state="normal"), seed=50)
    _check_snapshots(inp, 2, TOL["bf16"], "snapshots varlen P=128")


def test_prefill_snapshots_across_parts_f32():
    """One 8192-token sequence cut into parts; a snapshot every 192 tokens, so snapshots fall on
    both sides of part boundaries (fp32, 1e-5)."""
    inp = gi.make_inputs(gi.custom(dtype="f32", Hqk=1, Hv=1, dk=64, dv=64, seqlens=(8192,),
                                   init_state="normal"), seed=51)
    _check_snapshots(inp, 3, TOL["f32"], "snapshots parts P=192")


def test_prefill_snapshots_equal_lengths_without_offsets():
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=2, Hv=2, dk=64, dv=128, seqlens=(640, 640, 640),
                                   init_state="zero"), seed=52)
    _check_snapshots(inp, 1, TOL["bf16"], "snapshots 3x640 P=64 no offsets", num_seqs=3)


# ---------------------------------------------- raw projections (fused prologue)
def _check_raw_prefill(inp, tol, label):
    cu = None if inp.cu_seqlens is None else dev(inp.cu_seqlens)
    out, fin = B.gdn_prefill(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta),
                             None if inp.init_state is None else dev(inp.init_state), cu, raw=True)
    torch.cuda.synchronize()
    ro, rf = c_oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state, inp.cu_seqlens, raw=True)
    eo, ef = rel_err(host64(out), ro), rel_err(host64(fin), rf)
    say(f"[parity] {label}: out {eo:.3e} final {ef:.3e}")
    assert np.all(np.isfinite(host64(out)))
    assert eo <= tol and ef <= tol


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (128, 64)])
def test_prefill_raw_packed(dtype, dk, dv):
    """Unnormalised q, k (per-token scales 0.1 .. 10) and gate logits; packed ragged sequences."""
    inp = gi.make_inputs(gi.custom(dtype=dtype, Hqk=2, Hv=4, dk=dk, dv=dv, seqlens=(200, 7, 130),
                                   init_state="normal", raw=True), seed=70)
    _check_raw_prefill(inp, TOL[dtype], f"prefill_raw {dtype} dk={dk} dv={dv}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_raw_long_sequence_in_parts(dtype):
    inp = gi.make_inputs(gi.custom(dtype=dtype, Hqk=1, Hv=1, dk=128, dv=128, seqlens=(4096,),
                                   init_state="normal", raw=True), seed=71)
    _check_raw_prefill(inp, TOL[dtype], f"prefill_raw parts {dtype}")


def _guard_rows(inp, dtype):
    """Tokens t = 0 mod 5 get q, k rows of squared norm 1e-6 (the guard's own size), tokens t = 0 mod 7
    get zero q, k rows (normalised to zero by the guard instead of dividing by zero)."""
    for name in ("q", "k"):
        x = gi.to_f64(getattr(inp, name), dtype)
        x[::5] *= 1e-3 / np.linalg.norm(x[::5], axis=-1, keepdims=True)
        x[::7] = 0.0
        x = x.astype(np.float32)
        setattr(inp, name, gi.f32_to_bf16_bits(x) if dtype == "bf16" else x)
    return inp


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_raw_guard_sized_and_zero_rows(dtype):
    inp = gi.make_inputs(gi.custom(dtype=dtype, Hqk=2, Hv=4, dk=128, dv=64, seqlens=(150, 64, 33),
                                   init_state="normal", raw=True), seed=74)
    _check_raw_prefill(_guard_rows(inp, dtype), TOL[dtype], f"prefill_raw guard rows {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_tokens_raw_guard_sized_and_zero_rows(dtype):
    T = 5
    inp = _guard_rows(gi.make_inputs(gi.custom(dtype=dtype, Hqk=2, Hv=4, dk=128, dv=128, seqlens=(T,) * 7,
                                                init_state="normal", raw=True), seed=75), dtype)
    state = dev(inp.init_state)
    out, _ = B.gdn_decode_tokens(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), state, T,
                                 raw=True)
    torch.cuda.synchronize()
    ro, _, rf = c_oracle.decode_tokens(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state, T, raw=True)
    eo, ef = rel_err(host64(out), ro), rel_err(host64(state), rf)
    say(f"[parity] decode_tokens_raw guard rows {dtype}: out {eo:.3e} state {ef:.3e}")
    assert eo <= TOL[dtype] and ef <= TOL[dtype]


@pytest.mark.parametrize("dtype,T", [("f32", 1), ("f32", 4), ("bf16", 3)])
def test_decode_tokens_raw(dtype, T):
    inp = gi.make_inputs(gi.custom(dtype=dtype, Hqk=2, Hv=4, dk=128, dv=64, seqlens=(T,) * 5,
                                   init_state="normal", raw=True), seed=72 + T)
    state = dev(inp.init_state)
    out, ts = B.gdn_decode_tokens(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), state, T,
                                  token_states=True, raw=True)
    torch.cuda.synchronize()
    ro, rs, rf = c_oracle.decode_tokens(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state, T, raw=True)
    eo, es, et = rel_err(host64(out), ro), rel_err(host64(state), rf), rel_err(host64(ts), rs)
    say(f"[parity] decode_tokens_raw {dtype} T={T}: out {eo:.3e} state {es:.3e} token states {et:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype] and et <= TOL[dtype]


# ------------------------------------------------- caller-owned workspace
@pytest.mark.parametrize("dtype,lens,packed", [("bf16", (4096,), False), ("f32", (300, 0, 1000, 65), True),
                                               ("bf16", (128, 128, 128), False)])
def test_prefill_with_caller_workspace_matches_pool_workspace(dtype, lens, packed):
    """gdn_prefill_ws on a caller buffer gives gdn_prefill's bits, on parts (one long sequence) and on
    packed ragged sequences; the buffer's prior contents do not matter; and the oracle agrees."""
    inp = gi.make_inputs(gi.custom(dtype=dtype, Hqk=2, Hv=4, dk=128, dv=128, seqlens=lens,
                                   init_state="normal"), seed=80)
    q, k, v, g, beta = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    init = dev(inp.init_state)
    cu = dev(inp.cu_seqlens) if packed else None
    N = len(lens)
    kw = dict(cu_seqlens=cu) if packed else dict(num_seqs=N)
    need = B.gdn_prefill_workspace_size(q, v, **kw)
    assert need > 0
    ref_o, ref_f = B.gdn_prefill(q, k, v, g, beta, init, use_pool=True, **kw)
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    for _ in range(2):   # the second call finds the first call's leftovers in the workspace
        o, f = B.gdn_prefill(q, k, v, g, beta, init, workspace=ws, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(f, ref_f)
    if packed:
        ro, rf = c_oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state, inp.cu_seqlens)
        assert rel_err(host64(o), ro) <= TOL[dtype] and rel_err(host64(f), rf) <= TOL[dtype]


def test_prefill_with_too_small_workspace_is_rejected():
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=1, Hv=1, dk=128, dv=128, seqlens=(4096,)), seed=81)
    q, k, v, g, beta = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    need = B.gdn_prefill_workspace_size(q, v)
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.GdnError, match="workspace of"):
        B.gdn_prefill(q, k, v, g, beta, workspace=ws)
    # the raw-projection form needs more (1 / |k| per token): the plain size is too small for it
    assert B.gdn_prefill_workspace_size(q, v, raw=True) > need
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.GdnError, match="workspace of"):
        B.gdn_prefill(q, k, v, g, beta, workspace=ws, raw=True)


# ------------------------------------------------------ seeded shape sweep
def _sweep_case(i):
    r = np.random.default_rng(1000 + i)
    dtype = ["f32", "bf16"][int(r.integers(2))]
    dk, dv = (int(x) for x in r.choice([64, 128], size=2))
    hqk = int(r.choice([1, 2, 4]))
    hv = hqk * int(r.choice([1, 2])) if hqk == 4 else hqk * int(r.choice([1, 2, 4]))
    n = int(r.integers(1, 6))
    edge = [0, 1, 63, 64, 65, 127, 128, 129]
    lens = [int(r.choice(edge)) if r.random() < 0.5 else int(r.integers(1, 600)) for _ in range(n)]
    if i % 4 == 1:
        lens[0] = int(r.integers(1500, 3000))   # few chains, long sequence: cut into parts
    init = "normal" if r.random() < 0.6 else "zero"
    raw = i % 4 == 3
    return dict(dtype=dtype, Hqk=hqk, Hv=hv, dk=dk, dv=dv, seqlens=tuple(lens), init_state=init, raw=raw)


@pytest.mark.parametrize("i", range(16))
def test_seeded_shape_sweep(i):
    """Random shapes (dtype, head dims, grouped value heads, ragged and edge lengths, parts, initial
    state, raw projections) against the oracle; the caller-workspace path must give the same bits."""
    c = _sweep_case(i)
    say(f"[sweep {i}] {c}")
    inp = gi.make_inputs(gi.custom(**c), seed=2000 + i)
    if c["raw"]:
        _check_raw_prefill(inp, TOL[c["dtype"]], f"sweep {i} raw")
        return
    check_prefill(inp, label=f"sweep {i}")
    q, k, v, g, beta = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    cu = dev(inp.cu_seqlens) if inp.cu_seqlens is not None else None
    kw = dict(cu_seqlens=cu) if cu is not None else dict(num_seqs=len(c["seqlens"]))
    s0 = dev(inp.init_state)
    ref_o, ref_f = B.gdn_prefill(q, k, v, g, beta, s0, use_pool=True, **kw)
    ws = torch.empty(max(B.gdn_prefill_workspace_size(q, v, **kw), 256), dtype=torch.uint8, device="cuda")
    o, f = B.gdn_prefill(q, k, v, g, beta, s0, workspace=ws, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(f, ref_f)


# -------------------------------------------------- degenerate gate values
def _gates(kind, T, hv, rng):
    if kind == "no_write":            # beta = 0: the state only decays
        return rng.uniform(-1.0, 0.0, (T, hv)), np.zeros((T, hv))
    if kind == "total_decay":         # alpha = e^-60: every step forgets (gamma underflows in fp32)
        return np.full((T, hv), -60.0), rng.uniform(0.0, 1.0, (T, hv))
    if kind == "no_decay_full_write": # alpha = 1, beta = 1
        return np.zeros((T, hv)), np.ones((T, hv))
    # alternating extremes token by token
    t = np.arange(T)[:, None] % 4
    g = np.where(t == 0, -30.0, 0.0) + np.zeros((T, hv))
    b = np.where(t % 2 == 0, 1.0, 0.0) + np.zeros((T, hv))
    return g, b


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["no_write", "total_decay", "no_decay_full_write", "alternating"])
@pytest.mark.parametrize("lens", [(700, 5, 129), (3000,)])
def test_degenerate_gates(dtype, kind, lens):
    """Gate values at the ends of their ranges, on ragged sequences and on one sequence cut into parts."""
    inp = gi.make_inputs(gi.custom(dtype=dtype, Hqk=1, Hv=2, dk=128, dv=64, seqlens=lens,
                                   init_state="normal"), seed=90)
    rng = np.random.default_rng(91)
    g, b = _gates(kind, inp.q.shape[0], 2, rng)
    inp.g, inp.beta = g.astype(np.float32), b.astype(np.float32)
    check_prefill(inp, label=f"degenerate {kind} {dtype} {lens}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind", ["no_write", "total_decay", "no_decay_full_write", "alternating"])
def test_decode_tokens_degenerate_gates(dtype, kind):
    T = 4
    inp = gi.make_inputs(gi.custom(dtype=dtype, Hqk=2, Hv=4, dk=128, dv=128, seqlens=(T,) * 6,
                                   init_state="normal"), seed=92)
    g, b = _gates(kind, inp.q.shape[0], 4, np.random.default_rng(93))
    inp.g, inp.beta = g.astype(np.float32), b.astype(np.float32)
    state = dev(inp.init_state)
    out, ts = B.gdn_decode_tokens(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), state, T,
                                  token_states=True)
    torch.cuda.synchronize()
    ro, rs, rf = c_oracle.decode_tokens(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state, T)
    eo, es, et = rel_err(host64(out), ro), rel_err(host64(state), rf), rel_err(host64(ts), rs)
    say(f"[parity] decode_tokens degenerate {kind} {dtype}: out {eo:.3e} state {es:.3e} token states {et:.3e}")
    assert eo <= TOL[dtype] and es <= TOL[dtype] and et <= TOL[dtype]


# ------------------------------------- affine state map of a token range
def _mild_gates(inp, decay):
    """Gates under which the transition of a few thousand tokens stays of order one: beta scaled by
    0.02, and g scaled by 0.0002 (decay) or zero.  Every token's factor alpha (I - beta k k^T) then
    shrinks a state by little, so an error in M is not hidden by M fading to nothing."""
    inp.beta = (inp.beta * 0.02).astype(np.float32)
    inp.g = (inp.g * 0.0002).astype(np.float32) if decay else np.zeros_like(inp.g)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("decay", [True, False])
@pytest.mark.parametrize("dk,dv,lens", [(128, 128, (300, 0, 65, 1)), (64, 128, (200, 7)), (128, 64, (2500,)),
                                        (64, 64, (130,)), (128, 128, (4096,))])
def test_prefill_affine_matches_oracle(dtype, decay, dk, dv, lens):
    """M and B against the oracle, both with the plain metric max|err| / max|ref|, under gates that keep
    M of order one (the single-sequence cases of 2500 and 4096 tokens are cut into 5 and 8 parts)."""
    inp = gi.make_inputs(gi.custom(dtype=dtype, Hqk=1, Hv=2 if lens != (4096,) else 1, dk=dk, dv=dv, seqlens=lens),
                         seed=100)
    _mild_gates(inp, decay)
    cu = dev(inp.cu_seqlens) if inp.cu_seqlens is not None else None
    kw = dict(cu_seqlens=cu) if cu is not None else dict(num_seqs=len(lens))
    m, b = B.gdn_prefill_affine(dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), **kw)
    torch.cuda.synchronize()
    rm, rb = oracle_affine(inp)
    em, eb = rel_err(host64(m), rm), rel_err(host64(b), rb)
    # smallest of the sequences' largest transition entries: every M here is of order one
    mmin = min(float(np.abs(rm[n]).max()) for n in range(len(lens)))
    say(f"[parity] affine {dtype} decay={decay} dk={dk} dv={dv} {lens}: transition {em:.3e} offset {eb:.3e} "
        f"(smallest max|M| {mmin:.3f})")
    assert mmin >= 0.1
    assert em <= TOL[dtype] and eb <= TOL[dtype]
    if 0 in lens:   # an empty sequence maps S to S
        z = lens.index(0)
        assert torch.equal(m[z], torch.eye(dk, device="cuda").expand(2, dk, dk)) and not b[z].any()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (128, 64), (64, 128)])
def test_prefill_affine_under_strong_decay(dtype, dk, dv):
    """The workload's gates (mean alpha 0.5) over 3000 tokens in parts: B against the oracle (plain
    metric).  Every token's factor alpha (I - beta k k^T) has spectral norm at most alpha (|k| = 1 to
    bf16 rounding, beta in [0, 1]), so |M_ij| <= exp(sum g), which is below 1e-300 here: the computed
    transition must vanish to within fp32 rounding of the identity it starts from."""
    inp = gi.make_inputs(gi.custom(dtype=dtype, Hqk=1, Hv=2, dk=dk, dv=dv, seqlens=(3000,)), seed=102)
    m, b = B.gdn_prefill_affine(dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta))
    torch.cuda.synchronize()
    rm, rb = oracle_affine(inp)
    bound = float(np.exp(inp.g.astype(np.float64).sum(axis=0)).max())
    eb, mg = rel_err(host64(b), rb), float(host64(m).__abs__().max())
    say(f"[parity] affine strong decay {dtype} dk={dk} dv={dv}: offset {eb:.3e}, max|M| {mg:.3e} (bound {bound:.1e})")
    assert bound < 1e-300 and np.abs(rm).max() <= bound
    assert eb <= TOL[dtype] and mg <= 1e-6


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("decay", [True, False])
def test_sequence_sharded_prefill_on_one_gpu(dtype, decay):
    """Four ranges of one sequence as four ranks would run them: each range's affine map, the maps
    composed in order from the initial state, then each range rerun from its composed start state;
    the concatenated outputs and the last final state against the oracle's single run.  decay=False
    (g = 0, beta / 50) keeps every range's transition of order one, so the composed start states
    depend on M as much as on B."""
    T, cuts = 4096, (0, 1000, 2100, 3333, 4096)
    inp = gi.make_inputs(gi.custom(dtype=dtype, Hqk=1, Hv=2, dk=128, dv=128, seqlens=(T,), init_state="normal"),
                         seed=101)
    if not decay:
        _mild_gates(inp, False)
    q, k, v, g, beta = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    maps = [B.gdn_prefill_affine(k[a:e], v[a:e], g[a:e], beta[a:e]) for a, e in zip(cuts, cuts[1:])]
    torch.cuda.synchronize()
    s = inp.init_state.astype(np.float64)                      # composed on the host in fp64
    starts = []
    for m, b in maps:
        starts.append(s.astype(np.float32))
        s = s @ host64(m) + host64(b)
    outs, fin = [], None
    for (a, e), s0 in zip(zip(cuts, cuts[1:]), starts):
        o, fin = B.gdn_prefill(q[a:e], k[a:e], v[a:e], g[a:e], beta[a:e], torch.from_numpy(s0).cuda())
        outs.append(o)
    torch.cuda.synchronize()
    ro, rf = c_oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state, None)
    eo, ef = rel_err(host64(torch.cat(outs)), ro), rel_err(host64(fin), rf)
    mmin = min(float(host64(m).__abs__().max()) for m, _ in maps)
    say(f"[parity] sharded over 4 ranges {dtype} decay={decay}: out {eo:.3e} final {ef:.3e} "
        f"(smallest max|M| {mmin:.3g})")
    assert eo <= TOL[dtype] and ef <= TOL[dtype]
    if not decay:
        assert mmin >= 0.1


@pytest.mark.parametrize("kind", ["plain", "raw", "snapshots", "affine"])
@pytest.mark.parametrize("lens", [(40000,), (300, 0, 65, 1)])
def test_workspace_forms_equal_pool_forms(kind, lens):
    """Every prefill entry point on a caller workspace (*_ws) gives the bits of its pool form."""
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=2, Hv=2, dk=128, dv=128, seqlens=lens, init_state="normal",
                                   raw=kind == "raw"), seed=103)
    q, k, v, g, beta, s0 = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state))
    cu = dev(inp.cu_seqlens) if len(lens) > 1 else None
    kw = dict(cu_seqlens=cu) if cu is not None else {}
    res = []
    for pool in (True, False):
        if kind == "affine":
            res.append(B.gdn_prefill_affine(k, v, g, beta, use_pool=pool, **kw))
        elif kind == "snapshots":
            res.append(B.gdn_prefill_snapshots(q, k, v, g, beta, 5, init_state=s0, use_pool=pool, **kw))
        else:
            res.append(B.gdn_prefill(q, k, v, g, beta, s0, raw=kind == "raw", use_pool=pool, **kw))
    torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a, b)


# ------------------------------- seeded sweep over the other entry points
def _sweep2_case(i):
    r = np.random.default_rng(3000 + i)
    dtype = ["f32", "bf16"][int(r.integers(2))]
    dk, dv = (int(x) for x in r.choice([64, 128], size=2))
    hqk = int(r.choice([1, 2, 4]))
    hv = hqk * int(r.choice([1, 2]))
    n = int(r.integers(1, 5))
    lens = [int(r.choice([0, 1, 63, 64, 65, int(r.integers(1, 900)), int(r.integers(900, 3000))])) for _ in range(n)]
    kind = ["decode_tokens", "decode_tokens_raw", "snapshots", "affine"][i % 4]
    return dict(dtype=dtype, dk=dk, dv=dv, hqk=hqk, hv=hv, lens=lens, kind=kind,
                init="normal" if r.random() < 0.6 else "zero", T=int(r.integers(1, 6)), P=int(r.choice([1, 2, 5])))


@pytest.mark.parametrize("i", range(48))
def test_seeded_entry_point_sweep(i):
    """Random shapes for multi-token decode (plain and raw), prefill with snapshots and the affine
    state map, against the oracle."""
    c = _sweep2_case(i)
    say(f"[sweep2 {i}] {c}")
    dt, kind = c["dtype"], c["kind"]
    if kind.startswith("decode_tokens"):
        T, raw = c["T"], kind.endswith("raw")
        inp = gi.make_inputs(gi.custom(dtype=dt, Hqk=c["hqk"], Hv=c["hv"], dk=c["dk"], dv=c["dv"],
                                       seqlens=(T,) * len(c["lens"]), init_state="normal", raw=raw), seed=4000 + i)
        st = dev(inp.init_state)
        o, ts = B.gdn_decode_tokens(dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta), st, T,
                                    token_states=True, raw=raw)
        torch.cuda.synchronize()
        ro, rs, rf = c_oracle.decode_tokens(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state, T, raw=raw)
        errs = [rel_err(host64(o), ro), rel_err(host64(st), rf), rel_err(host64(ts), rs)]
    else:
        inp = gi.make_inputs(gi.custom(dtype=dt, Hqk=c["hqk"], Hv=c["hv"], dk=c["dk"], dv=c["dv"],
                                       seqlens=tuple(c["lens"]), init_state=c["init"]), seed=4000 + i)
        q, k, v, g, b = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
        cu = dev(inp.cu_seqlens) if inp.cu_seqlens is not None else None
        kw = dict(cu_seqlens=cu) if cu is not None else dict(num_seqs=len(c["lens"]))
        if kind == "affine":
            _mild_gates(inp, c["T"] % 2 == 0)
            g, b = dev(inp.g), dev(inp.beta)
            m, bb = B.gdn_prefill_affine(k, v, g, b, **kw)
            torch.cuda.synchronize()
            rm, rb = oracle_affine(inp)
            errs = [rel_err(host64(m), rm), rel_err(host64(bb), rb)]
        else:
            P = c["P"]
            o, f, sn = B.gdn_prefill_snapshots(q, k, v, g, b, P, init_state=dev(inp.init_state), **kw)
            torch.cuda.synchronize()
            ro, rf = oracle_prefill(inp)
            errs = [rel_err(host64(o), ro), rel_err(host64(f), rf)]
            errs += [rel_err(host64(sn[slot]), ref) for slot, ref in oracle_snapshots(inp, 64 * P).items()]
    say(f"[parity] sweep2 {i} {kind} {dt}: worst {max(errs):.3e}")
    assert max(errs) <= TOL[dt]
