"""Race check of the prefill's shared-memory protocol on the GPU.

libgdn_poison.so is the same source built with GDN_POISON_LDS: every prefill
kernel fills its shared memory with all-ones words (NaN in fp64, fp32 and bf16)
at entry, and the chunk kernels refill each input slice with them just before
the direct loads that reuse it.  A read of a slice that the protocol has not
(re)written since -- a missing wait or barrier, a buffer recycled too early --
would then return NaN or other bits.  The poisoned build must give exactly the
normal build's results; both are also repeated to check determinism.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_rule_amd import binding as B
from gated_deltanet_linear_rule_amd import inputs as gi
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return B.lib(), B.open_library(B.POISON_LIB_PATH)


def _run(monkeypatch, L, kind, inp, **kw):
    monkeypatch.setattr(B, "_lib", L)
    q, k, v, g, beta, s0 = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state))
    cu = dev(inp.cu_seqlens) if inp.cu_seqlens is not None and len(inp.wl.seqlens) > 1 else None
    a = dict(cu_seqlens=cu) if cu is not None else {}
    if kind == "affine":
        res = B.gdn_prefill_affine(k, v, g, beta, **a)
    elif kind == "snapshots":
        res = B.gdn_prefill_snapshots(q, k, v, g, beta, 3, init_state=s0, **a)
    else:
        res = B.gdn_prefill(q, k, v, g, beta, s0, raw=kind == "raw", **a)
    torch.cuda.synchronize()
    return [t.clone() for t in res]


CASES = [
    ("plain", "bf16", 128, 128, 2, 2, (40000,)),           # one sequence in parts: summary, link, rerun
    ("plain", "f32", 128, 64, 1, 2, (9000, 0, 130, 1)),    # fp32 path (single buffer set), ragged, empty
    ("plain", "bf16", 64, 128, 2, 4, (300, 64, 5000)),     # grouped value heads
    ("raw", "bf16", 128, 128, 2, 2, (20000, 77)),          # raw projections (1 / |k| slice)
    ("snapshots", "bf16", 128, 128, 1, 1, (12000,)),       # snapshots across parts
    ("affine", "bf16", 128, 128, 1, 2, (10000, 3000)),     # summary over every part, link in composing mode
    ("affine", "f32", 64, 64, 1, 1, (5000,)),
]


@pytest.mark.parametrize("kind,dtype,dk,dv,hqk,hv,lens", CASES)
def test_poisoned_shared_memory_changes_nothing(libs, monkeypatch, kind, dtype, dk, dv, hqk, hv, lens):
    inp = gi.make_inputs(gi.custom(dtype=dtype, Hqk=hqk, Hv=hv, dk=dk, dv=dv, seqlens=lens, init_state="normal",
                                   raw=kind == "raw"), seed=500)
    normal, poisoned = libs
    ref = _run(monkeypatch, normal, kind, inp)
    for rep in range(2):
        got = _run(monkeypatch, poisoned, kind, inp)
        for a, b in zip(ref, got):
            assert torch.isfinite(b.float()).all()
            assert torch.equal(a, b), f"{kind} {dtype} {lens}: poisoned build differs (repeat {rep})"
    say(f"[poison] {kind} {dtype} dk={dk} dv={dv} {hqk}/{hv} {lens}: identical to the normal build")


@pytest.mark.parametrize("name", ["prefill_4k", "varlen_8x"])
def test_poisoned_shared_memory_workloads(libs, monkeypatch, name):
    inp = gi.make_inputs(name, seed=0)
    normal, poisoned = libs
    ref = _run(monkeypatch, normal, "plain", inp)
    got = _run(monkeypatch, poisoned, "plain", inp)
    for a, b in zip(ref, got):
        assert torch.equal(a, b)
    say(f"[poison] {name}: identical to the normal build")


@pytest.mark.parametrize("kind", ["plain", "raw", "mixed"])
def test_poisoned_shared_memory_two_launch_schedule(libs, monkeypatch, kind):
    """A packed batch with as many (sequence, value head) chains as compute units and one long sequence:
    the two-launch schedule (first parts, summaries and the later parts after a near decay horizon in
    one launch, sharing its shared memory between the kinds of workgroup; the link with two row blocks
    per workgroup; the other later parts).  "mixed": stretches of g = 0 among the standard gates, so
    that later parts run in both launches."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    n = max(2, cus // 16)
    lens = ([9000] + [700, 0, 1, 1500, 64, 300] * n)[:n]
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=8, Hv=16, dk=128, dv=128, seqlens=lens, init_state="normal",
                                   raw=kind == "raw"), seed=501)
    if kind == "mixed":
        weak = (np.arange(inp.g.shape[0]) // 1100) % 2 == 1
        inp.g[weak] = 0
        inp.beta[weak] *= 0.05
        kind = "plain"
    normal, poisoned = libs
    ref = _run(monkeypatch, normal, kind, inp)
    got = _run(monkeypatch, poisoned, kind, inp)
    for a, b in zip(ref, got):
        assert torch.isfinite(b.float()).all()
        assert torch.equal(a, b)
    say(f"[poison] two-launch {kind} {n} seqs: identical to the normal build")
