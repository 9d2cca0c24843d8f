"""gdn_prefill_static (the prefill on the library's static device scratch, which
allocates nothing) against gdn_prefill_ws on the same inputs: two calls in a
row, the second smaller, and a shape beyond the scratch rejected."""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_rule_amd import binding as B
from gated_deltanet_linear_rule_amd import inputs as gi
from oracle import c_oracle
from tests.gpu_util import TOL, dev, host64, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()


def _call_both(inp, num_seqs=None):
    q, k, v, g, beta = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    s0 = dev(inp.init_state)
    cu = dev(inp.cu_seqlens) if inp.cu_seqlens is not None else None
    kw = dict(cu_seqlens=cu) if cu is not None else dict(num_seqs=num_seqs or inp.wl.num_seqs)
    need = B.gdn_prefill_workspace_size(q, v, **kw)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    ref = B.gdn_prefill(q, k, v, g, beta, s0, workspace=ws, **kw)
    got = B.gdn_prefill(q, k, v, g, beta, s0, use_static=True, **kw)
    torch.cuda.synchronize()
    return need, ref, got


def test_static_scratch_prefill_two_calls_second_smaller():
    # first call: one 8,192-token sequence, 16 heads, d = 128 (about 63 MiB of scratch, cut into parts)
    big = gi.make_inputs(gi.custom(dtype="bf16", Hqk=16, Hv=16, dk=128, dv=128, seqlens=(8192,),
                                   init_state="normal"), seed=300)
    need, ref, got = _call_both(big)
    say(f"[no-alloc] call 1: 8192 tokens x 16 heads, scratch {need} bytes")
    assert 0 < need <= B.GDN_STATIC_SCRATCH_BYTES
    assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
    ro, rf = c_oracle.prefill(big.q[:, :2], big.k[:, :2], big.v[:, :2], big.g[:, :2], big.beta[:, :2],
                              big.init_state[:, :2], None)
    eo, ef = rel_err(host64(got[0][:, :2]), ro), rel_err(host64(got[1][:, :2]), rf)
    say(f"[no-alloc] call 1 heads 0-1 against the oracle: out {eo:.3e} final {ef:.3e}")
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]
    # second call, smaller: packed ragged sequences in fp32 with grouped value heads; the scratch still
    # holds the first call's leftovers
    small = gi.make_inputs(gi.custom(dtype="f32", Hqk=2, Hv=4, dk=64, dv=128, seqlens=(300, 0, 65, 1),
                                     init_state="normal"), seed=301)
    need2, ref2, got2 = _call_both(small)
    say(f"[no-alloc] call 2: packed (300, 0, 65, 1) fp32, scratch {need2} bytes")
    assert need2 < need
    assert torch.equal(got2[0], ref2[0]) and torch.equal(got2[1], ref2[1])
    ro, rf = c_oracle.prefill(small.q, small.k, small.v, small.g, small.beta, small.init_state, small.cu_seqlens)
    assert rel_err(host64(got2[0]), ro) <= TOL["f32"] and rel_err(host64(got2[1]), rf) <= TOL["f32"]


def test_static_scratch_rejects_a_shape_beyond_its_size():
    T, H, d = 16384, 16, 128
    q = torch.zeros((T, H, d), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((T, H), dtype=torch.float32, device="cuda")
    assert B.gdn_prefill_workspace_size(q, q) > B.GDN_STATIC_SCRATCH_BYTES
    out = torch.full((T, H, d), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(B.GdnError, match="static scratch holds"):
        B.gdn_prefill(q, q, q, g, g, out=out, use_static=True)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())   # nothing was enqueued
