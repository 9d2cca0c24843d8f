"""GPU tests of the part summary's decay horizon.

A part summary (the state map S -> S M_p + B_p of a part) may start at a later
chunk c of the part when every token of the part is a contraction (g_t <= 0,
0 <= beta_t |k_t|^2 <= 2) and the gates of chunks [c, end) multiply to at most
2^-160: what the chunks before c contribute then reaches the part's end scaled
by at most that factor.  These tests place the horizon at different depths of
long parts (the gates scaled so that it falls after a few, a few tens, or no
chunks of a part) and compare with the fp64 oracle; and they check on the
affine map entry point, which runs the summaries alone, that the horizon is
taken exactly when the part's tokens allow it: a NaN value at the first token
stays out of the map when the horizon is taken and reaches it when a
non-contracting token (beta |k|^2 > 2, or g > 0) anywhere in the part forbids
it.  Parts of both kinds in one sequence exercise the link, which takes
S_{p+1} = B_p after a part with a horizon and S_p M_p + B_p after one without.
"""
import numpy as np
import pytest
import torch

from gated_deltanet_linear_rule_amd import binding as B
from gated_deltanet_linear_rule_amd import inputs as gi
from tests.gpu_util import TOL, check_prefill, dev, host64, oracle_affine, rel_err, say

pytestmark = pytest.mark.gpu

BF16_NAN = np.uint16(0x7FC0)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()   # fails loudly if the HIP library is missing


def _long(dtype, scale, seed, hv=8, T=65536):
    """One T-token sequence, hv heads of d = 128 (at 256 compute units: parts of 32 chunks, 32 per
    head), the standard gates times `scale`.  A chunk's mean log2 decay is about -74 * scale, so the
    horizon lies about 3 / scale chunks before a part's end (no horizon within a part below scale
    0.15 at parts of 32 chunks)."""
    inp = gi.make_inputs(gi.custom(dtype=dtype, Hqk=hv, Hv=hv, dk=128, dv=128, seqlens=(T,),
                                   init_state="normal"), seed=seed)
    inp.g = (inp.g * scale).astype(np.float32)
    return inp


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("scale", [1.0, 0.3, 0.15, 0.02])
def test_horizon_at_different_depths(dtype, scale):
    check_prefill(_long(dtype, scale, 200), label=f"horizon {dtype} gates x{scale}")


def test_horizon_packed_varlen_with_raw_projections():
    """The raw-projection entry point (gates from logits inside the kernels) over packed sequences
    cut into parts: the prep kernel's contraction check runs on the normalised keys."""
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=4, Hv=8, dk=128, dv=128, seqlens=(30000, 17, 41000),
                                   init_state="normal", raw=True), seed=202)
    q, k, v, g, b = (dev(x) for x in (inp.q, inp.k, inp.v, inp.g, inp.beta))
    out, fin = B.gdn_prefill(q, k, v, g, b, dev(inp.init_state), dev(inp.cu_seqlens), raw=True)
    torch.cuda.synchronize()
    from oracle import c_oracle
    ro, rf = c_oracle.prefill(inp.q, inp.k, inp.v, inp.g, inp.beta, inp.init_state, inp.cu_seqlens, raw=True)
    eo, ef = rel_err(host64(out), ro), rel_err(host64(fin), rf)
    say(f"[parity] horizon raw packed: out {eo:.3e} final {ef:.3e}")
    assert eo <= TOL["bf16"] and ef <= TOL["bf16"]


@pytest.mark.parametrize("T", [384, 65536])
@pytest.mark.parametrize("refuse", [None, "beta", "gate"])
def test_horizon_is_taken_exactly_on_contracting_parts(refuse, T):
    """Affine map of one sequence (every part summarised) with v = NaN at token 0.  With the standard
    gates every part's horizon is a few chunks from its end, so the NaN cannot reach the map: M and B
    are finite and match the oracle run with v = 0 at token 0.  One token of the first chunk with
    beta |k|^2 = 2.5, or with g = +0.25, makes the first part non-contracting: its summary then runs
    from its first chunk, and with T = 384 (one part of six chunks) the NaN reaches B in every head.
    (Over 65536 tokens the later parts' horizons cut the NaN off again: S_{p+1} = B_p.)"""
    inp = _long("bf16", 1.0, 201, T=T)
    if refuse == "beta":
        inp.beta[5, :] = 2.5
    elif refuse == "gate":
        inp.g[5, :] = 0.25
    vn = inp.v.copy()
    vn[0] = BF16_NAN
    m, b = B.gdn_prefill_affine(dev(inp.k), dev(vn), dev(inp.g), dev(inp.beta))
    torch.cuda.synchronize()
    nan_heads = int(torch.isnan(b).flatten(2).any(dim=2).sum().item())
    say(f"[horizon] T={T} refuse={refuse}: heads with NaN in B {nan_heads} of {b.shape[1]}, max|M| "
        f"{float(torch.nan_to_num(m, nan=0.0).abs().max()):.3e}")
    if refuse is None or T > 384:
        inp.v[0] = 0
        rm, rb = oracle_affine(inp)
        eb = rel_err(host64(b), rb)
        say(f"[parity] horizon affine T={T}: offset {eb:.3e}, oracle max|M| {np.abs(rm).max():.3e}")
        assert nan_heads == 0 and torch.isfinite(m).all()
        assert eb <= TOL["bf16"] and float(m.abs().max()) <= 1e-6 and np.abs(rm).max() <= 1e-6
    else:
        assert nan_heads == b.shape[1]


def _mixed_gates(inp, period=3000):
    """Alternating stretches of `period` tokens: the standard gates, then g = 0 with beta / 20 (no
    decay, a transition of order one), so that some parts of a long sequence are summarised from a
    decay horizon and others in full, and the link chains both kinds."""
    t = np.arange(inp.g.shape[0])
    weak = (t // period) % 2 == 1
    inp.g[weak] = 0
    inp.beta[weak] *= 0.05


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_link_over_parts_with_and_without_horizon(dtype):
    inp = _long(dtype, 1.0, 203)
    _mixed_gates(inp)
    check_prefill(inp, label=f"mixed horizons {dtype}")


def test_affine_map_over_parts_with_and_without_horizon():
    """The map's offset chains parts of both kinds; its transition passes through a part with a
    horizon, so it vanishes (as the oracle's does)."""
    inp = _long("bf16", 1.0, 204, T=40000)
    _mixed_gates(inp)
    m, b = B.gdn_prefill_affine(dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta))
    torch.cuda.synchronize()
    rm, rb = oracle_affine(inp)
    eb = rel_err(host64(b), rb)
    say(f"[parity] affine, mixed horizons: offset {eb:.3e}, max|M| {float(m.abs().max()):.3e} "
        f"(oracle {np.abs(rm).max():.3e})")
    assert eb <= TOL["bf16"] and float(m.abs().max()) <= 1e-6 and np.abs(rm).max() <= 1e-6


def test_balanced_schedule_with_and_without_horizon():
    """Packed batch under the two-launch schedule: a later part whose predecessor has a horizon at most
    six chunks from its end reruns those chunks from zero in the first launch; the others start from B
    of the part before (a deeper horizon) or from the link's state, in the second launch."""
    from tests.test_gpu_parity import _balanced_batch
    inp = _balanced_batch(205)
    _mixed_gates(inp, period=1100)
    check_prefill(inp, label="balanced, mixed horizons")
