"""Seeded generator properties and the frozen oracle fixture."""
import json
import os

import numpy as np
import pytest
import torch

from gated_deltanet_linear_rule_amd import inputs as gi

HERE = os.path.dirname(os.path.abspath(__file__))


def test_bf16_rounding_is_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-6, 6, 100000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0], np.float32)])
    x = x.astype(np.float32)
    ours = gi.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    back = gi.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_slab_independent(monkeypatch):
    a = gi.make_inputs(gi.custom(Hqk=2, Hv=4, dk=16, dv=8, seqlens=(300, 5)), seed=3)
    monkeypatch.setattr(gi, "_SLAB_TOKENS", 7)
    b = gi.make_inputs(gi.custom(Hqk=2, Hv=4, dk=16, dv=8, seqlens=(300, 5)), seed=3)
    for name in ("q", "k", "v", "g", "beta"):
        assert np.array_equal(getattr(a, name), getattr(b, name)), name
    c = gi.make_inputs(gi.custom(Hqk=2, Hv=4, dk=16, dv=8, seqlens=(300, 5)), seed=4)
    assert not np.array_equal(a.q, c.q)


def test_distributions():
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=4, Hv=8, dk=128, dv=128, seqlens=(2048,)), seed=0)
    q = gi.bf16_bits_to_f32(inp.q)
    n = np.linalg.norm(q.astype(np.float64), axis=-1)
    assert np.all(np.abs(n - 1) < 2 ** -7)          # unit norm up to bf16 rounding
    assert np.all((inp.beta > 0) & (inp.beta < 1))
    assert np.all(inp.g < 0)
    assert abs(float(np.mean(np.exp(inp.g))) - 0.50) < 0.02   # mean alpha of -softplus(N(0,1))
    v = gi.bf16_bits_to_f32(inp.v)
    assert abs(float(v.std()) - 1) < 0.01


def test_packed_lengths_and_offsets():
    wl = gi._workload("varlen_8x")
    rng = np.random.default_rng(0)
    lens = rng.integers(1024, 16384, endpoint=True, size=8)
    assert np.all((lens >= 1024) & (lens <= 16384))
    small = gi.make_inputs(gi.custom(Hqk=2, Hv=4, dk=16, dv=16, seqlens=(5, 0, 9), init_state="normal"))
    assert small.cu_seqlens.tolist() == [0, 5, 5, 14]
    assert small.init_state.shape == (3, 4, 16, 16)
    assert wl.num_v_heads == 2 * wl.num_qk_heads


def test_decode_workload_shapes():
    wl = gi.custom(Hqk=2, Hv=2, dk=16, dv=16, seqlens=(1,) * 4, init_state="normal", decode_steps=3)
    inp = gi.make_inputs(wl)
    assert len(inp.steps) == 3 and inp.init_state.shape == (4, 2, 16, 16)
    assert inp.steps[0]["q"].shape == (4, 2, 16)


def test_oracle_matches_frozen_fixture():
    from tests.golden.make_golden import summarize  # calls only the oracle
    with open(os.path.join(HERE, "golden", "tiny_f32_oracle.json")) as f:
        want = json.load(f)
    got = summarize()
    for key in ("out_sum", "out_abs_sum", "out_max_abs", "final_sum", "final_abs_sum"):
        assert got[key] == pytest.approx(want[key], rel=1e-12, abs=1e-12), key
    for a, b in zip(got["out_samples"] + got["final_samples"], want["out_samples"] + want["final_samples"]):
        assert a[:3] == b[:3] and a[3] == pytest.approx(b[3], rel=1e-12, abs=1e-14)
