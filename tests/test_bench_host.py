"""Host-side logic of bench.py, on the CPU: the algorithmic byte and flop counts
that the roofline divides by, the matching of profiler kernel names, the
comment-insensitive source hash and the reduction of the HBM counters.

The expected counts are written out by hand from the layouts: q, k, v, out
[T, H, d] in bf16, g and beta [T, H] fp32, states [N, H, d_v, d_k] fp32; the
flop count is that of the chunk-64 form with dense 64 x 64 tiles.
"""
import csv
import json

import pytest

import bench


def test_prefill_bytes_of_the_262144_token_workload():
    io = 262144 * 16 * 128 * 2 * 4          # q, k, v read and out written, bf16
    gates = 262144 * 16 * 4 * 2             # g and beta, fp32
    final = 16 * 128 * 128 * 4              # final state, fp32
    assert bench.prefill_bytes(262144, 1, 16, 16, 128, 128) == io + gates + final == 4_329_570_304
    assert bench.prefill_bytes(262144, 1, 16, 16, 128, 128, init=True) == 4_329_570_304 + final
    assert bench.prefill_bytes(262144, 1, 16, 16, 128, 128, final=False) == io + gates


def test_prefill_bytes_with_grouped_value_heads():
    # q and k are read per q/k head, v and out per value head; gates and states per value head.
    T, N = 1000, 3
    b = bench.prefill_bytes(T, N, 16, 32, 128, 128, init=True)
    assert b == T * (2 * 16 * 128 + 2 * 32 * 128) * 2 + T * 32 * 8 + 2 * N * 32 * 128 * 128 * 4


def test_prefill_flops_per_token():
    # per value head: K S^T, Q S^T and the state update (3 x 2 d_k d_v), A's half (2 C d_k),
    # T~R and P U (2 x 2 C d_v), the triangular inverse (C^2 / 3); per q/k head: K K^T and Q K^T.
    per_v = 6 * 128 * 128 + 2 * 64 * 128 + 4 * 64 * 128 + 64 * 64 / 3
    per_qk = 4 * 64 * 128
    f = bench.prefill_flops_per_token(16, 16, 128, 128)
    assert f == pytest.approx(16 * per_v + 16 * per_qk, rel=1e-15)
    assert int(f) == 2_905_429


def test_decode_bytes_of_the_256_sequence_step():
    state = 256 * 16 * 128 * 128 * 4
    assert bench.decode_bytes(256, 16, 16, 128, 128) == 2 * state + 256 * 16 * 128 * 2 * 4 + 256 * 16 * 8
    assert bench.decode_bytes(256, 16, 16, 128, 128) == 541_097_984
    # one token per sequence with no per-token states is a plain decode step
    assert bench.decode_tokens_bytes(256, 1, 16, 16, 128, 128, token_states=False) == \
        bench.decode_bytes(256, 16, 16, 128, 128)
    assert bench.decode_tokens_bytes(256, 4, 16, 16, 128, 128) - \
        bench.decode_tokens_bytes(256, 4, 16, 16, 128, 128, token_states=False) == 4 * state


PREP = "_ZN3gdn12_GLOBAL__N_115gdn_prep_kernelIDF16bLi128ELb0EEEvNS_11PrefillArgsE"
SUMMARY = "_ZN3gdn12_GLOBAL__N_116gdn_chunk_kernelIDF16bLi128ELi128ELb0ELb0EEEvNS_11PrefillArgsE"
OUTPUT = "_ZN3gdn12_GLOBAL__N_116gdn_chunk_kernelIDF16bLi128ELi128ELb1ELb0EEEvNS_11PrefillArgsE"
LINK = "void gdn::(anonymous namespace)::gdn_link_kernel<128>(gdn::PrefillArgs)"
DECODE = "_ZN3gdn12_GLOBAL__N_117gdn_decode_kernelIDF16bLi128ELi128EEEvNS_10DecodeArgsE"
CALIB = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int, float*)"


def test_kernel_name_matching():
    m = bench._kernel_matches
    assert m("gdn_chunk_kernel<summary>", SUMMARY) and not m("gdn_chunk_kernel<summary>", OUTPUT)
    assert m("gdn_chunk_kernel<output>", OUTPUT) and not m("gdn_chunk_kernel<output>", SUMMARY)
    assert m("gdn_prep_kernel", PREP) and not m("gdn_chunk_kernel<output>", PREP)
    assert m("gdn_link_kernel", LINK) and m("gdn_decode_kernel", DECODE)
    assert not m("gdn_decode_kernel", PREP)


def test_source_hash_ignores_comments_but_not_code():
    base = "int f(int x) {\n  return x + 1;  // add one\n}\n"
    texts = {
        "base": base,
        "comment": "/* header\n   block */\nint f(int x) {\n\n  return x + 1;  // add 1\n}\n",
        "indent": "int f(int x) {\n        return   x + 1;\n}\n",
        "code": base.replace("x + 1", "x + 2"),
    }
    h = {k: bench._sha(["a"], read=lambda p, t=t: t) for k, t in texts.items()}
    assert h["base"] == h["comment"] == h["indent"]
    assert h["base"] != h["code"]


def _write_pmc(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, name, vals in rows:
            for v in vals:                   # one row per counter instance, summed per dispatch
                w.writerow([d, name, counter, v])


def test_traffic_summary_scales_by_the_calibration_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "_sha", lambda paths, read=None: "sha-" + paths[0].rsplit("/", 1)[-1])
    gib_kib = (1 << 30) / 1024
    # the calibration copy's FETCH_SIZE reads half its true bytes, WRITE_SIZE all of them
    fetch = [(1, CALIB, [gib_kib / 4, gib_kib / 4])]
    write = [(1, CALIB, [gib_kib])]
    d = 2
    for _ in range(2):                       # two prefill calls of four dispatches each
        for name, fk, wk in ((PREP, 100, 40), (SUMMARY, 200, 2), (LINK, 10, 1), (OUTPUT, 300, 100)):
            fetch.append((d, name, [fk / 2, fk / 2]))
            write.append((d, name, [wk]))
            d += 1
    for _ in range(3):                       # three decode dispatches
        fetch.append((d, DECODE, [50]))
        write.append((d, DECODE, [60]))
        d += 1
    _write_pmc(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _write_pmc(tmp_path / "w.csv", "WRITE_SIZE", write)
    bench.write_traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), prefill_calls=2)
    rec = json.loads((tmp_path / "profiles" / "hbm_traffic.json").read_text())
    assert rec["calibration"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["calibration"]["write_scale"] == pytest.approx(1.0)
    pre = rec["gdn_prefill"]
    assert pre["source_sha"] == "sha-gdn_prefill.hip"
    # per call: reads (100 + 200 + 10 + 300) KiB x 2, writes (40 + 2 + 1 + 100) KiB
    assert pre["bytes_per_call"] == pytest.approx((610 * 2 + 143) * 1024)
    assert pre["kernels"]["gdn_chunk_kernel<output>"]["read_bytes"] == pytest.approx(600 * 1024)
    assert pre["kernels"]["gdn_chunk_kernel<summary>"]["write_bytes"] == pytest.approx(2 * 1024)
    assert pre["kernels"]["gdn_prep_kernel"]["dispatches"] == 2
    dec = rec["gdn_decode"]
    assert dec["bytes_per_call"] == pytest.approx((50 * 2 + 60) * 1024)
    assert dec["source_sha"] == "sha-gdn_decode.hip"


def _write_pmc_multi(path, rows):
    """rows: (dispatch, kernel, {counter: value})."""
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, name, vals in rows:
            for c, v in vals.items():
                w.writerow([d, name, c, v])


def test_sq_summary_per_call_rates(tmp_path, monkeypatch):
    """Two passes over two calls of one kernel: cycles from GRBM_GUI_ACTIVE / 8 XCDs per call,
    matrix-core busy over 1024 SIMDs, LDS over 256 CUs, per-wave-chunk instruction counts."""
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "_sha", lambda paths, read=None: "sha")
    cyc = 1000
    p1 = [(d, OUTPUT, {"GRBM_GUI_ACTIVE": 8 * cyc, "SQ_WAVES": 16, "SQ_INSTS_VALU": 3200, "SQ_INSTS_MFMA": 640})
          for d in (1, 2)]
    p2 = [(d, OUTPUT, {"GRBM_GUI_ACTIVE": 8 * cyc, "SQ_VALU_MFMA_BUSY_CYCLES": 1024 * cyc / 4,
                       "SQ_LDS_IDX_ACTIVE": 256 * cyc / 2, "SQ_LDS_BANK_CONFLICT": 256 * cyc / 20,
                       "SQ_WAVE_CYCLES": 400, "SQ_ACTIVE_INST_ANY": 100, "SQ_WAIT_ANY": 200, "SQ_WAIT_INST_ANY": 50})
          for d in (1, 2)]
    _write_pmc_multi(tmp_path / "p1.csv", p1)
    _write_pmc_multi(tmp_path / "p2.csv", p2)
    bench.write_sq_summary([str(tmp_path / "p1.csv"), str(tmp_path / "p2.csv")], "w", calls=2,
                           wave_chunks={"gdn_chunk_kernel<output>": 16 * 10})
    rec = json.loads((tmp_path / "profiles" / "sq_counters.json").read_text())["w"]
    k = rec["kernels"]["gdn_chunk_kernel<output>"]
    assert rec["source_sha"] == "sha" and k["cycles"] == cyc
    assert k["mfma_busy"] == pytest.approx(0.25) and k["lds_active"] == pytest.approx(0.5)
    assert k["lds_bank_conflict_share"] == pytest.approx(0.1)
    assert (k["issuing"], k["waiting_on_counters"], k["waiting_to_issue"]) == (0.25, 0.5, 0.125)
    # per call 3200 VALU and 640 MFMA instructions over 16 waves x 10 chunks
    assert k["per_wave_chunk"] == {"valu": 20.0, "mfma": 4.0}
    assert bench.counters_current("w") and not bench.counters_current("other")


def test_summary_steps_follow_the_decay_horizon():
    """Per-chunk counter figures count a summary's chunks from its decay horizon: about three chunks
    per head with the workload's gates (a chunk decays by about 2^-74), every chunk with g = 0 or when
    one token of the range has beta |k|^2 > 2 (not a contraction)."""
    from gated_deltanet_linear_rule_amd import inputs as gi
    inp = gi.make_inputs(gi.custom(dtype="bf16", Hqk=2, Hv=4, dk=128, dv=128, seqlens=(640,)), seed=1)
    assert 4 * 2 <= bench.summary_steps(inp, 0, 0, 10) <= 4 * 4
    beta = inp.beta.copy()
    inp.beta[100, 1] = 2.5
    got = bench.summary_steps(inp, 0, 0, 10)
    assert 3 * 2 + 10 <= got <= 3 * 4 + 10            # head 1 runs every chunk
    inp.beta = beta
    inp.g[:] = 0
    assert bench.summary_steps(inp, 0, 0, 10) == 4 * 10


def test_wave_chunks_place_later_parts_by_their_predecessors_horizon():
    """Per-chunk counter figures of the packed schedule: with the workload's gates every later part of
    varlen_8x follows a part whose horizon is a few chunks from its end, so its chunks (and the rerun
    ones) count in the first launch; with g = 0 none does, and they count in the second launch, as
    without inputs."""
    from gated_deltanet_linear_rule_amd import inputs as gi
    inp = gi.make_inputs("varlen_8x", seed=0)
    plain = bench.wave_chunks(inp.wl)
    fast = bench.wave_chunks(inp.wl, inp)
    assert fast["gdn_chunk_kernel<output>"] == 0
    assert fast["gdn_chunk_first_kernel"] > plain["gdn_chunk_first_kernel"]
    inp.g[:] = 0
    slow = bench.wave_chunks(inp.wl, inp)
    assert slow["gdn_chunk_kernel<output>"] == plain["gdn_chunk_kernel<output>"] > 0
