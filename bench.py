"""Benchmark of the GDN hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Headline: prefill tokens/s on the native-context workload (B=1, T=262,144,
16 heads, d_k = d_v = 128, bf16 q/k/v/out, fp32 gates, zero initial state,
final state returned).  One step = one gdn_prefill call over that sequence
with inputs already resident in HBM.  The decode leg (256 sequences x 16
heads, fp32 state 256 MiB updated in place, 64 consecutive steps with fresh
tokens) is reported in the same JSON line as state GB/s.

Timing uses HIP events on the stream the library launches on (torch's
current stream, handed to the C ABI).  `roofline` uses algorithmic bytes and
flops per call (prefill_bytes, prefill_flops_per_token below); `cpu_baseline`
times the fp64 oracle on a bounded sample of the same prefill workload on
host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 matrix peak, TFLOP/s
CHUNK = 64

# What the pages report about speed (context only, never a target or a baseline).
VENDOR_CONTEXT = {
    "vendor_claims": "up to 7.6x faster prefill and up to 4.9x faster decode at 1M-token sequences",
    "what_it_compares": "the model's sparse attention layer (QSA) against dense attention, at kernel level; not "
                        "end-to-end, and not a measurement of the GDN layer timed here",
    "hardware": "not stated", "precision": "not stated",
    "sources": ["studioglobal.ai, 'Hybride Aufmerksamkeit fuer sehr lange Kontexte'",
                "flozi.net, 'Der Weg eines Tokens durch das Modell', item 2"],
}


def prefill_bytes(T, N, hqk, hv, dk, dv, elem=2, init=False, final=True):
    """Compulsory HBM bytes of one prefill call: q, k, v read, out written,
    g and beta read, initial state read (if given) and final state written."""
    b = T * (2 * hqk * dk + 2 * hv * dv) * elem + T * hv * 8
    st = N * hv * dv * dk * 4
    return b + (st if init else 0) + (st if final else 0)


def prefill_flops_per_token(hqk, hv, dk, dv, C=CHUNK):
    """Algorithmic flops per token of the chunk-C WY/UT form (dense C x C tiles):
    per value head the state products 6 dk dv (K S^T, Q S^T, state update),
    2 C dk for A's scaling-free half, 4 C dv for T~R and P U, C^2/3 for the
    triangular inverse; per q/k head 4 C dk for K K^T and Q K^T."""
    return hv * (6 * dk * dv + 2 * C * dk + 4 * C * dv + C * C / 3) + hqk * (4 * C * dk)


def decode_bytes(N, hqk, hv, dk, dv, elem=2):
    return 2 * N * hv * dv * dk * 4 + N * (2 * hqk * dk + 2 * hv * dv) * elem + N * hv * 8


def decode_tokens_bytes(N, T, hqk, hv, dk, dv, elem=2, token_states=True):
    """State read and written once, T per-token states written, T tokens of inputs and outputs."""
    st = N * hv * dv * dk * 4
    return 2 * st + (T * st if token_states else 0) + N * T * (2 * hqk * dk + 2 * hv * dv) * elem + N * T * hv * 8


def _code_text(text):
    """Source text without comments, blank lines and indentation, runs of spaces as one (so that
    a comment edit or a re-indent does not count as a change of the kernels; string literals in
    these files hold no comment marks)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(" ".join(ln.split()) for ln in text.splitlines() if ln.strip())


def _sha(paths, read=None):
    """Hash of the kernel sources' code (comments and blank lines dropped)."""
    h = hashlib.sha256()
    for p in paths:
        if read is None:
            with open(os.path.join(ROOT, p), encoding="utf-8") as f:
                text = f.read()
        else:
            text = read(p)
        h.update(_code_text(text).encode())
    return h.hexdigest()[:16]


PREFILL_SOURCES = ["gated_deltanet_linear_rule_amd/csrc/gdn_prefill.hip",
                   "gated_deltanet_linear_rule_amd/csrc/gdn_device.h"]
DECODE_SOURCES = ["gated_deltanet_linear_rule_amd/csrc/gdn_decode.hip",
                  "gated_deltanet_linear_rule_amd/csrc/gdn_device.h"]


def measured_traffic(name, sources):
    """HBM bytes per call from the committed rocprofv3 counter summary, or None
    if absent or taken on a different version of the kernel source."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)[name]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha") != _sha(sources):
        return None
    return rec.get("bytes_per_call")


CALIB_BYTES = 1 << 30      # bytes read and bytes written by the calibration kernel
KERNELS = {"gdn_prefill": ("gdn_prep_kernel", "gdn_chunk_kernel<summary>", "gdn_chunk_first_kernel", "gdn_link_kernel",
                           "gdn_chunk_kernel<output>"),
           "gdn_decode": ("gdn_decode_kernel",)}


def _kernel_matches(label, name):
    """Does a dispatch's (mangled) kernel name belong to `label`?  The two chunk kernels are one
    template; its fourth argument (OUT) tells them apart."""
    import re
    if label.startswith("gdn_chunk_kernel<"):
        m = re.search(r"gdn_chunk_kernelI\w+?Li\d+ELi\d+ELb([01])E", name)
        return bool(m) and m.group(1) == ("1" if label.endswith("<output>") else "0")
    return label in name


def _pmc_per_dispatch(path, counter):
    """{dispatch id: (kernel name, value in KiB)} for one counter of a rocprofv3 csv."""
    import csv
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] != counter:
                continue
            d = int(row["Dispatch_Id"])
            name, val = out.get(d, (row["Kernel_Name"], 0.0))
            out[d] = (name, val + float(row["Counter_Value"]))
    return out


def write_traffic_summary(fetch_csv, write_csv, prefill_calls):
    """HBM bytes per call from FETCH_SIZE / WRITE_SIZE (KiB per dispatch), each scaled
    by what the same counter reads for the calibration kernel (1 GiB in, 1 GiB out).
    A prefill call may launch its kernels several times (segments): its bytes are the
    counters summed over all dispatches divided by the number of calls profiled."""
    fetch = _pmc_per_dispatch(fetch_csv, "FETCH_SIZE")
    write = _pmc_per_dispatch(write_csv, "WRITE_SIZE")

    def mean_of(table, pred):
        v = [val for name, val in table.values() if pred(name)]
        return (sum(v) / len(v) if v else None), len(v)

    def per_call(table, pred, calls):
        v = [val for name, val in table.values() if pred(name)]
        return (sum(v) / calls if v else None), len(v)

    is_calib = lambda n: "neg_kernel" in n
    cf, _ = mean_of(fetch, is_calib)
    cw, _ = mean_of(write, is_calib)
    if not cf or not cw:
        raise SystemExit("calibration kernel (torch.neg) not found in the counter files")
    sf, sw = CALIB_BYTES / (cf * 1024), CALIB_BYTES / (cw * 1024)
    rec = {"calibration": {"kernel": "torch.neg fp32, 1 GiB read + 1 GiB written",
                           "fetch_kib": cf, "write_kib": cw, "fetch_scale": sf, "write_scale": sw}}
    for call, kernels in KERNELS.items():
        per = {}
        total = 0.0
        agg = (lambda t, p: per_call(t, p, prefill_calls)) if call == "gdn_prefill" else mean_of
        for kn in kernels:   # (a schedule runs some of the call's kernels only)
            f, nf = agg(fetch, lambda n, kn=kn: _kernel_matches(kn, n))
            w, nw = agg(write, lambda n, kn=kn: _kernel_matches(kn, n))
            if f is None or w is None:
                continue
            rb, wb = f * 1024 * sf, w * 1024 * sw
            per[kn] = {"read_bytes": rb, "write_bytes": wb, "dispatches": min(nf, nw)}
            total += rb + wb
        if per:
            srcs = PREFILL_SOURCES if call == "gdn_prefill" else DECODE_SOURCES
            rec[call] = {"bytes_per_call": total, "kernels": per, "source_sha": _sha(srcs)}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "hbm_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


SQ_PASSES = (
    ("GRBM_GUI_ACTIVE", "SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_INSTS_MFMA",
     "SQ_INSTS_VMEM_RD", "SQ_INSTS_VMEM_WR"),
    ("GRBM_GUI_ACTIVE", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_ANY", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY",
     "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU"),
    ("GRBM_GUI_ACTIVE", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_LDS",
     "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_ACTIVE_INST_SCA", "SQ_INSTS_SMEM"),
)
XCDS, CUS, SIMDS = 8, 256, 1024


def part_plan(wl, cus=CUS):
    """The library's part plan for a workload on a `cus`-CU device (mirrors prefill_part_plan and
    SeqParts in gdn_prefill.hip): per sequence, the chunk counts of its first part and of its later
    parts, and whether the balanced schedule runs."""
    chunks = -(-wl.total_tokens // 64)
    whole = max(chunks, 1)
    chains = wl.num_seqs * wl.num_v_heads
    L, cut, first, balanced = whole, 0, 1, False
    if chains < cus:
        L = min(max(-(-chunks * wl.num_v_heads // cus), 6), whole)
    elif (wl.dtype == "bf16" and wl.num_seqs > 1 and wl.head_dim_k == wl.head_dim_v and chains <= 2 * cus
          and (wl.packed or wl.num_seqs > 1)):
        share = chunks * wl.num_v_heads / cus
        Lb, cb = max(int(0.2 * share), 6), int(1.0 * share)
        cb = max(cb, Lb)
        if Lb < whole and cb < whole:
            L, cut, first, balanced = Lb, cb, cb // Lb, True
    seqs = []
    for n in wl.seqlens:
        nc = -(-n // 64)
        ns = max(-(-nc // L), 1)
        kk = min(first, ns) if nc > cut else ns
        head = min(kk * L, nc)
        seqs.append((head, [min((j + 1) * L, nc) - j * L for j in range(kk, ns)]))
    return seqs, balanced


HORIZON_LOG2 = -160.0
WARM_CHUNKS = 6            # deepest predecessor horizon a later part reruns in the first launch


def horizon_depths(inp, seq, a, e):
    """Per value head, the number of chunks from the decay horizon of chunks [a, e) of sequence
    `seq` to e, or None where there is none (every token a contraction, g <= 0 and 0 <= beta |k|^2 <=
    1.99, and the chunks' log2 decays summing to <= -160 from some chunk to the end; the prep and
    chunk kernels decide this on the device).  For the per-chunk counter figures."""
    wl = inp.wl
    cu = np.concatenate([[0], np.cumsum(wl.seqlens)])
    t0, t1 = int(cu[seq]) + 64 * a, min(int(cu[seq]) + 64 * e, int(cu[seq + 1]))
    g = inp.g[t0:t1].astype(np.float64)                         # [tokens, Hv]
    beta = inp.beta[t0:t1].astype(np.float64)
    k = inp.k[t0:t1]
    k = (k.astype(np.uint32) << 16).view(np.float32) if k.dtype == np.uint16 else k
    k2 = (k.astype(np.float64) ** 2).sum(axis=2)                # [tokens, Hqk]
    k2 = np.repeat(k2, wl.num_v_heads // wl.num_qk_heads, axis=1)
    ok = np.all((g <= 0) & (beta >= 0) & (beta * k2 <= 1.99), axis=0)
    pad = (-(t1 - t0)) % 64
    dec = np.concatenate([g, np.zeros((pad, g.shape[1]))]).reshape(-1, 64, g.shape[1]).sum(axis=1) / np.log(2)
    suffix = np.cumsum(dec[::-1], axis=0)[::-1]                 # sum over chunks [c, e)
    depths = []
    for h in range(g.shape[1]):
        hit = np.nonzero(suffix[:, h] <= HORIZON_LOG2)[0]
        depths.append((e - a) - int(hit[-1]) if ok[h] and len(hit) else None)
    return depths


def summary_steps(inp, seq, a, e):
    """Chunk steps the summary of chunks [a, e) of sequence `seq` runs, summed over the value heads:
    from its decay horizon when it has one, else all e - a."""
    return sum(e - a if d is None else d for d in horizon_depths(inp, seq, a, e))


def wave_chunks(wl, inp=None):
    """Chunk steps summed over the working waves of each chunk kernel in one prefill call (every wave
    of a part's workgroup runs the part's chunks; d_k = d_v here or d_v waves for outputs and
    max(d_k, d_v) for summaries).  A summary runs from its part's decay horizon when it has one
    (summary_steps, with the inputs `inp`; without them every chunk of the part is counted)."""
    seqs, balanced = part_plan(wl)
    nwo, nws = wl.head_dim_v // 16, max(wl.head_dim_v, wl.head_dim_k) // 16
    H = wl.num_v_heads

    def summ_of(n, head, rest, summarised):
        # chunk ranges of the summarised parts of sequence n: the first part (unless the balanced
        # schedule runs it from init_state), then the later parts but the last
        bounds = [(0, head)] + [(head + sum(rest[:j]), head + sum(rest[:j + 1])) for j in range(len(rest))]
        parts = bounds[:-1] if summarised else bounds[1:-1]
        if inp is None:
            return sum(e - a for a, e in parts) * H
        return sum(summary_steps(inp, n, a, e) for a, e in parts)
    if balanced:
        # first launch: first parts (outputs), the later parts' summaries but the last's, and the later
        # parts whose predecessor has a horizon at most WARM_CHUNKS from its end (their own chunks and
        # the rerun ones); second launch: the other later parts
        first = sum(h for h, _ in seqs) * H * nwo + sum(summ_of(n, h, r, False) for n, (h, r) in enumerate(seqs)) * nws
        later = 0
        for n, (h, r) in enumerate(seqs):
            bounds = [(0, h)] + [(h + sum(r[:j]), h + sum(r[:j + 1])) for j in range(len(r))]
            for (a0, e0), (a1, e1) in zip(bounds, bounds[1:]):
                depths = horizon_depths(inp, n, a0, e0) if inp is not None else [None] * H
                for d in depths:
                    if d is not None and d <= WARM_CHUNKS:
                        first += (e1 - a1 + d) * nwo
                    else:
                        later += (e1 - a1) * nwo
        return {"gdn_chunk_first_kernel": first, "gdn_chunk_kernel<output>": later}
    # one pass over every part; with no later parts the sequence is one part.  Summaries: every
    # part but the last (the first part of a cut sequence is the first slot, the rest follow)
    out = sum(h + sum(r) for h, r in seqs) * H * nwo
    summ = sum(summ_of(n, h, r, True) if r else 0 for n, (h, r) in enumerate(seqs)) * nws
    wcs = {"gdn_chunk_kernel<output>": out}
    if summ:
        wcs["gdn_chunk_kernel<summary>"] = summ
    return wcs


def write_sq_summary(csvs, workload, calls, wave_chunks):
    """Per-kernel shader-sequencer metrics from rocprofv3 --pmc counter files (the passes of
    SQ_PASSES, each a separate run of the same command).  Counters are summed over the
    dispatches of each prefill kernel and divided by the number of calls; `wave_chunks` maps a
    kernel label to its chunk steps summed over its working waves (for per-chunk figures).
    Cycles = GRBM_GUI_ACTIVE / 8 XCDs; SQ_*_CYCLES and SQ_ACTIVE_/WAIT_ counters are in
    units of 4 cycles per wave."""
    tot = {}
    for path in csvs:
        for name, vals in _pmc_all(path).items():
            lab = next((k for k in KERNELS["gdn_prefill"] if _kernel_matches(k, name)), None)
            if lab is None:
                continue
            agg = tot.setdefault(lab, {})
            for c, v in vals.items():
                agg.setdefault(c, []).append(v)
    out = {}
    for lab, agg in tot.items():
        m = {c: sum(v) / calls for c, v in agg.items() if c != "GRBM_GUI_ACTIVE"}
        # every pass holds GRBM_GUI_ACTIVE summed over its `calls` dispatches of the kernel
        cyc = sum(agg["GRBM_GUI_ACTIVE"]) / len(agg["GRBM_GUI_ACTIVE"]) / calls / XCDS
        waves = m.get("SQ_WAVES", 0.0)
        wc = wave_chunks.get(lab)
        rec = {"cycles": round(cyc), "waves": round(waves)}
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            rec["mfma_busy"] = round(m["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * SIMDS), 4)
        if "SQ_LDS_IDX_ACTIVE" in m:
            rec["lds_active"] = round(m["SQ_LDS_IDX_ACTIVE"] / (cyc * CUS), 4)
            rec["lds_bank_conflict_share"] = round(m["SQ_LDS_BANK_CONFLICT"] / max(m["SQ_LDS_IDX_ACTIVE"], 1), 4)
        if "SQ_WAVE_CYCLES" in m:
            wcyc = m["SQ_WAVE_CYCLES"]
            rec["issuing"] = round(m["SQ_ACTIVE_INST_ANY"] / wcyc, 4)
            rec["waiting_on_counters"] = round(m["SQ_WAIT_ANY"] / wcyc, 4)
            rec["waiting_to_issue"] = round(m["SQ_WAIT_INST_ANY"] / wcyc, 4)
        if wc:
            n = wc
            for c, key in (("SQ_INSTS_VALU", "valu"), ("SQ_INSTS_MFMA", "mfma"), ("SQ_INSTS_SALU", "salu"),
                           ("SQ_INSTS_LDS", "lds"), ("SQ_INSTS_VMEM_RD", "vmem_rd"), ("SQ_INSTS_VMEM_WR", "vmem_wr")):
                if c in m:
                    rec.setdefault("per_wave_chunk", {})[key] = round(m[c] / n, 1)
        out[lab] = rec
    path = os.path.join(ROOT, "profiles", "sq_counters.json")
    try:
        with open(path) as f:
            allrec = json.load(f)
    except (OSError, ValueError):
        allrec = {}
    allrec[workload] = {"kernels": out, "source_sha": _sha(PREFILL_SOURCES), "calls": calls}
    with open(path, "w") as f:
        json.dump(allrec, f, indent=1)
    print(json.dumps(allrec[workload], indent=1))


def _pmc_all(path):
    """{kernel name: {counter: value summed over that kernel's dispatches}} of a rocprofv3 csv."""
    import csv
    out = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            d = out.setdefault(row["Kernel_Name"], {})
            d[row["Counter_Name"]] = d.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
    return out


def counters_current(workload):
    """Whether profiles/sq_counters.json holds counters of `workload` taken on the current kernel code."""
    try:
        with open(os.path.join(ROOT, "profiles", "sq_counters.json")) as f:
            rec = json.load(f)[workload]
    except (OSError, KeyError, ValueError):
        return None
    return rec.get("source_sha") == _sha(PREFILL_SOURCES)


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the shader clock settles over the first ten or so calls of sustained load (calls right after
    # the inputs are uploaded run up to a third slower, then recover), so the default warmup covers them
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--decode-runs", type=int, default=3, help="timed 64-step decode runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="headline prefill and single-step decode only (no raw-projection, snapshot, "
                         "multi-token or state-pool legs): the run the counter summaries are taken on")
    ap.add_argument("--cpu-sample-tokens", type=int, default=262144)
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB -> 1 GiB elementwise kernel (torch.neg, fp32), the "
                         "known-size reference that scales rocprofv3 FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) of a --calib-copy run into profiles/hbm_traffic.json")
    ap.add_argument("--prefill-calls", type=int, default=3,
                    help="with --traffic-summary / --sq-summary: prefill calls in the profiled run (warmup + steps)")
    ap.add_argument("--sq-summary", nargs="+", metavar="CSV",
                    help="no GPU: reduce rocprofv3 --pmc counter files of the SQ_PASSES passes of one run into "
                         "profiles/sq_counters.json (with --prefill-workload naming the workload)")
    ap.add_argument("--prefill-workload", default="prefill_256k",
                    help="workload of the prefill leg (profiling runs of the smaller workloads); the headline "
                         "metric is the default, prefill_256k")
    args = ap.parse_args()
    if args.traffic_summary:
        write_traffic_summary(*args.traffic_summary, args.prefill_calls)
        return
    if args.sq_summary:
        from gated_deltanet_linear_rule_amd import inputs as gi
        winp = gi.make_inputs(args.prefill_workload, seed=0)
        # chunk steps per wave: every wave of a part's workgroup runs the part's chunks (a summary
        # from its decay horizon); parts are 64 L tokens, L as the library chooses on a 256-CU device
        # (one part per sequence when the (sequence, head) chains alone fill it)
        write_sq_summary(args.sq_summary, args.prefill_workload, args.prefill_calls, wave_chunks(winp.wl, winp))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the GDN path here is single-GPU); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_deltanet_linear_rule_amd import binding as B
    from gated_deltanet_linear_rule_amd import inputs as gi

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    B.lib()

    def dev(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    # ------------------------------------------------------------ prefill leg
    t_gen = time.time()
    inp = gi.make_inputs(args.prefill_workload, seed=0)
    wl = inp.wl
    T, hqk, hv, dk, dv = wl.total_tokens, wl.num_qk_heads, wl.num_v_heads, wl.head_dim_k, wl.head_dim_v
    NS = wl.num_seqs
    q, k, v, g, beta = dev(inp.q), dev(inp.k), dev(inp.v), dev(inp.g), dev(inp.beta)
    pcu = dev(inp.cu_seqlens) if NS > 1 else None
    ps0 = dev(inp.init_state) if inp.init_state is not None else None
    pkw = dict(cu_seqlens=pcu) if pcu is not None else {}
    out = torch.empty((T, hv, dv), dtype=torch.bfloat16, device="cuda")
    fin = torch.empty((NS, hv, dv, dk), dtype=torch.float32, device="cuda")
    log(f"prefill inputs generated and uploaded in {time.time() - t_gen:.1f}s")

    # every prefill leg runs on a workspace allocated here, outside the timed region
    ws_bytes = max(B.gdn_prefill_workspace_size(q, v, **pkw), B.gdn_prefill_workspace_size(q, v, raw=True, **pkw),
                   B.gdn_prefill_workspace_size(k, v, affine=True, **pkw))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")

    def step():
        B.gdn_prefill(q, k, v, g, beta, ps0, out=out, final_state=fin, workspace=ws, **pkw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_call_ms = [a.elapsed_time(b) for a, b in ev]
    ms = float(np.mean(per_call_ms))
    # every 16th token (a full fp32 copy of the 1 GB of outputs here left the next leg ~15% slower)
    assert torch.isfinite(out[::16]).all().item(), "non-finite prefill output"
    log(f"prefill: mean {ms:.3f} ms/call, median {np.median(per_call_ms):.3f}, wall {1e3 * wall / args.steps:.3f} ms/step")

    bytes_call = prefill_bytes(T, NS, hqk, hv, dk, dv, init=ps0 is not None)
    flops_call = prefill_flops_per_token(hqk, hv, dk, dv) * T
    gbs = bytes_call / (ms * 1e-3) / 1e9
    tflops = flops_call / (ms * 1e-3) / 1e12
    tok_s = T / (ms * 1e-3)
    traffic = measured_traffic("gdn_prefill", PREFILL_SOURCES)
    # shader counters of this workload's kernels (profiles/sq_counters.json), while taken on this code
    counters = None
    if counters_current(args.prefill_workload):
        with open(os.path.join(ROOT, "profiles", "sq_counters.json")) as f:
            crec = json.load(f)[args.prefill_workload]
        counters = {"source_sha": crec["source_sha"],
                    "kernels": {k: {m: v.get(m) for m in ("mfma_busy", "lds_active", "issuing", "waiting_on_counters")}
                                for k, v in crec["kernels"].items()}}

    raw_rec = snapshot_rec = affine_rec = slow_rec = None
    headline = args.prefill_workload == "prefill_256k"
    if not args.no_variants and headline:
        # The variants of the call, timed in alternating rounds together with the plain call (a leg
        # timed on its own right after the headline loop ran up to a third slower: the shader clock
        # drops under the sustained load and recovers, so each leg's figure is the median over
        # rounds that interleave all legs).
        snap_chunks = 64
        snaps = torch.empty((B.snapshot_slots(T, 1, snap_chunks), hv, dv, dk), dtype=torch.float32, device="cuda")
        aff_m = torch.empty((1, hv, dk, dk), dtype=torch.float32, device="cuda")
        aff_b = torch.empty((1, hv, dv, dk), dtype=torch.float32, device="cuda")
        # slowly decaying gates (g / 1000: about 19 bits of decay over a part of 256 chunks), so that no
        # part summary finds a decay horizon and every summary runs over its whole part: the time the
        # call takes when the gates keep a long memory
        g_slow = g * 1e-3
        legs = {
            "plain": lambda: B.gdn_prefill(q, k, v, g, beta, ps0, out=out, final_state=fin, workspace=ws, **pkw),
            # from raw projections (fused q/k normalisation and gate activations; the normalised inputs
            # and their gates stand in as values)
            "raw": lambda: B.gdn_prefill(q, k, v, g, beta, None, None, out=out, final_state=fin, raw=True,
                                         workspace=ws),
            # with a state snapshot every 4096 tokens (prefix reuse)
            "snapshots": lambda: B.gdn_prefill_snapshots(q, k, v, g, beta, snap_chunks, snapshots=snaps, out=out,
                                                         final_state=fin, workspace=ws),
            "slow_gates": lambda: B.gdn_prefill(q, k, v, g_slow, beta, ps0, out=out, final_state=fin, workspace=ws,
                                                **pkw),
            # the affine state map of the whole sequence (per-device half of a sequence-sharded prefill)
            "affine": lambda: B.gdn_prefill_affine(k, v, g, beta, transition=aff_m, offset=aff_b, workspace=ws),
        }
        leg_ms = {name: [] for name in legs}
        for rnd in range(7):
            for name, f in legs.items():
                f()
                f()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(5):
                    f()
                b.record(stream)
                torch.cuda.synchronize()
                if rnd > 0:
                    leg_ms[name].append(a.elapsed_time(b) / 5)
        med = {name: float(np.median(t)) for name, t in leg_ms.items()}
        for name, m_ in med.items():
            log(f"prefill leg {name} (alternating rounds): {m_:.3f} ms/call")
        alt_note = "median over 6 rounds that alternate the plain, raw, snapshot, slow-gate and affine calls"
        raw_rec = {"workload": "prefill_256k from raw projections (q, k normalised and gates activated inside the "
                               "kernels, gdn_prefill_raw)",
                   "ms_per_call": round(med["raw"], 4), "tokens_per_s": round(T / (med["raw"] * 1e-3), 1),
                   "plain_ms_same_rounds": round(med["plain"], 4), "timing": alt_note}
        snapshot_rec = {"workload": f"prefill_256k with a state snapshot every {64 * snap_chunks} tokens "
                                    f"({T // (64 * snap_chunks)} snapshots x 16 heads, gdn_prefill_snapshots)",
                        "ms_per_call": round(med["snapshots"], 4),
                        "tokens_per_s": round(T / (med["snapshots"] * 1e-3), 1),
                        "plain_ms_same_rounds": round(med["plain"], 4), "timing": alt_note}
        slow_rec = {"workload": "prefill_256k with the gates g scaled by 1/1000 (about 19 bits of decay per part: "
                                "no part summary starts at a decay horizon)",
                    "ms_per_call": round(med["slow_gates"], 4),
                    "tokens_per_s": round(T / (med["slow_gates"] * 1e-3), 1),
                    "hbm_frac": round(bytes_call / (med["slow_gates"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "plain_ms_same_rounds": round(med["plain"], 4), "timing": alt_note}
        affine_rec = {"workload": "prefill_256k summarised to its state map S -> S M + B (every part's map, "
                                  "composed; gdn_prefill_affine)",
                      "ms_per_call": round(med["affine"], 4), "tokens_per_s": round(T / (med["affine"] * 1e-3), 1),
                      "plain_ms_same_rounds": round(med["plain"], 4), "timing": alt_note}
        del snaps, aff_m, aff_b, g_slow, legs
    del q, k, v, g, beta, out, ws
    torch.cuda.empty_cache()

    # the two smaller prefill workloads, reported beside the headline: 4,096 tokens x 16 heads, and 8
    # packed sequences of U[1024, 16384] tokens with 32 value heads on 16 q/k heads and initial states
    other = None
    if not args.no_variants and headline:
        other = {}
        for name, reps in (("prefill_4k", 50), ("varlen_8x", 50)):
            o_inp = gi.make_inputs(name, seed=0)
            ow = o_inp.wl
            oq, ok, ov, og, ob = (dev(x) for x in (o_inp.q, o_inp.k, o_inp.v, o_inp.g, o_inp.beta))
            ocu = dev(o_inp.cu_seqlens) if o_inp.cu_seqlens is not None else None
            os0 = dev(o_inp.init_state) if o_inp.init_state is not None else None
            kw = dict(cu_seqlens=ocu) if ocu is not None else dict(num_seqs=ow.num_seqs)
            oo = torch.empty((ow.total_tokens, ow.num_v_heads, ow.head_dim_v), dtype=torch.bfloat16, device="cuda")
            of = torch.empty((ow.num_seqs, ow.num_v_heads, ow.head_dim_v, ow.head_dim_k), dtype=torch.float32,
                             device="cuda")
            ows = torch.empty(max(B.gdn_prefill_workspace_size(oq, ov, **kw), 256), dtype=torch.uint8,
                              device="cuda")
            for _ in range(args.warmup):
                B.gdn_prefill(oq, ok, ov, og, ob, os0, out=oo, final_state=of, workspace=ows, **kw)
            torch.cuda.synchronize()
            oev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for a, b in oev:
                a.record(stream)
                B.gdn_prefill(oq, ok, ov, og, ob, os0, out=oo, final_state=of, workspace=ows, **kw)
                b.record(stream)
            torch.cuda.synchronize()
            t = np.array([a.elapsed_time(b) for a, b in oev])
            tmed = float(np.median(t)) * 1e-3
            obytes = prefill_bytes(ow.total_tokens, ow.num_seqs, ow.num_qk_heads, ow.num_v_heads, ow.head_dim_k,
                                   ow.head_dim_v, init=os0 is not None)
            oflops = prefill_flops_per_token(ow.num_qk_heads, ow.num_v_heads, ow.head_dim_k, ow.head_dim_v) * \
                ow.total_tokens
            other[name] = {"workload": f"{name}: {ow.num_seqs} seq(s), {ow.total_tokens} tokens, H_qk={ow.num_qk_heads}, "
                                       f"H_v={ow.num_v_heads}, d={ow.head_dim_k}, bf16",
                           "ms_median": round(float(np.median(t)), 4),
                           "tokens_per_s": round(ow.total_tokens / tmed, 1),
                           "roofline": {"bound": "hbm", "achieved": round(obytes / tmed / 1e9, 1),
                                        "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                        "frac": round(obytes / tmed / 1e9 / HBM_PEAK_GBS, 4),
                                        "bytes_per_call": obytes,
                                        "mfma_tflops": round(oflops / tmed / 1e12, 1),
                                        "mfma_frac_of_bf16_peak": round(oflops / tmed / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}}
            log(f"{name}: median {np.median(t):.4f} ms/call, {other[name]['tokens_per_s'] / 1e6:.1f} M tokens/s")
            del oq, ok, ov, og, ob, ocu, os0, oo, of, o_inp, ows
        torch.cuda.empty_cache()

    # ------------------------------------------------------------- decode leg
    decode = None
    if not args.no_decode:
        t_gen = time.time()
        d = gi.make_inputs("decode_256x64", seed=0)
        N, dhqk, dhv, ddk, ddv = d.wl.num_seqs, d.wl.num_qk_heads, d.wl.num_v_heads, d.wl.head_dim_k, d.wl.head_dim_v
        state = dev(d.init_state)
        steps = [tuple(dev(s[n]) for n in ("q", "k", "v", "g", "beta")) for s in d.steps]
        dout = torch.empty((N, dhv, ddv), dtype=torch.bfloat16, device="cuda")
        log(f"decode inputs generated and uploaded in {time.time() - t_gen:.1f}s")

        def run64():
            for s in steps:
                B.gdn_decode_step(*s, state, out=dout)

        run64()
        torch.cuda.synchronize()
        dev_ms = []
        for _ in range(args.decode_runs):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run64()
            b.record(stream)
            torch.cuda.synchronize()
            dev_ms.append(a.elapsed_time(b) / len(steps))
        dms = float(np.mean(dev_ms))
        dbytes = decode_bytes(N, dhqk, dhv, ddk, ddv)
        dgbs = dbytes / (dms * 1e-3) / 1e9
        assert torch.isfinite(state).all().item()
        dtraffic = measured_traffic("gdn_decode", DECODE_SOURCES)
        decode = {
            "workload": "decode_256x64: 256 seqs x 16 heads, d=128, bf16 q/k/v, fp32 state [256,16,128,128] in place, 64 steps",
            "value": round(dgbs, 1), "unit": "GB/s", "ms_per_step": round(dms, 5),
            "tokens_per_s": round(N / (dms * 1e-3), 1),
            "roofline": {"bound": "hbm", "achieved": round(dgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(dgbs / HBM_PEAK_GBS, 4),
                         "traffic": None if dtraffic is None else round(dtraffic / (dms * 1e-3) / 1e9, 1),
                         "bytes_per_step": dbytes},
        }
        log(f"decode: {dms * 1e3:.1f} us/step, {dgbs:.0f} GB/s")
        del state, steps, d
        torch.cuda.empty_cache()

        if not args.no_variants:
            # multi-token decode: 256 sequences advance 4 tokens per call, with per-token states
            m = gi.make_inputs("draft_256x4", seed=0)
            MT = m.wl.seqlens[0]
            mN = m.wl.num_seqs
            mst = dev(m.init_state)
            margs = tuple(dev(x) for x in (m.q, m.k, m.v, m.g, m.beta))
            mout = torch.empty((mN * MT, dhv, ddv), dtype=torch.bfloat16, device="cuda")
            mts = torch.empty((mN, MT, dhv, ddv, ddk), dtype=torch.float32, device="cuda")

            def run_mt(n):
                for _ in range(n):
                    B.gdn_decode_tokens(*margs, mst, MT, out=mout, token_states=mts)

            run_mt(3)
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            run_mt(20)
            b.record(stream)
            torch.cuda.synchronize()
            mms = a.elapsed_time(b) / 20
            mbytes = decode_tokens_bytes(mN, MT, dhqk, dhv, ddk, ddv)
            mgbs = mbytes / (mms * 1e-3) / 1e9
            assert torch.isfinite(mst).all().item()
            decode["multi_token"] = {
                "workload": "draft_256x4: 256 seqs x 4 tokens x 16 heads, d=128, bf16, fp32 state in place, "
                            "per-token states written (gdn_decode_tokens)",
                "value": round(mgbs, 1), "unit": "GB/s", "ms_per_call": round(mms, 5),
                "tokens_per_s": round(mN * MT / (mms * 1e-3), 1),
                "roofline": {"bound": "hbm", "achieved": round(mgbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": round(mgbs / HBM_PEAK_GBS, 4), "bytes_per_call": mbytes},
            }
            log(f"multi-token decode: {mms * 1e3:.1f} us/call ({MT} tokens), {mgbs:.0f} GB/s")

            # one decode step over a pool of 512 states, the batch's 256 sequences on permuted slots
            pool = torch.zeros((2 * mN, dhv, ddv, ddk), dtype=torch.float32, device="cuda")
            sidx = torch.randperm(2 * mN, generator=torch.Generator().manual_seed(0))[:mN].to(torch.int32).cuda()
            sargs = tuple(x[::MT].contiguous() for x in margs)
            sout = torch.empty((mN, dhv, ddv), dtype=torch.bfloat16, device="cuda")
            for _ in range(3):
                B.gdn_decode_slots(*sargs, pool, sidx, 1, out=sout)
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(20):
                B.gdn_decode_slots(*sargs, pool, sidx, 1, out=sout)
            b.record(stream)
            torch.cuda.synchronize()
            pms = a.elapsed_time(b) / 20
            pbytes = decode_bytes(mN, dhqk, dhv, ddk, ddv)
            decode["state_pool"] = {
                "workload": "one decode step of 256 seqs x 16 heads over a pool of 512 states (permuted slots, "
                            "gdn_decode_slots)",
                "value": round(pbytes / (pms * 1e-3) / 1e9, 1), "unit": "GB/s", "ms_per_step": round(pms, 5)}
            log(f"decode over a state pool: {pms * 1e3:.1f} us/step, {pbytes / (pms * 1e-3) / 1e9:.0f} GB/s")
            del pool, sidx, sargs, sout
            del mst, margs, mout, mts, m
        torch.cuda.empty_cache()

    # ------------------------------------------------------------ CPU baseline
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import c_oracle
        Ts = min(args.cpu_sample_tokens, T)
        sub = inp
        threads = min(16, os.cpu_count() or 1, hv)
        t1 = time.perf_counter()
        c_oracle.prefill(sub.q[:Ts], sub.k[:Ts], sub.v[:Ts], sub.g[:Ts], sub.beta[:Ts], None, None,
                         nthreads=threads)
        cw = time.perf_counter() - t1
        cpu = {"value": round(Ts / cw, 1), "unit": "tokens/s", "cores": c_oracle.threads(threads),
               "kind": "oracle",
               "sample": (f"the whole T=262144, H=16, d=128 prefill (all 16 heads)" if Ts == T else
                          f"first {Ts} tokens of the T=262144, H=16, d=128 prefill (all 16 heads)")
                         + f", fp64 sequential oracle, {cw:.1f}s wall"}
        # One thread on a shorter prefix of the same workload, for the per-core rate.
        T1 = min(8192, Ts)
        t1 = time.perf_counter()
        c_oracle.prefill(sub.q[:T1], sub.k[:T1], sub.v[:T1], sub.g[:T1], sub.beta[:T1], None, None,
                         nthreads=1)
        cw1 = time.perf_counter() - t1
        cpu["single_thread"] = {"value": round(T1 / cw1, 1), "unit": "tokens/s",
                                "sample": f"first {T1} tokens, all 16 heads, {cw1:.1f}s wall"}
        cpu["host"] = {"cpus": os.cpu_count(), "model": _cpu_model()}
        log(f"cpu oracle: {Ts} tokens in {cw:.1f}s on {cpu['cores']} threads; "
            f"{T1} tokens in {cw1:.1f}s on 1 thread")

    if args.calib_copy:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    rec = {
        "metric": "GDN prefill tokens/sec (T=262144, H=16, d=128); decode state GB/s",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_p10_median_p90": [round(float(np.percentile(per_call_ms, x)), 4) for x in (10, 50, 90)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded: q,k ~ N(0,1) L2-normalised, v ~ N(0,1), beta = sigmoid(N(0,1)), g = -softplus(N(0,1)))",
        "config": {"workload": "prefill_256k: B=1, T=262144, H_qk=H_v=16, d_k=d_v=128, bf16 I/O, fp32 gates and state, zero initial state, chunk 64"
                   if headline else args.prefill_workload,
                   "global_batch": 1, "seq_len": T, "parallelism": "single GPU"},
        "counters": counters,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic / (ms * 1e-3) / 1e9, 1),
                     "kernel": "gdn_prefill call (prep, summary, link and output kernels)",
                     "bytes_per_call": bytes_call,
                     "mfma_tflops": round(tflops, 1),
                     "mfma_frac_of_bf16_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)},
        "cpu_baseline": cpu,
        "decode": decode,
        "prefill_snapshots": snapshot_rec,
        "prefill_raw": raw_rec,
        "prefill_affine": affine_rec,
        "prefill_slow_gates": slow_rec,
        "method_note": "with these gates every part summary starts at its decay horizon (the chunks before it reach "
                       "the part's end scaled by at most 2^-160, every token a contraction; checked on the device "
                       "per call): prefill_slow_gates is the same call with g / 1000, where no summary has one",
        "prefill_other_workloads": other,
        "context": VENDOR_CONTEXT,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
