// gdn_internal.h -- host-side launch interface between the C ABI (gdn_api.cpp)
// and the kernels.  Arguments here are already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    float* state;
    void* out;
    int32_t num_seqs;
    int32_t hqk;
    int32_t hv;
    int32_t tokens;          // tokens per sequence (multi-token decode; 1 for a step)
    float* token_states;     // [N, tokens, Hv, dv, dk] or nullptr (multi-token decode)
    const int32_t* slot_idx; // state of sequence n at state[slot_idx[n]] (nullptr: slot n)
    int64_t pool_slots;      // slots in `state` when slot_idx is given; others are skipped
};

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const float* init_state;   // nullable
    const int32_t* cu;         // nullable (equal lengths)
    void* out;
    float* final_state;        // nullable
    int64_t num_tokens;
    int64_t seqlen;            // equal length when cu == nullptr
    int32_t num_seqs;
    int32_t hqk;
    int32_t hv;
    int32_t dv;
    int64_t num_slots;         // chunk slots: ceil(num_tokens / 64) + num_seqs
    int64_t part_chunks;       // L: chunks per part
    int64_t first_chunks;      // F: chunks of a cut sequence's first part (later parts: L)
    int64_t cut_chunks;        // sequences of at most this many chunks (or of at most F) are
                               // one part
    int64_t num_part_slots;    // part slots: ceil(num_tokens / (64 L)) + num_seqs
    int32_t phase;             // 0: one output pass over every part; 1: two launches (first
                               // parts beside the later parts' summaries, later parts after
                               // the link)
    // Workspace.  Per (chunk slot, value head), written by the prep kernel:
    void* ws_t;                // T~ = (I + A)^{-1} diag(beta) without its diagonal, as operand
                               // fragments (5 KB bf16, 12 KB fp32)
    double* ws_g;              // 1.25 KB gate record: 64 log2-scaled cumulative gates (fp64),
                               // then 64 gamma, 64 D and 64 beta (fp32)
    float* ws_ik;              // raw projections only: 64 values 1 / |k_t| (256 B)
    float* ws_hz;              // the chunk's log2 decay sum_t g_t / ln 2 when every token of it is
                               // a contraction (0 <= beta_t |k_t|^2 <= 1.99, g_t <= 0), else +inf
                               // (4 B; read by the summary's decay horizon)
    // Per (part slot, value head), fp32 row-major; NULL when no sequence has
    // more than one part:
    float* ws_m;               // d_k x d_k transition M_p of the part, transposed (see m_pos)
    float* ws_b;               // d_v x d_k offset B_p of the part (state from zero)
    float* ws_s;               // d_v x d_k start state S_p of the part
    int32_t* ws_hf;            // 1 if the part's summary started at its decay horizon (M_p is
                               // negligible: S_{p+1} = B_p), else 0
    // Optional state snapshots every snap_chunks chunks of each sequence:
    // snapshot s (state after the first 64 s snap_chunks tokens) of sequence n
    // at slot floor(start(n) / (64 snap_chunks)) + n + s - 1.
    float* snapshots;          // [slots, Hv, dv, dk] or nullptr
    int32_t snap_chunks;
    // Affine map of each sequence (gdn_prefill_affine): the summary covers
    // every part and the link composes them, from zero (offset rows) and from
    // the identity (transition rows), into these instead of start states:
    float* aff_m;              // [N, Hv, dk, dk] transition, or nullptr (ordinary prefill)
    float* aff_b;              // [N, Hv, dv, dk] offset
};

// Workspace layout of one prefill call (byte offsets of each part and total),
// element size 2 for bf16, 4 for fp32.
struct PrefillWorkspace {
    int64_t t, g, ik, hz, m, b, s, hf, total;
    PrefillWorkspace(int64_t num_slots, int64_t num_part_slots, bool split, int hv, int dk, int dv, int elem_size,
                     bool raw = false) {
        auto up = [](int64_t x) { return (x + 255) / 256 * 256; };
        const int64_t blocks = num_slots * hv, pblocks = split ? num_part_slots * hv : 0;
        t = 0;
        g = t + up(blocks * (elem_size == 2 ? 5 : 12) * 1024);   // T~: 5 KB bf16, 12 KB fp32
        ik = g + up(blocks * 1280);                               // gate record: 1.25 KB
        hz = ik + (raw ? up(blocks * 256) : 0);
        m = hz + up(blocks * 4);                                  // chunk decay / contraction: 4 B
        b = m + up(pblocks * dk * dk * 4);
        s = b + up(pblocks * dv * dk * 4);
        hf = s + up(pblocks * dv * dk * 4);
        total = hf + up(pblocks * 4);                             // horizon flags: 4 B
    }
};

// How a prefill call cuts its sequences into parts (PrefillArgs::part_chunks,
// first_chunks, cut_chunks, phase).  two_launch: bf16, d_k = d_v, plain or
// raw-projection call; packed: cu_seqlens given.  With fewer (sequence, value
// head) chains than compute units every sequence is cut into parts of about
// one compute unit's share.  With one to two chains per compute unit on packed
// two_launch input, the sequences longer than one share keep a first part of
// about one share and are cut into short parts after it (two launches).
// Otherwise every sequence is one part.
struct PartPlan {
    int64_t part_chunks, first_chunks, cut_chunks;
    int32_t phase;
};
PartPlan prefill_part_plan(int64_t num_tokens, int num_seqs, int hv, int num_cus, bool two_launch, bool packed);

// Launchers: return hipSuccess or the launch error.  `bf16` selects the
// element type of q/k/v/out; dk/dv are 64 or 128.
hipError_t launch_decode(const DecodeArgs& a, bool bf16, int dk, int dv, hipStream_t s);
hipError_t launch_decode_tokens(const DecodeArgs& a, bool bf16, int dk, int dv, hipStream_t s, bool raw = false);
// raw: q, k unnormalised and g, beta given as logits (see gdn_prefill_raw).
hipError_t launch_prefill(const PrefillArgs& a, bool bf16, int dk, int dv, hipStream_t s, bool raw = false);
// The affine map of each sequence (a.aff_m, a.aff_b set; q and out unused).
hipError_t launch_prefill_affine(const PrefillArgs& a, bool bf16, int dk, int dv, hipStream_t s);

}  // namespace gdn
