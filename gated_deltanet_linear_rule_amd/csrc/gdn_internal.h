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
    int64_t num_slots;         // ceil(num_tokens / 64) + num_seqs
    // Workspace written by the prep kernel and read by the scan, per (slot,
    // value head), in the order of the scan's matrix-core operands:
    void* ws_w;                // 64 x dk  W  = T~ diag(gamma) K
    void* ws_q;                // 64 x dk  Q~ = diag(gamma) Q
    void* ws_k;                // dk x 64  K~^T = (diag(e^{G_last - G}) K)^T
    void* ws_u;                // 64 x dv  u  = T~ V
    void* ws_p;                // 64 x 64  P  = lower_incl(Gamma o Q K^T)
    float* ws_g;               // G2_last: log2 of the chunk's total decay
    // One launch covers chunk indices [seg_j0, seg_j1) of every sequence.  The
    // scan starts from state_in (NULL = zeros) and ends in state_out (NULL =
    // not kept).  seg_len = 0: the prep kernel walks every slot; seg_len > 0:
    // it walks (sequence, chunk in the range, value head) items.
    int64_t seg_j0, seg_j1;
    int32_t seg_len;
    const float* state_in;
    float* state_out;
};

// Workspace layout of one prefill call (byte offsets of each part and total),
// element size 2 for bf16, 4 for fp32.
struct PrefillWorkspace {
    int64_t w, q, k, u, p, g, total;
    PrefillWorkspace(int64_t num_slots, int hv, int dk, int dv, int elem_size) {
        const int64_t blocks = num_slots * hv;
        const int64_t mk = blocks * 64 * (int64_t)dk * elem_size;
        w = 0;
        q = w + mk;
        k = q + mk;
        u = k + mk;
        p = u + blocks * 64 * (int64_t)dv * elem_size;
        g = p + blocks * 64 * 64 * (int64_t)elem_size;
        total = g + ((blocks * 4 + 255) / 256) * 256;
    }
};

// Chunks per segment when the prefill is split into segments whose prep and
// scan overlap (0: one launch of each kernel).  Segmenting pays when the scan
// alone cannot fill the device (few sequences x heads) and sequences are long.
int64_t prefill_segment_chunks(int64_t num_tokens, int num_seqs, int hv, int dv);

// Launchers: return hipSuccess or the launch error.  `bf16` selects the
// element type of q/k/v/out; dk/dv are 64 or 128.
hipError_t launch_decode(const DecodeArgs& a, bool bf16, int dk, int dv, hipStream_t s);
// `state_ws` (N * hv * dv * dk floats) carries the state between segments;
// it may be NULL when prefill_segment_chunks() returned 0.
hipError_t launch_prefill(const PrefillArgs& a, bool bf16, int dk, int dv, float* state_ws, hipStream_t s);

}  // namespace gdn
