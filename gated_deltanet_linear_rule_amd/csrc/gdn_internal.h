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
    // Workspace written by the prep kernel and read by the scan, in the order
    // of the scan's operand fragments ("fragment-major"):
    void* ws_t;                // per (slot, value head): 64 x 64 T~ = (I + A)^-1 diag(beta)
    void* ws_p;                // per (slot, value head): 64 x 64 P = lower_incl(Gamma o Q K^T)
    float* ws_g;               // per (slot, value head): 64 pairs (G2_t, G2_last - G2_t)
    void* ws_k;                // per (slot, q/k head): the chunk's 64 x dk block of K
    void* ws_q;                // per (slot, q/k head): the chunk's 64 x dk block of Q
};

// Workspace layout of one prefill call (byte offsets of each part and total),
// element size 2 for bf16, 4 for fp32.
struct PrefillWorkspace {
    int64_t t, p, g, k, q, total;
    PrefillWorkspace(int64_t num_slots, int hqk, int hv, int dk, int elem_size) {
        const int64_t mat = num_slots * hv * 64 * 64 * (int64_t)elem_size;
        const int64_t gate = num_slots * hv * 64 * 2 * 4;
        const int64_t kq = num_slots * hqk * 64 * (int64_t)dk * elem_size;
        t = 0;
        p = t + mat;
        g = p + mat;
        k = g + gate;
        q = k + kq;
        total = q + kq;
    }
};

// Launchers: return hipSuccess or the launch error.  `bf16` selects the
// element type of q/k/v/out; dk/dv are 64 or 128.
hipError_t launch_decode(const DecodeArgs& a, bool bf16, int dk, int dv, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, bool bf16, int dk, hipStream_t s);

}  // namespace gdn
