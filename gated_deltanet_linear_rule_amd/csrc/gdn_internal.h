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
    // Workspace written by the prep kernel and read by the scan, per (slot, value head):
    void* ws_t;                // 64 x 64 T~ = (I + A)^-1 diag(beta), fragment-major order
    void* ws_p;                // 64 x 64 P = lower_incl(Gamma o Q K^T), fragment-major order
    float* ws_g;               // 64 pairs (G2_t, G2_last - G2_t): log2-scaled cumulative gates
};

// Workspace bytes per (slot, value head) of each part (element size 2 for bf16, 4 for fp32).
inline int64_t prefill_matrix_bytes(int elem_size) { return (int64_t)64 * 64 * elem_size; }
inline int64_t prefill_gate_bytes() { return (int64_t)64 * 2 * 4; }
// Workspace bytes for one prefill call: T~, P and the gates of every (slot, value head).
inline int64_t prefill_workspace_bytes(int64_t num_slots, int hv, int elem_size) {
    return num_slots * (int64_t)hv * (2 * prefill_matrix_bytes(elem_size) + prefill_gate_bytes());
}

// Launchers: return hipSuccess or the launch error.  `bf16` selects the
// element type of q/k/v/out; dk/dv are 64 or 128.
hipError_t launch_decode(const DecodeArgs& a, bool bf16, int dk, int dv, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs& a, bool bf16, int dk, hipStream_t s);

}  // namespace gdn
