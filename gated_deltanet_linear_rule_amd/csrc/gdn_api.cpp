// gdn_api.cpp -- the C ABI of libgdn.so (declared in include/gdn.h).
//
// Validates every host-checkable argument before touching HIP, picks the
// kernel variant, takes the prefill workspace from HIP's stream-ordered pool
// (or from the caller, gdn_prefill_ws) and enqueues the kernels on the
// caller's stream.  No exception or abort
// crosses the ABI; the text of the last failure is kept per thread.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "gdn.h"
#include "gdn_internal.h"

namespace {

thread_local char g_last_error[512] = "";

gdn_status fail(gdn_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Optional debugging aid: GDN_DEBUG_SYNC=1 synchronises the stream after each
// call and reports asynchronous kernel errors as GDN_ERROR_LAUNCH.
bool debug_sync() {
    static const bool on = [] {
        const char* s = std::getenv("GDN_DEBUG_SYNC");
        return s && s[0] && s[0] != '0';
    }();
    return on;
}

gdn_status check_shape(const gdn_shape* s, bool decode) {
    if (!s) return fail(GDN_ERROR_INVALID_VALUE, "shape is NULL");
    if (s->num_seqs < 0 || s->num_tokens < 0)
        return fail(GDN_ERROR_INVALID_VALUE, "negative size (num_seqs=%d, num_tokens=%lld)", s->num_seqs,
                    (long long)s->num_tokens);
    if (s->num_qk_heads <= 0 || s->num_v_heads <= 0 || s->head_dim_k <= 0 || s->head_dim_v <= 0)
        return fail(GDN_ERROR_INVALID_VALUE, "head counts and head dims must be positive");
    if (s->num_v_heads % s->num_qk_heads != 0)
        return fail(GDN_ERROR_INVALID_VALUE, "num_v_heads (%d) is not a multiple of num_qk_heads (%d)",
                    s->num_v_heads, s->num_qk_heads);
    if (s->dtype != GDN_DTYPE_F32 && s->dtype != GDN_DTYPE_BF16)
        return fail(GDN_ERROR_INVALID_VALUE, "unknown dtype %d", (int)s->dtype);
    if (decode && s->num_tokens != s->num_seqs)
        return fail(GDN_ERROR_INVALID_VALUE, "decode needs num_tokens == num_seqs (got %lld, %d)",
                    (long long)s->num_tokens, s->num_seqs);
    if (s->num_seqs == 0 && s->num_tokens != 0)
        return fail(GDN_ERROR_INVALID_VALUE, "tokens without sequences");
    if ((s->head_dim_k != 64 && s->head_dim_k != 128) || (s->head_dim_v != 64 && s->head_dim_v != 128))
        return fail(GDN_ERROR_NOT_SUPPORTED, "head dims (%d, %d) not in {64, 128}", s->head_dim_k,
                    s->head_dim_v);
    const int64_t units = (int64_t)s->num_seqs * s->num_v_heads;
    if (units > INT32_MAX) return fail(GDN_ERROR_NOT_SUPPORTED, "too many (sequence, head) pairs");
    return GDN_SUCCESS;
}

gdn_status check_ptr(const void* p, const char* name, uintptr_t align, bool required) {
    if (!p) return required ? fail(GDN_ERROR_INVALID_VALUE, "%s is NULL", name) : GDN_SUCCESS;
    if (!aligned(p, align)) return fail(GDN_ERROR_INVALID_VALUE, "%s is not %u-byte aligned", name, (unsigned)align);
    return GDN_SUCCESS;
}

#define GDN_TRY(expr)                         \
    do {                                      \
        gdn_status st_ = (expr);              \
        if (st_ != GDN_SUCCESS) return st_;   \
    } while (0)

// Keep freed workspace in HIP's default pool instead of returning it to the
// driver at every synchronisation (set once per device).
void keep_pool_memory(int dev) {
    static std::mutex mu;
    static bool done[64] = {};
    if (dev < 0 || dev >= 64) return;
    std::lock_guard<std::mutex> lk(mu);
    if (done[dev]) return;
    hipMemPool_t pool;
    if (hipDeviceGetDefaultMemPool(&pool, dev) == hipSuccess) {
        uint64_t thr = UINT64_MAX;
        (void)hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &thr);
    }
    done[dev] = true;
}

// Compute units of device `dev` (cached; 0 if the query fails).
int compute_units(int dev) {
    static std::mutex mu;
    static int cached[64] = {};
    if (dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lk(mu);
    if (cached[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
            (void)hipGetLastError();
            return 0;
        }
        cached[dev] = cus;
    }
    return cached[dev];
}

}  // namespace

extern "C" {

int gdn_abi_version(void) { return GDN_ABI_VERSION; }

const char* gdn_last_error(void) { return g_last_error; }

const char* gdn_status_string(gdn_status status) {
    switch (status) {
        case GDN_SUCCESS: return "success";
        case GDN_ERROR_INVALID_VALUE: return "invalid argument";
        case GDN_ERROR_NOT_SUPPORTED: return "shape or type not supported";
        case GDN_ERROR_LAUNCH: return "kernel launch failed";
        case GDN_ERROR_OUT_OF_MEMORY: return "workspace allocation failed";
    }
    return "unknown status";
}

gdn_status gdn_decode_step(const gdn_shape* shape, const void* q, const void* k, const void* v,
                           const float* g, const float* beta, float* state, void* out, void* stream) {
    g_last_error[0] = '\0';
    GDN_TRY(check_shape(shape, true));
    const bool any = shape->num_seqs > 0;
    GDN_TRY(check_ptr(q, "q", 16, any));
    GDN_TRY(check_ptr(k, "k", 16, any));
    GDN_TRY(check_ptr(v, "v", 16, any));
    GDN_TRY(check_ptr(g, "g", 4, any));
    GDN_TRY(check_ptr(beta, "beta", 4, any));
    GDN_TRY(check_ptr(state, "state", 16, any));
    GDN_TRY(check_ptr(out, "out", 16, any));
    if (!any) return GDN_SUCCESS;
    gdn::DecodeArgs a{q, k, v, g, beta, state, out, shape->num_seqs, shape->num_qk_heads, shape->num_v_heads, 1,
                      nullptr, nullptr, 0};
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = gdn::launch_decode(a, shape->dtype == GDN_DTYPE_BF16, shape->head_dim_k, shape->head_dim_v, st);
    if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(GDN_ERROR_LAUNCH, "decode: %s", hipGetErrorString(e));
    return GDN_SUCCESS;
}

}  // extern "C"

namespace {

gdn_status decode_tokens_impl(const char* who, const gdn_shape* shape, int32_t tokens_per_seq, const void* q,
                              const void* k, const void* v, const float* g, const float* beta, float* state,
                              int64_t pool_slots, const int32_t* slot_idx, void* out, float* token_states,
                              void* stream, bool raw = false) {
    g_last_error[0] = '\0';
    GDN_TRY(check_shape(shape, false));
    if (tokens_per_seq <= 0) return fail(GDN_ERROR_INVALID_VALUE, "tokens_per_seq must be positive (got %d)", tokens_per_seq);
    if (shape->num_tokens != (int64_t)shape->num_seqs * tokens_per_seq)
        return fail(GDN_ERROR_INVALID_VALUE, "num_tokens (%lld) must equal num_seqs * tokens_per_seq (%d * %d)",
                    (long long)shape->num_tokens, shape->num_seqs, tokens_per_seq);
    const bool any = shape->num_seqs > 0;
    const int64_t slots = slot_idx ? pool_slots : shape->num_seqs;
    if (slot_idx && pool_slots < 0) return fail(GDN_ERROR_INVALID_VALUE, "negative pool_slots (%lld)", (long long)pool_slots);
    GDN_TRY(check_ptr(q, "q", 16, any));
    GDN_TRY(check_ptr(k, "k", 16, any));
    GDN_TRY(check_ptr(v, "v", 16, any));
    GDN_TRY(check_ptr(g, "g", 4, any));
    GDN_TRY(check_ptr(beta, "beta", 4, any));
    GDN_TRY(check_ptr(state, "state", 16, any && slots > 0));
    GDN_TRY(check_ptr(out, "out", 16, any));
    GDN_TRY(check_ptr(slot_idx, "slot_idx", 4, false));
    GDN_TRY(check_ptr(token_states, "token_states", 16, false));
    if (token_states && state && any && slots > 0) {
        const size_t sb = (size_t)shape->num_v_heads * shape->head_dim_v * shape->head_dim_k * 4;
        const char* a0 = reinterpret_cast<const char*>(state);
        const char* b0 = reinterpret_cast<const char*>(token_states);
        if (a0 < b0 + sb * (size_t)shape->num_seqs * tokens_per_seq && b0 < a0 + sb * (size_t)slots)
            return fail(GDN_ERROR_INVALID_VALUE, "token_states overlaps state");
    }
    if (!any || slots == 0) return GDN_SUCCESS;
    gdn::DecodeArgs a{q, k, v, g, beta, state, out, shape->num_seqs, shape->num_qk_heads, shape->num_v_heads,
                      tokens_per_seq, token_states, slot_idx, pool_slots};
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = gdn::launch_decode_tokens(a, shape->dtype == GDN_DTYPE_BF16, shape->head_dim_k,
                                             shape->head_dim_v, st, raw);
    if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(GDN_ERROR_LAUNCH, "%s: %s", who, hipGetErrorString(e));
    return GDN_SUCCESS;
}

}  // namespace

extern "C" {

gdn_status gdn_decode_tokens(const gdn_shape* shape, int32_t tokens_per_seq, const void* q, const void* k,
                             const void* v, const float* g, const float* beta, float* state, void* out,
                             float* token_states, void* stream) {
    return decode_tokens_impl("decode_tokens", shape, tokens_per_seq, q, k, v, g, beta, state, 0, nullptr, out,
                              token_states, stream);
}

gdn_status gdn_decode_slots(const gdn_shape* shape, int32_t tokens_per_seq, const void* q, const void* k,
                            const void* v, const float* g, const float* beta, float* state_pool,
                            int64_t pool_slots, const int32_t* slot_idx, void* out, float* token_states,
                            void* stream) {
    if (!slot_idx) {
        g_last_error[0] = '\0';
        return fail(GDN_ERROR_INVALID_VALUE, "slot_idx is NULL");
    }
    return decode_tokens_impl("decode_slots", shape, tokens_per_seq, q, k, v, g, beta, state_pool, pool_slots,
                              slot_idx, out, token_states, stream);
}

gdn_status gdn_decode_tokens_raw(const gdn_shape* shape, int32_t tokens_per_seq, const void* q, const void* k,
                                 const void* v, const float* a_gate, const float* b_beta, float* state, void* out,
                                 float* token_states, void* stream) {
    return decode_tokens_impl("decode_tokens_raw", shape, tokens_per_seq, q, k, v, a_gate, b_beta, state, 0,
                              nullptr, out, token_states, stream, true);
}

}  // extern "C"

namespace {

// The part length, slot counts and workspace layout of one prefill call on
// the current device; `packed` tells whether cu_seqlens will be given.
gdn_status plan_prefill(const gdn_shape* shape, bool packed, bool raw, gdn::PrefillArgs& a, bool& split,
                        int64_t& total) {
    a.num_tokens = shape->num_tokens;
    a.seqlen = shape->num_tokens / shape->num_seqs;
    a.num_seqs = shape->num_seqs;
    a.hqk = shape->num_qk_heads;
    a.hv = shape->num_v_heads;
    a.dv = shape->head_dim_v;
    a.num_slots = (shape->num_tokens + 63) / 64 + shape->num_seqs;
    if (a.num_slots > INT32_MAX) return fail(GDN_ERROR_NOT_SUPPORTED, "too many chunks");
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(GDN_ERROR_LAUNCH, "hipGetDevice failed");
    const int cus = compute_units(dev);
    if (cus <= 0) return fail(GDN_ERROR_LAUNCH, "cannot query the device's compute units");
    a.part_chunks = gdn::prefill_part_chunks(a.num_tokens, a.num_seqs, a.hv, cus);
    const int64_t span = a.part_chunks * 64;
    a.num_part_slots = (a.num_tokens + span - 1) / span + a.num_seqs;
    const int64_t longest = packed ? (a.num_tokens + 63) / 64 : (a.seqlen + 63) / 64;
    split = a.part_chunks < longest;
    if (a.num_part_slots * a.hv > INT32_MAX || a.num_seqs * (int64_t)a.hv * (a.dv / 16) > INT32_MAX)
        return fail(GDN_ERROR_NOT_SUPPORTED, "too many (part, head) pairs");
    const gdn::PrefillWorkspace wl(a.num_slots, a.num_part_slots, split, a.hv, shape->head_dim_k, shape->head_dim_v,
                                   shape->dtype == GDN_DTYPE_BF16 ? 2 : 4, raw);
    total = wl.total;
    return GDN_SUCCESS;
}

// `workspace` NULL: the workspace comes from HIP's stream-ordered pool.
gdn_status prefill_impl(const char* who, const gdn_shape* shape, const void* q, const void* k, const void* v,
                        const float* g, const float* beta, const float* init_state, const int32_t* cu_seqlens,
                        void* out, float* final_state, int32_t snapshot_chunks, float* snapshots, void* stream,
                        bool raw = false, void* workspace = nullptr, size_t workspace_bytes = 0) {
    g_last_error[0] = '\0';
    GDN_TRY(check_shape(shape, false));
    const bool tok = shape->num_tokens > 0;
    GDN_TRY(check_ptr(q, "q", 16, tok));
    GDN_TRY(check_ptr(k, "k", 16, tok));
    GDN_TRY(check_ptr(v, "v", 16, tok));
    GDN_TRY(check_ptr(g, "g", 4, tok));
    GDN_TRY(check_ptr(beta, "beta", 4, tok));
    GDN_TRY(check_ptr(out, "out", 16, tok));
    GDN_TRY(check_ptr(init_state, "init_state", 16, false));
    GDN_TRY(check_ptr(final_state, "final_state", 16, false));
    GDN_TRY(check_ptr(cu_seqlens, "cu_seqlens", 4, false));
    GDN_TRY(check_ptr(workspace, "workspace", 256, false));
    if (!cu_seqlens && shape->num_seqs > 0 && shape->num_tokens % shape->num_seqs != 0)
        return fail(GDN_ERROR_INVALID_VALUE, "num_tokens (%lld) is not a multiple of num_seqs (%d) and no cu_seqlens",
                    (long long)shape->num_tokens, shape->num_seqs);
    if (init_state && final_state && init_state != final_state) {
        const size_t bytes = (size_t)shape->num_seqs * shape->num_v_heads * shape->head_dim_v * shape->head_dim_k * 4;
        const char* a0 = reinterpret_cast<const char*>(init_state);
        const char* b0 = reinterpret_cast<const char*>(final_state);
        if (a0 < b0 + bytes && b0 < a0 + bytes)
            return fail(GDN_ERROR_INVALID_VALUE, "init_state and final_state overlap partially");
    }
    GDN_TRY(check_ptr(snapshots, "snapshots", 16, false));
    if (snapshots && snapshot_chunks <= 0)
        return fail(GDN_ERROR_INVALID_VALUE, "snapshot_chunks must be positive (got %d)", snapshot_chunks);
    if (shape->num_seqs == 0) return GDN_SUCCESS;

    const bool bf16 = shape->dtype == GDN_DTYPE_BF16;
    gdn::PrefillArgs a{};
    a.snapshots = snapshots;
    a.snap_chunks = snapshots ? snapshot_chunks : 0;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.init_state = init_state; a.cu = cu_seqlens; a.out = out; a.final_state = final_state;
    bool split = false;
    int64_t total = 0;
    GDN_TRY(plan_prefill(shape, cu_seqlens != nullptr, raw, a, split, total));
    const gdn::PrefillWorkspace wl(a.num_slots, a.num_part_slots, split, a.hv, shape->head_dim_k, shape->head_dim_v,
                                   bf16 ? 2 : 4, raw);
    hipStream_t st = static_cast<hipStream_t>(stream);
    void* ws = workspace;
    if (workspace) {
        if (workspace_bytes < (size_t)total)
            return fail(GDN_ERROR_INVALID_VALUE, "workspace of %zu bytes, this call needs %lld", workspace_bytes,
                        (long long)total);
    } else {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return fail(GDN_ERROR_LAUNCH, "hipGetDevice failed");
        keep_pool_memory(dev);
        if (hipMallocAsync(&ws, (size_t)total, st) != hipSuccess || !ws) {
            (void)hipGetLastError();
            return fail(GDN_ERROR_OUT_OF_MEMORY, "prefill workspace of %lld bytes", (long long)total);
        }
    }
    char* wc = static_cast<char*>(ws);
    a.ws_t = wc + wl.t;
    a.ws_g = reinterpret_cast<double*>(wc + wl.g);
    a.ws_ik = raw ? reinterpret_cast<float*>(wc + wl.ik) : nullptr;
    a.ws_m = split ? reinterpret_cast<float*>(wc + wl.m) : nullptr;
    a.ws_b = split ? reinterpret_cast<float*>(wc + wl.b) : nullptr;
    a.ws_s = split ? reinterpret_cast<float*>(wc + wl.s) : nullptr;
    hipError_t e = gdn::launch_prefill(a, bf16, shape->head_dim_k, shape->head_dim_v, st, raw);
    if (!workspace) {
        const hipError_t ef = hipFreeAsync(ws, st);
        if (e == hipSuccess) e = ef;
    }
    if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(GDN_ERROR_LAUNCH, "%s: %s", who, hipGetErrorString(e));
    return GDN_SUCCESS;
}

}  // namespace

extern "C" {

gdn_status gdn_prefill(const gdn_shape* shape, const void* q, const void* k, const void* v, const float* g,
                       const float* beta, const float* init_state, const int32_t* cu_seqlens, void* out,
                       float* final_state, void* stream) {
    return prefill_impl("prefill", shape, q, k, v, g, beta, init_state, cu_seqlens, out, final_state, 0, nullptr,
                        stream);
}

gdn_status gdn_prefill_workspace_size(const gdn_shape* shape, int32_t packed, size_t* bytes) {
    g_last_error[0] = '\0';
    if (!bytes) return fail(GDN_ERROR_INVALID_VALUE, "bytes is NULL");
    *bytes = 0;
    GDN_TRY(check_shape(shape, false));
    if (!packed && shape->num_seqs > 0 && shape->num_tokens % shape->num_seqs != 0)
        return fail(GDN_ERROR_INVALID_VALUE, "num_tokens (%lld) is not a multiple of num_seqs (%d) and not packed",
                    (long long)shape->num_tokens, shape->num_seqs);
    if (shape->num_seqs == 0) return GDN_SUCCESS;
    gdn::PrefillArgs a{};
    bool split = false;
    int64_t total = 0;
    GDN_TRY(plan_prefill(shape, packed != 0, false, a, split, total));
    *bytes = (size_t)total;
    return GDN_SUCCESS;
}

gdn_status gdn_prefill_ws(const gdn_shape* shape, const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const float* init_state, const int32_t* cu_seqlens, void* out,
                          float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
    if (!workspace) {
        g_last_error[0] = '\0';
        return fail(GDN_ERROR_INVALID_VALUE, "workspace is NULL");
    }
    return prefill_impl("prefill_ws", shape, q, k, v, g, beta, init_state, cu_seqlens, out, final_state, 0, nullptr,
                        stream, false, workspace, workspace_bytes);
}

gdn_status gdn_prefill_affine(const gdn_shape* shape, const void* k, const void* v, const float* g,
                              const float* beta, const int32_t* cu_seqlens, float* transition, float* offset,
                              void* stream) {
    g_last_error[0] = '\0';
    GDN_TRY(check_shape(shape, false));
    const bool tok = shape->num_tokens > 0;
    GDN_TRY(check_ptr(k, "k", 16, tok));
    GDN_TRY(check_ptr(v, "v", 16, tok));
    GDN_TRY(check_ptr(g, "g", 4, tok));
    GDN_TRY(check_ptr(beta, "beta", 4, tok));
    GDN_TRY(check_ptr(cu_seqlens, "cu_seqlens", 4, false));
    const bool any = shape->num_seqs > 0;
    GDN_TRY(check_ptr(transition, "transition", 16, any));
    GDN_TRY(check_ptr(offset, "offset", 16, any));
    if (!cu_seqlens && shape->num_seqs > 0 && shape->num_tokens % shape->num_seqs != 0)
        return fail(GDN_ERROR_INVALID_VALUE, "num_tokens (%lld) is not a multiple of num_seqs (%d) and no cu_seqlens",
                    (long long)shape->num_tokens, shape->num_seqs);
    if (!any) return GDN_SUCCESS;
    {
        const size_t mb = (size_t)shape->num_seqs * shape->num_v_heads * shape->head_dim_k * shape->head_dim_k * 4;
        const size_t bb = (size_t)shape->num_seqs * shape->num_v_heads * shape->head_dim_v * shape->head_dim_k * 4;
        const char* m0 = reinterpret_cast<const char*>(transition);
        const char* b0 = reinterpret_cast<const char*>(offset);
        if (m0 < b0 + bb && b0 < m0 + mb) return fail(GDN_ERROR_INVALID_VALUE, "transition and offset overlap");
    }
    const bool bf16 = shape->dtype == GDN_DTYPE_BF16;
    gdn::PrefillArgs a{};
    a.q = k; a.k = k; a.v = v; a.g = g; a.beta = beta;
    a.cu = cu_seqlens;
    a.aff_m = transition;
    a.aff_b = offset;
    bool split = false;
    int64_t total = 0;
    GDN_TRY(plan_prefill(shape, cu_seqlens != nullptr, false, a, split, total));
    // every sequence gets its part maps, split or not
    const gdn::PrefillWorkspace wl(a.num_slots, a.num_part_slots, true, a.hv, shape->head_dim_k, shape->head_dim_v,
                                   bf16 ? 2 : 4);
    hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(GDN_ERROR_LAUNCH, "hipGetDevice failed");
    keep_pool_memory(dev);
    void* ws = nullptr;
    if (hipMallocAsync(&ws, (size_t)wl.total, st) != hipSuccess || !ws) {
        (void)hipGetLastError();
        return fail(GDN_ERROR_OUT_OF_MEMORY, "prefill_affine workspace of %lld bytes", (long long)wl.total);
    }
    char* wc = static_cast<char*>(ws);
    a.ws_t = wc + wl.t;
    a.ws_g = reinterpret_cast<double*>(wc + wl.g);
    a.ws_m = reinterpret_cast<float*>(wc + wl.m);
    a.ws_b = reinterpret_cast<float*>(wc + wl.b);
    a.ws_s = reinterpret_cast<float*>(wc + wl.s);
    hipError_t e = gdn::launch_prefill_affine(a, bf16, shape->head_dim_k, shape->head_dim_v, st);
    const hipError_t ef = hipFreeAsync(ws, st);
    if (e == hipSuccess) e = ef;
    if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(GDN_ERROR_LAUNCH, "prefill_affine: %s", hipGetErrorString(e));
    return GDN_SUCCESS;
}

gdn_status gdn_prefill_snapshots(const gdn_shape* shape, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const float* init_state,
                                 const int32_t* cu_seqlens, void* out, float* final_state, int32_t snapshot_chunks,
                                 float* snapshots, void* stream) {
    if (!snapshots) {
        g_last_error[0] = '\0';
        return fail(GDN_ERROR_INVALID_VALUE, "snapshots is NULL");
    }
    return prefill_impl("prefill_snapshots", shape, q, k, v, g, beta, init_state, cu_seqlens, out, final_state,
                        snapshot_chunks, snapshots, stream);
}

gdn_status gdn_prefill_raw(const gdn_shape* shape, const void* q, const void* k, const void* v, const float* a_gate,
                           const float* b_beta, const float* init_state, const int32_t* cu_seqlens, void* out,
                           float* final_state, void* stream) {
    return prefill_impl("prefill_raw", shape, q, k, v, a_gate, b_beta, init_state, cu_seqlens, out, final_state, 0,
                        nullptr, stream, true);
}

}  // extern "C"
