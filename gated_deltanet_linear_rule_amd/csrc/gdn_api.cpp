// gdn_api.cpp -- the C ABI of libgdn.so (declared in include/gdn.h).
//
// Validates every host-checkable argument before touching HIP, picks the
// kernel variant, takes the prefill workspace from the caller (the *_ws entry
// points) or from the device's default stream-ordered pool, and enqueues the
// kernels on the caller's stream.  No exception or abort crosses the ABI; the
// text of the last failure is kept per thread.  The library keeps no state
// between calls and changes no process-wide setting.
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
    const char* s = std::getenv("GDN_DEBUG_SYNC");
    return s && s[0] && s[0] != '0';
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

// Compute units of the current device (0 if the query fails); queried on every
// call, so the library keeps no per-device state.
int current_compute_units() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return cus;
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

// Which prefill entry point a call comes from (selects the kernels and the
// workspace layout).
enum PrefillKind { kPlain, kRaw, kSnapshots, kAffine };

// The part length, slot counts and workspace layout of one prefill call on
// the current device; `packed` tells whether cu_seqlens will be given.
gdn_status plan_prefill(const gdn_shape* shape, bool packed, PrefillKind kind, gdn::PrefillArgs& a, bool& split,
                        int64_t& total) {
    a.num_tokens = shape->num_tokens;
    a.seqlen = shape->num_tokens / shape->num_seqs;
    a.num_seqs = shape->num_seqs;
    a.hqk = shape->num_qk_heads;
    a.hv = shape->num_v_heads;
    a.dv = shape->head_dim_v;
    a.num_slots = (shape->num_tokens + 63) / 64 + shape->num_seqs;
    if (a.num_slots > INT32_MAX) return fail(GDN_ERROR_NOT_SUPPORTED, "too many chunks");
    const int cus = current_compute_units();
    if (cus <= 0) return fail(GDN_ERROR_LAUNCH, "cannot query the device's compute units");
    // the two-launch schedule of packed batches: plain and raw-projection calls,
    // bf16, d_k = d_v
    const gdn::PartPlan pp = gdn::prefill_part_plan(
        a.num_tokens, a.num_seqs, a.hv, cus,
        (kind == kPlain || kind == kRaw) && shape->head_dim_k == shape->head_dim_v && shape->dtype == GDN_DTYPE_BF16,
        packed);
    a.part_chunks = pp.part_chunks;
    a.first_chunks = pp.first_chunks;
    a.cut_chunks = pp.cut_chunks;
    a.phase = pp.phase;
    const int64_t span = a.part_chunks * 64;
    a.num_part_slots = (a.num_tokens + span - 1) / span + a.num_seqs;
    const int64_t longest = packed ? (a.num_tokens + 63) / 64 : (a.seqlen + 63) / 64;
    // the affine map needs every sequence's part maps, split or not
    split = kind == kAffine || longest > (a.first_chunks > a.cut_chunks ? a.first_chunks : a.cut_chunks);
    if (3 * a.num_part_slots * a.hv > INT32_MAX ||
        (a.num_seqs * (int64_t)a.hv + 7) * (a.dv / 16 + shape->head_dim_k / 16) > INT32_MAX)
        return fail(GDN_ERROR_NOT_SUPPORTED, "too many (part, head) pairs");
    const gdn::PrefillWorkspace wl(a.num_slots, a.num_part_slots, split, a.hv, shape->head_dim_k, shape->head_dim_v,
                                   shape->dtype == GDN_DTYPE_BF16 ? 2 : 4, kind == kRaw);
    total = wl.total;
    return GDN_SUCCESS;
}

// The arguments of every prefill entry point (unused ones NULL / 0).
struct PrefillCall {
    const void *q, *k, *v;
    const float *g, *beta, *init_state;
    const int32_t* cu;
    void* out;
    float* final_state;
    int32_t snapshot_chunks;
    float* snapshots;
    float *transition, *offset;   // affine map
};

// Static scratch for gdn_prefill_static: one array per device, allocated when
// the library's code object is loaded onto that device and held until the
// process ends.  In host code `scratch` is only a host-side stand-in for the
// symbol; its device address comes from hipGetSymbolAddress, looked up once
// per device (with that device current) and kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[GDN_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the first
// call on that device), or NULL with the error recorded.
void* scratch_address(gdn_status& st) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        st = fail(GDN_ERROR_LAUNCH, "prefill_static: no usable current device (%d)", dev);
        return nullptr;
    }
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            st = fail(GDN_ERROR_LAUNCH, "prefill_static: scratch address lookup on device %d: %s", dev,
                      hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

// Where a prefill call's workspace comes from: the current device's default
// stream-ordered pool (hipMallocAsync / hipFreeAsync on the call's stream; the
// pool's settings are left as the caller set them), the caller, or the static
// scratch array.
enum WsSource { kPoolWs, kCallerWs, kStaticWs };

// Validates a prefill call, lays out its workspace and enqueues its kernels.
gdn_status prefill_impl(const char* who, PrefillKind kind, const gdn_shape* shape, const PrefillCall& c, void* stream,
                        WsSource src, void* workspace = nullptr, size_t workspace_bytes = 0) {
    g_last_error[0] = '\0';
    const bool caller_ws = src == kCallerWs;
    if (caller_ws && !workspace) return fail(GDN_ERROR_INVALID_VALUE, "workspace is NULL");
    if (kind == kSnapshots && !c.snapshots) return fail(GDN_ERROR_INVALID_VALUE, "snapshots is NULL");
    GDN_TRY(check_shape(shape, false));
    const bool tok = shape->num_tokens > 0, any = shape->num_seqs > 0;
    const bool affine = kind == kAffine;
    if (!affine) GDN_TRY(check_ptr(c.q, "q", 16, tok));
    GDN_TRY(check_ptr(c.k, "k", 16, tok));
    GDN_TRY(check_ptr(c.v, "v", 16, tok));
    GDN_TRY(check_ptr(c.g, "g", 4, tok));
    GDN_TRY(check_ptr(c.beta, "beta", 4, tok));
    if (affine) {
        GDN_TRY(check_ptr(c.transition, "transition", 16, any));
        GDN_TRY(check_ptr(c.offset, "offset", 16, any));
    } else {
        GDN_TRY(check_ptr(c.out, "out", 16, tok));
        GDN_TRY(check_ptr(c.init_state, "init_state", 16, false));
        GDN_TRY(check_ptr(c.final_state, "final_state", 16, false));
    }
    GDN_TRY(check_ptr(c.cu, "cu_seqlens", 4, false));
    GDN_TRY(check_ptr(workspace, "workspace", 256, false));
    if (!c.cu && any && shape->num_tokens % shape->num_seqs != 0)
        return fail(GDN_ERROR_INVALID_VALUE, "num_tokens (%lld) is not a multiple of num_seqs (%d) and no cu_seqlens",
                    (long long)shape->num_tokens, shape->num_seqs);
    const size_t sbytes = (size_t)shape->num_seqs * shape->num_v_heads * shape->head_dim_v * shape->head_dim_k * 4;
    if (c.init_state && c.final_state && c.init_state != c.final_state) {
        const char* a0 = reinterpret_cast<const char*>(c.init_state);
        const char* b0 = reinterpret_cast<const char*>(c.final_state);
        if (a0 < b0 + sbytes && b0 < a0 + sbytes)
            return fail(GDN_ERROR_INVALID_VALUE, "init_state and final_state overlap partially");
    }
    if (affine && any) {
        const size_t mb = (size_t)shape->num_seqs * shape->num_v_heads * shape->head_dim_k * shape->head_dim_k * 4;
        const char* m0 = reinterpret_cast<const char*>(c.transition);
        const char* b0 = reinterpret_cast<const char*>(c.offset);
        if (m0 < b0 + sbytes && b0 < m0 + mb) return fail(GDN_ERROR_INVALID_VALUE, "transition and offset overlap");
    }
    if (kind == kSnapshots) {
        GDN_TRY(check_ptr(c.snapshots, "snapshots", 16, true));
        if (c.snapshot_chunks <= 0)
            return fail(GDN_ERROR_INVALID_VALUE, "snapshot_chunks must be positive (got %d)", c.snapshot_chunks);
    }
    if (!any) return GDN_SUCCESS;

    const bool bf16 = shape->dtype == GDN_DTYPE_BF16;
    gdn::PrefillArgs a{};
    a.q = affine ? c.k : c.q;
    a.k = c.k; a.v = c.v; a.g = c.g; a.beta = c.beta;
    a.init_state = c.init_state; a.cu = c.cu; a.out = c.out; a.final_state = c.final_state;
    a.snapshots = kind == kSnapshots ? c.snapshots : nullptr;
    a.snap_chunks = kind == kSnapshots ? c.snapshot_chunks : 0;
    a.aff_m = affine ? c.transition : nullptr;
    a.aff_b = affine ? c.offset : nullptr;
    bool split = false;
    int64_t total = 0;
    GDN_TRY(plan_prefill(shape, c.cu != nullptr, kind, a, split, total));
    const gdn::PrefillWorkspace wl(a.num_slots, a.num_part_slots, split, a.hv, shape->head_dim_k, shape->head_dim_v,
                                   bf16 ? 2 : 4, kind == kRaw);
    hipStream_t st = static_cast<hipStream_t>(stream);
    void* ws = workspace;
    if (caller_ws) {
        if (workspace_bytes < (size_t)total)
            return fail(GDN_ERROR_INVALID_VALUE, "workspace of %zu bytes, this call needs %lld", workspace_bytes,
                        (long long)total);
    } else if (src == kStaticWs) {
        if ((size_t)total > (size_t)GDN_STATIC_SCRATCH_BYTES)
            return fail(GDN_ERROR_NOT_SUPPORTED,
                        "%s: this call needs %lld bytes of scratch, the static scratch holds %zu (use "
                        "gdn_prefill_ws with a caller workspace)", who, (long long)total,
                        (size_t)GDN_STATIC_SCRATCH_BYTES);
        gdn_status sst = GDN_SUCCESS;
        ws = scratch_address(sst);
        if (!ws) return sst;
    } else if (hipMallocAsync(&ws, (size_t)total, st) != hipSuccess || !ws) {
        (void)hipGetLastError();
        return fail(GDN_ERROR_OUT_OF_MEMORY, "%s workspace of %lld bytes", who, (long long)total);
    }
    char* wc = static_cast<char*>(ws);
    a.ws_t = wc + wl.t;
    a.ws_g = reinterpret_cast<double*>(wc + wl.g);
    a.ws_ik = kind == kRaw ? reinterpret_cast<float*>(wc + wl.ik) : nullptr;
    a.ws_hz = reinterpret_cast<float*>(wc + wl.hz);
    a.ws_m = split ? reinterpret_cast<float*>(wc + wl.m) : nullptr;
    a.ws_b = split ? reinterpret_cast<float*>(wc + wl.b) : nullptr;
    a.ws_s = split ? reinterpret_cast<float*>(wc + wl.s) : nullptr;
    a.ws_hf = split ? reinterpret_cast<int32_t*>(wc + wl.hf) : nullptr;
    const int dk = shape->head_dim_k, dv = shape->head_dim_v;
    hipError_t e = affine ? gdn::launch_prefill_affine(a, bf16, dk, dv, st)
                          : gdn::launch_prefill(a, bf16, dk, dv, st, kind == kRaw);
    if (src == kPoolWs) {
        const hipError_t ef = hipFreeAsync(ws, st);
        if (e == hipSuccess) e = ef;
    }
    if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(GDN_ERROR_LAUNCH, "%s: %s", who, hipGetErrorString(e));
    return GDN_SUCCESS;
}

PrefillCall call_of(const void* q, const void* k, const void* v, const float* g, const float* beta,
                    const float* init_state, const int32_t* cu, void* out, float* final_state) {
    PrefillCall c{};
    c.q = q; c.k = k; c.v = v; c.g = g; c.beta = beta;
    c.init_state = init_state; c.cu = cu; c.out = out; c.final_state = final_state;
    return c;
}

PrefillCall affine_call(const void* k, const void* v, const float* g, const float* beta, const int32_t* cu,
                        float* transition, float* offset) {
    PrefillCall c{};
    c.k = k; c.v = v; c.g = g; c.beta = beta; c.cu = cu;
    c.transition = transition; c.offset = offset;
    return c;
}

}  // namespace

extern "C" {

gdn_status gdn_prefill_workspace_size(const gdn_shape* shape, uint32_t flags, size_t* bytes) {
    g_last_error[0] = '\0';
    if (!bytes) return fail(GDN_ERROR_INVALID_VALUE, "bytes is NULL");
    *bytes = 0;
    if (flags & ~(uint32_t)(GDN_WS_PACKED | GDN_WS_RAW | GDN_WS_AFFINE))
        return fail(GDN_ERROR_INVALID_VALUE, "unknown workspace flags 0x%x", (unsigned)flags);
    if ((flags & GDN_WS_RAW) && (flags & GDN_WS_AFFINE))
        return fail(GDN_ERROR_INVALID_VALUE, "GDN_WS_RAW and GDN_WS_AFFINE exclude each other");
    GDN_TRY(check_shape(shape, false));
    const bool packed = (flags & GDN_WS_PACKED) != 0;
    if (!packed && shape->num_seqs > 0 && shape->num_tokens % shape->num_seqs != 0)
        return fail(GDN_ERROR_INVALID_VALUE, "num_tokens (%lld) is not a multiple of num_seqs (%d) and not packed",
                    (long long)shape->num_tokens, shape->num_seqs);
    if (shape->num_seqs == 0) return GDN_SUCCESS;
    gdn::PrefillArgs a{};
    bool split = false;
    int64_t total = 0;
    const PrefillKind kind = (flags & GDN_WS_RAW) ? kRaw : (flags & GDN_WS_AFFINE) ? kAffine : kPlain;
    GDN_TRY(plan_prefill(shape, packed, kind, a, split, total));
    *bytes = (size_t)total;
    return GDN_SUCCESS;
}

gdn_status gdn_prefill(const gdn_shape* shape, const void* q, const void* k, const void* v, const float* g,
                       const float* beta, const float* init_state, const int32_t* cu_seqlens, void* out,
                       float* final_state, void* stream) {
    return prefill_impl("prefill", kPlain, shape, call_of(q, k, v, g, beta, init_state, cu_seqlens, out, final_state),
                        stream, kPoolWs);
}

gdn_status gdn_prefill_ws(const gdn_shape* shape, const void* q, const void* k, const void* v, const float* g,
                          const float* beta, const float* init_state, const int32_t* cu_seqlens, void* out,
                          float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl("prefill_ws", kPlain, shape,
                        call_of(q, k, v, g, beta, init_state, cu_seqlens, out, final_state), stream, kCallerWs, workspace,
                        workspace_bytes);
}

gdn_status gdn_prefill_static(const gdn_shape* shape, const void* q, const void* k, const void* v, const float* g,
                              const float* beta, const float* init_state, const int32_t* cu_seqlens, void* out,
                              float* final_state, void* stream) {
    return prefill_impl("prefill_static", kPlain, shape,
                        call_of(q, k, v, g, beta, init_state, cu_seqlens, out, final_state), stream, kStaticWs);
}

gdn_status gdn_prefill_raw(const gdn_shape* shape, const void* q, const void* k, const void* v, const float* a_gate,
                           const float* b_beta, const float* init_state, const int32_t* cu_seqlens, void* out,
                           float* final_state, void* stream) {
    return prefill_impl("prefill_raw", kRaw, shape,
                        call_of(q, k, v, a_gate, b_beta, init_state, cu_seqlens, out, final_state), stream, kPoolWs);
}

gdn_status gdn_prefill_raw_ws(const gdn_shape* shape, const void* q, const void* k, const void* v,
                              const float* a_gate, const float* b_beta, const float* init_state,
                              const int32_t* cu_seqlens, void* out, float* final_state, void* workspace,
                              size_t workspace_bytes, void* stream) {
    return prefill_impl("prefill_raw_ws", kRaw, shape,
                        call_of(q, k, v, a_gate, b_beta, init_state, cu_seqlens, out, final_state), stream, kCallerWs,
                        workspace, workspace_bytes);
}

gdn_status gdn_prefill_snapshots(const gdn_shape* shape, const void* q, const void* k, const void* v,
                                 const float* g, const float* beta, const float* init_state,
                                 const int32_t* cu_seqlens, void* out, float* final_state, int32_t snapshot_chunks,
                                 float* snapshots, void* stream) {
    PrefillCall c = call_of(q, k, v, g, beta, init_state, cu_seqlens, out, final_state);
    c.snapshot_chunks = snapshot_chunks;
    c.snapshots = snapshots;
    return prefill_impl("prefill_snapshots", kSnapshots, shape, c, stream, kPoolWs);
}

gdn_status gdn_prefill_snapshots_ws(const gdn_shape* shape, const void* q, const void* k, const void* v,
                                    const float* g, const float* beta, const float* init_state,
                                    const int32_t* cu_seqlens, void* out, float* final_state,
                                    int32_t snapshot_chunks, float* snapshots, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    PrefillCall c = call_of(q, k, v, g, beta, init_state, cu_seqlens, out, final_state);
    c.snapshot_chunks = snapshot_chunks;
    c.snapshots = snapshots;
    return prefill_impl("prefill_snapshots_ws", kSnapshots, shape, c, stream, kCallerWs, workspace, workspace_bytes);
}

gdn_status gdn_prefill_affine(const gdn_shape* shape, const void* k, const void* v, const float* g,
                              const float* beta, const int32_t* cu_seqlens, float* transition, float* offset,
                              void* stream) {
    return prefill_impl("prefill_affine", kAffine, shape, affine_call(k, v, g, beta, cu_seqlens, transition, offset),
                        stream, kPoolWs);
}

gdn_status gdn_prefill_affine_ws(const gdn_shape* shape, const void* k, const void* v, const float* g,
                                 const float* beta, const int32_t* cu_seqlens, float* transition, float* offset,
                                 void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_impl("prefill_affine_ws", kAffine, shape,
                        affine_call(k, v, g, beta, cu_seqlens, transition, offset), stream, kCallerWs, workspace,
                        workspace_bytes);
}

}  // extern "C"
