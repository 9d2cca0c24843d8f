// gdn_decode.hip -- GDN state updates for decoding, fused into a single pass
// over the fp32 state (HBM-bound): one token per sequence, or several tokens
// per sequence with the state held in registers between them.
//
// Per (sequence n, value head h) with state S (d_v x d_k, fp32, row-major),
// alpha = exp(g), and the gated delta rule expanded into its rank-1 form:
//     s_k = S k,  s_q = S q,  u = beta (v - alpha s_k),
//     S  <- alpha S + u k^T,   o = S q = alpha s_q + (k . q) u.
// Row i of the new state depends only on row i of the old one, on v_i and on
// the shared k, q, alpha, beta, so each state row is read once, reduced
// against k and q, and written back at once: 2 x 64 KiB of HBM traffic per
// (n, h) at d = 128 and no other state traffic.  The recurrence is the
// layer's fixed-size per-head state (flozi.net, "Qwen3.8-Flash-Next
// architecture", "Der Weg eines Tokens durch das Modell", item 1: no
// per-token KV entry, hence O(1) memory per decoded token).
//
// Layout of the work: one 256-thread workgroup per (n, h).  Eight
// consecutive lanes share a state row; lane `sub` holds the float4 columns
// 4*sub + 32*j, so each wave-wide load covers eight full 128-byte lines.
// Every lane issues all of its state loads (DV/32 rows x DK/32 float4) before
// the first reduction, keeping 16 KiB per wave in flight.  Row sums over the
// eight lanes use DPP (quad swaps, then the half-row mirror).  State traffic
// is marked non-temporal: each byte is touched exactly once per step.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

// DPP lane move; the patterns used here give every lane a source, so no "old"
// value is needed.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 8 consecutive lanes (a half DPP row) that share a state row.
__device__ __forceinline__ float sum8(float x) {
    x += dpp_mov<0xB1>(x);   // quad_perm [1,0,3,2]: swap neighbours
    x += dpp_mov<0x4E>(x);   // quad_perm [2,3,0,1]: swap pairs -> quad sum
    x += dpp_mov<0x141>(x);  // row_half_mirror: lane i <- lane 7-i (other quad)
    return x;
}

template <typename IO>
__device__ __forceinline__ void load4(const IO* p, float* dst) {
    if constexpr (sizeof(IO) == 2) {
        bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
        dst[0] = (float)v[0]; dst[1] = (float)v[1]; dst[2] = (float)v[2]; dst[3] = (float)v[3];
    } else {
        f32x4 v = *reinterpret_cast<const f32x4*>(p);
        dst[0] = v[0]; dst[1] = v[1]; dst[2] = v[2]; dst[3] = v[3];
    }
}

template <typename IO, int DK, int DV>
__global__ __launch_bounds__(256) void gdn_decode_kernel(DecodeArgs a) {
    constexpr int LPR = 8;                 // lanes per state row
    constexpr int NJ = DK / (4 * LPR);     // float4 per lane per row
    constexpr int RPP = 256 / LPR;         // rows per pass
    constexpr int NM = DV / RPP;           // rows per lane
    static_assert(NJ >= 1 && NM >= 1, "unsupported head dims");

    const int unit = blockIdx.x;           // n * hv + h
    const int n = unit / a.hv;
    const int h = unit - n * a.hv;
    const int hq = (h * a.hqk) / a.hv;
    const int tid = threadIdx.x;
    const int sub = tid & (LPR - 1);
    const int rg = tid / LPR;

    const IO* qp = static_cast<const IO*>(a.q) + ((size_t)n * a.hqk + hq) * DK;
    const IO* kp = static_cast<const IO*>(a.k) + ((size_t)n * a.hqk + hq) * DK;
    const IO* vp = static_cast<const IO*>(a.v) + (size_t)unit * DV;
    IO* op = static_cast<IO*>(a.out) + (size_t)unit * DV;
    float* S = a.state + (size_t)unit * DV * DK;

    // state rows first: all loads in flight before any arithmetic
    f32x4 s[NM][NJ];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            s[m][j] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4*>(S + (size_t)(rg + RPP * m) * DK + 4 * sub + 32 * j));

    float kr[4 * NJ], qr[4 * NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        load4<IO>(kp + 4 * sub + 32 * j, kr + 4 * j);
        load4<IO>(qp + 4 * sub + 32 * j, qr + 4 * j);
    }
    float vr[NM];
#pragma unroll
    for (int m = 0; m < NM; ++m) vr[m] = to_f32(vp[rg + RPP * m]);
    const float alpha = expf(a.g[unit]);
    const float beta = a.beta[unit];

    float kq = 0.f;
#pragma unroll
    for (int e = 0; e < 4 * NJ; ++e) kq += kr[e] * qr[e];
    kq = sum8(kq);

#pragma unroll
    for (int m = 0; m < NM; ++m) {
        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sk += s[m][j][e] * kr[4 * j + e];
                sq += s[m][j][e] * qr[4 * j + e];
            }
        sk = sum8(sk);
        sq = sum8(sq);
        const float u = beta * (vr[m] - alpha * sk);
        const float o = alpha * sq + kq * u;
        const int row = rg + RPP * m;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            f32x4 nv;
#pragma unroll
            for (int e = 0; e < 4; ++e) nv[e] = alpha * s[m][j][e] + u * kr[4 * j + e];
            __builtin_nontemporal_store(nv, reinterpret_cast<f32x4*>(S + (size_t)row * DK + 4 * sub + 32 * j));
        }
        if (sub == 0) op[row] = from_f32<IO>(o);
    }
}

// Several tokens per sequence in one pass over the state (draft verification
// and multi-token decode): the state rows stay in the lanes' registers while
// the T tokens of the sequence are applied in order, exactly as T single
// steps would (same rank-1 form, same per-row order of operations).  The
// next token's inputs are fetched while the current one is applied.  If
// token_states is given, the state after every token is written there
// ([N, T, Hv, dv, dk]), so that a caller can roll back to any accepted
// prefix; the final state always goes back to `state`.  With slot_idx, the
// state of sequence n is slot slot_idx[n] of a state pool (serving engines
// keep the states of all live requests in one pool and pass each batch's
// slots); negative slots mark padding rows and are skipped.  HBM traffic per
// (n, h): the state read and written once (plus T states when requested) and
// the T tokens' q, k, v, out, gates.
template <typename IO, int DK, int DV, bool RAW>
__global__ __launch_bounds__(256) void gdn_decode_tokens_kernel(DecodeArgs a) {
    constexpr int LPR = 8, NJ = DK / (4 * LPR), RPP = 256 / LPR, NM = DV / RPP;
    static_assert(NJ >= 1 && NM >= 1, "unsupported head dims");
    const int unit = blockIdx.x;           // n * hv + h
    const int n = unit / a.hv;
    const int h = unit - n * a.hv;
    const int hq = (h * a.hqk) / a.hv;
    const int tid = threadIdx.x, sub = tid & (LPR - 1), rg = tid / LPR;
    const int T = a.tokens;
    int64_t slot = n;
    if (a.slot_idx) {
        slot = a.slot_idx[n];
        if (slot < 0 || slot >= a.pool_slots) return;   // padding entry (or out of the pool): skipped
    }
    float* S = a.state + ((size_t)slot * a.hv + h) * DV * DK;

    f32x4 s[NM][NJ];
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            s[m][j] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4*>(S + (size_t)(rg + RPP * m) * DK + 4 * sub + 32 * j));

    struct Tok {
        float kr[4 * NJ], qr[4 * NJ], vr[NM], alpha, beta;
    };
    auto fetch = [&](int t, Tok& x) {
        const size_t tok = (size_t)n * T + t;
        const IO* qp = static_cast<const IO*>(a.q) + (tok * a.hqk + hq) * DK;
        const IO* kp = static_cast<const IO*>(a.k) + (tok * a.hqk + hq) * DK;
        const IO* vp = static_cast<const IO*>(a.v) + (tok * a.hv + h) * DV;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            load4<IO>(kp + 4 * sub + 32 * j, x.kr + 4 * j);
            load4<IO>(qp + 4 * sub + 32 * j, x.qr + 4 * j);
        }
#pragma unroll
        for (int m = 0; m < NM; ++m) x.vr[m] = to_f32(vp[rg + RPP * m]);
        if constexpr (RAW) {   // the eight lanes of a row group hold all of k and q
            float kk2 = 0.f, qq2 = 0.f;
#pragma unroll
            for (int e = 0; e < 4 * NJ; ++e) {
                kk2 += x.kr[e] * x.kr[e];
                qq2 += x.qr[e] * x.qr[e];
            }
            const float ik = 1.f / sqrtf(sum8(kk2) + kNormEps), iq = 1.f / sqrtf(sum8(qq2) + kNormEps);
#pragma unroll
            for (int e = 0; e < 4 * NJ; ++e) {
                x.kr[e] *= ik;
                x.qr[e] *= iq;
            }
            x.alpha = expf(gate_from_logit(a.g[tok * a.hv + h]));
            x.beta = beta_from_logit(a.beta[tok * a.hv + h]);
        } else {
            x.alpha = expf(a.g[tok * a.hv + h]);
            x.beta = a.beta[tok * a.hv + h];
        }
    };

    Tok cur, nxt;
    fetch(0, cur);
    for (int t = 0; t < T; ++t) {
        if (t + 1 < T) fetch(t + 1, nxt);
        float kq = 0.f;
#pragma unroll
        for (int e = 0; e < 4 * NJ; ++e) kq += cur.kr[e] * cur.qr[e];
        kq = sum8(kq);
        IO* op = static_cast<IO*>(a.out) + ((size_t)n * T + t) * a.hv * DV + (size_t)h * DV;
        float* ts = a.token_states ? a.token_states + (((size_t)n * T + t) * a.hv + h) * DV * DK : nullptr;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    sk += s[m][j][e] * cur.kr[4 * j + e];
                    sq += s[m][j][e] * cur.qr[4 * j + e];
                }
            sk = sum8(sk);
            sq = sum8(sq);
            const float u = cur.beta * (cur.vr[m] - cur.alpha * sk);
            const float o = cur.alpha * sq + kq * u;
            const int row = rg + RPP * m;
#pragma unroll
            for (int j = 0; j < NJ; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) s[m][j][e] = cur.alpha * s[m][j][e] + u * cur.kr[4 * j + e];
            if (ts) {
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    __builtin_nontemporal_store(s[m][j], reinterpret_cast<f32x4*>(ts + (size_t)row * DK + 4 * sub + 32 * j));
            }
            if (sub == 0) op[row] = from_f32<IO>(o);
        }
        cur = nxt;
    }
#pragma unroll
    for (int m = 0; m < NM; ++m)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            __builtin_nontemporal_store(s[m][j], reinterpret_cast<f32x4*>(S + (size_t)(rg + RPP * m) * DK + 4 * sub + 32 * j));
}

template <typename IO>
hipError_t launch_decode_t(const DecodeArgs& a, int dk, int dv, hipStream_t st) {
    dim3 grid((unsigned)((int64_t)a.num_seqs * a.hv)), block(256);
    if (dk == 128 && dv == 128) hipLaunchKernelGGL((gdn_decode_kernel<IO, 128, 128>), grid, block, 0, st, a);
    else if (dk == 128 && dv == 64) hipLaunchKernelGGL((gdn_decode_kernel<IO, 128, 64>), grid, block, 0, st, a);
    else if (dk == 64 && dv == 128) hipLaunchKernelGGL((gdn_decode_kernel<IO, 64, 128>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((gdn_decode_kernel<IO, 64, 64>), grid, block, 0, st, a);
    return hipGetLastError();
}

template <typename IO, bool RAW>
hipError_t launch_decode_tokens_t(const DecodeArgs& a, int dk, int dv, hipStream_t st) {
    dim3 grid((unsigned)((int64_t)a.num_seqs * a.hv)), block(256);
    if (dk == 128 && dv == 128) hipLaunchKernelGGL((gdn_decode_tokens_kernel<IO, 128, 128, RAW>), grid, block, 0, st, a);
    else if (dk == 128 && dv == 64) hipLaunchKernelGGL((gdn_decode_tokens_kernel<IO, 128, 64, RAW>), grid, block, 0, st, a);
    else if (dk == 64 && dv == 128) hipLaunchKernelGGL((gdn_decode_tokens_kernel<IO, 64, 128, RAW>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((gdn_decode_tokens_kernel<IO, 64, 64, RAW>), grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_tokens(const DecodeArgs& a, bool bf16, int dk, int dv, hipStream_t st, bool raw) {
    if (a.num_seqs == 0) return hipSuccess;
    if (raw)
        return bf16 ? launch_decode_tokens_t<__bf16, true>(a, dk, dv, st) : launch_decode_tokens_t<float, true>(a, dk, dv, st);
    return bf16 ? launch_decode_tokens_t<__bf16, false>(a, dk, dv, st) : launch_decode_tokens_t<float, false>(a, dk, dv, st);
}

hipError_t launch_decode(const DecodeArgs& a, bool bf16, int dk, int dv, hipStream_t st) {
    if (a.num_seqs == 0) return hipSuccess;
    return bf16 ? launch_decode_t<__bf16>(a, dk, dv, st) : launch_decode_t<float>(a, dk, dv, st);
}

}  // namespace gdn
