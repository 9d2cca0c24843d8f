// gdn_prefill.hip -- chunk-wise (WY / UT transform) GDN prefill for gfx950.
//
// The recurrence S_t = alpha_t S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
// o_t = S_t q_t (the GDN layer's fixed-size per-head state: flozi.net,
// "Qwen3.8-Flash-Next architecture", "Der Weg eines Tokens durch das
// Modell", item 1) is evaluated over chunks of C = 64 tokens.  Within a chunk
// with start state S, cumulative log-decay G_t = g_1 + ... + g_t (so every
// exponent below is <= 0), gamma_t = e^{G_t}, Gamma_ts = e^{G_t - G_s}:
//
//   A  = strict_lower(diag(beta) (Gamma o K K^T)),   T = (I + A)^{-1}
//   T~ = T diag(beta),   P = lower_incl(Gamma o Q K^T)         [state-free]
//   R  = V - diag(gamma) K S^T
//   U  = T~ R                       (the chunk's effective writes u_t)
//   O  = diag(gamma) Q S^T + P U
//   S' = gamma_n S + U^T diag(e^{G_n - G}) K
//
// Two kernels:
//  * gdn_prep_kernel  -- one workgroup per (chunk, value head), all chunks in
//    parallel: stages K and Q in LDS, the gate cumsum, Gamma-weighted K K^T and
//    Q K^T on bf16 (or fp32) matrix cores, the unit-lower-triangular inverse
//    in LDS (16x16 diagonal blocks by forward substitution, off-diagonal
//    blocks by fp32 MFMA block products), and writes T~ and P to a workspace.
//  * gdn_scan_kernel  -- sequential over the chunks of one sequence, parallel
//    over (sequence, value head, 16-column block of d_v): rows of S are
//    independent, so each wave owns 16 rows of S (as S^T tiles in fp32
//    accumulators: d_k x 16) for the whole sequence and never exchanges them.
//    Per chunk a wave runs X = K S^T, Y = Q S^T, U = T~ R, O = gamma Y + P U
//    and the state update on the matrix cores, with every intermediate kept in
//    registers (accumulator tiles double as operand fragments, see
//    gdn_device.h).  The workgroup's waves share one LDS copy of K (row-major
//    and transposed) and Q per chunk.
//
// Padding: a final partial chunk is padded with k = q = v = 0, g = 0,
// beta = 0; padded rows then carry u = 0 and leave S and the real rows
// untouched, and gamma_n = e^{G_63} equals the decay up to the last real token.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kPrepThreads = 256;

template <typename OP> constexpr int pad_elems() { return 16 / (int)sizeof(OP); }

// Lower 16x16 tiles (tm >= tn) of a 64x64 matrix, in a fixed order.
__constant__ int kLowerTiles[10][2] = {{0, 0}, {1, 0}, {1, 1}, {2, 0}, {2, 1},
                                       {2, 2}, {3, 0}, {3, 1}, {3, 2}, {3, 3}};

// Find the (sequence, chunk) that owns workspace slot `slot`; returns false if
// the slot is a gap.  Slots of sequence n: [base(n), base(n) + ceil(len/64)).
__device__ __forceinline__ bool locate_slot(const SeqIndex& si, int nseq, int64_t slot, int& n_out,
                                            int64_t& t0, int64_t& t1) {
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (slot_base(si.start(mid), mid) <= slot) lo = mid;
        else hi = mid - 1;
    }
    const int64_t s0 = si.start(lo), s1 = si.start(lo + 1);
    const int64_t b = slot_base(s0, lo);
    if (slot < b) return false;
    t0 = s0 + (slot - b) * kChunk;
    t1 = s1;
    n_out = lo;
    return t0 < s1;
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_cumsum(float x) {
    const int l = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        float y = __shfl_up(x, off, kWave);
        if (l >= off) x += y;
    }
    return x;
}

template <typename OP, int DK>
struct PrepSmem {
    static constexpr int LD = DK + pad_elems<OP>();
    OP K[kChunk * LD];
    OP Q[kChunk * LD];
    float A[kChunk][kChunk + 4];
    float T[kChunk][kChunk + 4];
    float G[kChunk];
    float B[kChunk];
};

template <typename OP, int DK>
__global__ __launch_bounds__(kPrepThreads) void gdn_prep_kernel(PrefillArgs a) {
    using Ops = Op<OP>;
    constexpr int LD = PrepSmem<OP, DK>::LD;
    constexpr int VE = 16 / (int)sizeof(OP);      // elements per 16-byte vector
    constexpr int NV = DK / VE;                    // vectors per row
    __shared__ PrepSmem<OP, DK> sm;

    const int64_t slot = blockIdx.x;
    const int h = blockIdx.y;
    const SeqIndex si{a.cu, a.seqlen};
    int n;
    int64_t t0, t1;
    if (!locate_slot(si, a.num_seqs, slot, n, t0, t1)) return;   // uniform over the workgroup
    const int nt = (int)((t1 - t0) < kChunk ? (t1 - t0) : kChunk);
    const int hq = (h * a.hqk) / a.hv;
    const int tid = threadIdx.x, l = lane_id(), w = wave_id(), r = l & 15, gq = l >> 4;

    // ---- stage K, Q (zero rows past the end of the sequence) and gates
    const OP* kg = static_cast<const OP*>(a.k);
    const OP* qg = static_cast<const OP*>(a.q);
    for (int e = tid; e < kChunk * NV; e += kPrepThreads) {
        const int row = e / NV, cv = e - row * NV;
        u32x4 kv = {0u, 0u, 0u, 0u}, qv = {0u, 0u, 0u, 0u};
        if (row < nt) {
            const size_t off = ((size_t)(t0 + row) * a.hqk + hq) * DK + (size_t)cv * VE;
            kv = *reinterpret_cast<const u32x4*>(kg + off);
            qv = *reinterpret_cast<const u32x4*>(qg + off);
        }
        *reinterpret_cast<u32x4*>(&sm.K[row * LD + cv * VE]) = kv;
        *reinterpret_cast<u32x4*>(&sm.Q[row * LD + cv * VE]) = qv;
    }
    if (w == 0) {
        const bool ok = l < nt;
        const float gv = ok ? a.g[(size_t)(t0 + l) * a.hv + h] : 0.f;
        const float bv = ok ? a.beta[(size_t)(t0 + l) * a.hv + h] : 0.f;
        sm.G[l] = wave_cumsum(gv);
        sm.B[l] = bv;
    }
    __syncthreads();

    // ---- Gamma-weighted K K^T (-> A, fp32 in LDS) and Q K^T (-> P, workspace)
    OP* Pw = static_cast<OP*>(a.ws_p) + ((size_t)slot * a.hv + h) * (kChunk * kChunk);
    OP* Tw = static_cast<OP*>(a.ws_t) + ((size_t)slot * a.hv + h) * (kChunk * kChunk);
    for (int job = w; job < 20; job += kPrepThreads / kWave) {
        const bool qk = job >= 10;
        const int tm = kLowerTiles[job % 10][0], tn = kLowerTiles[job % 10][1];
        const OP* X = qk ? sm.Q : sm.K;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk)
            acc = Ops::mma(frag_rows(X, LD, 16 * tm + r, 32 * kk), frag_rows(sm.K, LD, 16 * tn + r, 32 * kk), acc);
        const int s = 16 * tn + r;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * tm + 4 * gq + i;
            if (!qk) {
                sm.A[t][s] = (s < t) ? sm.B[t] * expf(sm.G[t] - sm.G[s]) * acc[i] : 0.f;
            } else {
                Pw[t * kChunk + s] = from_f32<OP>((s <= t) ? expf(sm.G[t] - sm.G[s]) * acc[i] : 0.f);
            }
        }
    }
    // zero the strictly-upper 16x16 tiles of P and T~ (read as padding by the scan)
    for (int e = tid; e < kChunk * kChunk; e += kPrepThreads) {
        const int t = e >> 6, s = e & 63;
        if ((s >> 4) > (t >> 4)) {
            Pw[e] = from_f32<OP>(0.f);
            Tw[e] = from_f32<OP>(0.f);
        }
    }
    __syncthreads();

    // ---- T = (I + A)^{-1}: diagonal 16x16 blocks by forward substitution
    // (lane c of wave b solves column c of block b), fp32.
    if (l < 16) {
        const int b = w, c = l;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float acc = (i == c) ? 1.f : 0.f;
#pragma unroll
            for (int j = 0; j < i; ++j) acc -= sm.A[16 * b + i][16 * b + j] * x[j];
            x[i] = acc;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) sm.T[16 * b + i][16 * b + c] = x[i];
    }
    __syncthreads();
    // Off-diagonal blocks, by distance from the diagonal:
    //   T_mb = -T_mm * sum_{b <= k < m} A_mk T_kb     (fp32 matrix cores)
#pragma unroll
    for (int dist = 1; dist <= 3; ++dist) {
        if (w < 4 - dist) {
            const int b = w, m = w + dist;
            f32x4 z = zero4();
            for (int kb = b; kb < m; ++kb) {
                const f32x4 arow = *reinterpret_cast<const f32x4*>(&sm.A[16 * m + r][16 * kb + 4 * gq]);
                f32x4 tcol;
#pragma unroll
                for (int i = 0; i < 4; ++i) tcol[i] = sm.T[16 * kb + 4 * gq + i][16 * b + r];
                z = mm16_f32(arow, tcol, z);
            }
            const f32x4 trow = *reinterpret_cast<const f32x4*>(&sm.T[16 * m + r][16 * m + 4 * gq]);
            const f32x4 res = mm16_f32(trow, z, zero4());
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.T[16 * m + 4 * gq + i][16 * b + r] = -res[i];
        }
        __syncthreads();
    }

    // ---- T~ = T diag(beta), lower blocks (upper blocks were zeroed above)
    for (int e = tid; e < kChunk * kChunk; e += kPrepThreads) {
        const int t = e >> 6, s = e & 63;
        if ((s >> 4) <= (t >> 4)) Tw[e] = from_f32<OP>((s <= t) ? sm.T[t][s] * sm.B[s] : 0.f);
    }
}

template <typename OP, int DK>
struct ScanSmem {
    static constexpr int LD = DK + pad_elems<OP>();      // K, Q rows (token-major)
    static constexpr int LDT = kChunk + pad_elems<OP>(); // K^T rows (d_k-major)
    OP K[kChunk * LD];
    OP Q[kChunk * LD];
    OP Kt[DK * LDT];
    float G[kChunk];
};

template <typename OP, int DK, int NW>
__global__ __launch_bounds__(NW * kWave) void gdn_scan_kernel(PrefillArgs a) {
    using Ops = Op<OP>;
    using frag = typename Ops::frag;
    constexpr int LD = ScanSmem<OP, DK>::LD;
    constexpr int LDT = ScanSmem<OP, DK>::LDT;
    constexpr int VE = 16 / (int)sizeof(OP);
    constexpr int NV = DK / VE;
    constexpr int NT = NW * kWave;
    constexpr int NTI = DK / 16;   // S^T tiles along d_k
    __shared__ ScanSmem<OP, DK> sm;

    const int chain = blockIdx.x;
    const int n = chain / a.hv;
    const int h = chain - n * a.hv;
    const int hq = (h * a.hqk) / a.hv;
    const int tid = threadIdx.x, l = lane_id(), w = wave_id(), r = l & 15, gq = l >> 4;
    const int c = (blockIdx.y * NW + w) * 16 + r;          // this lane's d_v column
    const int dv = a.dv;

    const SeqIndex si{a.cu, a.seqlen};
    const int64_t s0 = si.start(n), s1 = si.start(n + 1);
    const int64_t base = slot_base(s0, n);

    // S^T tiles: St[ti] holds S[c][16 ti + 4 gq + i], i = 0..3
    f32x4 St[NTI];
    const size_t srow = ((size_t)chain * dv + c) * DK;
#pragma unroll
    for (int ti = 0; ti < NTI; ++ti)
        St[ti] = a.init_state ? *reinterpret_cast<const f32x4*>(a.init_state + srow + 16 * ti + 4 * gq) : zero4();

    const OP* kg = static_cast<const OP*>(a.k);
    const OP* qg = static_cast<const OP*>(a.q);
    const OP* vg = static_cast<const OP*>(a.v);
    OP* og = static_cast<OP*>(a.out);

    int64_t slot = base;
    for (int64_t t0 = s0; t0 < s1; t0 += kChunk, ++slot) {
        const int nt = (int)((s1 - t0) < kChunk ? (s1 - t0) : kChunk);
        __syncthreads();   // previous chunk's LDS reads are complete
        // ---- stage: Q row-major; K row-major and transposed.  A task is 4
        // consecutive tokens x one 16-byte column vector.
        for (int e = tid; e < (kChunk / 4) * NV; e += NT) {
            const int rq = e % (kChunk / 4), cv = e / (kChunk / 4);
            u32x4 kv[4], qv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * rq + i;
                kv[i] = u32x4{0u, 0u, 0u, 0u};
                qv[i] = u32x4{0u, 0u, 0u, 0u};
                if (row < nt) {
                    const size_t off = ((size_t)(t0 + row) * a.hqk + hq) * DK + (size_t)cv * VE;
                    kv[i] = *reinterpret_cast<const u32x4*>(kg + off);
                    qv[i] = *reinterpret_cast<const u32x4*>(qg + off);
                }
                *reinterpret_cast<u32x4*>(&sm.K[row * LD + cv * VE]) = kv[i];
                *reinterpret_cast<u32x4*>(&sm.Q[row * LD + cv * VE]) = qv[i];
            }
#pragma unroll
            for (int e2 = 0; e2 < VE; ++e2) {
                typename Ops::quad col;
#pragma unroll
                for (int i = 0; i < 4; ++i) col[i] = reinterpret_cast<const OP*>(&kv[i])[e2];
                *reinterpret_cast<typename Ops::quad*>(&sm.Kt[(cv * VE + e2) * LDT + 4 * rq]) = col;
            }
        }
        if (w == 0) sm.G[l] = wave_cumsum(l < nt ? a.g[(size_t)(t0 + l) * a.hv + h] : 0.f);
        __syncthreads();

        // ---- X = K S^T, Y = Q S^T (64 tokens x 16 columns)
        frag Sb[DK / 32];
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) Sb[kk] = Ops::pack(St[2 * kk], St[2 * kk + 1]);
        f32x4 X[4], Y[4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            X[tm] = zero4();
            Y[tm] = zero4();
#pragma unroll
            for (int kk = 0; kk < DK / 32; ++kk) {
                X[tm] = Ops::mma(frag_rows(sm.K, LD, 16 * tm + r, 32 * kk), Sb[kk], X[tm]);
                Y[tm] = Ops::mma(frag_rows(sm.Q, LD, 16 * tm + r, 32 * kk), Sb[kk], Y[tm]);
            }
        }
        // ---- gates for this lane's rows
        const float Glast = sm.G[kChunk - 1];
        f32x4 Gv[4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) Gv[tm] = *reinterpret_cast<const f32x4*>(&sm.G[16 * tm + 4 * gq]);
        // ---- R = V - diag(gamma) X
        f32x4 R[4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tm + 4 * gq + i;
                const float vv = (t < nt) ? to_f32(vg[((size_t)(t0 + t) * a.hv + h) * dv + c]) : 0.f;
                R[tm][i] = vv - expf(Gv[tm][i]) * X[tm][i];
            }
        // ---- U = T~ R (T~ lower triangular: skip zero K steps)
        const OP* Tw = static_cast<const OP*>(a.ws_t) + ((size_t)slot * a.hv + h) * (kChunk * kChunk);
        const OP* Pw = static_cast<const OP*>(a.ws_p) + ((size_t)slot * a.hv + h) * (kChunk * kChunk);
        const frag Rb0 = Ops::pack(R[0], R[1]), Rb1 = Ops::pack(R[2], R[3]);
        f32x4 U[4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            U[tm] = Ops::mma(frag_rows(Tw, kChunk, 16 * tm + r, 0), Rb0, zero4());
            if (tm >= 2) U[tm] = Ops::mma(frag_rows(Tw, kChunk, 16 * tm + r, 32), Rb1, U[tm]);
        }
        // ---- O = diag(gamma) Y + P U
        const frag Ub0 = Ops::pack(U[0], U[1]), Ub1 = Ops::pack(U[2], U[3]);
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            f32x4 O;
#pragma unroll
            for (int i = 0; i < 4; ++i) O[i] = expf(Gv[tm][i]) * Y[tm][i];
            O = Ops::mma(frag_rows(Pw, kChunk, 16 * tm + r, 0), Ub0, O);
            if (tm >= 2) O = Ops::mma(frag_rows(Pw, kChunk, 16 * tm + r, 32), Ub1, O);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tm + 4 * gq + i;
                if (t < nt) og[((size_t)(t0 + t) * a.hv + h) * dv + c] = from_f32<OP>(O[i]);
            }
        }
        // ---- S^T <- gamma_n S^T + K^T diag(e^{G_n - G}) U
        f32x4 UD[4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int i = 0; i < 4; ++i) UD[tm][i] = U[tm][i] * expf(Glast - Gv[tm][i]);
        const frag Db0 = Ops::pack(UD[0], UD[1]), Db1 = Ops::pack(UD[2], UD[3]);
        const float gl = expf(Glast);
#pragma unroll
        for (int ti = 0; ti < NTI; ++ti) {
            f32x4 acc = gl * St[ti];
            acc = Ops::mma(frag_rows(sm.Kt, LDT, 16 * ti + r, 0), Db0, acc);
            St[ti] = Ops::mma(frag_rows(sm.Kt, LDT, 16 * ti + r, 32), Db1, acc);
        }
    }
    if (a.final_state) {
#pragma unroll
        for (int ti = 0; ti < NTI; ++ti)
            *reinterpret_cast<f32x4*>(a.final_state + srow + 16 * ti + 4 * gq) = St[ti];
    }
}

template <typename OP, int DK>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
    {
        dim3 grid((unsigned)a.num_slots, (unsigned)a.hv), block(kPrepThreads);
        hipLaunchKernelGGL((gdn_prep_kernel<OP, DK>), grid, block, 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    constexpr int NW = 4;
    const int groups = a.dv / (16 * NW);
    dim3 grid((unsigned)((int64_t)a.num_seqs * a.hv), (unsigned)groups), block(NW * kWave);
    hipLaunchKernelGGL((gdn_scan_kernel<OP, DK, NW>), grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, bool bf16, int dk, hipStream_t st) {
    if (a.num_seqs == 0) return hipSuccess;
    if (bf16) return dk == 128 ? launch_prefill_t<__bf16, 128>(a, st) : launch_prefill_t<__bf16, 64>(a, st);
    return dk == 128 ? launch_prefill_t<float, 128>(a, st) : launch_prefill_t<float, 64>(a, st);
}

}  // namespace gdn
