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
//    gdn_device.h).  The workgroup's waves share one LDS copy of the chunk's
//    K (row-major and transposed), Q, V columns, T~ and P; the global loads
//    of chunk j+1 are issued before chunk j is computed so that their latency
//    overlaps the matrix work, and outputs leave through LDS as 16-byte rows.
//
// Exponentials use exp2 of log2-scaled cumulative gates (G2 = G log2 e).
// Padding: a final partial chunk is padded with k = q = v = 0, g = 0,
// beta = 0; padded rows then carry u = 0 and leave S and the real rows
// untouched, and gamma_n = e^{G_63} equals the decay up to the last real token.
// All global loads are unconditional with the row index clamped into the
// sequence (the padding value is selected afterwards), so no load sits behind
// a branch.
#include <cstdlib>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kPrepThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

template <typename OP> constexpr int pad_elems() { return 16 / (int)sizeof(OP); }

template <typename OP> struct VecE;                       // 16 bytes as elements
template <> struct VecE<__bf16> { using type = bf16x8; };
template <> struct VecE<float> { using type = f32x4; };

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ u32x4 zero_u4() { return u32x4{0u, 0u, 0u, 0u}; }

template <typename T>
__device__ __forceinline__ u32x4 ld16(const T* p) { return *reinterpret_cast<const u32x4*>(p); }

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

// Lane shuffle of a double by a DPP control (two 32-bit halves); lanes whose
// source is outside the pattern (or whose row is masked off) read 0.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_f64(double x) {
    const long long b = __builtin_bit_cast(long long, x);
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(b & 0xffffffff), CTRL, ROW_MASK, 0xF, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(b >> 32), CTRL, ROW_MASK, 0xF, true);
    return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned)lo);
}

// Inclusive prefix sum over the 64 lanes of a wave, in fp64, on DPP lane
// moves only: shifts by 1, 2, 4, 8 inside each row of 16 lanes, then lane 15
// of a row into the next row (rows 1, 3) and lane 31 into rows 2, 3.
__device__ __forceinline__ double wave_cumsum_f64(double x) {
    x += dpp_f64<0x111, 0xF>(x);   // row_shr:1
    x += dpp_f64<0x112, 0xF>(x);   // row_shr:2
    x += dpp_f64<0x114, 0xF>(x);   // row_shr:4
    x += dpp_f64<0x118, 0xF>(x);   // row_shr:8
    x += dpp_f64<0x142, 0xA>(x);   // row_bcast:15
    x += dpp_f64<0x143, 0xC>(x);   // row_bcast:31
    return x;
}

__device__ __forceinline__ double lane63_f64(double x) {
    const long long b = __builtin_bit_cast(long long, x);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xffffffff), 63);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), 63);
    return __builtin_bit_cast(double, ((long long)hi << 32) | (unsigned)lo);
}

// Gates of one chunk, computed by one wave: lane l holds g_l (0 past the end
// of the sequence).  With G_t = g_1 + ... + g_t accumulated in fp64 (so that
// differences of nearby prefix sums keep full fp32 accuracy), writes
// gam[t] = e^{G_t}, dec[t] = e^{G_last - G_t} and gam[64] = e^{G_last}.
__device__ __forceinline__ void chunk_gates(float g, float* gam, float* dec) {
    const int l = lane_id();
    const double G = wave_cumsum_f64((double)g * 1.4426950408889634);
    const double Gl = lane63_f64(G);
    gam[l] = fast_exp2((float)G);
    dec[l] = fast_exp2((float)(Gl - G));
    if (l == 0) gam[kChunk] = fast_exp2((float)Gl);
}

// ===========================================================================
// prep: T~ and P for one (chunk, value head)
// ===========================================================================
template <typename OP, int DK>
struct PrepSmem {
    static constexpr int LD = DK + pad_elems<OP>();
    static constexpr int LDP = kChunk + pad_elems<OP>();
    alignas(16) OP K[kChunk * LD];     // later: T~ (LDP rows) for the store
    alignas(16) OP Q[kChunk * LD];
    alignas(16) OP P[kChunk * LDP];    // P staged for the store
    alignas(16) float A[kChunk][kChunk + 4];
    alignas(16) float T[kChunk][kChunk + 4];
    alignas(16) double G[kChunk];      // log2-scaled cumulative gates (fp64)
    alignas(16) float B[kChunk];
};

template <typename OP, int DK>
__global__ __launch_bounds__(kPrepThreads) void gdn_prep_kernel(PrefillArgs a) {
    using Ops = Op<OP>;
    using Sm = PrepSmem<OP, DK>;
    constexpr int LD = Sm::LD, LDP = Sm::LDP;
    constexpr int VE = 16 / (int)sizeof(OP);      // elements per 16-byte vector
    constexpr int NV = DK / VE;                    // vectors per K/Q row
    constexpr int MV = kChunk / VE;                // vectors per T~/P row
    __shared__ Sm sm;

    const int64_t slot = blockIdx.x;
    const int h = blockIdx.y;
    const SeqIndex si{a.cu, a.seqlen};
    int n;
    int64_t t0, t1;
    if (!locate_slot(si, a.num_seqs, slot, n, t0, t1)) return;   // uniform over the workgroup
    const int nt = (int)((t1 - t0) < kChunk ? (t1 - t0) : kChunk);
    const int hq = (h * a.hqk) / a.hv;
    const int tid = threadIdx.x, l = lane_id(), w = wave_id(), r = l & 15, gq = l >> 4;

    // ---- stage K, Q (rows past the end are zero) and the gates
    const OP* kg = static_cast<const OP*>(a.k);
    const OP* qg = static_cast<const OP*>(a.q);
    for (int e = tid; e < kChunk * NV; e += kPrepThreads) {
        const int row = e / NV, cv = e - row * NV;
        const int rc = row < nt ? row : nt - 1;
        const size_t off = ((size_t)(t0 + rc) * a.hqk + hq) * DK + (size_t)cv * VE;
        u32x4 kv = ld16(kg + off), qv = ld16(qg + off);
        if (row >= nt) { kv = zero_u4(); qv = zero_u4(); }
        *reinterpret_cast<u32x4*>(&sm.K[row * LD + cv * VE]) = kv;
        *reinterpret_cast<u32x4*>(&sm.Q[row * LD + cv * VE]) = qv;
    }
    if (w == 0) {
        const int lc = l < nt ? l : nt - 1;
        float gv = a.g[(size_t)(t0 + lc) * a.hv + h];
        float bv = a.beta[(size_t)(t0 + lc) * a.hv + h];
        if (l >= nt) { gv = 0.f; bv = 0.f; }
        sm.G[l] = wave_cumsum_f64((double)gv * 1.4426950408889634);
        sm.B[l] = bv;
    }
    __syncthreads();

    // ---- Gamma-weighted K K^T (-> A, fp32) and Q K^T (-> P, staged as OP)
    for (int job = w; job < 20; job += kPrepThreads / kWave) {
        const bool qk = job >= 10;
        const int tm = kLowerTiles[job % 10][0], tn = kLowerTiles[job % 10][1];
        const OP* X = qk ? sm.Q : sm.K;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk)
            acc = Ops::mma(frag_rows(X, LD, 16 * tm + r, 32 * kk), frag_rows(sm.K, LD, 16 * tn + r, 32 * kk), acc);
        const int s = 16 * tn + r;
        if (!qk) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tm + 4 * gq + i;
                sm.A[t][s] = (s < t) ? sm.B[t] * fast_exp2((float)(sm.G[t] - sm.G[s])) * acc[i] : 0.f;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * tm + 4 * gq + i;
                sm.P[t * LDP + s] = from_f32<OP>((s <= t) ? fast_exp2((float)(sm.G[t] - sm.G[s])) * acc[i] : 0.f);
            }
        }
    }
    __syncthreads();   // K no longer read: its space holds T~ from here on

    OP* Pl = sm.P;
    OP* Tl = sm.K;     // T~ staged as [64][LDP]
    // strictly-upper 16x16 tiles of P and T~ are zero (read as padding by the scan)
    for (int e = tid; e < kChunk * kChunk; e += kPrepThreads) {
        const int t = e >> 6, s = e & 63;
        if ((s >> 4) > (t >> 4)) {
            Pl[t * LDP + s] = from_f32<OP>(0.f);
            Tl[t * LDP + s] = from_f32<OP>(0.f);
        }
    }
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

    // ---- T~ = T diag(beta) on the lower blocks, staged as OP
    for (int e = tid; e < kChunk * kChunk; e += kPrepThreads) {
        const int t = e >> 6, s = e & 63;
        if ((s >> 4) <= (t >> 4)) Tl[t * LDP + s] = from_f32<OP>((s <= t) ? sm.T[t][s] * sm.B[s] : 0.f);
    }
    __syncthreads();

    // ---- coalesced 16-byte stores of T~ and P
    OP* Pw = static_cast<OP*>(a.ws_p) + ((size_t)slot * a.hv + h) * (kChunk * kChunk);
    OP* Tw = static_cast<OP*>(a.ws_t) + ((size_t)slot * a.hv + h) * (kChunk * kChunk);
    for (int e = tid; e < kChunk * MV; e += kPrepThreads) {
        const int row = e / MV, cv = e - row * MV;
        *reinterpret_cast<u32x4*>(Tw + row * kChunk + cv * VE) = ld16(Tl + row * LDP + cv * VE);
        *reinterpret_cast<u32x4*>(Pw + row * kChunk + cv * VE) = ld16(Pl + row * LDP + cv * VE);
    }
}

// ===========================================================================
// scan: sequential over chunks, 16 state rows per wave
// ===========================================================================
template <typename OP, int DK, int NW>
struct ScanSmem {
    static constexpr int PAD = pad_elems<OP>();
    static constexpr int LD = DK + PAD;          // K, Q rows (token-major)
    static constexpr int LDT = kChunk + PAD;     // K^T rows (d_k-major), T~ and P rows
    static constexpr int LDV = 16 * NW + PAD;    // V and O rows (this workgroup's columns)
    alignas(16) OP K[kChunk * LD];
    alignas(16) OP Q[kChunk * LD];
    alignas(16) OP Kt[DK * LDT];
    alignas(16) OP T[kChunk * LDT];
    alignas(16) OP P[kChunk * LDT];
    alignas(16) OP V[kChunk * LDV];
    alignas(16) OP O[kChunk * LDV];
    alignas(16) float gam[kChunk + 4];           // e^{G_t}; [64] = e^{G_last}
    alignas(16) float dec[kChunk];               // e^{G_last - G_t}
};

// Per-thread register staging of one chunk's inputs (16-byte vectors).
template <typename OP, int DK, int NW>
struct ScanStage {
    static constexpr int NT = NW * kWave;
    static constexpr int VE = 16 / (int)sizeof(OP);
    static constexpr int NV = DK / VE;                       // vectors per K/Q row
    static constexpr int KTASKS = (kChunk / 4) * NV;         // 4 tokens x 1 vector
    static constexpr int KT = (KTASKS + NT - 1) / NT;
    static constexpr int QTASKS = kChunk * NV;
    static constexpr int QT = (QTASKS + NT - 1) / NT;
    static constexpr int VV = 16 * NW / VE;                  // vectors per V/O row
    static constexpr int VTASKS = kChunk * VV;
    static constexpr int VT = (VTASKS + NT - 1) / NT;
    static constexpr int MV = kChunk / VE;                   // vectors per T~/P row
    static constexpr int MTASKS = kChunk * MV;
    static constexpr int MT = (MTASKS + NT - 1) / NT;
    u32x4 k[KT][4];
    u32x4 q[QT];
    u32x4 v[VT];
    u32x4 t[MT];
    u32x4 p[MT];
    float g;
    int nt;   // valid rows; padding is applied when the stage is committed
};

template <typename OP, int DK, int NW>
struct ScanCtx {
    using St = ScanStage<OP, DK, NW>;
    const OP* kg;
    const OP* qg;
    const OP* vg;
    const float* gg;
    const OP* tws;
    const OP* pws;
    int hqk, hv, dv, hq, h, col0;

    // Issue the global loads of the chunk starting at t0 (nt >= 1 tokens).
    __device__ __forceinline__ void load(St& s, int64_t t0, int nt, int64_t slot) const {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < St::KT; ++i) {
            const int e = tid + i * St::NT;
            if (St::KTASKS % St::NT == 0 || e < St::KTASKS) {
                const int rq = e % (kChunk / 4), cv = e / (kChunk / 4);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int row = 4 * rq + j;
                    const int rc = row < nt ? row : nt - 1;
                    s.k[i][j] = ld16(kg + ((size_t)(t0 + rc) * hqk + hq) * DK + (size_t)cv * St::VE);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < St::QT; ++i) {
            const int e = tid + i * St::NT;
            if (St::QTASKS % St::NT == 0 || e < St::QTASKS) {
                const int row = e / St::NV, cv = e - row * St::NV;
                const int rc = row < nt ? row : nt - 1;
                s.q[i] = ld16(qg + ((size_t)(t0 + rc) * hqk + hq) * DK + (size_t)cv * St::VE);
            }
        }
#pragma unroll
        for (int i = 0; i < St::VT; ++i) {
            const int e = tid + i * St::NT;
            if (St::VTASKS % St::NT == 0 || e < St::VTASKS) {
                const int row = e / St::VV, cv = e - row * St::VV;
                const int rc = row < nt ? row : nt - 1;
                s.v[i] = ld16(vg + ((size_t)(t0 + rc) * hv + h) * dv + col0 + cv * St::VE);
            }
        }
        const OP* tw = tws + ((size_t)slot * hv + h) * (kChunk * kChunk);
        const OP* pw = pws + ((size_t)slot * hv + h) * (kChunk * kChunk);
#pragma unroll
        for (int i = 0; i < St::MT; ++i) {
            const int e = tid + i * St::NT;
            if (St::MTASKS % St::NT == 0 || e < St::MTASKS) {
                s.t[i] = ld16(tw + (size_t)e * St::VE);
                s.p[i] = ld16(pw + (size_t)e * St::VE);
            }
        }
        if (wave_id() == 0) {
            const int l = lane_id();
            const int lc = l < nt ? l : nt - 1;
            s.g = gg[(size_t)(t0 + lc) * hv + h];
        }
        s.nt = nt;
    }

    // Write a staged chunk into LDS (K row-major and transposed, Q, V, T~, P, G).
    __device__ __forceinline__ void commit(const St& s, ScanSmem<OP, DK, NW>& sm) const {
        using SS = ScanSmem<OP, DK, NW>;
        using vecE = typename VecE<OP>::type;
        using quad = typename Op<OP>::quad;
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < St::KT; ++i) {
            const int e = tid + i * St::NT;
            if (St::KTASKS % St::NT == 0 || e < St::KTASKS) {
                const int rq = e % (kChunk / 4), cv = e / (kChunk / 4);
                u32x4 kv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    kv[j] = (4 * rq + j) < s.nt ? s.k[i][j] : zero_u4();
                    *reinterpret_cast<u32x4*>(&sm.K[(4 * rq + j) * SS::LD + cv * St::VE]) = kv[j];
                }
#pragma unroll
                for (int e2 = 0; e2 < St::VE; ++e2) {
                    quad col;
#pragma unroll
                    for (int j = 0; j < 4; ++j) col[j] = __builtin_bit_cast(vecE, kv[j])[e2];
                    *reinterpret_cast<quad*>(&sm.Kt[(cv * St::VE + e2) * SS::LDT + 4 * rq]) = col;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < St::QT; ++i) {
            const int e = tid + i * St::NT;
            if (St::QTASKS % St::NT == 0 || e < St::QTASKS) {
                const int row = e / St::NV, cv = e - row * St::NV;
                *reinterpret_cast<u32x4*>(&sm.Q[row * SS::LD + cv * St::VE]) = row < s.nt ? s.q[i] : zero_u4();
            }
        }
#pragma unroll
        for (int i = 0; i < St::VT; ++i) {
            const int e = tid + i * St::NT;
            if (St::VTASKS % St::NT == 0 || e < St::VTASKS) {
                const int row = e / St::VV, cv = e - row * St::VV;
                *reinterpret_cast<u32x4*>(&sm.V[row * SS::LDV + cv * St::VE]) = row < s.nt ? s.v[i] : zero_u4();
            }
        }
#pragma unroll
        for (int i = 0; i < St::MT; ++i) {
            const int e = tid + i * St::NT;
            if (St::MTASKS % St::NT == 0 || e < St::MTASKS) {
                const int row = e / St::MV, cv = e - row * St::MV;
                *reinterpret_cast<u32x4*>(&sm.T[row * SS::LDT + cv * St::VE]) = s.t[i];
                *reinterpret_cast<u32x4*>(&sm.P[row * SS::LDT + cv * St::VE]) = s.p[i];
            }
        }
        if (wave_id() == 0) chunk_gates(lane_id() < s.nt ? s.g : 0.f, sm.gam, sm.dec);
    }

    // 16-byte stores of the O rows of a finished chunk (rows < nt).
    __device__ __forceinline__ void store_out(const ScanSmem<OP, DK, NW>& sm, OP* og, int64_t t0, int nt) const {
        using SS = ScanSmem<OP, DK, NW>;
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < St::VT; ++i) {
            const int e = tid + i * St::NT;
            if (St::VTASKS % St::NT == 0 || e < St::VTASKS) {
                const int row = e / St::VV, cv = e - row * St::VV;
                if (row < nt)
                    *reinterpret_cast<u32x4*>(og + ((size_t)(t0 + row) * hv + h) * dv + col0 + cv * St::VE) =
                        ld16(&sm.O[row * SS::LDV + cv * St::VE]);
            }
        }
    }
};

template <typename OP, int DK, int NW, bool PREFETCH>
__global__ __launch_bounds__(NW * kWave) void gdn_scan_kernel(PrefillArgs a) {
    using Ops = Op<OP>;
    using frag = typename Ops::frag;
    using SS = ScanSmem<OP, DK, NW>;
    using St = ScanStage<OP, DK, NW>;
    constexpr int LD = SS::LD, LDT = SS::LDT, LDV = SS::LDV;
    constexpr int NTI = DK / 16;   // S^T tiles along d_k
    __shared__ SS sm;

    const int chain = blockIdx.x;
    const int n = chain / a.hv;
    const int h = chain - n * a.hv;
    const int l = lane_id(), w = wave_id(), r = l & 15, gq = l >> 4;
    const int col0 = blockIdx.y * NW * 16;                  // workgroup's first d_v column
    const int cl = w * 16 + r;                               // this lane's column within the workgroup
    const int c = col0 + cl;                                 // this lane's d_v column

    ScanCtx<OP, DK, NW> ctx{static_cast<const OP*>(a.k), static_cast<const OP*>(a.q),
                            static_cast<const OP*>(a.v), a.g,
                            static_cast<const OP*>(a.ws_t), static_cast<const OP*>(a.ws_p),
                            a.hqk, a.hv, a.dv, (h * a.hqk) / a.hv, h, col0};
    OP* og = static_cast<OP*>(a.out);

    const SeqIndex si{a.cu, a.seqlen};
    const int64_t s0 = si.start(n), s1 = si.start(n + 1);
    const int64_t base = slot_base(s0, n);

    // S^T tiles: St[ti] holds S[c][16 ti + 4 gq + i], i = 0..3
    f32x4 S[NTI];
    const size_t srow = ((size_t)chain * a.dv + c) * DK;
    if (a.init_state) {
#pragma unroll
        for (int ti = 0; ti < NTI; ++ti) S[ti] = *reinterpret_cast<const f32x4*>(a.init_state + srow + 16 * ti + 4 * gq);
    } else {
#pragma unroll
        for (int ti = 0; ti < NTI; ++ti) S[ti] = zero4();
    }

    St stage;
    if (PREFETCH && s0 < s1) ctx.load(stage, s0, (int)((s1 - s0) < kChunk ? (s1 - s0) : kChunk), base);

    int64_t prev_t0 = 0;
    int prev_nt = 0;
    int64_t slot = base;
    for (int64_t t0 = s0; t0 < s1; t0 += kChunk, ++slot) {
        const int nt = (int)((s1 - t0) < kChunk ? (s1 - t0) : kChunk);
        __syncthreads();                       // LDS of the previous chunk is free, its O rows complete
        if (prev_nt > 0) ctx.store_out(sm, og, prev_t0, prev_nt);
        if (!PREFETCH) ctx.load(stage, t0, nt, slot);
        ctx.commit(stage, sm);
        __syncthreads();
        if (PREFETCH && t0 + kChunk < s1) {
            const int64_t rem = s1 - t0 - kChunk;
            ctx.load(stage, t0 + kChunk, (int)(rem < kChunk ? rem : kChunk), slot + 1);
        }

        // ---- X = K S^T, Y = Q S^T (64 tokens x 16 columns)
        frag Sb[DK / 32];
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) Sb[kk] = Ops::pack(S[2 * kk], S[2 * kk + 1]);
        f32x4 X[4], Y[4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) { X[tm] = zero4(); Y[tm] = zero4(); }
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk) {
            frag kf[4], qf[4];
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) {
                kf[tm] = frag_rows(sm.K, LD, 16 * tm + r, 32 * kk);
                qf[tm] = frag_rows(sm.Q, LD, 16 * tm + r, 32 * kk);
            }
#pragma unroll
            for (int tm = 0; tm < 4; ++tm) {
                X[tm] = Ops::mma(kf[tm], Sb[kk], X[tm]);
                Y[tm] = Ops::mma(qf[tm], Sb[kk], Y[tm]);
            }
        }
        // ---- gates for this lane's rows
        f32x4 gam[4], dec[4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            gam[tm] = *reinterpret_cast<const f32x4*>(&sm.gam[16 * tm + 4 * gq]);
            dec[tm] = *reinterpret_cast<const f32x4*>(&sm.dec[16 * tm + 4 * gq]);
        }
        // ---- R = V - diag(gamma) X
        f32x4 R[4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                R[tm][i] = to_f32(sm.V[(16 * tm + 4 * gq + i) * LDV + cl]) - gam[tm][i] * X[tm][i];
        // ---- U = T~ R (T~ lower triangular: skip zero K steps)
        const frag Rb0 = Ops::pack(R[0], R[1]), Rb1 = Ops::pack(R[2], R[3]);
        f32x4 U[4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            U[tm] = Ops::mma(frag_rows(sm.T, LDT, 16 * tm + r, 0), Rb0, zero4());
            if (tm >= 2) U[tm] = Ops::mma(frag_rows(sm.T, LDT, 16 * tm + r, 32), Rb1, U[tm]);
        }
        // ---- O = diag(gamma) Y + P U  (staged in LDS for 16-byte stores)
        const frag Ub0 = Ops::pack(U[0], U[1]), Ub1 = Ops::pack(U[2], U[3]);
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            f32x4 O = gam[tm] * Y[tm];
            O = Ops::mma(frag_rows(sm.P, LDT, 16 * tm + r, 0), Ub0, O);
            if (tm >= 2) O = Ops::mma(frag_rows(sm.P, LDT, 16 * tm + r, 32), Ub1, O);
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.O[(16 * tm + 4 * gq + i) * LDV + cl] = from_f32<OP>(O[i]);
        }
        // ---- S^T <- gamma_n S^T + K^T diag(e^{G_n - G}) U
        f32x4 UD[4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) UD[tm] = U[tm] * dec[tm];
        const frag Db0 = Ops::pack(UD[0], UD[1]), Db1 = Ops::pack(UD[2], UD[3]);
        const float gl = sm.gam[kChunk];
#pragma unroll
        for (int ti = 0; ti < NTI; ++ti) {
            f32x4 acc = gl * S[ti];
            acc = Ops::mma(frag_rows(sm.Kt, LDT, 16 * ti + r, 0), Db0, acc);
            S[ti] = Ops::mma(frag_rows(sm.Kt, LDT, 16 * ti + r, 32), Db1, acc);
        }
        prev_t0 = t0;
        prev_nt = nt;
    }
    __syncthreads();
    if (prev_nt > 0) ctx.store_out(sm, og, prev_t0, prev_nt);
    if (a.final_state) {
#pragma unroll
        for (int ti = 0; ti < NTI; ++ti)
            *reinterpret_cast<f32x4*>(a.final_state + srow + 16 * ti + 4 * gq) = S[ti];
    }
}


// ===========================================================================
// split scan: one workgroup per (sequence, value head, 16-column block of d_v);
// its NWS = DK/32 waves split d_k, wave w owning state rows S[:, 32w .. 32w+32)
// as two fp32 accumulator tiles (d_k x 16).  Inside the slice the d_k order
// of the tiles is permuted (tile `sub`, row 4 gq + i  <->  d_k 8 gq + 4 sub + i)
// so that an operand fragment of K or Q is one contiguous 16-byte load.
// Wave w also owns token tiles tw = w + NWS j (j < TPW = 4 / NWS).  Per chunk:
//   wave w:  Xp^T = S_w K_w^T,  Yp^T = S_w Q_w^T          (partial over d_k)
//            K_w^T in operand layout via an exact identity product
//   E1 (LDS): partial sums -> owner of token tile tw holds X^T and Y^T there
//   owner:   R^T = V^T - X^T diag(gamma)        (one 8-byte V load per lane)
//   E2 (LDS): R for all tokens to every wave
//   owner:   U = T~_tw R,  D o U
//   E3 (LDS): U and D o U for all tokens to every wave
//   owner:   O^T = Y^T diag(gamma) + U^T P_tw^T  (one 8-byte store per lane)
//   wave w:  S_w^T <- gamma_n S_w^T + K_w^T (D o U)
// Loads come from buffer resources two chunks ahead of use (two register
// stages), with no load, store or use of a loaded value behind a branch, so
// the compiler's memory-counter waits stay exact.  Padded rows of a partial
// last chunk need no zeroing: the prep kernel padded K with zero rows and beta
// with zeros, so those rows carry u = 0 exactly.
// ===========================================================================
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// Buffer resource over [base, base + bytes): loads past the end read 0 and
// stores past the end are dropped by the hardware.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

template <typename OP> struct Buf;
template <> struct Buf<__bf16> {
    __device__ __forceinline__ static bf16x8 frag(__amdgpu_buffer_rsrc_t r, unsigned off) {
        return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
    __device__ __forceinline__ static bf16x4 quad(__amdgpu_buffer_rsrc_t r, unsigned off) {
        return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
    }
    __device__ __forceinline__ static void store4(bf16x4 x, __amdgpu_buffer_rsrc_t r, unsigned off) {
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, x), r, off, 0, 0);
    }
};
template <> struct Buf<float> {
    __device__ __forceinline__ static f32x8 frag(__amdgpu_buffer_rsrc_t r, unsigned off) {
        const i32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
        const i32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0);
        return __builtin_bit_cast(f32x8, i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    }
    __device__ __forceinline__ static f32x4 quad(__amdgpu_buffer_rsrc_t r, unsigned off) {
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
    }
    __device__ __forceinline__ static void store4(f32x4 x, __amdgpu_buffer_rsrc_t r, unsigned off) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x), r, off, 0, 0);
    }
};

// A/B fragment of a row-major LDS matrix in natural K order: k0 + 8 gq + (0..7).
template <typename T>
__device__ __forceinline__ typename Op<T>::frag frag_nat(const T* M, int ld, int row, int k0) {
    using frag = typename Op<T>::frag;
    return *reinterpret_cast<const frag*>(M + (size_t)row * ld + k0 + 8 * (lane_id() >> 4));
}

template <typename OP, int TPW>
struct SplitStage {
    using frag = typename Op<OP>::frag;
    using quad = typename Op<OP>::quad;
    frag kf[4];          // K[16 tm + r][32 w + 8 gq + (0..7)]
    frag qf[4];          // Q, same positions
    frag tf[TPW][2];     // T~[16 tw + r][32 kk + 8 gq + (0..7)]
    frag pf[TPW][2];     // P, same positions
    quad v[TPW];         // V[16 tw + r][16 blk + 4 gq + (0..3)]
    float g;             // g of token `lane` (0 past the end of the sequence)
};

template <typename OP, int DK>
struct SplitSmem {
    static constexpr int NWS = DK / 32;
    static constexpr int RLD = kChunk + (sizeof(OP) == 2 ? 8 : 4);   // 16-byte rows, staggered banks
    f32x4 part[NWS][8][kWave];          // E1: X^T partials (0..3) and Y^T partials (4..7)
    alignas(16) OP Rt[16 * RLD];        // E2: R as [column][token]
    alignas(16) OP Ut[16 * RLD];        // E3: U as [column][token]
    alignas(16) OP Dt[16 * RLD];        // E3: D o U as [column][token]
    alignas(16) float gam[2][kChunk + 4];   // gates by chunk parity: e^{G_t}, [64] = e^{G_last}
    alignas(16) float dec[2][kChunk];       // e^{G_last - G_t}
};

template <typename OP, int DK>
struct SplitCtx {
    static constexpr int NWS = DK / 32, TPW = 4 / NWS;
    static constexpr int E = (int)sizeof(OP);
    using St = SplitStage<OP, TPW>;
    using B = Buf<OP>;
    // per-sequence scalars: byte address of the sequence's first chunk in each
    // tensor and the bytes from there to the end of the tensor
    const char* kb; const char* qb; int64_t kqn;
    const char* vb; int64_t vn;
    const char* gb;
    const char* tb;
    const char* pb;
    int64_t kq_step, v_step, g_step, w_step;   // bytes per chunk step
    int64_t seq_tokens;
    int hv;
    // loop-invariant per-lane byte offsets
    unsigned koff[4];      // ((16 tm + r) * hqk * DK + 8 gq) * E
    unsigned voff[TPW];    // ((16 tw + r) * hv * dv + 4 gq) * E
    unsigned toff[TPW];    // ((16 tw + r) * 64 + 8 gq) * E
    unsigned goff;         // lane * hv * 4

    __device__ __forceinline__ void init(const PrefillArgs& a, int64_t s0, int64_t s1, int64_t base, int h,
                                         int blk, int w) {
        const int l = lane_id(), r = l & 15, gq = l >> 4;
        const int hq = (h * a.hqk) / a.hv;
        hv = a.hv;
        const size_t kq0 = ((size_t)s0 * a.hqk + hq) * DK + 32 * w;
        kb = reinterpret_cast<const char*>(static_cast<const OP*>(a.k) + kq0);
        qb = reinterpret_cast<const char*>(static_cast<const OP*>(a.q) + kq0);
        kqn = ((int64_t)a.num_tokens * a.hqk * DK - (int64_t)kq0) * E;
        const size_t v0 = ((size_t)s0 * a.hv + h) * a.dv + blk * 16;
        vb = reinterpret_cast<const char*>(static_cast<const OP*>(a.v) + v0);
        vn = ((int64_t)a.num_tokens * a.hv * a.dv - (int64_t)v0) * E;
        gb = reinterpret_cast<const char*>(a.g + (size_t)s0 * a.hv + h);
        const size_t w0 = ((size_t)base * a.hv + h) * (kChunk * kChunk);
        tb = reinterpret_cast<const char*>(static_cast<const OP*>(a.ws_t) + w0);
        pb = reinterpret_cast<const char*>(static_cast<const OP*>(a.ws_p) + w0);
        kq_step = (int64_t)kChunk * a.hqk * DK * E;
        v_step = (int64_t)kChunk * a.hv * a.dv * E;
        g_step = (int64_t)kChunk * a.hv * 4;
        w_step = (int64_t)a.hv * kChunk * kChunk * E;
        seq_tokens = s1 - s0;
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) koff[tm] = (unsigned)(((16 * tm + r) * a.hqk * DK + 8 * gq) * E);
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
            const int tw = w + NWS * jt;
            voff[jt] = (unsigned)(((16 * tw + r) * a.hv * a.dv + 4 * gq) * E);
            toff[jt] = (unsigned)(((16 * tw + r) * kChunk + 8 * gq) * E);
        }
        goff = (unsigned)(l * a.hv * 4);
    }

    // Fetch the operands of the sequence's chunk j (zeros when !valid), in the
    // order the chunk consumes them, so that each wait covers only the oldest
    // loads in flight.
    __device__ __forceinline__ void load(St& s, int64_t j, bool valid) const {
        const int64_t jc = valid ? j : 0;
        const int64_t kqo = jc * kq_step, vo = jc * v_step, go = jc * g_step, wo = jc * w_step;
        const int64_t nt = seq_tokens - jc * kChunk;              // g past the sequence reads 0
        const auto rg = make_rsrc(gb + go, (valid && nt > 0) ? ((nt - 1) * hv + 1) * 4 : 0);
        s.g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, goff, 0, 0));
        const int64_t kqb = valid ? kqn - kqo : 0;
        const auto rk = make_rsrc(kb + kqo, kqb);
        const auto rq = make_rsrc(qb + kqo, kqb);
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) s.kf[tm] = B::frag(rk, koff[tm]);
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) s.qf[tm] = B::frag(rq, koff[tm]);
        const auto rv = make_rsrc(vb + vo, valid ? vn - vo : 0);
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) s.v[jt] = B::quad(rv, voff[jt]);
        const int64_t wb = valid ? kChunk * kChunk * E : 0;
        const auto rt = make_rsrc(tb + wo, wb);
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) s.tf[jt][kk] = B::frag(rt, toff[jt] + 32 * kk * E);
        const auto rp = make_rsrc(pb + wo, wb);
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) s.pf[jt][kk] = B::frag(rp, toff[jt] + 32 * kk * E);
    }
};

template <typename OP, int DK>
__global__ __launch_bounds__(DK / 32 * kWave) void gdn_scan_split_kernel(PrefillArgs a, int xcd_map) {
    using Ops = Op<OP>;
    using frag = typename Ops::frag;
    using quad = typename Ops::quad;
    using SS = SplitSmem<OP, DK>;
    using Ctx = SplitCtx<OP, DK>;
    using St = typename Ctx::St;
    using B = Buf<OP>;
    constexpr int NWS = SS::NWS, RLD = SS::RLD, TPW = Ctx::TPW;
    __shared__ SS sm;

    // Work item (chain, 16-column block).  With xcd_map, the 8 column blocks of
    // a chain get workgroup ids that the dispatcher sends to one XCD, so they
    // share that XCD's L2 for K, Q, T~ and P.
    int chain, blk;
    {
        const int L = blockIdx.x, nblk = a.dv / 16;
        if (xcd_map) {
            chain = (L & 7) + 8 * (L / 64);
            blk = (L >> 3) & 7;
        } else {
            chain = L / nblk;
            blk = L - chain * nblk;
        }
    }
    const int n = chain / a.hv;
    const int h = chain - n * a.hv;
    const int l = lane_id(), w = wave_id(), r = l & 15, gq = l >> 4;
    const int c = blk * 16 + r;

    const SeqIndex si{a.cu, a.seqlen};
    const int64_t s0 = si.start(n), s1 = si.start(n + 1);
    const int64_t base = slot_base(s0, n);
    Ctx ctx;
    ctx.init(a, s0, s1, base, h, blk, w);

    // identity fragments: K slot (gq, i) <-> d_k 8 gq + i, state tile `sub`
    // row n <-> d_k 8 (n/4) + 4 sub + n%4
    frag Iden[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            Iden[sub][i] = from_f32<OP>((gq == (r >> 2) && i == 4 * sub + (r & 3)) ? 1.f : 0.f);

    // S[sub][i] = S[c][32 w + 8 gq + 4 sub + i]
    f32x4 S[2];
    const size_t srow = ((size_t)chain * a.dv + c) * DK + 32 * w + 8 * gq;
    if (a.init_state) {
        S[0] = *reinterpret_cast<const f32x4*>(a.init_state + srow);
        S[1] = *reinterpret_cast<const f32x4*>(a.init_state + srow + 4);
    } else {
        S[0] = zero4();
        S[1] = zero4();
    }

    const int64_t nchunks = (s1 - s0 + kChunk - 1) / kChunk;
    // One chunk; `nxt` holds the next chunk's operands (its gates are
    // prepared here, by wave 0, into the other parity buffer).
    auto chunk = [&](St& cur, const St& nxt, int64_t j, int par) {
        const int64_t t0 = s0 + j * kChunk;
        const int nt = (int)((s1 - t0) < kChunk ? (s1 - t0) : kChunk);
        // ---- partial products over the d_k slice
        const frag Sb = Ops::pack(S[0], S[1]);
        f32x4 Xp[4], Yp[4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            Xp[tm] = Ops::mma(Sb, cur.kf[tm], zero4());
            Yp[tm] = Ops::mma(Sb, cur.qf[tm], zero4());
        }
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            sm.part[w][tm][l] = Xp[tm];
            sm.part[w][4 + tm][l] = Yp[tm];
        }
        __syncthreads();                                                        // E1
        // K^T in operand layout (exact identity product), off the critical path
        frag Ktf[2][2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
                Ktf[sub][kk] = Ops::pack(Ops::mma(cur.kf[2 * kk], Iden[sub], zero4()),
                                         Ops::mma(cur.kf[2 * kk + 1], Iden[sub], zero4()));
        f32x4 Y[TPW];
        float gt[TPW];
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
            const int tw = w + NWS * jt;
            f32x4 X = sm.part[0][tw][l];
            Y[jt] = sm.part[0][4 + tw][l];
#pragma unroll
            for (int v2 = 1; v2 < NWS; ++v2) {
                X += sm.part[v2][tw][l];
                Y[jt] += sm.part[v2][4 + tw][l];
            }
            gt[jt] = sm.gam[par][16 * tw + r];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sm.Rt[(4 * gq + i) * RLD + 16 * tw + r] = from_f32<OP>(to_f32(cur.v[jt][i]) - gt[jt] * X[i]);
        }
        const float gn = sm.gam[par][kChunk];
        __syncthreads();                                                        // E2
        const frag Rb0 = frag_nat(sm.Rt, RLD, r, 0), Rb1 = frag_nat(sm.Rt, RLD, r, 32);
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
            const int tw = w + NWS * jt;
            const f32x4 U = Ops::mma(cur.tf[jt][1], Rb1, Ops::mma(cur.tf[jt][0], Rb0, zero4()));
            const f32x4 dc = *reinterpret_cast<const f32x4*>(&sm.dec[par][16 * tw + 4 * gq]);
            quad uq, dq;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uq[i] = from_f32<OP>(U[i]);
                dq[i] = from_f32<OP>(U[i] * dc[i]);
            }
            *reinterpret_cast<quad*>(&sm.Ut[r * RLD + 16 * tw + 4 * gq]) = uq;
            *reinterpret_cast<quad*>(&sm.Dt[r * RLD + 16 * tw + 4 * gq]) = dq;
        }
        __syncthreads();                                                        // E3
        // ---- S_w^T <- gamma_n S_w^T + K_w^T (D o U)   (the serial chain first)
        const frag Db0 = frag_rows(sm.Dt, RLD, r, 0), Db1 = frag_rows(sm.Dt, RLD, r, 32);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
            S[sub] = Ops::mma(Ktf[sub][1], Db1, Ops::mma(Ktf[sub][0], Db0, gn * S[sub]));
        // ---- O^T tiles: rows = columns 16 blk + 4 gq + i, column = token 16 tw + r
        const frag Ub0 = frag_nat(sm.Ut, RLD, r, 0), Ub1 = frag_nat(sm.Ut, RLD, r, 32);
        f32x4 Ot[TPW];
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt)
            Ot[jt] = Ops::mma(Ub1, cur.pf[jt][1], Ops::mma(Ub0, cur.pf[jt][0], gt[jt] * Y[jt]));
        // gates of the next chunk (read after the next E1 barrier)
        if (w == 0) chunk_gates(nxt.g, sm.gam[par ^ 1], sm.dec[par ^ 1]);
        // this stage is free: fetch the chunk two steps ahead
        ctx.load(cur, j + 2, j + 2 < nchunks);
        {
            // rows past the end of the sequence fall outside the resource
            const auto ro = make_rsrc(static_cast<OP*>(a.out) + ((size_t)t0 * a.hv + h) * a.dv + blk * 16,
                                      ((int64_t)(nt - 1) * a.hv * a.dv + 16) * (int64_t)sizeof(OP));
#pragma unroll
            for (int jt = 0; jt < TPW; ++jt) {
                quad oq;
#pragma unroll
                for (int i = 0; i < 4; ++i) oq[i] = from_f32<OP>(Ot[jt][i]);
                B::store4(oq, ro, ctx.voff[jt]);
            }
        }
    };

    // Chunks are processed in pairs (stages A, B).  An odd count gets one
    // trailing empty chunk, which is an exact no-op: its loads read zeros
    // (g = 0, so gamma_n = 1 and S is unchanged) and its stores are dropped.
    // Keeping the loop free of an early exit keeps the load order identical on
    // every path into the loop, so the memory-counter waits stay exact.
    St A, Bs;
    ctx.load(A, 0, nchunks > 0);
    ctx.load(Bs, 1, nchunks > 1);
    if (w == 0) chunk_gates(A.g, sm.gam[0], sm.dec[0]);
    for (int64_t j = 0; j < nchunks; j += 2) {
        chunk(A, Bs, j, 0);
        chunk(Bs, A, j + 1, 1);
    }
    if (a.final_state) {
        *reinterpret_cast<f32x4*>(a.final_state + srow) = S[0];
        *reinterpret_cast<f32x4*>(a.final_state + srow + 4) = S[1];
    }
}

// Scan variant: 1 = split (default), 0 = wide.  GDN_SCAN=wide|split overrides
// (both compute the same result; the choice only affects speed).
int scan_variant() {
    static const int v = [] {
        const char* e = getenv("GDN_SCAN");
        if (e && e[0] == 'w') return 0;
        return 1;
    }();
    return v;
}

template <typename OP, int DK>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
    {
        dim3 grid((unsigned)a.num_slots, (unsigned)a.hv), block(kPrepThreads);
        hipLaunchKernelGGL((gdn_prep_kernel<OP, DK>), grid, block, 0, st, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t chains = (int64_t)a.num_seqs * a.hv;
    const int nblk = a.dv / 16;
    if (scan_variant() == 1) {
        // split scan: DK/32 waves per 16-column block
        const int xcd = (nblk == 8 && chains % 8 == 0) ? 1 : 0;
        dim3 grid((unsigned)(chains * nblk)), block(DK / 32 * kWave);
        hipLaunchKernelGGL((gdn_scan_split_kernel<OP, DK>), grid, block, 0, st, a, xcd);
        return hipGetLastError();
    }
    // wide scan.  bf16: 4 waves (64 columns) per workgroup with register
    // prefetch of the next chunk; fp32: 2 waves (LDS budget), loads at the top
    // of each chunk.
    constexpr bool BF = sizeof(OP) == 2;
    constexpr int NW = BF ? 4 : 2;
    const int groups = a.dv / (16 * NW);
    dim3 grid((unsigned)chains, (unsigned)groups), block(NW * kWave);
    hipLaunchKernelGGL((gdn_scan_kernel<OP, DK, NW, BF>), grid, block, 0, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, bool bf16, int dk, hipStream_t st) {
    if (a.num_seqs == 0) return hipSuccess;
    if (bf16) return dk == 128 ? launch_prefill_t<__bf16, 128>(a, st) : launch_prefill_t<__bf16, 64>(a, st);
    return dk == 128 ? launch_prefill_t<float, 128>(a, st) : launch_prefill_t<float, 64>(a, st);
}

}  // namespace gdn
