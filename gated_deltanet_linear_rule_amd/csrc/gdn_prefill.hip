// gdn_prefill.hip -- chunk-wise (WY / UT transform) GDN prefill for gfx950.
//
// The recurrence S_t = alpha_t S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
// o_t = S_t q_t (the GDN layer's fixed-size per-head state: flozi.net,
// "Qwen3.8-Flash-Next architecture", "Der Weg eines Tokens durch das
// Modell", item 1) is evaluated over chunks of C = 64 tokens.  Within a chunk
// with start state S, cumulative log-decay G_t = g_1 + ... + g_t (so every
// exponent below is <= 0), gamma_t = e^{G_t}, Gamma_ts = e^{G_t - G_s},
// D_t = e^{G_last - G_t}:
//
//   A  = strict_lower(diag(beta) (Gamma o K K^T)),   T = (I + A)^{-1}
//   T~ = T diag(beta)
//   W  = T~ diag(gamma) K,   u = T~ V                            [state-free]
//   K~ = diag(D) K,   Q~ = diag(gamma) Q,   P = lower_incl(Gamma o Q K^T)
//   U  = u - W S^T            (the chunk's effective writes u_t)
//   O  = Q~ S^T + P U
//   S' = gamma_last S + U^T K~
//
// (U = T~ (V - diag(gamma) K S^T) is the WY / UT form of the chunk's
// sequential delta-rule writes; the rest follows by expanding the product of
// the per-token transitions over the chunk.)
//
// Two kernels:
//  * gdn_prep_kernel  -- one workgroup per (chunk, value head), all chunks in
//    parallel: the gate cumsum (fp64), Gamma-weighted K K^T and Q K^T on the
//    matrix cores, the unit-lower-triangular inverse (16x16 diagonal blocks by
//    forward substitution, off-diagonal blocks by fp32 MFMA block products),
//    then W, u, K~^T, Q~ and P, written to a workspace in exactly the
//    register layout in which the scan feeds them to its matrix cores.
//  * gdn_scan_kernel  -- sequential over the chunks of one sequence, parallel
//    over (sequence, value head, 16-column block of d_v); the d_k rows of the
//    state block are split over the workgroup's waves and stay in fp32
//    matrix-core accumulators for the whole sequence (details above the
//    kernel).
//
// Exponentials use exp2 of log2-scaled cumulative gates (G2 = G log2 e).
// Padding: a final partial chunk is padded with k = q = v = 0, g = 0,
// beta = 0 in the prep kernel; padded rows then carry u = 0 and zero rows of
// W and K~, so they leave S and the real rows untouched, and
// gamma_last = e^{G2_63} equals the decay up to the last real token.
#include <mutex>
#include <vector>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kPrepThreads = 256;

template <typename OP> constexpr int pad_elems() { return 16 / (int)sizeof(OP); }

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

// A/B fragment of a row-major LDS matrix in natural K order: k0 + 8 gq + (0..7).
template <typename T>
__device__ __forceinline__ typename Op<T>::frag frag_nat(const T* M, int ld, int row, int k0) {
    using frag = typename Op<T>::frag;
    return *reinterpret_cast<const frag*>(M + (size_t)row * ld + k0 + 8 * (lane_id() >> 4));
}

// ===========================================================================
// workspace layout shared by the two kernels
// ===========================================================================
// Operand fragments are stored fragment-major: 16-byte unit
//     e = (f * FU + u) * 64 + lane
// holds unit u of fragment f for that lane (FU = 1 for bf16, 2 for fp32), so
// a wave reads a fragment as one contiguous 1 KB block.  Lane (r, gq) =
// (lane & 15, lane >> 4) of a fragment holds 8 elements of row r of a
// 16-row tile.  Per (chunk, value head), with slice ws = d_k columns
// 32 ws .. 32 ws + 31 (scan wave ws) and "paired" column order
//     slot i < 4  <->  c0 + 4 gq + i,     slot 4 + i  <->  c0 + 16 + 4 gq + i:
//  * W, Q~ : f = ws * 4 + tm, row = token 16 tm + r, paired columns from 32 ws;
//  * K~^T  : f = (ws * 2 + sub) * 2 + kk, row = d_k 32 ws + 16 sub + r,
//            paired columns (tokens) from 32 kk;
//  * P     : f = tw * 2 + kk, row = token 16 tw + r, natural columns
//            (tokens) 32 kk + 8 gq + (0..7);
//  * u     : accumulator-major: per (token tile tw, 16-column block cb),
//            lane (r, gq) holds u[16 tw + 4 gq + i][16 cb + r], i = 0..3;
//  * G2_last of the chunk as one float (0, as read past the end, means no
//    decay).
template <typename OP> struct Frag {
    static constexpr int VE = 16 / (int)sizeof(OP);      // elements per 16-byte unit
    static constexpr int FU = 8 / VE;                    // units per operand fragment
};

// Workspace stores are non-temporal: the scan reads them back much later (or
// on other compute units), and they should not push its working set out of
// the caches meanwhile.
template <typename T>
__device__ __forceinline__ void ws_store(T* p, const T& x) { __builtin_nontemporal_store(x, p); }

template <typename OP>
__device__ __forceinline__ void store_frag(OP* base, int f, const typename Op<OP>::frag& x) {
    constexpr int VE = Frag<OP>::VE, FU = Frag<OP>::FU;
    const int l = lane_id();
    if constexpr (FU == 1) {
        ws_store(reinterpret_cast<typename Op<OP>::frag*>(base + ((size_t)f * 64 + l) * VE), x);
    } else {
        ws_store(reinterpret_cast<f32x4*>(base + ((size_t)(f * 2) * 64 + l) * VE),
                 f32x4(__builtin_shufflevector(x, x, 0, 1, 2, 3)));
        ws_store(reinterpret_cast<f32x4*>(base + ((size_t)(f * 2 + 1) * 64 + l) * VE),
                 f32x4(__builtin_shufflevector(x, x, 4, 5, 6, 7)));
    }
}

// Identity fragment for exact transposes on the matrix cores: as the B
// operand of a product whose K range is 32 consecutive columns c0 + (0..31)
// (natural order), it selects column c0 + 16 sub + n into output column n.
template <typename OP>
__device__ __forceinline__ typename Op<OP>::frag iden_frag(int sub) {
    typename Op<OP>::frag x;
    const int l = lane_id(), n = l & 15, gq = l >> 4;
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = from_f32<OP>((8 * gq + i == 16 * sub + n) ? 1.f : 0.f);
    return x;
}

// Rows 32 kk + (0..31) of a row-major LDS matrix, columns c0 + 16 sub +
// (0..15), transposed into an operand fragment whose K order is the paired
// row order: lane (n, gq) gets M[32 kk + 4 gq + i][c0 + 16 sub + n] and
// M[32 kk + 16 + 4 gq + i][c0 + 16 sub + n].  Exact (products with 0 and 1);
// I = iden_frag(sub).
template <typename OP>
__device__ __forceinline__ typename Op<OP>::frag transpose_frag(const OP* M, int ld, int kk, int c0,
                                                               const typename Op<OP>::frag& I) {
    using Ops = Op<OP>;
    const int r = lane_id() & 15;
    const f32x4 lo = Ops::mma(frag_nat(M, ld, 32 * kk + r, c0), I, zero4());
    const f32x4 hi = Ops::mma(frag_nat(M, ld, 32 * kk + 16 + r, c0), I, zero4());
    return Ops::pack(lo, hi);
}

// ===========================================================================
// prep: W, u, K~^T, Q~, P and G2_last for one (chunk, value head)
// ===========================================================================
template <typename OP, int DK, int DV>
struct PrepSmem {
    static constexpr int PAD = pad_elems<OP>();
    static constexpr int LD = DK + PAD;                      // K rows
    static constexpr int LDQV = (DK > DV ? DK : DV) + PAD;   // Q rows, later V rows
    static constexpr int LDP = kChunk + PAD;                 // P, T~, T~ diag(gamma) rows
    alignas(16) OP K[kChunk * LD];
    alignas(16) OP QV[kChunk * LDQV];
    alignas(16) OP P[kChunk * LDP];                          // P, later T~
    alignas(16) float A[kChunk][kChunk + 4];                 // A, later T~ diag(gamma) (OP, LDP rows)
    alignas(16) float T[kChunk][kChunk + 4];
    alignas(16) double G[kChunk];                            // log2-scaled cumulative gates (fp64)
    alignas(16) float B[kChunk];                             // beta
    alignas(16) float gam[kChunk];                           // e^{G_t}
    alignas(16) float dec[kChunk];                           // e^{G_last - G_t}
};

template <typename OP, int DK, int DV>
__global__ __launch_bounds__(kPrepThreads, 2) void gdn_prep_kernel(PrefillArgs a) {
    using Ops = Op<OP>;
    using frag = typename Ops::frag;
    using quad = typename Ops::quad;
    using Sm = PrepSmem<OP, DK, DV>;
    constexpr int LD = Sm::LD, LDQV = Sm::LDQV, LDP = Sm::LDP;
    constexpr int VE = Frag<OP>::VE;                       // elements per 16-byte vector
    constexpr int FU = Frag<OP>::FU;
    constexpr int NV = DK / VE;                            // vectors per K/Q row
    constexpr int NVV = DV / VE;                           // vectors per V row
    constexpr int KQREG = kChunk * NV / kPrepThreads;      // K (and Q) vectors per thread
    constexpr int VREG = kChunk * NVV / kPrepThreads;      // V vectors per thread
    constexpr int NS = DK / 32;                            // scan slices of d_k
    constexpr int NCP = DV / 32;                           // pairs of 16-column blocks of d_v
    static_assert(VREG * kPrepThreads == kChunk * NVV && KQREG * kPrepThreads == kChunk * NV, "staging");
    static_assert(sizeof(OP) * kChunk * LDP <= sizeof(float) * kChunk * (kChunk + 4), "T~ diag(gamma) in A");
    __shared__ Sm sm;

    const int tid = threadIdx.x, l = lane_id(), w = wave_id(), r = l & 15, gq = l >> 4;
    const SeqIndex si{a.cu, a.seqlen};
    const OP* kg = static_cast<const OP*>(a.k);
    const OP* qg = static_cast<const OP*>(a.q);
    const OP* vg = static_cast<const OP*>(a.v);
    const int64_t nitems = a.seg_len > 0 ? (int64_t)a.num_seqs * a.seg_len * a.hv : a.num_slots * a.hv;

    // One work item = one (slot, value head); a workgroup walks the items
    // blockIdx.x, blockIdx.x + gridDim.x, ..., fetching the next item's
    // inputs into registers while it computes the current one.
    struct Item {
        bool ok;           // a real chunk (not past the end, not a gap slot)
        int64_t slot, t0;
        int h, nt, hq;
    };
    auto locate = [&](int64_t item) {
        Item it{};
        it.ok = false;
        if (item < nitems) {
            int64_t t1;
            if (a.seg_len > 0) {
                // (sequence, chunk j in [seg_j0, seg_j1), value head)
                const int64_t per_seq = (int64_t)a.seg_len * a.hv;
                const int n = (int)(item / per_seq);
                const int64_t rem = item - n * per_seq;
                const int64_t j = a.seg_j0 + rem / a.hv;
                it.h = (int)(rem - (rem / a.hv) * a.hv);
                const int64_t s0 = si.start(n);
                t1 = si.start(n + 1);
                it.t0 = s0 + j * kChunk;
                it.slot = slot_base(s0, n) + j;
                it.ok = j < a.seg_j1 && it.t0 < t1;
            } else {
                // every slot
                it.slot = item / a.hv;
                it.h = (int)(item - it.slot * a.hv);
                int n;
                it.ok = locate_slot(si, a.num_seqs, it.slot, n, it.t0, t1);
            }
            it.nt = it.ok ? (int)((t1 - it.t0) < kChunk ? (t1 - it.t0) : kChunk) : 0;
            it.hq = (it.h * a.hqk) / a.hv;
        }
        return it;
    };
    // rows past the end of the sequence are clamped here and zeroed when staged
    u32x4 kreg[KQREG], qreg[KQREG], vreg[VREG];
    float gv = 0.f, bv = 0.f;
    auto fetch = [&](const Item& it) {
#pragma unroll
        for (int i = 0; i < KQREG; ++i) {
            const int e = tid + i * kPrepThreads;
            const int row = e / NV, cv = e - row * NV;
            const int rc = row < it.nt ? row : it.nt - 1;
            const size_t off = ((size_t)(it.t0 + rc) * a.hqk + it.hq) * DK + (size_t)cv * VE;
            kreg[i] = ld16(kg + off);
            qreg[i] = ld16(qg + off);
        }
#pragma unroll
        for (int i = 0; i < VREG; ++i) {
            const int e = tid + i * kPrepThreads;
            const int row = e / NVV, cv = e - row * NVV;
            const int rc = row < it.nt ? row : it.nt - 1;
            vreg[i] = ld16(vg + ((size_t)(it.t0 + rc) * a.hv + it.h) * DV + (size_t)cv * VE);
        }
        const int lc = l < it.nt ? l : it.nt - 1;
        gv = a.g[(size_t)(it.t0 + lc) * a.hv + it.h];
        bv = a.beta[(size_t)(it.t0 + lc) * a.hv + it.h];
    };

    Item cur = locate(blockIdx.x);
    if (cur.ok) fetch(cur);
    for (int64_t item = blockIdx.x; item < nitems; item += gridDim.x) {
    const Item nxt = locate(item + gridDim.x);
    if (!cur.ok) {
        if (nxt.ok) fetch(nxt);
        cur = nxt;
        continue;
    }
    const int64_t slot = cur.slot;
    const int h = cur.h, nt = cur.nt, hq = cur.hq;
    const size_t blk = (size_t)slot * a.hv + h;
    OP* const Ww = static_cast<OP*>(a.ws_w) + blk * (kChunk * DK);
    OP* const Qw = static_cast<OP*>(a.ws_q) + blk * (kChunk * DK);
    OP* const Kw = static_cast<OP*>(a.ws_k) + blk * (kChunk * DK);
    OP* const Uw = static_cast<OP*>(a.ws_u) + blk * (kChunk * DV);
    OP* const Pw = static_cast<OP*>(a.ws_p) + blk * (kChunk * kChunk);

    // ---- stage K and Q into LDS (zero past the end); V stays in registers
    // until Q's space is free
#pragma unroll
    for (int i = 0; i < KQREG; ++i) {
        const int e = tid + i * kPrepThreads;
        const int row = e / NV, cv = e - row * NV;
        *reinterpret_cast<u32x4*>(&sm.K[row * LD + cv * VE]) = row < nt ? kreg[i] : zero_u4();
        *reinterpret_cast<u32x4*>(&sm.QV[row * LDQV + cv * VE]) = row < nt ? qreg[i] : zero_u4();
    }
    u32x4 vcur[VREG];
#pragma unroll
    for (int i = 0; i < VREG; ++i) {
        const int row = (tid + i * kPrepThreads) / NVV;
        vcur[i] = row < nt ? vreg[i] : zero_u4();
    }
    float gc = gv, bc = bv;
    // the next item's inputs are in flight from here on
    if (nxt.ok) fetch(nxt);
    if (w == 0) {
        if (l >= nt) { gc = 0.f; bc = 0.f; }
        const double G = wave_cumsum_f64((double)gc * 1.4426950408889634);
        const double Gl = lane63_f64(G);
        sm.G[l] = G;
        sm.B[l] = bc;
        sm.gam[l] = fast_exp2((float)G);
        sm.dec[l] = fast_exp2((float)(Gl - G));
        if (l == 0) a.ws_g[blk] = (float)Gl;
    }
    __syncthreads();

    // ---- per wave (scan slice ws = w): Q~ fragments, and K^T fragments by
    // exact identity products -- kept for W, stored as K~^T = K^T diag(D)
    frag Ktr[2][2];
    if (w < NS) {
        const int ws = w;
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            const int row = 16 * tm + r;
            const frag q = frag_rows(sm.QV, LDQV, row, 32 * ws);
            const float gm = sm.gam[row];
            frag qs;
#pragma unroll
            for (int i = 0; i < 8; ++i) qs[i] = from_f32<OP>(to_f32(q[i]) * gm);
            store_frag(Qw, ws * 4 + tm, qs);
        }
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const frag I = iden_frag<OP>(sub);
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                Ktr[sub][kk] = transpose_frag(sm.K, LD, kk, 32 * ws, I);
                frag ks;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int s = 32 * kk + (i < 4 ? 4 * gq + i : 16 + 4 * gq + i - 4);
                    ks[i] = from_f32<OP>(to_f32(Ktr[sub][kk][i]) * sm.dec[s]);
                }
                store_frag(Kw, (ws * 2 + sub) * 2 + kk, ks);
            }
        }
    }

    // ---- Gamma-weighted K K^T (-> A, fp32) and Q K^T (-> P, staged as OP)
    for (int job = w; job < 20; job += kPrepThreads / kWave) {
        const bool qk = job >= 10;
        const int tm = kLowerTiles[job % 10][0], tn = kLowerTiles[job % 10][1];
        const OP* X = qk ? sm.QV : sm.K;
        const int ldx = qk ? LDQV : LD;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < DK / 32; ++kk)
            acc = Ops::mma(frag_rows(X, ldx, 16 * tm + r, 32 * kk), frag_rows(sm.K, LD, 16 * tn + r, 32 * kk), acc);
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
    __syncthreads();   // Q done: its space takes V; P is complete

    // ---- P to the workspace (strictly-upper tiles are zero), V into LDS
    for (int e = tid; e < kChunk * kChunk / VE; e += kPrepThreads) {
        const int f = (e >> 6) / FU, ln = e & 63;
        const int row = 16 * (f >> 1) + (ln & 15);
        const int col = 32 * (f & 1) + 8 * (ln >> 4) + VE * ((e >> 6) % FU);
        const u32x4 x = ((col >> 4) > (row >> 4)) ? zero_u4() : ld16(sm.P + row * LDP + col);
        ws_store(reinterpret_cast<u32x4*>(Pw + (size_t)e * VE), x);
    }
#pragma unroll
    for (int i = 0; i < VREG; ++i) {
        const int e = tid + i * kPrepThreads;
        const int row = e / NVV, cv = e - row * NVV;
        *reinterpret_cast<u32x4*>(&sm.QV[row * LDQV + cv * VE]) = vcur[i];
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

    // ---- T~ = T diag(beta) (into P's space) and T~ diag(gamma) (into A's)
    OP* const Tb = sm.P;
    OP* const Tg = reinterpret_cast<OP*>(&sm.A[0][0]);
    for (int e = tid; e < kChunk * kChunk / 8; e += kPrepThreads) {
        const int t = e >> 3, c0 = (e & 7) * 8;     // row t, columns c0 .. c0 + 7
        const f32x4 t0v = *reinterpret_cast<const f32x4*>(&sm.T[t][c0]);
        const f32x4 t1v = *reinterpret_cast<const f32x4*>(&sm.T[t][c0 + 4]);
        const f32x4 b0v = *reinterpret_cast<const f32x4*>(&sm.B[c0]);
        const f32x4 b1v = *reinterpret_cast<const f32x4*>(&sm.B[c0 + 4]);
        const f32x4 g0v = *reinterpret_cast<const f32x4*>(&sm.gam[c0]);
        const f32x4 g1v = *reinterpret_cast<const f32x4*>(&sm.gam[c0 + 4]);
        frag tb, tg;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float tv = i < 4 ? t0v[i] : t1v[i - 4];
            const float x = (c0 + i <= t) ? tv * (i < 4 ? b0v[i] : b1v[i - 4]) : 0.f;
            tb[i] = from_f32<OP>(x);
            tg[i] = from_f32<OP>(x * (i < 4 ? g0v[i] : g1v[i - 4]));
        }
        *reinterpret_cast<frag*>(&Tb[t * LDP + c0]) = tb;
        *reinterpret_cast<frag*>(&Tg[t * LDP + c0]) = tg;
    }
    __syncthreads();

    // ---- W^T = K^T (T~ diag(gamma))^T for scan slice ws = w; the two 16-row
    // halves of the slice form the scan's paired-order W fragment
    if (w < NS) {
        const int ws = w;
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            f32x4 acc[2];
#pragma unroll
            for (int sub = 0; sub < 2; ++sub) {
                acc[sub] = zero4();
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    acc[sub] = Ops::mma(Ktr[sub][kk], frag_rows(Tg, LDP, 16 * tm + r, 32 * kk), acc[sub]);
            }
            store_frag(Ww, ws * 4 + tm, Ops::pack(acc[0], acc[1]));
        }
    }
    // ---- u = T~ V for the column-block pair cp = w, in the scan's
    // accumulator layout
    if (w < NCP) {
        const int cp = w;
        constexpr int NCB = DV / 16;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const frag I = iden_frag<OP>(sub);
            frag Vtr[2];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) Vtr[kk] = transpose_frag(sm.QV, LDQV, kk, 32 * cp, I);
#pragma unroll
            for (int tw = 0; tw < 4; ++tw) {
                f32x4 acc = zero4();
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) acc = Ops::mma(frag_rows(Tb, LDP, 16 * tw + r, 32 * kk), Vtr[kk], acc);
                quad uq;
#pragma unroll
                for (int i = 0; i < 4; ++i) uq[i] = from_f32<OP>(acc[i]);
                ws_store(reinterpret_cast<quad*>(Uw + ((size_t)(tw * NCB + 2 * cp + sub) * 64 + l) * 4), uq);
            }
        }
    }
    __syncthreads();   // LDS is restaged for the next item
    cur = nxt;
    }
}

// ===========================================================================
// scan: sequential over the chunks of one sequence
// ===========================================================================
// One workgroup per (sequence, value head, 16-column block of d_v), with
// NWS = DK / 32 waves.  The state block S (16 columns x d_k) is split by d_k:
// wave w owns S[:, 32w .. 32w+32) as two fp32 accumulator tiles S^T (tile
// `sub` holding d_k 32 w + 16 sub + (0..15)); packed to the operand type they
// are the state's operand fragment for slice w in paired d_k order.  Token
// tiles are split too: wave w owns tiles tw = w + NWS jt (jt < TPW = 4 / NWS).
// Per chunk:
//   B1 (LDS): every wave publishes its state slice (operand fragment), so
//             each wave sees the whole start state S
//   wave w:  Z = W_tw S^T, Y^T = S Q~_tw^T for its token tiles (full d_k)
//            U = u - Z for its tokens, to LDS
//   B2 (LDS): U for all tokens to every wave
//   wave w:  S_w^T <- gamma_last S_w^T + K~_w^T U        (its d_k slice)
//            O^T = Y^T + U^T P_tw^T                       (its token tiles)
// Nothing is reduced across waves; the only exchanges are the state slices
// (in the operand type the products use anyway) and U.
//
// Global memory.  The vector memory path serves a wave request four lanes at
// a time, and four lanes on four different rows cost four times as much as
// four lanes on one 64-byte piece, so every access keeps consecutive lanes on
// consecutive bytes: all operands come fragment-major from the prep kernel's
// workspace (one 1 KB block per fragment; u as 8-byte lane records), and O
// passes through a small wave-private LDS area between the lanes' tile layout
// and row-wise global stores.  Operands are fetched several chunks ahead,
// each group issued right after the product that consumes the registers it
// refills, so that the vector memory queue is fed evenly through the chunk.
// All loads go through buffer resources (reads past the end of a resource
// return 0, writes past it are dropped), and no load, store or use of a
// loaded value sits behind a branch, so the compiler's memory-counter waits
// stay exact.
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + bytes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
    const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

template <typename OP> struct Buf;
template <> struct Buf<__bf16> {
    // operand fragment: one 16-byte unit
    __device__ __forceinline__ static bf16x8 frag(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
        return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    }
    __device__ __forceinline__ static bf16x4 quad(__amdgpu_buffer_rsrc_t r, unsigned voff) {
        return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, voff, 0, 0));
    }
    __device__ __forceinline__ static void store4(bf16x4 x, __amdgpu_buffer_rsrc_t r, unsigned voff) {
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(i32x2, x), r, voff, 0, 0);
    }
};
template <> struct Buf<float> {
    // operand fragment: two units, the second 1 KB after the first
    __device__ __forceinline__ static f32x8 frag(__amdgpu_buffer_rsrc_t r, unsigned voff, unsigned soff) {
        const f32x4 lo = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
        const f32x4 hi = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff + 1024, 0));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    __device__ __forceinline__ static f32x4 quad(__amdgpu_buffer_rsrc_t r, unsigned voff) {
        return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
    }
    __device__ __forceinline__ static void store4(f32x4 x, __amdgpu_buffer_rsrc_t r, unsigned voff) {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x), r, voff, 0, 0);
    }
};

// XOR swizzle of the O staging tiles (16 rows of four 4-element quads): the
// quad index is XORed with a function of the row so that both the row-wise
// side (four lanes per row) and the tile side (one row per lane) spread over
// the LDS banks.
__device__ __forceinline__ int swz_vo(int row, int elem) {
    return elem == 2 ? ((row >> 2) & 3) : (((row >> 1) ^ (row >> 3)) & 3);
}

// Keeps a group of loads where it stands: no memory operation moves across
// this point, in either direction, at any stage of compilation.
__device__ __forceinline__ void pin() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// Orders this wave's LDS writes before its later LDS reads of the same area.
// LDS executes one wave's operations in issue order; the fence only keeps the
// compiler from moving them.
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

template <typename OP, int DK>
struct ScanGeom {
    static constexpr int NWS = DK / 32;                 // d_k slices = waves per role
    static constexpr int TPW = 4 / NWS;                 // token tiles per wave
    static constexpr int NT = 2 * NWS * kWave;          // threads per workgroup
    static constexpr int E = (int)sizeof(OP);
    static constexpr int FU = Frag<OP>::FU;             // 16-byte units per operand fragment
    static constexpr int QE = 4 * E;                    // bytes per 4-element quad
    static constexpr int VROWB = 16 * E;                // bytes per O tile row
    static constexpr int VB = 16 * VROWB;               // bytes per O tile
    static constexpr int RLD = kChunk + (E == 2 ? 8 : 4);   // 16-byte rows, staggered banks
};

template <typename OP, int DK>
struct ScanSmem {
    using G = ScanGeom<OP, DK>;
    typename Op<OP>::frag sfr[G::NWS][kWave];   // state slices as operand fragments
    alignas(16) OP Ut[16 * G::RLD];             // U as [column][token]
    alignas(16) char ost[G::NWS][G::TPW][G::VB];   // output waves' private O tiles
};

// Per-wave addressing of one sequence's operands in the workspace.
template <typename OP, int DK>
struct ScanCtx {
    using G = ScanGeom<OP, DK>;
    using B = Buf<OP>;
    using frag = typename Op<OP>::frag;
    using quad = typename Op<OP>::quad;
    static constexpr int NWS = G::NWS, TPW = G::TPW, E = G::E, FU = G::FU;
    // operands of one chunk for a state wave and for an output wave
    struct StateStage {
        frag wf[TPW][NWS];   // W[16 tw + r][paired d_k of slice s]
        quad u[TPW];         // u[16 tw + 4 gq + i][16 blk + r]
        frag kt[2][2];       // K~^T[32 w + 16 sub + r][paired tokens from 32 kk]
        float gl;            // G2_last
    };
    struct OutStage {
        frag qf[TPW][NWS];   // Q~[16 tw + r][paired d_k of slice s]
        frag p[TPW][2];      // P[16 tw + r][32 kk + 8 gq + (0..7)]
    };

    // per-sequence: byte address of the sequence's first chunk in each part
    const char* wb; const char* qb; const char* kb; const char* ub; const char* pb; const char* gb;
    int64_t m_step, u_step, p_step, g_step;    // bytes per chunk step
    int u_bytes;                               // bytes of one u block
    int v_row;                                 // bytes per token row of O
    int w;
    // Loop-invariant per-lane byte offsets.  Row offsets that a bounds check
    // must see stay in the per-lane offset; the scalar offset only carries
    // fragment offsets inside a fully valid block.
    unsigned o_voff[TPW];   // row-wise O of tile tw: row 16 tw + (l >> 2), quad l & 3
    unsigned u_voff[TPW];   // u record of (tw, blk) for this lane
    unsigned f_voff;        // fragment-major blocks: unit `lane`

    __device__ __forceinline__ void init(const PrefillArgs& a, int64_t base, int h, int blk, int wave) {
        const int l = lane_id();
        w = wave;
        const size_t b0 = (size_t)base * a.hv + h;
        wb = reinterpret_cast<const char*>(static_cast<const OP*>(a.ws_w) + b0 * (kChunk * DK));
        qb = reinterpret_cast<const char*>(static_cast<const OP*>(a.ws_q) + b0 * (kChunk * DK));
        kb = reinterpret_cast<const char*>(static_cast<const OP*>(a.ws_k) + b0 * (kChunk * DK));
        ub = reinterpret_cast<const char*>(static_cast<const OP*>(a.ws_u) + b0 * ((size_t)kChunk * a.dv));
        pb = reinterpret_cast<const char*>(static_cast<const OP*>(a.ws_p) + b0 * (kChunk * kChunk));
        gb = reinterpret_cast<const char*>(a.ws_g + b0);
        m_step = (int64_t)a.hv * kChunk * DK * E;
        u_step = (int64_t)a.hv * kChunk * a.dv * E;
        p_step = (int64_t)a.hv * kChunk * kChunk * E;
        g_step = (int64_t)a.hv * 4;
        u_bytes = kChunk * a.dv * E;
        v_row = a.hv * a.dv * E;
        const int ncb = a.dv / 16;
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
            const int tw = w + NWS * jt;
            o_voff[jt] = (unsigned)((16 * tw + (l >> 2)) * v_row + (l & 3) * G::QE);
            u_voff[jt] = (unsigned)(((tw * ncb + blk) * 64 + l) * G::QE);
        }
        f_voff = (unsigned)(l * 16);
    }

    __device__ __forceinline__ static int64_t cj(int64_t j, bool valid) { return valid ? j : 0; }
    // Fetch parts of the sequence's chunk j (zeros when !valid).
    template <typename S>
    __device__ __forceinline__ void load_tiles(frag (&f)[TPW][NWS], const char* base, int64_t j, bool valid) const {
        const auto rs = make_rsrc(base + cj(j, valid) * m_step, valid ? (int64_t)kChunk * DK * E : 0);
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt)
#pragma unroll
            for (int sl = 0; sl < NWS; ++sl)
                f[jt][sl] = B::frag(rs, f_voff, (unsigned)((sl * 4 + w + NWS * jt) * FU * 1024));
    }
    __device__ __forceinline__ void load_w(StateStage& s, int64_t j, bool valid) const {
        load_tiles<StateStage>(s.wf, wb, j, valid);
    }
    __device__ __forceinline__ void load_u(StateStage& s, int64_t j, bool valid) const {
        const auto ru = make_rsrc(ub + cj(j, valid) * u_step, valid ? u_bytes : 0);
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) s.u[jt] = B::quad(ru, u_voff[jt]);
    }
    __device__ __forceinline__ void load_k(StateStage& s, int64_t j, bool valid) const {
        const int64_t jc = cj(j, valid);
        const auto rk = make_rsrc(kb + jc * m_step, valid ? (int64_t)kChunk * DK * E : 0);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                s.kt[sub][kk] = B::frag(rk, f_voff, (unsigned)(((w * 2 + sub) * 2 + kk) * FU * 1024));
        const auto rg = make_rsrc(gb + jc * g_step, valid ? 4 : 0);
        s.gl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rg, 0, 0, 0));
    }
    __device__ __forceinline__ void load_q(OutStage& s, int64_t j, bool valid) const {
        load_tiles<OutStage>(s.qf, qb, j, valid);
    }
    __device__ __forceinline__ void load_p(OutStage& s, int64_t j, bool valid) const {
        const auto rp = make_rsrc(pb + cj(j, valid) * p_step, valid ? kChunk * kChunk * E : 0);
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                s.p[jt][kk] = B::frag(rp, f_voff, (unsigned)(((w + NWS * jt) * 2 + kk) * FU * 1024));
    }
};

// Sequence bookkeeping shared by both roles.
struct ScanSeq {
    int n, h;
    int64_t s0, s1, base, jb, je;
};
__device__ __forceinline__ ScanSeq scan_seq(const PrefillArgs& a, int chain) {
    ScanSeq q;
    q.n = chain / a.hv;
    q.h = chain - q.n * a.hv;
    const SeqIndex si{a.cu, a.seqlen};
    q.s0 = si.start(q.n);
    q.s1 = si.start(q.n + 1);
    q.base = slot_base(q.s0, q.n);
    // this launch's chunks of the sequence: [jb, je)
    const int64_t nchunks = (q.s1 - q.s0 + kChunk - 1) / kChunk;
    q.jb = a.seg_j0 < nchunks ? a.seg_j0 : nchunks;
    q.je = a.seg_j1 < nchunks ? a.seg_j1 : nchunks;
    return q;
}

// Both roles walk the same chunk sequence with the same two barriers per
// chunk.  Operands are fetched kStages chunks ahead into a ring of kStages
// register stages (measured on MI355X: 2, 3, 4 and 6 stages stream equally
// fast; the compute unit's own limit on outstanding misses, not the depth,
// bounds the rate).  The loop starts kStages chunks
// early on zeroed stages, so that every load is issued inside the loop body
// and the memory-counter waits see the same load order on every path.  An
// empty chunk -- the leading ones, and the trailing ones that round the count
// up to a multiple of kStages -- is an exact no-op: its operands are zeros
// (G2_last = 0, so gamma_last = 1, and U = 0 leaves S unchanged) and its
// stores are dropped.
#ifndef GDN_SCAN_STAGES
#define GDN_SCAN_STAGES 2
#endif
template <typename OP> constexpr int scan_stages() { return sizeof(OP) == 2 ? GDN_SCAN_STAGES : 2; }

// State wave W: owns d_k slice W of the state and token tiles W + NWS jt.
template <typename OP, int DK, int W>
__device__ __forceinline__ void scan_state_wave(const PrefillArgs& a, ScanSmem<OP, DK>& sm, int chain, int blk) {
    using Ops = Op<OP>;
    using frag = typename Ops::frag;
    using quad = typename Ops::quad;
    using G = ScanGeom<OP, DK>;
    using Ctx = ScanCtx<OP, DK>;
    using St = typename Ctx::StateStage;
    constexpr int NWS = G::NWS, TPW = G::TPW, RLD = G::RLD;
    constexpr int kStages = scan_stages<OP>();
    constexpr int w = W;
    const int l = lane_id(), r = l & 15, gq = l >> 4;
    const ScanSeq q = scan_seq(a, chain);
    Ctx ctx;
    ctx.init(a, q.base, q.h, blk, w);

    // S[sub][i] = S[c][32 w + 16 sub + 4 gq + i], c = 16 blk + r
    f32x4 S[2];
    const size_t srow = ((size_t)chain * a.dv + blk * 16 + r) * DK + 32 * w + 4 * gq;
    if (a.state_in) {
        S[0] = *reinterpret_cast<const f32x4*>(a.state_in + srow);
        S[1] = *reinterpret_cast<const f32x4*>(a.state_in + srow + 16);
    } else {
        S[0] = zero4();
        S[1] = zero4();
    }

    auto chunk = [&](St& cur, int64_t j) {
        const bool pre = j + kStages < q.je;
        // ---- publish this wave's state slice; read the others
        frag Sf[NWS];
        Sf[w] = Ops::pack(S[0], S[1]);
        sm.sfr[w][l] = Sf[w];
        __syncthreads();                                                        // B1
#pragma unroll
        for (int sl = 0; sl < NWS; ++sl)
            if (sl != w) Sf[sl] = sm.sfr[sl][l];
        // ---- Z = W S^T for the wave's token tiles; U = u - Z to LDS
        f32x4 Z[TPW];
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
            f32x4 z0 = zero4(), z1 = zero4();
#pragma unroll
            for (int sl = 0; sl < NWS; sl += 2) {
                z0 = Ops::mma(cur.wf[jt][sl], Sf[sl], z0);
                if (sl + 1 < NWS) z1 = Ops::mma(cur.wf[jt][sl + 1], Sf[sl + 1], z1);
            }
            Z[jt] = z0 + z1;
        }
        pin();
        ctx.load_w(cur, j + kStages, pre);
        pin();
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
            const int tw = w + NWS * jt;
            quad uq;
#pragma unroll
            for (int i = 0; i < 4; ++i) uq[i] = from_f32<OP>(to_f32(cur.u[jt][i]) - Z[jt][i]);
            *reinterpret_cast<quad*>(&sm.Ut[r * RLD + 16 * tw + 4 * gq]) = uq;
        }
        pin();
        ctx.load_u(cur, j + kStages, pre);
        pin();
        __syncthreads();                                                        // B2
        // ---- S_w^T <- gamma_last S_w^T + K~_w^T U
        const float gn = fast_exp2(cur.gl);
        const frag Db0 = frag_rows(sm.Ut, RLD, r, 0), Db1 = frag_rows(sm.Ut, RLD, r, 32);
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
            S[sub] = Ops::mma(cur.kt[sub][1], Db1, Ops::mma(cur.kt[sub][0], Db0, gn * S[sub]));
        pin();
        ctx.load_k(cur, j + kStages, pre);
        pin();
    };

    St st[kStages] = {};
    // Let the initial-state load land here, outside the loop: otherwise the
    // loop head would have to wait for every load in flight on each pass.
    __builtin_amdgcn_s_waitcnt(0);
    for (int64_t j = q.jb - kStages; j < q.je; j += kStages) {
#pragma unroll
        for (int i = 0; i < kStages; ++i) chunk(st[i], j + i);
    }
    if (a.state_out) {
        *reinterpret_cast<f32x4*>(a.state_out + srow) = S[0];
        *reinterpret_cast<f32x4*>(a.state_out + srow + 16) = S[1];
    }
}

// Output wave W: token tiles W + NWS jt; reads the published state and U.
template <typename OP, int DK, int W>
__device__ __forceinline__ void scan_output_wave(const PrefillArgs& a, ScanSmem<OP, DK>& sm, int chain, int blk) {
    using Ops = Op<OP>;
    using frag = typename Ops::frag;
    using quad = typename Ops::quad;
    using G = ScanGeom<OP, DK>;
    using Ctx = ScanCtx<OP, DK>;
    using St = typename Ctx::OutStage;
    using B = Buf<OP>;
    constexpr int NWS = G::NWS, TPW = G::TPW, RLD = G::RLD, E = G::E;
    constexpr int kStages = scan_stages<OP>();
    constexpr int w = W;
    const int l = lane_id(), r = l & 15, gq = l >> 4;
    const ScanSeq q = scan_seq(a, chain);
    Ctx ctx;
    ctx.init(a, q.base, q.h, blk, w);

    // O staging: row-wise side (row l >> 2, quad l & 3) and tile side
    // (row r, quad gq), byte offsets inside a tile
    const unsigned o_rw = (unsigned)((l >> 2) * G::VROWB + G::QE * ((l & 3) ^ swz_vo(l >> 2, E)));
    const unsigned o_tl = (unsigned)(r * G::VROWB + G::QE * (gq ^ swz_vo(r, E)));

    auto chunk = [&](St& cur, int64_t j) {
        const int64_t t0 = q.s0 + j * kChunk;
        const bool pre = j + kStages < q.je;
        __syncthreads();                                                        // B1
        frag Sf[NWS];
#pragma unroll
        for (int sl = 0; sl < NWS; ++sl) Sf[sl] = sm.sfr[sl][l];
        // ---- Y^T = S Q~^T for the wave's token tiles
        f32x4 Y[TPW];
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
            f32x4 y0 = zero4(), y1 = zero4();
#pragma unroll
            for (int sl = 0; sl < NWS; sl += 2) {
                y0 = Ops::mma(Sf[sl], cur.qf[jt][sl], y0);
                if (sl + 1 < NWS) y1 = Ops::mma(Sf[sl + 1], cur.qf[jt][sl + 1], y1);
            }
            Y[jt] = y0 + y1;
        }
        pin();
        ctx.load_q(cur, j + kStages, pre);
        pin();
        __syncthreads();                                                        // B2
        // ---- O^T tiles: rows = columns 16 blk + 4 gq + i, column = token 16 tw + r
        const frag Ub0 = frag_nat(sm.Ut, RLD, r, 0), Ub1 = frag_nat(sm.Ut, RLD, r, 32);
        f32x4 Ot[TPW];
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt)
            Ot[jt] = Ops::mma(Ub1, cur.p[jt][1], Ops::mma(Ub0, cur.p[jt][0], Y[jt]));
        pin();
        ctx.load_p(cur, j + kStages, pre);
        pin();
        // O through the wave's staging area to row-wise stores; rows past the
        // end of the sequence fall outside the resource
        const bool mine = j >= q.jb && j < q.je;
        const int64_t ntl = mine ? q.s1 - t0 : 0;
        const auto ro = make_rsrc(static_cast<OP*>(a.out) + ((size_t)(mine ? t0 : q.s0) * a.hv + q.h) * a.dv + blk * 16,
                                  ntl > 0 ? (ntl - 1) * ctx.v_row + 16 * E : 0);
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
            quad oq;
#pragma unroll
            for (int i = 0; i < 4; ++i) oq[i] = from_f32<OP>(Ot[jt][i]);
            *reinterpret_cast<quad*>(sm.ost[w][jt] + o_tl) = oq;
        }
        wave_lds_fence();
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt)
            B::store4(*reinterpret_cast<const quad*>(sm.ost[w][jt] + o_rw), ro, ctx.o_voff[jt]);
    };

    St st[kStages] = {};
    __builtin_amdgcn_s_waitcnt(0);
    for (int64_t j = q.jb - kStages; j < q.je; j += kStages) {
#pragma unroll
        for (int i = 0; i < kStages; ++i) chunk(st[i], j + i);
    }
}

template <typename OP, int DK>
__global__ __launch_bounds__(2 * (DK / 32) * kWave) void gdn_scan_kernel(PrefillArgs a, int xcd_map) {
    __shared__ ScanSmem<OP, DK> sm;
    // Work item (chain, 16-column block).  With xcd_map, the 8 column blocks of
    // a chain get workgroup ids that the dispatcher sends to one XCD, so they
    // share that XCD's L2 for the chunk operands.
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
    // waves 0 .. NWS-1: state role; NWS .. 2 NWS - 1: output role
    constexpr int NWS = DK / 32;
    switch (wave_id()) {
        case 0: scan_state_wave<OP, DK, 0>(a, sm, chain, blk); break;
        case 1: scan_state_wave<OP, DK, 1>(a, sm, chain, blk); break;
        case 2:
            if constexpr (NWS > 2) scan_state_wave<OP, DK, 2>(a, sm, chain, blk);
            else scan_output_wave<OP, DK, 0>(a, sm, chain, blk);
            break;
        case 3:
            if constexpr (NWS > 2) scan_state_wave<OP, DK, 3>(a, sm, chain, blk);
            else scan_output_wave<OP, DK, 1>(a, sm, chain, blk);
            break;
        case 4: if constexpr (NWS > 2) scan_output_wave<OP, DK, 0>(a, sm, chain, blk); break;
        case 5: if constexpr (NWS > 2) scan_output_wave<OP, DK, 1>(a, sm, chain, blk); break;
        case 6: if constexpr (NWS > 2) scan_output_wave<OP, DK, 2>(a, sm, chain, blk); break;
        default: if constexpr (NWS > 2) scan_output_wave<OP, DK, 3>(a, sm, chain, blk); break;
    }
}

// cu_share: the fraction (1 / cu_share) of the device's compute units the
// stream st may use.
template <typename OP, int DK, int DV>
hipError_t launch_prep(const PrefillArgs& a, hipStream_t st, int cu_share = 1) {
    // persistent: as many workgroups as fit on the device at once
    static int resident[64] = {};   // per device, filled on first use
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    if (resident[dev] == 0) {
        int cus = 0, per_cu = 0;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, gdn_prep_kernel<OP, DK, DV>, kPrepThreads, 0);
        if (e != hipSuccess) return e;
        resident[dev] = (cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
    }
    const int64_t items = a.seg_len > 0 ? (int64_t)a.num_seqs * a.seg_len * a.hv : a.num_slots * a.hv;
    const int64_t fit = resident[dev] / cu_share > 0 ? resident[dev] / cu_share : 1;
    const unsigned nwg = (unsigned)(items < fit ? items : fit);
    hipLaunchKernelGGL((gdn_prep_kernel<OP, DK, DV>), dim3(nwg), dim3(kPrepThreads), 0, st, a);
    return hipGetLastError();
}

template <typename OP, int DK>
hipError_t launch_scan(const PrefillArgs& a, hipStream_t st) {
    const int64_t chains = (int64_t)a.num_seqs * a.hv;
    const int nblk = a.dv / 16;
    const int xcd = (nblk == 8 && chains % 8 == 0) ? 1 : 0;
    dim3 grid((unsigned)(chains * nblk)), block(ScanGeom<OP, DK>::NT);
    hipLaunchKernelGGL((gdn_scan_kernel<OP, DK>), grid, block, 0, st, a, xcd);
    return hipGetLastError();
}

// Per-device resources of the segmented launch: one stream for the prep
// kernels and one for the scan kernels, each confined to one half of the
// compute units (alternate CUs, so each half spans every XCD), so that the
// two kernels overlap without sharing a CU; plus a pool of events.  Created
// on first use (default priority; plain streams if CU masks are unavailable)
// and kept for the life of the process.
constexpr int kMaxSegments = 64;
struct SegmentResources {
    hipStream_t prep = nullptr, scan = nullptr;
    int cu_share = 1;              // 2 when each stream has half of the CUs
    hipEvent_t ev[kMaxSegments + 2] = {};
};

hipError_t segment_resources(int dev, SegmentResources** out) {
    static SegmentResources res[64];
    static std::mutex mu;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    SegmentResources& r = res[dev];
    if (!r.prep) {
        int cus = 0;
        hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        std::vector<uint32_t> even((cus + 31) / 32, 0u), odd((cus + 31) / 32, 0u);
        for (int c = 0; c < cus; ++c) (c % 2 ? odd : even)[c / 32] |= 1u << (c % 32);
        if (cus < 2 ||
            hipExtStreamCreateWithCUMask(&r.scan, (uint32_t)even.size(), even.data()) != hipSuccess ||
            hipExtStreamCreateWithCUMask(&r.prep, (uint32_t)odd.size(), odd.data()) != hipSuccess) {
            (void)hipGetLastError();
            if (r.scan) (void)hipStreamDestroy(r.scan);
            r.scan = nullptr;
            if ((e = hipStreamCreateWithFlags(&r.scan, hipStreamNonBlocking)) != hipSuccess) { r.scan = nullptr; return e; }
            if ((e = hipStreamCreateWithFlags(&r.prep, hipStreamNonBlocking)) != hipSuccess) { r.prep = nullptr; return e; }
        } else {
            r.cu_share = 2;
        }
        for (auto& ev : r.ev) {
            e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
            if (e != hipSuccess) return e;
        }
    }
    *out = &r;
    return hipSuccess;
}

template <typename OP, int DK, int DV>
hipError_t launch_prefill_t(const PrefillArgs& a0, float* state_ws, hipStream_t st) {
    PrefillArgs a = a0;
    const int64_t cs = prefill_segment_chunks(a0.num_tokens, a0.num_seqs, a0.hv, a0.dv);
    if (cs == 0 || !state_ws) {
        a.seg_j0 = 0;
        a.seg_j1 = INT64_MAX / 2;
        a.seg_len = 0;
        a.state_in = a0.init_state;
        a.state_out = a0.final_state;
        hipError_t e = launch_prep<OP, DK, DV>(a, st);
        if (e != hipSuccess) return e;
        return launch_scan<OP, DK>(a, st);
    }
    // Segments of cs chunks: the prep of segment k+1 runs while the scan
    // works through segment k; the state passes from segment to segment
    // through state_ws.  Both internal streams start after everything already
    // queued on st, and st resumes after the last scan.
    const int64_t max_chunks = a0.cu ? (a0.num_tokens + kChunk - 1) / kChunk : (a0.seqlen + kChunk - 1) / kChunk;
    const int nseg = (int)((max_chunks + cs - 1) / cs);
    if (nseg > kMaxSegments) return hipErrorInvalidValue;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    SegmentResources* R = nullptr;
    if ((e = segment_resources(dev, &R)) != hipSuccess) return e;
    if ((e = hipEventRecord(R->ev[0], st)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(R->prep, R->ev[0], 0)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(R->scan, R->ev[0], 0)) != hipSuccess) return e;
    for (int k = 0; k < nseg; ++k) {
        a.seg_j0 = k * cs;
        a.seg_j1 = (k + 1) * cs;
        a.seg_len = (int32_t)cs;
        a.state_in = k == 0 ? a0.init_state : state_ws;
        a.state_out = k == nseg - 1 ? a0.final_state : state_ws;
        if ((e = launch_prep<OP, DK, DV>(a, R->prep, R->cu_share)) != hipSuccess) return e;
        if ((e = hipEventRecord(R->ev[k + 1], R->prep)) != hipSuccess) return e;
        if ((e = hipStreamWaitEvent(R->scan, R->ev[k + 1], 0)) != hipSuccess) return e;
        if ((e = launch_scan<OP, DK>(a, R->scan)) != hipSuccess) return e;
    }
    if ((e = hipEventRecord(R->ev[nseg + 1], R->scan)) != hipSuccess) return e;
    return hipStreamWaitEvent(st, R->ev[nseg + 1], 0);
}

template <typename OP>
hipError_t launch_prefill_dt(const PrefillArgs& a, int dk, int dv, float* state_ws, hipStream_t st) {
    if (dk == 128)
        return dv == 128 ? launch_prefill_t<OP, 128, 128>(a, state_ws, st) : launch_prefill_t<OP, 128, 64>(a, state_ws, st);
    return dv == 128 ? launch_prefill_t<OP, 64, 128>(a, state_ws, st) : launch_prefill_t<OP, 64, 64>(a, state_ws, st);
}

}  // namespace

int64_t prefill_segment_chunks(int64_t num_tokens, int num_seqs, int hv, int dv) {
    if (num_seqs <= 0 || num_seqs > 8) return 0;
    const int64_t scan_wgs = (int64_t)num_seqs * hv * (dv / 16);
    const int64_t avg_chunks = (num_tokens / num_seqs + kChunk - 1) / kChunk;
    if (scan_wgs > 192 || avg_chunks < 512) return 0;
    const int64_t max_chunks = (num_tokens + kChunk - 1) / kChunk;
    int64_t cs = 256;
    while ((max_chunks + cs - 1) / cs > 32) cs *= 2;
    return cs;
}

hipError_t launch_prefill(const PrefillArgs& a, bool bf16, int dk, int dv, float* state_ws, hipStream_t st) {
    if (a.num_seqs == 0) return hipSuccess;
    return bf16 ? launch_prefill_dt<__bf16>(a, dk, dv, state_ws, st) : launch_prefill_dt<float>(a, dk, dv, state_ws, st);
}

}  // namespace gdn
