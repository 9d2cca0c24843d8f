// gdn_prefill.hip -- chunk-parallel GDN prefill for gfx950.
//
// The recurrence S_t = alpha_t S_{t-1}(I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
// o_t = S_t q_t (the GDN layer's fixed-size per-head state: flozi.net,
// "Qwen3.8-Flash-Next architecture", "Der Weg eines Tokens durch das
// Modell", item 1) is evaluated over chunks of C = 64 tokens.  Within a chunk
// with start state S, cumulative log-decay G_t = g_1 + ... + g_t (every
// exponent below is <= 0), gamma_t = e^{G_t}, Gamma_ts = e^{G_t - G_s},
// D_t = e^{G_last - G_t}:
//
//   A  = strict_lower(diag(beta) (Gamma o K K^T)),   T = (I + A)^{-1}
//   T~ = T diag(beta)                                             [state-free]
//   U  = T~ (V - diag(gamma) K S^T)      (the chunk's effective writes u_t)
//   O  = diag(gamma) Q S^T + lower_incl(Gamma o Q K^T) U
//   S' = gamma_last S + U^T diag(D) K
//
// (U is the WY / UT form of the chunk's sequential delta-rule writes; the
// rest follows by expanding the product of the per-token transitions over the
// chunk.)  Over one chunk S maps affinely, S' = S M_c + B_c with
// M_c = gamma_last I - (T~ diag(gamma) K)^T diag(D) K, so a run of chunks
// composes to one affine map as well.  That gives the parallel schedule:
//
//  * gdn_prep_kernel   -- every (chunk, value head) in parallel: gate cumsum
//    in fp64, Gamma-weighted K K^T on the matrix cores, the unit-lower
//    triangular inverse, T~ written in operand-fragment order, and the
//    log2-scaled cumulative gates G2 (fp64).
//  * each sequence is cut into parts of L chunks.  gdn_chunk_kernel<summary>
//    runs every part but the last from a zero state and from the identity,
//    giving the part's offset B_p (d_v x d_k) and transition M_p (d_k x d_k).
//  * gdn_link_kernel   -- per (sequence, head, 16 state rows), sequentially
//    over parts: S_{p+1} = S_p M_p + B_p (fp32 matrix cores).
//  * decay horizon: when every token of a part contracts the state and its
//    gates multiply to at most 2^-160 over the part's last few chunks, the
//    summary starts there (value rows only) and S_{p+1} = B_p: see
//    horizon_start.
//  * gdn_chunk_kernel<output> runs every part from its true start state and
//    writes the outputs (and the final state, from the last part).
//
// Packed batches whose chains alone fill the device run in two launches
// instead: the sequences longer than one compute unit's share keep a first
// part of about one share and are cut into short parts after it.
// gdn_chunk_first_kernel runs every first part (outputs, from init_state; its
// end state starts the second part) beside the summaries of the later parts,
// the link runs over the later parts, and gdn_chunk_kernel<output> runs them.
//
// A workgroup of the chunk kernels holds the whole state of its (part, head)
// in fp32 accumulator tiles, 16 state rows per wave; the chunk's K, Q, V rows
// sit in LDS, and every product reads its operands from there (K^T and V
// tiles through the LDS transpose read), so no wave ever waits for another's
// state.
//
// Padding: a partial last chunk is padded with k = q = v = 0, g = 0, beta = 0;
// padded rows then carry u = 0 and zero rows of K, so they leave the state and
// the real rows untouched, and gamma_last = e^{G_63} equals the decay up to
// the last real token.  Padded output rows are never stored.
#include <algorithm>
#include <mutex>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kTriFrags = 6;       // lower operand fragments of a 64 x 64 matrix
constexpr int kLinkThreads = 256;
// Gate record of one (chunk, value head): G2_t = log2-scaled cumulative gate
// (fp64), then gamma_t = 2^{G2_t}, D_t = 2^{G2_63 - G2_t} and beta_t (fp32).
constexpr int kGateRecord = kChunk * 8 + 3 * kChunk * 4;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T>
__device__ __forceinline__ u32x4 ld16(const T* p) { return *reinterpret_cast<const u32x4*>(p); }

// Operand fragments of a lower-triangular 64 x 64 matrix X (T~ or P): for token
// tile tb and 32-wide K step kk <= tb / 2, fragment f = tri_frag(tb, kk).  Lane
// (r, gq) of fragment f holds X[16 tb + r][32 kk + 4 gq + i] and
// X[16 tb + r][32 kk + 16 + 4 gq + i] (i = 0..3), entries above the diagonal
// zero.  Stored fragment-major: 16-byte unit u of fragment f for lane l at
// element ((f * FU + u) * 64 + l) * VE.
__host__ __device__ constexpr int tri_frag(int tb, int kk) { return tb < 2 ? tb : 2 + 2 * (tb - 2) + kk; }
__device__ __forceinline__ void tri_frag_pos(int f, int& tb, int& kk) {
    tb = f < 2 ? f : 2 + ((f - 2) >> 1);
    kk = f < 2 ? 0 : ((f - 2) & 1);
}

template <typename OP> struct Units {
    static constexpr int VE = 16 / (int)sizeof(OP);   // elements per 16-byte unit
    static constexpr int FU = 8 / VE;                 // units per operand fragment
    // T~ per (chunk, value head), in 1 KB units (64 lanes x 16 bytes).  bf16:
    // the four full lower fragments (1, 2, 4, 5), then the lower halves of
    // fragments 0 and 3, whose upper halves (tiles above the diagonal) are
    // zero: 5 units.  fp32: all six fragments, two units each.
    static constexpr int TU = sizeof(OP) == 2 ? 5 : 12;
};

// bf16 T~ storage: unit of full fragment f (1, 2, 4, 5), and element offset
// of the lane's lower half of fragment f (0, 3) in the fifth unit.
__host__ __device__ constexpr int tri_full_unit(int f) { return f - 1 - (f > 3 ? 1 : 0); }
__host__ __device__ constexpr int tri_half_elem(int f, int lane) { return 4 * 512 + (f == 3 ? 256 : 0) + 4 * lane; }

// Slots of width `span` tokens: part j of sequence n (first token
// start(n) + span j) gets slot floor(start(n) / span) + n + j.  Slots are
// distinct and increase with (n, j); sequence n owns
// [base(n), base(n) + max(1, ceil(len / span))), so ceil(tokens / span) + N
// slots cover every sequence.  An empty sequence owns one slot.
__device__ __forceinline__ int64_t span_base(int64_t start, int n, int64_t span) { return start / span + n; }

// Sequence owning slot `slot` and the slot's index within it (may be past the
// sequence's last part: a gap).
__device__ __forceinline__ void locate_span(const SeqIndex& si, int nseq, int64_t span, int64_t slot, int& n_out,
                                            int64_t& idx) {
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (span_base(si.start(mid), mid, span) <= slot) lo = mid;
        else hi = mid - 1;
    }
    n_out = lo;
    idx = slot - span_base(si.start(lo), lo, span);
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

// Workspace stores are non-temporal: the chunk kernels read them back after
// this kernel has finished, and they should not push its working set out of
// the caches meanwhile.
template <typename T>
__device__ __forceinline__ void ws_store(T* p, const T& x) { __builtin_nontemporal_store(x, p); }

// Race-check builds (GDN_POISON_LDS): every kernel fills its shared memory with
// all-ones words (NaN in fp64, fp32 and bf16) at entry, and the chunk kernels
// refill each input slice with them just before its next direct load.  A read
// of LDS that the protocol has not (re)written since then returns NaN and
// shows up in the results; the arithmetic is unchanged otherwise.
#ifdef GDN_POISON_LDS
constexpr bool kPoisonLds = true;
#else
constexpr bool kPoisonLds = false;
#endif
__device__ __forceinline__ void poison_lds(void* p, int bytes, int tid, int nthreads) {
    u32x4* q = reinterpret_cast<u32x4*>(p);
    for (int i = tid; i < bytes / 16; i += nthreads) q[i] = u32x4{~0u, ~0u, ~0u, ~0u};
}

// ===========================================================================
// prep: T~ fragments and the gate record of one (chunk, value head) per wave
// ===========================================================================
// The four waves of a workgroup take four consecutive items and share nothing,
// so the kernel has no workgroup barrier.  A wave keeps its chunk's K as
// matrix-core operand fragments in registers (loaded straight from memory),
// forms the ten lower 16x16 tiles of the gated A, solves the diagonal blocks
// by forward substitution and the off-diagonal blocks on the fp32 matrix
// cores, and writes T~ = T diag(beta) directly in the chunk kernels' operand
// order.  Only the gates and the diagonal 16 x 16 blocks pass through LDS.
constexpr int kPrepWaves = 4;
constexpr int kDiagLd = 16 * 16 + 8;   // floats per stored 16 x 16 block (padded)

// Workgroups are dispatched to the eight XCDs in turn (workgroup b to XCD
// b mod 8), and each XCD has its own L2.  The value heads of one chunk read
// the same 128-byte lines of g and beta ([tokens, Hv] fp32), so the prep
// kernel hands kPrepGroup consecutive runs of items (kPrepGroup * 4 items: all
// 16 heads of a chunk at Hv = 16) to workgroups of one XCD: in every full
// block of 8 * kPrepGroup workgroups, workgroup 8 i + x takes run
// kPrepGroup x + (i mod kPrepGroup) of that block; the rest keep their order.
constexpr int kXcds = 8, kPrepGroup = 4;
__device__ __forceinline__ int64_t prep_run(int64_t b, int64_t nwg) {
    constexpr int64_t B = kXcds * kPrepGroup;
    if (b >= nwg - nwg % B) return b;
    const int64_t base = b - b % B, i = (b % B) / kXcds, x = b % kXcds;
    return base + kPrepGroup * x + i;
}

struct PrepWaveSmem {
    alignas(16) float D[4 * kDiagLd];  // diagonal blocks of A, then of T; column-major
    alignas(16) double G[kChunk];      // log2-scaled cumulative gates (fp64)
    alignas(16) float B[kChunk];       // beta
    alignas(16) float IK[kChunk];      // raw projections: 1 / |k_t|
};

// Raw projections (see gdn_device.h): the norms are not applied to the stored
// rows; 1 / |k_t| and 1 / |q_t| scale the products in which k_t and q_t appear.

// Sum over the four lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ float sum_groups(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Squares of the eight elements of an operand fragment, summed (bf16: four
// two-term dot products with fp32 accumulation).
template <typename OP>
__device__ __forceinline__ float frag_sq(const typename Op<OP>::frag& f) {
    float s2 = 0.f;
    if constexpr (sizeof(OP) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bf16x2 x = {f[2 * e], f[2 * e + 1]};
            s2 = __builtin_amdgcn_fdot2_f32_bf16(x, x, s2, false);
        }
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) s2 += f[e] * f[e];
    }
    return s2;
}

// Orders a wave's LDS accesses: its earlier LDS writes complete before any
// later LDS read by another lane of the same wave, and the compiler moves no
// memory access across.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Eight consecutive elements p[0..7] as an operand fragment in natural K order.
template <typename OP>
__device__ __forceinline__ typename Op<OP>::frag load_frag8(const OP* p) {
    if constexpr (sizeof(OP) == 2) {
        return *reinterpret_cast<const bf16x8*>(p);
    } else {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

// Index of lower tile (tm, tn), tn <= tm, in row order.
__host__ __device__ constexpr int lower_tile(int tm, int tn) { return tm * (tm + 1) / 2 + tn; }

template <typename OP, int DK, bool RAW>
__global__ __launch_bounds__(kWave * kPrepWaves) void gdn_prep_kernel(PrefillArgs a) {
    using Ops = Op<OP>;
    using frag = typename Ops::frag;
    constexpr int VE = Units<OP>::VE, FU = Units<OP>::FU;
    constexpr int NK = DK / 32;
    __shared__ PrepWaveSmem smem[kPrepWaves];

    const int l = lane_id(), w = wave_id(), r = l & 15, gq = l >> 4;
    PrepWaveSmem& sm = smem[w];
    const int64_t item = prep_run(blockIdx.x, gridDim.x) * kPrepWaves + w;
    if (item >= a.num_slots * a.hv) return;
    const int64_t slot = item / a.hv;
    const int h = (int)(item - slot * a.hv);
    const SeqIndex si{a.cu, a.seqlen};
    int n;
    int64_t j;
    locate_span(si, a.num_seqs, kChunk, slot, n, j);
    const int64_t s1 = si.start(n + 1), t0 = si.start(n) + j * kChunk;
    if (j < 0 || t0 >= s1) return;   // a gap slot (the whole wave leaves)
    if constexpr (kPoisonLds) {
        poison_lds(&sm, (int)sizeof(PrepWaveSmem), l, kWave);
        wave_lds_sync();
    }
    const int nt = (int)((s1 - t0) < kChunk ? (s1 - t0) : kChunk);
    const int hq = (h * a.hqk) / a.hv;
    const size_t blk = (size_t)slot * a.hv + h;

    // ---- loads.  Lane (r, gq) takes K[16 tb + r][32 kk + 8 gq .. + 7]: the A
    // and B operand fragments of K K^T at once.  Rows past the end repeat the
    // last row: their beta is 0, so they never reach A, T~ or the gates.
    frag kf[4][NK];
    const OP* kg = static_cast<const OP*>(a.k);
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const int row = 16 * tb + r;
        const OP* src = kg + ((size_t)(t0 + (row < nt ? row : nt - 1)) * a.hqk + hq) * DK + 8 * gq;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) kf[tb][kk] = load_frag8<OP>(src + 32 * kk);
    }
    const size_t gi = (size_t)(t0 + (l < nt ? l : nt - 1)) * a.hv + h;
    float gl = l < nt ? a.g[gi] : 0.f;
    float bl = l < nt ? a.beta[gi] : 0.f;
    // raw projections: gates from logits; ikr[tb] = 1 / |k| of row 16 tb + r
    float ikr[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (RAW) {
        gl = l < nt ? gate_from_logit(gl) : 0.f;
        bl = l < nt ? beta_from_logit(bl) : 0.f;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            float s2 = 0.f;
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) s2 += frag_sq<OP>(kf[tb][kk]);
            ikr[tb] = 1.f / sqrtf(sum_groups(s2) + kNormEps);
            if (gq == 0) sm.IK[16 * tb + r] = ikr[tb];
        }
    }

    const double G = wave_cumsum_f64((double)gl * 1.4426950408889634);
    const double Gl = lane63_f64(G);
    sm.G[l] = G;
    sm.B[l] = bl;
    wave_lds_sync();

    // ---- whether every token's factor alpha_t (I - beta_t k_t k_t^T) is a
    // contraction of spectral norm <= alpha_t <= 1: g_t <= 0 and 0 <= beta_t
    // |k_t|^2 <= 2 (taken as <= 1.99 against the rounding of |k_t|^2).  Lane (r, gq)
    // checks row 16 tb + r of K (the four lane groups alike) and its own token's
    // gates; NaN anywhere fails every comparison.  Decided here, while K is in
    // registers anyway; the summary's decay horizon reads the result.
    bool contracting;
    {
        bool ok = gl <= 0.f && bl >= 0.f;
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            float s2 = 0.f;
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) s2 += frag_sq<OP>(kf[tb][kk]);
            s2 = sum_groups(s2) * ikr[tb] * ikr[tb];
            ok = ok && sm.B[16 * tb + r] * s2 <= 1.99f;
        }
        contracting = __ballot(!ok) == 0;
    }

    // ---- A = strict_lower(diag(beta) (Gamma o K K^T)): the ten lower tiles in
    // accumulator layout (lane (n, gq) holds A[16 tm + 4 gq + i][16 tn + n]).
    f32x4 at[10];
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
        double gt[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) gt[i] = sm.G[16 * tm + 4 * gq + i];
        f32x4 bt = *reinterpret_cast<const f32x4*>(&sm.B[16 * tm + 4 * gq]);
        if constexpr (RAW) bt = bt * *reinterpret_cast<const f32x4*>(&sm.IK[16 * tm + 4 * gq]);
#pragma unroll
        for (int tn = 0; tn <= tm; ++tn) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < NK; ++kk) acc = Ops::mma(kf[tm][kk], kf[tn][kk], acc);
            if constexpr (RAW) acc = acc * ikr[tn];
            const double gs = sm.G[16 * tn + r];
            f32x4 x;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                x[i] = bt[i] * fast_exp2((float)(gt[i] - gs)) * acc[i];
                if (tn == tm) x[i] = r < 4 * gq + i ? x[i] : 0.f;
            }
            at[lower_tile(tm, tn)] = x;
        }
    }

    // ---- diagonal blocks of T = (I + A)^{-1}, fp32 forward substitution.
    // The A blocks go to LDS column-major; lane (c, q) then solves column c of
    // block q, x_i = delta_ic - sum_{j < i} A_ij x_j, taking column j of the
    // block (a broadcast read within the lane group) once x_j is final.
#pragma unroll
    for (int b = 0; b < 4; ++b)
        *reinterpret_cast<f32x4*>(&sm.D[b * kDiagLd + 16 * r + 4 * gq]) = at[lower_tile(b, b)];
    wave_lds_sync();
    {
        const float* Dq = sm.D + gq * kDiagLd;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) x[i] = i == r ? 1.f : 0.f;
#pragma unroll
        for (int jc = 0; jc < 15; ++jc) {
#pragma unroll
            for (int u = (jc + 1) >> 2; u < 4; ++u) {
                const f32x4 col = *reinterpret_cast<const f32x4*>(Dq + 16 * jc + 4 * u);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (4 * u + e > jc) x[4 * u + e] -= col[e] * x[jc];
            }
        }
        wave_lds_sync();
        float* Tq = sm.D + gq * kDiagLd + 16 * r;
#pragma unroll
        for (int u = 0; u < 4; ++u)
            *reinterpret_cast<f32x4*>(Tq + 4 * u) = f32x4{x[4 * u], x[4 * u + 1], x[4 * u + 2], x[4 * u + 3]};
    }
    wave_lds_sync();
    // T_bb in accumulator layout (tc) and in A-operand layout (ta: lane (r, gq)
    // holds T_bb[r][4 gq + i]); the latter is exactly zero above the diagonal.
    f32x4 tc[4], ta[4][4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        tc[b] = *reinterpret_cast<const f32x4*>(&sm.D[b * kDiagLd + 16 * r + 4 * gq]);
#pragma unroll
        for (int i = 0; i < 4; ++i) ta[b][b][i] = sm.D[b * kDiagLd + 16 * (4 * gq + i) + r];
    }

    // ---- off-diagonal blocks, by distance from the diagonal.  Block row m of
    // T (I + A) = I gives T_mb = -(sum_{b < k <= m} T_mk A_kb) T_bb; it is formed
    // transposed, y^T = sum_k A_kb^T T_mk^T, then T_mb^T = -T_bb^T y^T, so that
    // every operand is at hand in the layout the matrix core wants and the
    // result comes out in A-operand layout.
#pragma unroll
    for (int d = 1; d < 4; ++d) {
#pragma unroll
        for (int b = 0; b + d < 4; ++b) {
            const int m = b + d;
            f32x4 yT = zero4();
#pragma unroll
            for (int k = b + 1; k <= m; ++k) yT = mm16_f32(at[lower_tile(k, b)], ta[m][k], yT);
            ta[m][b] = -mm16_f32(tc[b], yT, zero4());
        }
    }

    // ---- T~ = T diag(beta) as operand fragments, with its diagonal (beta_t:
    // T is unit lower triangular) left out: the chunk kernels add beta_t r_t
    // to u_t in fp32, so the largest entries are never rounded to the operand
    // type.  Then the gate record.
    f32x4 bc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) bc[c] = *reinterpret_cast<const f32x4*>(&sm.B[16 * c + 4 * gq]);
    OP* const Tw = static_cast<OP*>(a.ws_t) + blk * (Units<OP>::TU * 1024 / sizeof(OP));
    auto off_diag = [&](f32x4 x) {   // lane (r, gq) holds entries (r, 4 gq + i) of a diagonal tile
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = r == 4 * gq + i ? 0.f : x[i];
        return x;
    };
#pragma unroll
    for (int f = 0; f < kTriFrags; ++f) {
        const int tb = f < 2 ? f : 2 + ((f - 2) >> 1), kk = f < 2 ? 0 : ((f - 2) & 1);
        f32x4 lo = ta[tb][2 * kk] * bc[2 * kk];
        f32x4 hi = 2 * kk + 1 <= tb ? ta[tb][2 * kk + 1] * bc[2 * kk + 1] : zero4();
        if (2 * kk == tb) lo = off_diag(lo);
        if (2 * kk + 1 == tb) hi = off_diag(hi);
        if constexpr (FU == 1) {
            if (f == 0 || f == 3) {   // the upper half is zero: only the lower is stored
                typename Ops::quad q;
#pragma unroll
                for (int i = 0; i < 4; ++i) q[i] = from_f32<OP>(lo[i]);
                ws_store(reinterpret_cast<typename Ops::quad*>(Tw + tri_half_elem(f, l)), q);
            } else {
                ws_store(reinterpret_cast<frag*>(Tw + ((size_t)tri_full_unit(f) * 64 + l) * VE), Ops::pack(lo, hi));
            }
        } else {
            ws_store(reinterpret_cast<f32x4*>(Tw + ((size_t)(f * 2) * 64 + l) * VE), lo);
            ws_store(reinterpret_cast<f32x4*>(Tw + ((size_t)(f * 2 + 1) * 64 + l) * VE), hi);
        }
    }
    // (raw projections: gamma and D carry 1 / |k_t|, as they only ever scale
    // products with k_t; the chunk kernels take gamma itself from G2)
    double* rec = a.ws_g + blk * (kGateRecord / 8);
    const float ikl = RAW ? sm.IK[l] : 1.f;
    ws_store(rec + l, G);
    ws_store(reinterpret_cast<float*>(rec + kChunk) + l, fast_exp2((float)G) * ikl);
    ws_store(reinterpret_cast<float*>(rec + kChunk) + kChunk + l, fast_exp2((float)(Gl - G)) * ikl);
    ws_store(reinterpret_cast<float*>(rec + kChunk) + 2 * kChunk + l, bl);
    // and 1 / |k_t| itself, for the output kernel's intra-chunk products
    if constexpr (RAW) ws_store(a.ws_ik + blk * kChunk + l, ikl);
    // the chunk's entry for the summary's decay horizon: its log2 decay G2_63
    // if every token is a contraction, else +inf
    if (l == 0 && a.ws_hz) a.ws_hz[blk] = contracting ? (float)Gl : __builtin_inff();
}

// ===========================================================================
// chunk kernels: one workgroup per (part, value head)
// ===========================================================================
// LDS row tiles: 64 rows x D elements, row-major, with the 16-byte units of row
// r permuted by XOR with swz(r).  The pattern was chosen by measuring the LDS
// bank-conflict counters on gfx950 for the accesses used here; with it these
// are free of bank conflicts for D = 128 bf16:
//   * 16-byte row stores (the direct loads: consecutive bytes of LDS),
//   * operand fragments: lane (r, gq) reads unit k0 / 8 + gq of row r, one
//     16-byte read,
//   * the LDS transpose read of a contiguous 16 x 16 tile (lane L: row L / 4).
// The transpose read of the K^T fragments (eight bytes from each of four
// units of a row, all in the same half of their unit) meets each bank twice,
// the least any layout allows for it.  (Rows 8..15 of the pattern differ from
// rows 0..7 by XOR 8, not XOR 1: the latter makes the fragment reads of rows r
// and r + 8 collide.)
template <typename OP, int D>
struct RowTile {
    static constexpr int VE = 16 / (int)sizeof(OP);    // elements per unit
    static constexpr int UPR = D / VE;                  // units per row
    __device__ __forceinline__ static int swz(int r) { return ((((r << 1) | ((r >> 3) & 1)) ^ (r & 8)) & 15) & (UPR - 1); }
    __device__ __forceinline__ static int unit(int r, int u) { return r * D + (u ^ swz(r)) * VE; }
    __device__ __forceinline__ static int elem(int r, int c) { return unit(r, c / VE) + c % VE; }
};

// Operand fragment of row `row`, 32-wide K step from column k0, natural order:
// lane (r, gq) holds columns k0 + 8 gq .. k0 + 8 gq + 7.
template <typename OP, int D>
__device__ __forceinline__ typename Op<OP>::frag rt_frag(const OP* t, int row, int k0) {
    using RT = RowTile<OP, D>;
    const int gq = lane_id() >> 4;
    if constexpr (sizeof(OP) == 2) {
        return *reinterpret_cast<const bf16x8*>(t + RT::unit(row, (k0 >> 3) + gq));
    } else {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(t + RT::unit(row, (k0 >> 2) + 2 * gq));
        const f32x4 hi = *reinterpret_cast<const f32x4*>(t + RT::unit(row, (k0 >> 2) + 2 * gq + 1));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) __bf16 lds_bf16;

// A 16 x 16 tile in accumulator layout: rows row0 .. row0 + 15, and the 16
// columns col0 + cs a + c (a, c = 0..3; cs = 4 for a contiguous tile); lane
// (n, gq) gets M[row0 + 4 gq + i][col0 + cs (n / 4) + n % 4], i = 0..3.
// bf16: one LDS transpose read, for which lane L supplies the 8 bytes at row
// row0 + L / 4, columns col0 + cs (L & 3) .. + 3 (gfx950 delivers element b of
// lane 16 G + 4 j + a's read to lane 16 G + 4 a + b as its element j).
// fp32: four scalar reads.
template <typename OP, int D>
__device__ __forceinline__ typename Op<OP>::quad rt_ctile(const OP* t, int row0, int col0, int cs = 4) {
    using RT = RowTile<OP, D>;
    const int l = lane_id();
    if constexpr (sizeof(OP) == 2) {
        const OP* p = t + RT::elem(row0 + (l >> 2), col0 + cs * (l & 3));
        lds_s16x4* lp = (lds_s16x4*)((lds_bf16*)const_cast<OP*>(p));
        return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(lp));
    } else {
        const int n = l & 15, gq = l >> 4, c = col0 + cs * (n >> 2) + (n & 3);
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = t[RT::elem(row0 + 4 * gq + i, c)];
        return x;
    }
}

// The state's d_k columns are kept in a permuted order, so that a pair of
// state tiles is an operand fragment of eight consecutive d_k columns (one
// 16-byte LDS read of K or Q for the other operand).  Row rho of state tile
// db is d_k column pi_dk(db, rho); tiles 2 kk and 2 kk + 1 together cover the
// columns 32 kk .. 32 kk + 31.
__device__ __forceinline__ int pi_dk(int db, int rho) {
    return 32 * (db >> 1) + 8 * (rho >> 2) + 4 * (db & 1) + (rho & 3);
}

// K^T operand of the state update for state tile db and token half kk: lane
// (r, gq) holds K[32 kk + 4 gq + i][pi_dk(db, r)] and
// K[32 kk + 16 + 4 gq + i][pi_dk(db, r)], i = 0..3.
template <typename OP, int DK>
__device__ __forceinline__ typename Op<OP>::frag kt_frag(const OP* K, int db, int kk) {
    const int c0 = 32 * (db >> 1) + 4 * (db & 1);
    return Op<OP>::join(rt_ctile<OP, DK>(K, 32 * kk, c0, 8), rt_ctile<OP, DK>(K, 32 * kk + 16, c0, 8));
}

template <typename OP>
__device__ __forceinline__ f32x4 quad_f32(const typename Op<OP>::quad& x) {
    return f32x4{to_f32(x[0]), to_f32(x[1]), to_f32(x[2]), to_f32(x[3])};
}

// Operand fragment f (fragment-major storage, see tri_frag).
template <typename OP>
__device__ __forceinline__ typename Op<OP>::frag lds_frag(const OP* base, int f) {
    const int l = lane_id();
    if constexpr (sizeof(OP) == 2) {
        return *reinterpret_cast<const bf16x8*>(base + ((size_t)f * 64 + l) * 8);
    } else {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(base + ((size_t)(2 * f) * 64 + l) * 4);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(base + ((size_t)(2 * f + 1) * 64 + l) * 4);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

// Fragment f of T~ as stored by the prep kernel (see Units::TU).
template <typename OP>
__device__ __forceinline__ typename Op<OP>::frag t_frag(const OP* base, int f) {
    if constexpr (sizeof(OP) == 2) {
        const int l = lane_id();
        if (f == 0 || f == 3) {
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(base + tri_half_elem(f, l));
            return Op<OP>::join(lo, bf16x4{});
        }
        return *reinterpret_cast<const bf16x8*>(base + ((size_t)tri_full_unit(f) * 64 + l) * 8);
    } else {
        return lds_frag(base, f);
    }
}

// Half h (K slots 4h .. 4h + 3) of the lane's share of fragment f.
template <typename OP>
__device__ __forceinline__ void lds_frag_half(OP* base, int f, int h, const typename Op<OP>::quad& x) {
    using quad = typename Op<OP>::quad;
    const int l = lane_id();
    if constexpr (sizeof(OP) == 2) *reinterpret_cast<quad*>(base + ((size_t)f * 64 + l) * 8 + 4 * h) = x;
    else *reinterpret_cast<quad*>(base + ((size_t)(2 * f + h) * 64 + l) * 4) = x;
}

typedef __attribute__((address_space(3))) void lds_void;

// Direct loads into LDS (gfx950: lane l of the wave writes its 16 bytes to the
// LDS address given plus 16 l; lanes whose range check fails write zeros).
// Instruction i of a 64-row tile fills LDS bytes [1024 i, 1024 i + 1024) of the
// row tile `dst` (RowTile layout): rows past the resource's end read as 0.
template <typename OP, int D>
__device__ __forceinline__ void rows_to_lds(OP* dst, __amdgpu_buffer_rsrc_t rs, unsigned rstride, int i) {
    constexpr int RB = D * (int)sizeof(OP);           // bytes per row
    constexpr int RPI = 1024 / RB;                    // rows per instruction
    constexpr int UPR = RB / 16;                      // 16-byte units per row
    const int l = lane_id();
    const int r = i * RPI + l / UPR, p = l % UPR;
    const int u = p ^ RowTile<OP, D>::swz(r);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(dst + i * (1024 / (int)sizeof(OP))), 16,
                                             (unsigned)r * rstride + (unsigned)u * 16, 0, 0, 0);
}
// Plain copy: instruction i fills LDS bytes [1024 i, 1024 i + 1024) from the same
// bytes of the resource.
__device__ __forceinline__ void bytes_to_lds(void* dst, __amdgpu_buffer_rsrc_t rs, int i) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)((char*)dst + 1024 * i), 16,
                                             (unsigned)(1024 * i + 16 * lane_id()), 0, 0, 0);
}

// s_waitcnt vmcnt(0): this wave's loads (and stores) are complete.
constexpr int kWaitVm0 = 0x0F70;
// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses,
// then s_barrier.  Unlike __syncthreads() it does not wait for direct-to-LDS
// loads still in flight (those target the other buffer set).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// One chunk's inputs in LDS.  IKB: also 1 / |k_t| of the raw-projection
// prefill (64 values; the 1 KB region is what one direct load writes).
template <typename OP, int DK, int DV, bool OUT, bool IKB = false>
struct ChunkBuf {
    alignas(16) OP K[kChunk * DK];
    alignas(16) OP V[kChunk * DV];
    alignas(16) OP Q[OUT ? kChunk * DK : 8];
    alignas(16) OP T[kTriFrags * 64 * 8];   // T~ fragments
    alignas(16) double G2[kChunk];          // gate record: G2, gamma, D, beta
    alignas(16) float gam[kChunk];
    alignas(16) float dec[kChunk];
    alignas(16) float bet[kChunk];
    float gpad[(2048 - kGateRecord) / 4];   // the gate record's second 1 KB load writes up to here
    alignas(16) float IK[IKB ? 256 : 4];
};

// Geometry of the chunk kernels: one wave per 16 state rows (two waves per
// SIMD, so one wave's LDS latency hides behind the other's matrix work).
// Summary: value block w and transition block w per wave, so every K operand
// read from LDS feeds two products (with d_v != d_k, the waves past the
// smaller block count hold one block).
template <typename OP, int DK, int DV, bool OUT>
struct ChunkGeom {
    static constexpr int NR = OUT ? 1 : 2;
    static constexpr int NW = OUT ? DV / 16 : (DV > DK ? DV : DK) / 16;
    static constexpr int NT = NW * kWave;
    // input buffer sets: bf16 output 2, bf16 summary 3 (its K^T fragments are
    // formed a chunk ahead, see gdn_chunk_kernel), fp32 1 (rows do not fit twice)
    static constexpr int NBUF = sizeof(OP) == 2 ? (OUT ? 2 : 3) : 1;
    static constexpr bool KTA = !OUT && sizeof(OP) == 2;   // K^T fragments one chunk ahead
};

// Row block R0 .. R0 + 15 of a row-major (rows x DK) fp32 state, as S^T tiles:
// tile db, lane (n, gq) holds S[R0 + n][pi_dk(db, 4 gq + i)] (four consecutive
// columns).
template <int DK>
__device__ __forceinline__ void load_state(const float* S, int R0, f32x4 (&ST)[DK / 16]) {
    const int l = lane_id(), n = l & 15, gq = l >> 4;
#pragma unroll
    for (int db = 0; db < DK / 16; ++db)
        ST[db] = S ? *reinterpret_cast<const f32x4*>(S + (size_t)(R0 + n) * DK + pi_dk(db, 4 * gq)) : zero4();
}
template <int DK>
__device__ __forceinline__ void store_state(float* S, int R0, const f32x4 (&ST)[DK / 16]) {
    const int l = lane_id(), n = l & 15, gq = l >> 4;
#pragma unroll
    for (int db = 0; db < DK / 16; ++db) *reinterpret_cast<f32x4*>(S + (size_t)(R0 + n) * DK + pi_dk(db, 4 * gq)) = ST[db];
}
// The transition M_p in the workspace, transposed: entry M[r][c] at c DK + tr(c, r)
// with tr(c, r) = r XOR 4 (c mod 16).  The link kernel's B operand for
// column c is M[r .. r + 3][c] for aligned r: 16 contiguous bytes, and the XOR
// spreads the 16 columns of a read over all 64 banks.
__host__ __device__ constexpr int m_pos(int c, int r, int dk) { return c * dk + (r ^ ((c & 15) << 2)); }
template <int DK>
__device__ __forceinline__ void store_transition(float* M, int R0, const f32x4 (&ST)[DK / 16]) {
    const int l = lane_id(), n = l & 15, gq = l >> 4;
#pragma unroll
    for (int db = 0; db < DK / 16; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) M[m_pos(pi_dk(db, 4 * gq + i), R0 + n, DK)] = ST[db][i];
}


// The chunk's K^T operand fragments (2 per state tile), transposed once per
// chunk and shared by all waves: wave w writes fragments w, w + NW, ...
template <typename OP, int DK, int NW>
__device__ __forceinline__ void transpose_kt(const OP* K, OP* kt, int w) {
    constexpr int KTF = 2 * (DK / 16);
    const int l = lane_id();
#pragma unroll
    for (int r = 0; r < (KTF + NW - 1) / NW; ++r) {
        const int f = w + NW * r;
        if (KTF % NW == 0 || f < KTF)
            *reinterpret_cast<bf16x8*>(kt + ((size_t)f * 64 + l) * 8) = kt_frag<OP, DK>(K, f >> 1, f & 1);
    }
}

// Keeps the compiler's scheduler from moving instructions across this point,
// so that each group of LDS reads is issued ahead of the products that use the
// previous group (the reads are then in flight while the matrix cores work).
// Measured: this helps the summary kernel (two state blocks per wave) and hurts
// the output kernel (one block per wave, two waves per SIMD), which is left to
// the compiler's own schedule.
template <bool ON>
__device__ __forceinline__ void sched_fence() {
    if constexpr (ON) __builtin_amdgcn_sched_barrier(0);
}

// Lane move inside groups of four lanes (DPP quad permutation CTRL; every lane
// is written, so no "old" value is needed).
template <int CTRL>
__device__ __forceinline__ float quad_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// 4 x 4 transpose across the four lanes of a group: lane a's element i becomes
// lane i's element a.  Two exchange steps, with lanes a ^ 1 (elements whose
// index differs from a in bit 0) and a ^ 2 (bit 1).
__device__ __forceinline__ f32x4 quad_transpose(f32x4 x) {
    const int a = lane_id() & 3;
    f32x4 p, m;
    p[0] = quad_mov<0xB1>(x[1]); p[1] = quad_mov<0xB1>(x[0]); p[2] = quad_mov<0xB1>(x[3]); p[3] = quad_mov<0xB1>(x[2]);
#pragma unroll
    for (int i = 0; i < 4; ++i) m[i] = ((i ^ a) & 1) ? p[i] : x[i];
    p[0] = quad_mov<0x4E>(m[2]); p[1] = quad_mov<0x4E>(m[3]); p[2] = quad_mov<0x4E>(m[0]); p[3] = quad_mov<0x4E>(m[1]);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = ((i ^ a) & 2) ? p[i] : m[i];
    return x;
}

template <int CTRL>
__device__ __forceinline__ unsigned quad_mov_u(unsigned x) {
    return (unsigned)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, false);
}

// The same transpose after rounding to bf16: lane a packs its four values as
// (x0, x1), (x2, x3) and ends with the four lanes' element a, as bf16x4.
// Step 1 swaps 16-bit halves with lane a ^ 1 (v_perm with the lane-parity
// selector sel: even lanes keep their low halves, odd lanes their high
// halves), step 2 swaps whole dwords with lane a ^ 2.
__device__ __forceinline__ bf16x4 quad_transpose_bf16(f32x4 x, unsigned sel) {
    const int a = lane_id() & 3;
    const bf16x2 p0 = {(__bf16)x[0], (__bf16)x[1]}, p1 = {(__bf16)x[2], (__bf16)x[3]};
    const unsigned d0 = __builtin_bit_cast(unsigned, p0), d1 = __builtin_bit_cast(unsigned, p1);
    const unsigned e0 = __builtin_amdgcn_perm(d0, quad_mov_u<0xB1>(d0), sel);
    const unsigned e1 = __builtin_amdgcn_perm(d1, quad_mov_u<0xB1>(d1), sel);
    const unsigned q0 = quad_mov_u<0x4E>(e0), q1 = quad_mov_u<0x4E>(e1);
    const unsigned f0 = (a & 2) ? q1 : e0, f1 = (a & 2) ? e1 : q0;
    const bf16x2 r0 = __builtin_bit_cast(bf16x2, f0), r1 = __builtin_bit_cast(bf16x2, f1);
    return bf16x4{r0[0], r0[1], r1[0], r1[1]};
}

// One chunk for the wave's NR state blocks (rows R0[b] .. R0[b] + 15; block b
// has a V term when bit b of VMASK is set, else it is a transition block whose
// V is zero).  ST[b][db] holds block b's S^T tile for d_k columns
// pi_dk(db, .): lane (n, gq) has S[R0 + n][pi_dk(db, 4 gq + i)].  Packed
// pairwise, these tiles are the B operand of K S^T and of Q S^T.
//   Y  = K S^T,  R = V - diag(gamma) Y,  U = T~_off R + diag(beta) R
//   S^T <- gamma_last S^T + K^T diag(D) U
//   O  = diag(gamma) (Q S^T) + P_off U + diag(P) U                 (OUT)
// T~_off and P_off are T~ and P without their diagonals; the diagonal terms
// (beta_t and q_t . k_t, the largest entries) multiply u_t and r_t in fp32,
// lane by lane, since Y, R, U, Z and O share one tile layout (tokens x state
// rows).  Only the off-diagonal entries are rounded to the operand type.
// Output (and fp32): before the barrier in the middle, the wave also writes
// its share of the chunk's K^T operand fragments (bf16), P fragments and P
// diagonal (OUT); after it, it reads all of them.  OUT: the O tiles go to the
// row tile `ost` (RowTile layout).
// bf16 summary: `kt` already holds this chunk's K^T fragments (formed during
// the previous chunk) and there is no barrier.
// hook(stage) lets the caller place its other work: stage 0 once the wave's
// LDS writes of the state-free part are issued (the next chunk's direct loads
// go there, since the compiler orders any LDS write it cannot tell apart from
// their target after them), stage 1 once the products of Y are issued, stage
// 2 between U and the state update.
template <typename OP, int DK, int DV, bool OUT, int NR, int VMASK, int NW, bool RAW, typename F>
__device__ __forceinline__ void chunk_step(const ChunkBuf<OP, DK, DV, OUT, OUT && RAW>& cb, OP* P, OP* kt, OP* ost,
                                           f32x4 (&ST)[NR][DK / 16], const int (&R0)[NR], int w, F&& hook,
                                           float* nrm, float* pdg) {
    using Ops = Op<OP>;
    using frag = typename Ops::frag;
    using quad = typename Ops::quad;
    constexpr int NDB = DK / 16, NKK = DK / 32;
    constexpr bool KT = sizeof(OP) == 2;
    constexpr bool KTA = KT && !OUT;                            // kt was formed a chunk ahead
    const int l = lane_id(), n = l & 15, gq = l >> 4;

    // ---- state-free work of the chunk: P^T fragments and K^T fragments.
    // P[t][s] = Gamma_ts q_t . k_s for s <= t.  Wave w forms P fragments
    // w, w + NW, ... (< 6): fragment (tb, kk) is the token tiles 2 kk and
    // 2 kk + 1 of row tile tb, as B operand of U^T P^T (tile 2 kk + 1 lies above
    // the diagonal, all zero, when 2 kk + 1 > tb: not computed).
    if constexpr (OUT) {
#pragma unroll
        for (int f = w; f < kTriFrags; f += NW) {
            int tb, kk;
            tri_frag_pos(f, tb, kk);
            const bool two = 2 * kk + 1 <= tb;   // wave-uniform
            frag pq[NKK], p0[NKK], p1[NKK];
#pragma unroll
            for (int k2 = 0; k2 < NKK; ++k2) {
                pq[k2] = rt_frag<OP, DK>(cb.Q, 16 * tb + n, 32 * k2);
                p0[k2] = rt_frag<OP, DK>(cb.K, 32 * kk + n, 32 * k2);
                if (two) p1[k2] = rt_frag<OP, DK>(cb.K, 32 * kk + 16 + n, 32 * k2);
            }
            const int t = 16 * tb + n;
            const double gt = cb.G2[t];
            f32x4 a0 = zero4(), a1 = zero4();
#pragma unroll
            for (int k2 = 0; k2 < NKK; ++k2) a0 = Ops::mma(p0[k2], pq[k2], a0);
            if (two) {
#pragma unroll
                for (int k2 = 0; k2 < NKK; ++k2) a1 = Ops::mma(p1[k2], pq[k2], a1);
            }
            if constexpr (RAW) {
                // 1 / |q_t| for this lane's row t from the Q fragments already
                // loaded (gamma_t / |q_t| is kept in nrm for the outputs after the
                // barrier in the middle, written once per row tile); 1 / |k_s|
                // from the prep kernel, loaded with the chunk
                float sq = 0.f;
#pragma unroll
                for (int k2 = 0; k2 < NKK; ++k2) sq += frag_sq<OP>(pq[k2]);
                const float iq = 1.f / sqrtf(sum_groups(sq) + kNormEps);
                if (kk == 0 && gq == 0) nrm[t] = fast_exp2((float)gt) * iq;
                a0 = a0 * iq * *reinterpret_cast<const f32x4*>(&cb.IK[32 * kk + 4 * gq]);
                if (two) a1 = a1 * iq * *reinterpret_cast<const f32x4*>(&cb.IK[32 * kk + 16 + 4 * gq]);
            }
            // the diagonal P_tt goes to pdg in fp32 (applied to u_t in fp32), the
            // strictly lower entries to the operand fragment
            quad v0, v1;
            f32x4 x0, x1;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s0 = 32 * kk + 4 * gq + i, s1 = s0 + 16;
                x0[i] = fast_exp2((float)(gt - cb.G2[s0])) * a0[i];
                x1[i] = two ? fast_exp2((float)(gt - cb.G2[s1])) * a1[i] : 0.f;
                v0[i] = from_f32<OP>(s0 < t ? x0[i] : 0.f);
                v1[i] = from_f32<OP>(s1 < t ? x1[i] : 0.f);
            }
            // the diagonal tile of this row tile is token tile 2 kk (x0) or 2 kk + 1
            // (x1); lane (n, gq) holds its entry (n, n) iff gq = n / 4, as element n % 4.
            // Every lane stores (no branch): the others into a spare slot.
            if (2 * kk == tb || 2 * kk + 1 == tb) {   // wave-uniform
                const f32x4 xd = 2 * kk == tb ? x0 : x1;
                const int e = n & 3;
                const float d = e == 0 ? xd[0] : e == 1 ? xd[1] : e == 2 ? xd[2] : xd[3];
                pdg[gq == (n >> 2) ? t : kChunk + l] = d;
            }
            if constexpr (sizeof(OP) == 2) {
                *reinterpret_cast<frag*>(P + ((size_t)f * 64 + l) * 8) = Ops::join(v0, v1);
            } else {
                lds_frag_half(P, f, 0, v0);
                lds_frag_half(P, f, 1, v1);
            }
        }
        sched_fence<!OUT>();
    }
    if constexpr (KT && !KTA) {
        transpose_kt<OP, DK, NW>(cb.K, kt, w);
        sched_fence<!OUT>();
    }
    hook(0);
    sched_fence<!OUT>();

    // ---- Y = K S^T and Z = S Q^T; operands stream in groups of two token tiles
    frag Sb[NR][NKK];
#pragma unroll
    for (int b = 0; b < NR; ++b)
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) Sb[b][kk] = Ops::pack(ST[b][2 * kk], ST[b][2 * kk + 1]);
    f32x4 Y[NR][4], Z[NR][4];
    frag g0[2][NKK], g1[2][NKK];
    auto load2 = [&](frag (&g)[2][NKK], const OP* M, int tb0) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk) g[h][kk] = rt_frag<OP, DK>(M, 16 * (tb0 + h) + n, 32 * kk);
    };
    auto mmY = [&](const frag (&g)[2][NKK], int tb0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int b = 0; b < NR; ++b) Y[b][tb0 + h] = zero4();
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int b = 0; b < NR; ++b) Y[b][tb0 + h] = Ops::mma(g[h][kk], Sb[b][kk], Y[b][tb0 + h]);
        }
    };
    auto mmZ = [&](const frag (&g)[2][NKK], int tb0) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int b = 0; b < NR; ++b) Z[b][tb0 + h] = zero4();
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int b = 0; b < NR; ++b) Z[b][tb0 + h] = Ops::mma(g[h][kk], Sb[b][kk], Z[b][tb0 + h]);
        }
    };
    load2(g0, cb.K, 0);
    sched_fence<!OUT>();
    load2(g1, cb.K, 2);
    sched_fence<!OUT>();
    mmY(g0, 0);
    sched_fence<!OUT>();
    if constexpr (OUT) load2(g0, cb.Q, 0);
    sched_fence<!OUT>();
    mmY(g1, 2);
    sched_fence<!OUT>();
    hook(1);
    sched_fence<!OUT>();
    if constexpr (OUT) {
        load2(g1, cb.Q, 2);
        sched_fence<!OUT>();
        mmZ(g0, 0);
        sched_fence<!OUT>();
    }
    // operands of R and U
    f32x4 g4[4], vt[NR][4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        g4[tb] = *reinterpret_cast<const f32x4*>(&cb.gam[16 * tb + 4 * gq]);
#pragma unroll
        for (int b = 0; b < NR; ++b)
            vt[b][tb] = ((VMASK >> b) & 1) ? quad_f32<OP>(rt_ctile<OP, DV>(cb.V, 16 * tb, R0[b])) : zero4();
    }
    frag tf[kTriFrags];
#pragma unroll
    for (int f = 0; f < kTriFrags; ++f) tf[f] = t_frag(cb.T, f);
    f32x4 dd[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
        dd[kk][0] = *reinterpret_cast<const f32x4*>(&cb.dec[32 * kk + 4 * gq]);
        dd[kk][1] = *reinterpret_cast<const f32x4*>(&cb.dec[32 * kk + 16 + 4 * gq]);
    }
    // gamma_last (raw projections: from G2, the gamma slot carries 1 / |k|)
    const float gl = RAW ? fast_exp2((float)cb.G2[kChunk - 1]) : cb.gam[kChunk - 1];
    sched_fence<!OUT>();
    if constexpr (OUT) {
        mmZ(g1, 2);
        sched_fence<!OUT>();
    }
    // R = V - diag(gamma) Y (fp32, in Y's registers), packed pairwise as the B
    // operand of T~_off R; U = T~_off R + diag(beta) R, the product accumulating
    // onto the fp32 diagonal term
#pragma unroll
    for (int tb = 0; tb < 4; ++tb)
#pragma unroll
        for (int b = 0; b < NR; ++b) Y[b][tb] = vt[b][tb] - g4[tb] * Y[b][tb];
    frag Rb[NR][2];
#pragma unroll
    for (int tp = 0; tp < 2; ++tp)
#pragma unroll
        for (int b = 0; b < NR; ++b) Rb[b][tp] = Ops::pack(Y[b][2 * tp], Y[b][2 * tp + 1]);
    f32x4 U[NR][4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
        const f32x4 bt = *reinterpret_cast<const f32x4*>(&cb.bet[16 * tb + 4 * gq]);
#pragma unroll
        for (int b = 0; b < NR; ++b) U[b][tb] = Ops::mma(tf[tri_frag(tb, 0)], Rb[b][0], bt * Y[b][tb]);
        if (tb >= 2)
#pragma unroll
            for (int b = 0; b < NR; ++b) U[b][tb] = Ops::mma(tf[tri_frag(tb, 1)], Rb[b][1], U[b][tb]);
    }
    frag Ud[NR][2], Ua[NR][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int b = 0; b < NR; ++b) {
            Ud[b][kk] = Ops::pack(dd[kk][0] * U[b][2 * kk], dd[kk][1] * U[b][2 * kk + 1]);
            if constexpr (OUT) Ua[b][kk] = Ops::pack(U[b][2 * kk], U[b][2 * kk + 1]);
        }

    // K^T fragments (bf16) and P are complete after this barrier; so is every
    // wave's read of the previous chunk's O rows.
    if constexpr (OUT || (KT && !KTA)) lds_barrier();
    hook(2);
    sched_fence<!OUT>();

    // ---- S^T <- gamma_last S^T + K^T diag(D) U, operands in two groups
    constexpr int HD = NDB / 2;
    frag k0[HD][2], k1[HD][2];
    auto loadK = [&](frag (&g)[HD][2], int db0) {
#pragma unroll
        for (int d = 0; d < HD; ++d)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                if constexpr (KT) g[d][kk] = lds_frag(kt, 2 * (db0 + d) + kk);
                else g[d][kk] = kt_frag<OP, DK>(cb.K, db0 + d, kk);
            }
    };
    auto mmS = [&](const frag (&g)[HD][2], int db0) {
#pragma unroll
        for (int d = 0; d < HD; ++d)
#pragma unroll
            for (int b = 0; b < NR; ++b) {
                f32x4 acc = gl * ST[b][db0 + d];
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) acc = Ops::mma(g[d][kk], Ud[b][kk], acc);
                ST[b][db0 + d] = acc;
            }
    };
    loadK(k0, 0);
    sched_fence<!OUT>();
    loadK(k1, HD);
    sched_fence<!OUT>();
    mmS(k0, 0);
    sched_fence<!OUT>();
    frag pf[kTriFrags];
    f32x4 gt[4], pd[4];
    // byte selector of the first exchange step of quad_transpose_bf16 (by lane parity)
    const unsigned psel = (l & 1) ? 0x07060302u : 0x01000504u;
    if constexpr (OUT) {
#pragma unroll
        for (int f = 0; f < kTriFrags; ++f) pf[f] = lds_frag(P, f);
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            gt[tb] = *reinterpret_cast<const f32x4*>(RAW ? &nrm[16 * tb + 4 * gq] : &cb.gam[16 * tb + 4 * gq]);
            pd[tb] = *reinterpret_cast<const f32x4*>(&pdg[16 * tb + 4 * gq]);
        }
    }
    sched_fence<!OUT>();
    mmS(k1, HD);
    if constexpr (OUT) {
        sched_fence<!OUT>();
        // O tiles (tokens x rows): lane (n, gq) has O[16 tb + 4 gq + i][R0 + n]; after
        // the transpose inside each group of four lanes, O[16 tb + 4 gq + (n & 3)][R0 +
        // 4 (n >> 2) + i], four consecutive columns of one row for the LDS row tile
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
            for (int b = 0; b < NR; ++b) {
                f32x4 o = Ops::mma(pf[tri_frag(tb, 0)], Ua[b][0], gt[tb] * Z[b][tb] + pd[tb] * U[b][tb]);
                if (tb >= 2) o = Ops::mma(pf[tri_frag(tb, 1)], Ua[b][1], o);
                quad oq;
                if constexpr (sizeof(OP) == 2) {
                    oq = quad_transpose_bf16(o, psel);
                } else {
                    o = quad_transpose(o);
#pragma unroll
                    for (int i = 0; i < 4; ++i) oq[i] = from_f32<OP>(o[i]);
                }
                *reinterpret_cast<quad*>(ost + RowTile<OP, DV>::elem(16 * tb + 4 * gq + (n & 3), R0[b] + 4 * (n >> 2))) = oq;
            }
        }
    }
}

// Shared memory of a chunk-kernel workgroup.
template <typename OP, int DK, int DV, bool OUT, bool RAW>
struct ChunkSmem {
    using G = ChunkGeom<OP, DK, DV, OUT>;
    // bf16: the chunk's K^T operand fragments (2 per state tile), transposed once
    // per chunk instead of once per wave
    static constexpr int KTS = sizeof(OP) == 2 ? 2 * (DK / 16) * 64 * 8 : 8;
    ChunkBuf<OP, DK, DV, OUT, OUT && RAW> bufs[G::NBUF];
    alignas(16) OP Pf[OUT ? kTriFrags * 64 * 8 : 8];
    alignas(16) OP Ost[OUT ? kChunk * DV : 8];        // O rows of the previous chunk (RowTile layout)
    alignas(16) OP Kt[(G::KTA ? 2 : 1) * KTS];
    alignas(16) float Nrm[OUT && RAW ? kChunk : 1];   // raw projections: gamma_t / |q_t| of the chunk
    alignas(16) float Pdg[OUT ? kChunk + kWave : 1];  // diagonal of the chunk's P, fp32 (then spare slots)
};

// Where a workgroup's chunk-kernel arrays are (ChunkSmem's members, wherever
// they are placed).
template <typename OP, int DK, int DV, bool OUT, bool RAW>
struct ChunkLds {
    ChunkBuf<OP, DK, DV, OUT, OUT && RAW>* bufs;
    OP *Pf, *Ost, *Kt;
    float *Nrm, *Pdg;
    __device__ static ChunkLds of(ChunkSmem<OP, DK, DV, OUT, RAW>& m) { return {m.bufs, m.Pf, m.Ost, m.Kt, m.Nrm, m.Pdg}; }
};

// Decay horizon of a part summary.  Over chunks [c, je) the state maps as
// S -> S M' + B'.  If every token of the part is a contraction (each factor
// alpha_t (I - beta_t k_t k_t^T) of spectral norm <= alpha_t <= 1, checked by the
// prep kernel) then |M'| <= 2^(sum of the chunks' log2 decays), and the part's
// map (M_p, B_p) = (M_0 M', B_0 M' + B') differs from (M', B') by at most that
// factor times |M_0 - I| <= 2 and |B_0| <= sum_t beta_t |v_t| |k_t| (the state the
// chunks before c leave from zero).  Once the factor is below 2^-160 (under the
// smallest fp32 magnitude) the summary may start at c, from zero and from the
// identity, instead of at the part's first chunk.  Returns the latest such c
// (jb when there is none, or when some chunk of the part is not a contraction),
// and in `taken` whether there is one: then M_p is negligible and the link may
// take S_{p+1} = B_p.  Lane l reads the entries of chunks e - 1 - l, 64 chunks at
// a time from the end; every wave computes the same values.
constexpr double kHorizonLog2 = -160.0;
__device__ int64_t horizon_start(const float* hz, int64_t cbase, int hv, int h, int64_t jb, int64_t je, bool& taken) {
    taken = false;
    if (!hz) return jb;
    const int l = lane_id();
    double carry = 0.0;
    int64_t c = jb;
    bool found = false, ok = true;
    for (int64_t e = je; e > jb; e -= kWave) {
        const int64_t j = e - 1 - l;
        const float xj = hz[(cbase + (j >= jb ? j : jb)) * hv + h];   // (in bounds on every lane)
        const float x = j >= jb ? xj : 0.f;
        ok = ok && __ballot(!(x <= 0.f)) == 0;                  // +inf (not a contraction) or NaN
        const double sfx = carry + wave_cumsum_f64((double)x);  // sum over chunks [e - 1 - l, je)
        const unsigned long long m = __ballot(sfx <= kHorizonLog2);
        if (!found && m != 0) {
            found = true;
            c = e - 1 - __builtin_ctzll(m);
        }
        carry = lane63_f64(sfx);
    }
    taken = ok && found;
    return taken ? c : jb;
}

// The parts of a sequence of nc chunks (one part of no chunks when it is
// empty).  A sequence of at most `cut` chunks, or of at most F, is one part;
// any other has a first part of F chunks and later parts of L chunks (the last
// one shorter): part j >= 1 holds chunks [F + (j - 1) L, min(F + j L, nc)).
// One pass over every part: F = L, cut = 0.  Part j of sequence n has part
// slot span_base(start(n), n, 64 L) + j; with F >= L a sequence of len tokens
// has at most ceil(len / (64 L)) parts, which its slots cover.
struct SeqParts {
    int64_t nc, L, F, np;
    __device__ SeqParts(int64_t nc_, int64_t L_, int64_t F_, int64_t cut) : nc(nc_), L(L_), F(F_) {
        np = (nc <= cut || nc <= F) ? 1 : 1 + (nc - F + L - 1) / L;
    }
    __device__ int64_t begin(int64_t j) const { return j == 0 ? 0 : F + (j - 1) * L; }
    __device__ int64_t end(int64_t j) const {
        const int64_t e = F + j * L;
        return np == 1 || e > nc ? nc : e;
    }
};

// Chunks of the part before it that a later part reruns from zero (its decay
// horizon's depth) to find its own start state, at most.
constexpr int64_t kWarmChunks = 6;

// One (part slot, value head) of a chunk kernel, in phase ph (the launch's
// a.phase, or its role in the balanced schedule's first launch).
// OUT = false: summary of parts p < np - 1 (B_p into ws_b, M_p into ws_m).
// OUT = true: outputs of every part, from ws_s (np > 1) or init_state (np = 1);
// the last part writes final_state; SNAP: also the state snapshots.  In the
// balanced schedule (phases 1 to 3, see launch_prefill_t) the first part of
// every sequence runs in phase 1 from init_state and leaves its end state as
// the second part's start state.  A later part whose predecessor has a decay
// horizon at most kWarmChunks from its end runs in phase 3, in the same
// launch: from zero at that horizon, through the predecessor's last chunks
// (outputs not stored), then its own.  The other later parts run in phase 2,
// after the link.
template <typename OP, int DK, int DV, bool OUT, bool RAW, bool SNAP>
__device__ __forceinline__ void chunk_part(const PrefillArgs& a, int64_t item, const ChunkLds<OP, DK, DV, OUT, RAW>& sm,
                                           int ph) {
    using G = ChunkGeom<OP, DK, DV, OUT>;
    using Buf = ChunkBuf<OP, DK, DV, OUT, OUT && RAW>;
    constexpr int NR = G::NR, NW = G::NW, NBUF = G::NBUF;
    constexpr int NVB = DV / 16, NMB = DK / 16, NDB = DK / 16;
    constexpr int E = (int)sizeof(OP);
    constexpr int UK = kChunk * DK * E / 1024, UV = kChunk * DV * E / 1024, UT = Units<OP>::TU;
    Buf* const bufs = sm.bufs;
    OP* const Pf = sm.Pf;
    OP* const Ost = sm.Ost;
    constexpr int KTS = ChunkSmem<OP, DK, DV, OUT, RAW>::KTS;
    OP* const Kt = sm.Kt;
    float* const Nrm = sm.Nrm;
    float* const Pdg = sm.Pdg;

    const int l = lane_id(), w = wave_id(), n = l & 15, gq = l >> 4;
    const int64_t pslot = item / a.hv;
    const int h = (int)(item - pslot * a.hv);
    const SeqIndex si{a.cu, a.seqlen};
    const int64_t L = a.part_chunks;
    int seq;
    int64_t p;
    locate_span(si, a.num_seqs, L * kChunk, pslot, seq, p);
    const int64_t s0 = si.start(seq), len = si.start(seq + 1) - s0;
    const int64_t nc = (len + kChunk - 1) / kChunk;
    const SeqParts sp(nc, L, a.first_chunks, a.cut_chunks);
    if (p < 0 || p >= sp.np) return;                            // gap slot
    const bool last = p == sp.np - 1;
    const int64_t cbase = span_base(s0, seq, kChunk);
    if (OUT && ph == 1 && p != 0) return;                        // a later part
    int64_t jw = 0;                                              // phase 3: first chunk of the rerun
    if (OUT && (ph == 2 || ph == 3)) {
        if (p == 0) return;                                      // a first part
        bool t;
        jw = horizon_start(a.ws_hz, cbase, a.hv, h, sp.begin(p - 1), sp.begin(p), t);
        // (a last part that writes final_state in place of init_state stays in
        // phase 2: in phase 3 it would share a launch with the first part that
        // reads init_state)
        const bool in_place = last && a.init_state != nullptr && a.init_state == a.final_state;
        if ((t && sp.begin(p) - jw <= kWarmChunks && !in_place) != (ph == 3)) return;   // the other phase's part
    }
    const int64_t chain = (int64_t)seq * a.hv + h;
    const size_t sblk = (size_t)pslot * a.hv + h;

    // the wave's state blocks
    int R0[NR];
    if constexpr (OUT) {
        R0[0] = 16 * w;
    } else {
        R0[0] = w < NVB ? 16 * w : 0;   // value block (none when w >= NVB)
        R0[1] = w < NMB ? 16 * w : 0;   // transition block (none when w >= NMB)
    }
    f32x4 ST[NR][NDB];
    float* Send = nullptr;

    if constexpr (OUT) {
        if (nc == 0) {   // empty sequence: the state passes through
            if (a.final_state) {
#pragma unroll
                for (int b = 0; b < NR; ++b) {
                    load_state<DK>(a.init_state ? a.init_state + chain * DV * DK : nullptr, R0[b], ST[b]);
                    store_state<DK>(a.final_state + chain * DV * DK, R0[b], ST[b]);
                }
            }
            return;
        }
        // the part's start state: written by the link (one pass over more than
        // one part, and the later parts of the balanced schedule), else init_state;
        // B_{p-1} itself when the previous part was summarised from its decay
        // horizon (the link then writes nothing for this part)
        // (phase 3: zero, at the predecessor's horizon)
        const bool linked = ph == 2 || (ph == 0 && sp.np > 1);
        const bool from_b = linked && p >= (ph == 2 ? 2 : 1) && a.ws_hf[sblk - a.hv] != 0;
        const float* Sin = from_b ? a.ws_b + (sblk - a.hv) * DV * DK
                           : linked ? a.ws_s + sblk * DV * DK
                           : ph == 3 ? nullptr
                                     : (a.init_state ? a.init_state + chain * DV * DK : nullptr);
        // where the part's end state goes: final_state after the last part; in
        // the balanced schedule's first launch, the start of the first later part
        Send = last ? (a.final_state ? a.final_state + chain * DV * DK : nullptr)
                    : ph == 1 ? a.ws_s + ((size_t)(pslot + 1) * a.hv + h) * DV * DK : nullptr;
#pragma unroll
        for (int b = 0; b < NR; ++b) load_state<DK>(Sin, R0[b], ST[b]);
    } else {
        // every part but the last (its map is not needed to link), or every
        // part for the affine map of whole sequences; in the balanced schedule
        // not the first part either (its outputs give the next start state)
        if (a.aff_m ? nc == 0 : last || (ph == 1 && p == 0)) return;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            ST[0][db] = zero4();
#pragma unroll
            for (int i = 0; i < 4; ++i) ST[1][db][i] = (pi_dk(db, 4 * gq + i) == R0[1] + n) ? 1.f : 0.f;
        }
    }
    const int64_t jb = sp.begin(p), je = sp.end(p);
    const int hq = (h * a.hqk) / a.hv;
    // first chunk this workgroup runs: the summary starts at its decay horizon,
    // and records whether it found one; phase 3 at its predecessor's
    bool taken = false;
    const int64_t js = OUT ? (ph == 3 ? jw : jb) : horizon_start(a.ws_hz, cbase, a.hv, h, jb, je, taken);
    if (!OUT && w == 0 && l == 0) a.ws_hf[sblk] = taken ? 1 : 0;
    const unsigned kstride = (unsigned)(a.hqk * DK * E), vstride = (unsigned)(a.hv * DV * E);

    // Buffer resources of chunk j (js <= j < je).  Bases are taken once per part:
    // chunk j's rows start (j - js) * 64 rows after chunk js's, its T~ fragments
    // and gate record (j - js) * Hv records after; only the sequence's last
    // chunk may be partial, and its resources end at its last row, so rows past
    // the end read as 0 and stores to them are dropped.  (Per chunk this is a
    // few scalar adds: all eight waves compute these resources at the same
    // point of every chunk, on scalar issue slots they share.)
    const size_t row0 = (size_t)(s0 + js * kChunk);
    const char* const kB0 = static_cast<const char*>(a.k) + ((row0 * a.hqk + hq) * DK) * E;
    const char* const qB0 = static_cast<const char*>(a.q) + ((row0 * a.hqk + hq) * DK) * E;
    const char* const vB0 = static_cast<const char*>(a.v) + ((row0 * a.hv + h) * DV) * E;
    char* const oB0 = static_cast<char*>(a.out) + ((row0 * a.hv + h) * DV) * E;
    const char* const tB0 = static_cast<const char*>(a.ws_t) + ((size_t)(cbase + js) * a.hv + h) * (UT * 1024);
    const char* const gB0 = reinterpret_cast<const char*>(a.ws_g) + ((size_t)(cbase + js) * a.hv + h) * kGateRecord;
    const uint32_t kstep = kChunk * kstride, vstep = kChunk * vstride;
    const uint32_t tstep = (uint32_t)a.hv * (UT * 1024), gstep = (uint32_t)a.hv * kGateRecord;
    const int64_t jl = nc - 1;                                  // the sequence's last chunk
    const int lrows = (int)(len - jl * kChunk);                  // its rows, 1 .. 64
    const int kfull = (kChunk - 1) * (int)kstride + DK * E, klast = (lrows - 1) * (int)kstride + DK * E;
    const int vfull = (kChunk - 1) * (int)vstride + DV * E, vlast = (lrows - 1) * (int)vstride + DV * E;
    auto rsrc = [](const void* ptr, int bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(ptr), 0, bytes, 0x00020000);
    };
    auto at = [&](const char* base, uint32_t step, int64_t j) { return base + (uint64_t)(uint32_t)(j - js) * step; };
    auto res_k = [&](int64_t j) { return rsrc(at(kB0, kstep, j), j == jl ? klast : kfull); };
    auto res_q = [&](int64_t j) { return rsrc(at(qB0, kstep, j), j == jl ? klast : kfull); };
    auto res_v = [&](int64_t j) { return rsrc(at(vB0, vstep, j), j == jl ? vlast : vfull); };
    auto res_o = [&](int64_t j) { return rsrc(at(oB0, vstep, j), j == jl ? vlast : vfull); };
    auto res_t = [&](int64_t j) { return rsrc(at(tB0, tstep, j), UT * 1024); };
    auto res_g = [&](int64_t j) { return rsrc(at(gB0, gstep, j), kGateRecord); };
    const char* const ikB0 = OUT && RAW ? reinterpret_cast<const char*>(a.ws_ik) + ((size_t)(cbase + js) * a.hv + h) * (kChunk * 4)
                                        : nullptr;
    auto res_ik = [&](int64_t j) { return rsrc(at(ikB0, (uint32_t)a.hv * (kChunk * 4), j), kChunk * 4); };

    // Direct loads of chunk j's rows, T~ and gates into `B` (spread over the waves).
    auto issue = [&](int64_t j, Buf& B) {
        if constexpr (kPoisonLds) {   // this wave's target slices, then the loads
            constexpr int EK = 1024 / (int)sizeof(OP);
            for (int k = w; k < UK; k += NW) poison_lds(B.K + k * EK, 1024, l, kWave);
            if constexpr (OUT)
                for (int k = w; k < UK; k += NW) poison_lds(B.Q + k * EK, 1024, l, kWave);
            for (int k = w; k < UV; k += NW) poison_lds(B.V + k * EK, 1024, l, kWave);
            for (int k = w; k < UT; k += NW) poison_lds(B.T + k * EK, 1024, l, kWave);
            if (w == NW - 1) poison_lds(B.G2, 2048, l, kWave);
            if constexpr (OUT && RAW) {
                if (w == NW - 2) poison_lds(B.IK, 1024, l, kWave);
            }
            wave_lds_sync();
        }
        const auto rk = res_k(j);
#pragma unroll
        for (int k = 0; k < (UK + NW - 1) / NW; ++k)
            if (UK % NW == 0 || w + NW * k < UK) rows_to_lds<OP, DK>(B.K, rk, kstride, w + NW * k);
        if constexpr (OUT) {
            const auto rq = res_q(j);
#pragma unroll
            for (int k = 0; k < (UK + NW - 1) / NW; ++k)
                if (UK % NW == 0 || w + NW * k < UK) rows_to_lds<OP, DK>(B.Q, rq, kstride, w + NW * k);
        }
        const auto rv = res_v(j);
#pragma unroll
        for (int k = 0; k < (UV + NW - 1) / NW; ++k)
            if (UV % NW == 0 || w + NW * k < UV) rows_to_lds<OP, DV>(B.V, rv, vstride, w + NW * k);
        const auto rt = res_t(j);
#pragma unroll
        for (int k = 0; k < (UT + NW - 1) / NW; ++k)
            if (UT % NW == 0 || w + NW * k < UT) bytes_to_lds(B.T, rt, w + NW * k);
        if (w == NW - 1) {   // gate record: 1.25 KB in two loads (the second fills the pad with zeros)
            bytes_to_lds(B.G2, res_g(j), 0);
            bytes_to_lds(B.G2, res_g(j), 1);
        }
        if constexpr (OUT && RAW) {
            if (w == NW - 2) bytes_to_lds(B.IK, res_ik(j), 0);   // 256 B; the rest reads as zero
        }
    };

    // O rows of chunk j, staged in Ost, to global memory (rows past the end dropped)
    auto store_o = [&](int64_t j) {
        constexpr int VU = kChunk * DV * E / 16, UPR = DV * E / 16;
        const auto ro = res_o(j);
        const int tid = threadIdx.x;
#pragma unroll
        for (int k = 0; k < (VU + G::NT - 1) / G::NT; ++k) {
            const int e = tid + k * G::NT;
            if (VU % G::NT == 0 || e < VU) {
                const int row = e / UPR, u = e - row * UPR;
                const u32x4 x = *reinterpret_cast<const u32x4*>(Ost + RowTile<OP, DV>::unit(row, u));
                __builtin_amdgcn_raw_buffer_store_b128(x, ro, (unsigned)row * vstride + (unsigned)u * 16, 0, 0);
            }
        }
    };
    // Summary chunk step over the wave's blocks.  With d_v != d_k the waves
    // past the smaller block count have one block only and run a one-block step
    // (a wave-uniform branch; every wave still meets the same barriers).  From a
    // decay horizon only the value block runs (M_p is not needed).
    auto summary_blocks = [&](const Buf& cb, OP* ktc, auto&& hook) {
        if constexpr (!OUT) {
            using One = f32x4(&)[1][NDB];
            using OneR = const int(&)[1];
            if (taken && w < NVB)   // from a decay horizon M_p is not needed: the value block only
                chunk_step<OP, DK, DV, OUT, 1, 1, NW, RAW>(cb, nullptr, ktc, nullptr, reinterpret_cast<One>(ST[0]),
                                                           reinterpret_cast<OneR>(R0[0]), w, hook, Nrm, Pdg);
            else if (NVB == NMB || (w < NVB && w < NMB))
                chunk_step<OP, DK, DV, OUT, NR, 1, NW, RAW>(cb, nullptr, ktc, nullptr, ST, R0, w, hook, Nrm, Pdg);
            else if (w < NMB)   // d_v < d_k: a transition block only
                chunk_step<OP, DK, DV, OUT, 1, 0, NW, RAW>(cb, nullptr, ktc, nullptr, reinterpret_cast<One>(ST[1]),
                                                           reinterpret_cast<OneR>(R0[1]), w, hook, Nrm, Pdg);
            else                // d_k < d_v: a value block only
                chunk_step<OP, DK, DV, OUT, 1, 1, NW, RAW>(cb, nullptr, ktc, nullptr, reinterpret_cast<One>(ST[0]),
                                                           reinterpret_cast<OneR>(R0[0]), w, hook, Nrm, Pdg);
        }
    };
    // output: the next count of finished chunks at which a snapshot is due
    int64_t next_snap = SNAP ? (jb / a.snap_chunks + 1) * a.snap_chunks : -1;
    auto body = [&](int64_t j, const Buf& cur, Buf& nxt) {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);   // this wave's loads of chunk j have landed
        lds_barrier();                          // everyone's have; the previous chunk is done everywhere
        if constexpr (OUT) {
            if (j > jb) store_o(j - 1);
        }
        auto next_loads = [&](int stage) {
            if (stage != 0) return;
            if (NBUF == 2 && j + 1 < je) issue(j + 1, nxt);
        };
        if constexpr (OUT) {
            chunk_step<OP, DK, DV, OUT, NR, 1, NW, RAW>(cur, Pf, Kt, Ost, ST, R0, w, next_loads, Nrm, Pdg);
            if (SNAP && j + 1 == next_snap) {   // state after a full snapshot interval
                if ((j + 1) * kChunk <= len) {
                    const int64_t slot = span_base(s0, seq, (int64_t)a.snap_chunks * kChunk) + (j + 1) / a.snap_chunks - 1;
#pragma unroll
                    for (int b = 0; b < NR; ++b)
                        store_state<DK>(a.snapshots + ((size_t)slot * a.hv + h) * DV * DK, R0[b], ST[b]);
                }
                next_snap += a.snap_chunks;
            }
        } else {
            summary_blocks(cur, Kt, next_loads);
        }
        if (NBUF == 1 && j + 1 < je) {
            lds_barrier();                      // everyone is done with this chunk's rows
            issue(j + 1, nxt);
        }
    };

    if constexpr (kPoisonLds) {
        using SM = ChunkSmem<OP, DK, DV, OUT, RAW>;
        poison_lds(bufs, (int)sizeof(SM::bufs), threadIdx.x, G::NT);
        poison_lds(Pf, (int)sizeof(SM::Pf), threadIdx.x, G::NT);
        poison_lds(Ost, (int)sizeof(SM::Ost), threadIdx.x, G::NT);
        poison_lds(Kt, (int)sizeof(SM::Kt), threadIdx.x, G::NT);
        poison_lds(Pdg, (int)sizeof(SM::Pdg), threadIdx.x, G::NT);
        if constexpr (OUT && RAW) poison_lds(Nrm, (int)sizeof(SM::Nrm), threadIdx.x, G::NT);
        __syncthreads();
    }
    if constexpr (G::KTA) {
        // Summary, bf16: chunk j's inputs sit in buffer set (j - js) mod 3 and
        // its K^T fragments in Kt half j mod 2.  During chunk j the waves form chunk
        // j + 1's K^T fragments (its rows landed before the barrier that opens
        // chunk j) and load chunk j + 2 into the set chunk j - 1 used, so a
        // chunk needs one barrier.
        issue(js, bufs[0]);
        if (js + 1 < je) issue(js + 1, bufs[1]);
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        lds_barrier();
        transpose_kt<OP, DK, NW>(bufs[0].K, Kt + (js & 1) * KTS, w);
        int bc = 0;                                   // buffer set of chunk j
        auto body3 = [&](int64_t j) {
            // chunk j + 1's rows have landed; everyone's K^T fragments of chunk
            // j are written and chunk j - 1 is done everywhere
            __builtin_amdgcn_s_waitcnt(kWaitVm0);
            lds_barrier();
            const int b1 = bc == 2 ? 0 : bc + 1, b2 = b1 == 2 ? 0 : b1 + 1;
            OP* const ktc = Kt + (j & 1) * KTS;
            OP* const ktn = Kt + ((j + 1) & 1) * KTS;
            auto ahead = [&](int stage) {   // placed between U and the state update (measured best)
                if (stage != 2) return;
                if (j + 1 < je) transpose_kt<OP, DK, NW>(bufs[b1].K, ktn, w);
                if (j + 2 < je) issue(j + 2, bufs[b2]);
            };
            summary_blocks(bufs[bc], ktc, ahead);
            bc = b1;
        };
        for (int64_t j = js; j < je; ++j) body3(j);
    } else {
        issue(js, bufs[0]);
        for (int64_t j = js; j < je; j += NBUF) {
            body(j, bufs[0], bufs[NBUF == 2 ? 1 : 0]);
            if (NBUF == 2 && j + 1 < je) body(j + 1, bufs[NBUF == 2 ? 1 : 0], bufs[0]);
        }
    }
    if constexpr (OUT) {
        lds_barrier();
        store_o(je - 1);
    }

    if constexpr (OUT) {
        if (Send)
#pragma unroll
            for (int b = 0; b < NR; ++b) store_state<DK>(Send, R0[b], ST[b]);
    } else {
        if (w < NVB) store_state<DK>(a.ws_b + sblk * DV * DK, R0[0], ST[0]);
        if (w < NMB && !taken) store_transition<DK>(a.ws_m + sblk * DK * DK, R0[1], ST[1]);   // (no reader after a horizon)
    }
}

// Workgroup b: (part slot, value head) b of chunk_part.
template <typename OP, int DK, int DV, bool OUT, bool RAW, bool SNAP = false>
__global__ __launch_bounds__(64 * (OUT ? DV / 16 : (DV > DK ? DV : DK) / 16)) void gdn_chunk_kernel(PrefillArgs a) {
    static_assert(ChunkGeom<OP, DK, DV, OUT>::NT == 64 * (OUT ? DV / 16 : (DV > DK ? DV : DK) / 16),
                  "launch bound must equal the launch size");
    // separate arrays (the compiler's own placement needs fewer registers than
    // one ChunkSmem here)
    using SM = ChunkSmem<OP, DK, DV, OUT, RAW>;
    __shared__ decltype(SM::bufs) bufs;
    __shared__ decltype(SM::Pf) Pf;
    __shared__ decltype(SM::Ost) Ost;
    __shared__ decltype(SM::Kt) Kt;
    __shared__ decltype(SM::Nrm) Nrm;
    __shared__ decltype(SM::Pdg) Pdg;
    chunk_part<OP, DK, DV, OUT, RAW, SNAP>(a, blockIdx.x, ChunkLds<OP, DK, DV, OUT, RAW>{bufs, Pf, Ost, Kt, Nrm, Pdg},
                                           a.phase);
}

// The first launch of the balanced schedule (d_k = d_v): workgroups [0, n) run
// the first part of every sequence from init_state (outputs, phase 1),
// workgroups [n, 2n) the summaries, workgroups [2n, 3n) the later parts whose
// predecessor has a near decay horizon (outputs, phase 3), n = part slots x
// value heads.  The kinds share the shared memory, one at a time.
template <typename OP, int D, bool RAW>
__global__ __launch_bounds__(64 * D / 16) void gdn_chunk_first_kernel(PrefillArgs a) {
    using SO = ChunkSmem<OP, D, D, true, RAW>;
    using SS = ChunkSmem<OP, D, D, false, RAW>;
    static_assert(ChunkGeom<OP, D, D, true>::NT == 64 * D / 16 && ChunkGeom<OP, D, D, false>::NT == 64 * D / 16,
                  "both kinds use the launch size");
    __shared__ __attribute__((aligned(16))) unsigned char smem[sizeof(SO) > sizeof(SS) ? sizeof(SO) : sizeof(SS)];
    const int64_t n = a.num_part_slots * a.hv, b = blockIdx.x;
    if (b < n || b >= 2 * n)
        chunk_part<OP, D, D, true, RAW, false>(a, b < n ? b : b - 2 * n,
                                               ChunkLds<OP, D, D, true, RAW>::of(*reinterpret_cast<SO*>(smem)),
                                               b < n ? 1 : 3);
    else
        chunk_part<OP, D, D, false, RAW, false>(a, b - n, ChunkLds<OP, D, D, false, RAW>::of(*reinterpret_cast<SS*>(smem)),
                                                1);
}

// ===========================================================================
// link: start states of the parts, S_{p+1} = S_p M_p + B_p
// ===========================================================================
// One workgroup per (sequence, value head, RB 16-row blocks of the state);
// rows of S never mix, so the blocks are independent (the RB blocks of a
// workgroup share the loads of M_p).  S_0 (init_state or zeros) and
// every later S_p go to ws_s at the part's slot.  For the affine map of whole
// sequences (aff_m set) the chain runs over every part from zero (offset
// rows) and from the identity (transition rows, without B_p) and ends in
// aff_b and aff_m.  With NWV waves per row block, wave w computes the d_k
// column blocks w, w + NWV, ... of S_{p+1} on the fp32 matrix cores (NWV =
// d_k / 16: one block each, so a step's products are one block deep).  M_p does
// not depend on S, so M_{p+1} streams into the second LDS buffer (direct
// loads) while step p computes: a step waits for one load, not a chain of them.
// A step whose part was summarised from its decay horizon takes S_{p+1} = B_p
// without M_p; when every step of a chain is such, the workgroup only copies
// S_0 (the output kernel then starts each later part from the B before it).
template <int DK, int DV, int RB = 1, int NWV = kLinkThreads / kWave>
__global__ __launch_bounds__(kWave * NWV * RB) void gdn_link_kernel(PrefillArgs a) {
    constexpr int NVB = DV / 16, NDB = DK / 16, NKK = DK / 32, LD = DK + 4;
    constexpr int NT = kWave * NWV, PER = (NDB + NWV - 1) / NWV;   // threads per row block
    constexpr int MI = DK * DK * 4 / 1024;               // 1 KB direct loads per M
    static_assert(MI % (NWV * RB) == 0, "M loads per wave");
    static_assert(NVB % RB == 0 && NDB % RB == 0, "row blocks of a workgroup are all offset or all transition rows");
    __shared__ float Sall[RB][16][LD];
    __shared__ float Mb[2][DK * DK];                      // M_p, transposed (m_pos)
    // RB row blocks per workgroup (NWV waves each), sharing M_p
    const int l = lane_id(), n = l & 15, gq = l >> 4;
    const int sub = wave_id() / NWV, w = wave_id() - sub * NWV, tid = (int)threadIdx.x - sub * NT;
    float (&S)[16][LD] = Sall[sub];
    // affine map: row blocks 0 .. NVB - 1 are offset rows (from zero, + B_p),
    // NVB .. NVB + NDB - 1 transition rows (from the identity, no B_p)
    const bool aff = a.aff_m != nullptr;
    const int NBK = aff ? NVB + NDB : NVB;
    // Workgroup b takes row blocks RB (b / C) .. + RB - 1 of chain b mod C (C =
    // chains rounded up to a multiple of the 8 XCDs): all row blocks of a chain
    // then run on one XCD, and every M_p they all load comes from that XCD's L2
    // after the first.
    const int64_t nchain = (int64_t)a.num_seqs * a.hv, C = (nchain + kXcds - 1) / kXcds * kXcds;
    const int vg = (int)(blockIdx.x / C), vb = RB * vg + sub;
    const int64_t chain = blockIdx.x - (int64_t)vg * C;
    if (chain >= nchain) return;
    const bool trans = vb >= NVB;
    const int seq = (int)(chain / a.hv), h = (int)(chain - (int64_t)seq * a.hv);
    const SeqIndex si{a.cu, a.seqlen};
    const int64_t L = a.part_chunks;
    const int64_t s0 = si.start(seq), len = si.start(seq + 1) - s0;
    const int64_t nc = (len + kChunk - 1) / kChunk;
    const SeqParts sp(nc, L, a.first_chunks, a.cut_chunks);
    // S_{j+1} = S_j M_j + B_j for parts j0 <= j < j0 + steps.  One pass over
    // every part: from S_0 (init_state) over every part but the last (the
    // affine map: from zero / the identity over every part).  Two launches:
    // from S_1 (written by the first part's outputs) over the later parts but
    // the last.
    const bool bal = a.phase != 0;
    const int64_t j0 = bal ? 1 : 0;
    const int64_t steps = bal ? sp.np - 2 : aff ? (nc > 0 ? sp.np : 0) : (nc > 0 ? sp.np - 1 : 0);
    const int R0 = trans ? 16 * (vb - NVB) : 16 * vb;
    float* const outp = !aff ? nullptr
                             : trans ? a.aff_m + (chain * DK + R0) * DK : a.aff_b + (chain * DV + R0) * DK;
    if (aff && steps == 0) {                             // empty sequence: M = I, B = 0
        for (int e = tid; e < 16 * DK; e += NT) {
            const int row = e / DK, c = e - row * DK;
            outp[(size_t)row * DK + c] = trans && R0 + row == c ? 1.f : 0.f;
        }
        return;
    }
    if (steps <= 0) return;
    if constexpr (kPoisonLds) {
        poison_lds(Sall, (int)sizeof(Sall), (int)threadIdx.x, NT * RB);
        poison_lds(Mb, (int)sizeof(Mb), (int)threadIdx.x, NT * RB);
        __syncthreads();
    }
    const int64_t pbase = span_base(s0, seq, L * kChunk) + j0;   // slot of step 0

    // Steps whose part was summarised from its decay horizon: M_p is negligible
    // and S_{p+1} = B_p (the transition rows of the affine map become 0).  Bit
    // p mod 64 of `neg` covers step p of the current group of 64 steps.
    auto neg_group = [&](int64_t p0) {
        const int64_t p = p0 + l;
        const int f = a.ws_hf[(pbase + (p < steps ? p : p0)) * a.hv + h];   // (in bounds on every lane)
        return __ballot(p < steps && f != 0);
    };
    bool all_neg = true;
    for (int64_t p0 = 0; p0 < steps; p0 += kWave) {
        const unsigned long long m = neg_group(p0);
        const int64_t left = steps - p0;
        all_neg = all_neg && m == (left >= kWave ? ~0ull : (1ull << left) - 1);
    }
    if (all_neg) {
        // every step: nothing to chain.  The output kernel starts each later
        // part from B_{p-1} itself; S_0 still goes to ws_s (one pass), and the
        // affine map is (0, B of the last part).
        for (int e = tid; e < 16 * DK / 4; e += NT) {
            const int row = e / (DK / 4), c = 4 * (e - row * (DK / 4));
            if (aff) {
                const f32x4 x = trans ? zero4()
                                      : *reinterpret_cast<const f32x4*>(
                                            a.ws_b + (((size_t)(pbase + steps - 1) * a.hv + h) * DV + R0 + row) * DK + c);
                *reinterpret_cast<f32x4*>(outp + (size_t)row * DK + c) = x;
            } else if (!bal) {
                const f32x4 x = a.init_state ? *reinterpret_cast<const f32x4*>(a.init_state + (chain * DV + R0 + row) * DK + c) : zero4();
                *reinterpret_cast<f32x4*>(a.ws_s + (((size_t)pbase * a.hv + h) * DV + R0 + row) * DK + c) = x;
            }
        }
        return;
    }
    unsigned long long neg = neg_group(0);

    auto load_m = [&](int64_t p, int buf) {
        const float* M = a.ws_m + ((size_t)(pbase + p) * a.hv + h) * DK * DK;
        const auto rm = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(M), 0, DK * DK * 4, 0x00020000);
#pragma unroll
        for (int k = 0; k < MI / (NWV * RB); ++k) bytes_to_lds(&Mb[buf][0], rm, wave_id() + NWV * RB * k);
    };
    if (!(neg & 1)) load_m(0, 0);
    for (int e = tid; e < 16 * DK / 4; e += NT) {
        const int row = e / (DK / 4), c = 4 * (e - row * (DK / 4));
        if (aff) {
            f32x4 x = zero4();
            if (trans)
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = R0 + row == c + i ? 1.f : 0.f;
            *reinterpret_cast<f32x4*>(&S[row][c]) = x;
        } else if (bal) {
            *reinterpret_cast<f32x4*>(&S[row][c]) =
                *reinterpret_cast<const f32x4*>(a.ws_s + (((size_t)pbase * a.hv + h) * DV + R0 + row) * DK + c);
        } else {
            const f32x4 x = a.init_state ? *reinterpret_cast<const f32x4*>(a.init_state + (chain * DV + R0 + row) * DK + c) : zero4();
            *reinterpret_cast<f32x4*>(&S[row][c]) = x;
            *reinterpret_cast<f32x4*>(a.ws_s + (((size_t)pbase * a.hv + h) * DV + R0 + row) * DK + c) = x;
        }
    }
    // this lane's share of B_p (accumulator layout), fetched a step ahead
    auto load_b = [&](int64_t p, f32x4 (&c)[PER]) {
        const float* B = a.ws_b + ((size_t)(pbase + p) * a.hv + h) * DV * DK + (size_t)R0 * DK;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int db = w + NWV * k;
#pragma unroll
            for (int i = 0; i < 4; ++i) c[k][i] = db < NDB && !trans ? B[(size_t)(4 * gq + i) * DK + 16 * db + n] : 0.f;
        }
    };
    f32x4 bnext[PER];
    load_b(0, bnext);
    for (int64_t p = 0; p < steps; ++p) {
        const int cb = (int)(p & 1);
        f32x4 bcur[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) bcur[k] = bnext[k];
        // this wave's share of M_p is in: at the first step everything is
        // waited for; later the PER * 4 newest memory operations, the stores
        // of S_p, may still be in flight
        if (p == 0) __builtin_amdgcn_s_waitcnt(kWaitVm0);
        else __builtin_amdgcn_s_waitcnt(kWaitVm0 | ((PER * 4) & 15) | (((PER * 4) >> 4) << 14));
        __syncthreads();                                 // everyone's is; S_p is written
        const bool neg_p = (neg >> (p & 63)) & 1;
        if (((p + 1) & 63) == 0 && p + 1 < steps) neg = neg_group(p + 1);
        if (p + 1 < steps) {
            if (!((neg >> ((p + 1) & 63)) & 1)) load_m(p + 1, cb ^ 1);   // the other buffer was read in step p - 1
            load_b(p + 1, bnext);
        }
        f32x4 res[PER];
        if (neg_p) {                                     // S_{p+1} = B_p (transition rows: 0)
#pragma unroll
            for (int k = 0; k < PER; ++k) res[k] = trans ? zero4() : bcur[k];
        } else {
            const float* M = Mb[cb];
            // every operand of the step's products is read from LDS first, then the
            // products run (one wait for LDS instead of one per K step)
            f32x8 av[NKK], bv[PER][NKK];
#pragma unroll
            for (int kk = 0; kk < NKK; ++kk)
#pragma unroll
                for (int i = 0; i < 8; ++i) av[kk][i] = S[n][32 * kk + (i < 4 ? 4 * gq + i : 16 + 4 * gq + i - 4)];
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int db = w + NWV * k < NDB ? w + NWV * k : w;   // (an unused block reads a valid one)
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) {
                    const int c = 16 * db + n;
                    const f32x4 lo = *reinterpret_cast<const f32x4*>(&M[m_pos(c, 32 * kk + 4 * gq, DK)]);
                    const f32x4 hi = *reinterpret_cast<const f32x4*>(&M[m_pos(c, 32 * kk + 16 + 4 * gq, DK)]);
                    bv[k][kk] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < PER; ++k) {
                const int db = w + NWV * k;
                if (db >= NDB) break;
                f32x4 c = bcur[k];
#pragma unroll
                for (int kk = 0; kk < NKK; ++kk) c = Op<float>::mma(av[kk], bv[k][kk], c);
                res[k] = c;
            }
        }
        lds_barrier();                                   // S_p read by everyone (M_{p+1} may be in flight)
        float* Sn = aff ? outp : a.ws_s + ((size_t)(pbase + p + 1) * a.hv + h) * DV * DK + (size_t)R0 * DK;
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int db = w + NWV * k;
            if (db >= NDB) break;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                S[4 * gq + i][16 * db + n] = res[k][i];
                Sn[(size_t)(4 * gq + i) * DK + 16 * db + n] = res[k][i];
            }
        }
    }
}

// ===========================================================================
// host side
// ===========================================================================
template <typename OP, int DK, bool RAW>
hipError_t launch_prep(const PrefillArgs& a, hipStream_t st) {
    const int64_t items = a.num_slots * a.hv;
    const unsigned nwg = (unsigned)((items + kPrepWaves - 1) / kPrepWaves);
    if (nwg == 0) return hipSuccess;
    hipLaunchKernelGGL((gdn_prep_kernel<OP, DK, RAW>), dim3(nwg), dim3(kWave * kPrepWaves), 0, st, a);
    return hipGetLastError();
}

template <typename OP, int DK, int DV, bool RAW>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
    hipError_t e = launch_prep<OP, DK, RAW>(a, st);
    if (e != hipSuccess) return e;
    const unsigned parts = (unsigned)(a.num_part_slots * a.hv);
    if constexpr (DK == DV && sizeof(OP) == 2) {
        if (a.phase != 0 && a.ws_m && !a.snapshots) {
            // Balanced schedule: phase 1 runs the first part of every sequence
            // (outputs; the whole sequence when it is not cut) in the same
            // launch as the summaries of the cut sequences' later parts (all
            // but the last) and, as phase 3, the later parts whose predecessor
            // has a near decay horizon (each reruns that predecessor's last
            // chunks from zero); the link gives the other later parts' start
            // states, and phase 2 runs them.  The first parts, which need no
            // start state, fill the compute units that a single pass leaves
            // idle while the longest sequences finish.
            PrefillArgs b = a;
            b.phase = 1;
            hipLaunchKernelGGL((gdn_chunk_first_kernel<OP, DK, RAW>), dim3(3 * parts),
                               dim3(ChunkGeom<OP, DK, DV, true>::NT), 0, st, b);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            // two row blocks per workgroup: the link's workgroups hold 140 KB of
            // shared memory (one per compute unit), and here many chains link
            // at once
            const unsigned links = (unsigned)(((int64_t)a.num_seqs * a.hv + kXcds - 1) / kXcds * kXcds * (DV / 32));
            hipLaunchKernelGGL((gdn_link_kernel<DK, DV, 2, DK / 16>), dim3(links), dim3(2 * kWave * (DK / 16)), 0, st, a);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            b.phase = 2;
            hipLaunchKernelGGL((gdn_chunk_kernel<OP, DK, DV, true, RAW>), dim3(parts),
                               dim3(ChunkGeom<OP, DK, DV, true>::NT), 0, st, b);
            return hipGetLastError();
        }
    }
    PrefillArgs c = a;   // one output pass over every part
    c.phase = 0;
    if (c.ws_m) {
        hipLaunchKernelGGL((gdn_chunk_kernel<OP, DK, DV, false, RAW>), dim3(parts),
                           dim3(ChunkGeom<OP, DK, DV, false>::NT), 0, st, c);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const unsigned links = (unsigned)(((int64_t)c.num_seqs * c.hv + kXcds - 1) / kXcds * kXcds * (DV / 16));
        hipLaunchKernelGGL((gdn_link_kernel<DK, DV, 1, DK / 16>), dim3(links), dim3(kWave * (DK / 16)), 0, st, c);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if constexpr (!RAW) {   // snapshots come with the plain prefill only
        if (c.snapshots) {
            hipLaunchKernelGGL((gdn_chunk_kernel<OP, DK, DV, true, false, true>), dim3(parts),
                               dim3(ChunkGeom<OP, DK, DV, true>::NT), 0, st, c);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gdn_chunk_kernel<OP, DK, DV, true, RAW>), dim3(parts), dim3(ChunkGeom<OP, DK, DV, true>::NT),
                       0, st, c);
    return hipGetLastError();
}

template <typename OP, int DK, int DV>
hipError_t launch_prefill_affine_t(const PrefillArgs& a, hipStream_t st) {
    hipError_t e = launch_prep<OP, DK, false>(a, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gdn_chunk_kernel<OP, DK, DV, false, false>), dim3((unsigned)(a.num_part_slots * a.hv)),
                       dim3(ChunkGeom<OP, DK, DV, false>::NT), 0, st, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const unsigned links = (unsigned)(((int64_t)a.num_seqs * a.hv + kXcds - 1) / kXcds * kXcds * (DV / 16 + DK / 16));
    hipLaunchKernelGGL((gdn_link_kernel<DK, DV, 1, DK / 16>), dim3(links), dim3(kWave * (DK / 16)), 0, st, a);
    return hipGetLastError();
}

template <typename OP, bool RAW>
hipError_t launch_prefill_dt(const PrefillArgs& a, int dk, int dv, hipStream_t st) {
    if (dk == 128)
        return dv == 128 ? launch_prefill_t<OP, 128, 128, RAW>(a, st) : launch_prefill_t<OP, 128, 64, RAW>(a, st);
    return dv == 128 ? launch_prefill_t<OP, 64, 128, RAW>(a, st) : launch_prefill_t<OP, 64, 64, RAW>(a, st);
}

}  // namespace

PartPlan prefill_part_plan(int64_t num_tokens, int num_seqs, int hv, int num_cus, bool two_launch, bool packed) {
    const int64_t chunks = (num_tokens + kChunk - 1) / kChunk;
    const int64_t whole = chunks > 1 ? chunks : 1;             // no sequence has more chunks
    const int64_t chains = (int64_t)num_seqs * hv;
    constexpr int64_t kMinPartChunks = 6;
    if (num_seqs <= 0 || num_cus <= 0) return {whole, whole, 0, 0};
    if (chains < num_cus) {
        // about one part per compute unit, at least kMinPartChunks chunks each.
        // (A short first part whose outputs run beside the other parts'
        // summaries measured slower: among summary workgroups an output
        // workgroup's chunk step took about twice as long.)
        int64_t L = (chunks * hv + num_cus - 1) / num_cus;
        L = L > kMinPartChunks ? L : kMinPartChunks;
        L = L < whole ? L : whole;
        return {L, L, 0, 0};
    }
    if (two_launch && packed && num_seqs > 1 && chains <= 2 * (int64_t)num_cus) {
        // share = chunk steps per compute unit.  A chain of more than one share
        // keeps a first part of about one share (it needs no start state, so
        // it runs beside the summaries) and is cut into parts of 0.2 shares
        // after it, which run after the link.  (Chosen with a list-scheduling
        // model of the two launches over random length mixes, and measured.)
        const double share = (double)chunks * hv / num_cus;
        int64_t L = (int64_t)(0.2 * share), cut = (int64_t)(1.0 * share);
        L = L > kMinPartChunks ? L : kMinPartChunks;
        cut = cut > L ? cut : L;
        if (L < whole && cut < whole) return {L, cut / L * L, cut, 1};
    }
    return {whole, whole, 0, 0};
}

hipError_t launch_prefill_affine(const PrefillArgs& a, bool bf16, int dk, int dv, hipStream_t st) {
    if (a.num_seqs == 0) return hipSuccess;
    auto go = [&](auto op) {
        using OP = decltype(op);
        if (dk == 128)
            return dv == 128 ? launch_prefill_affine_t<OP, 128, 128>(a, st) : launch_prefill_affine_t<OP, 128, 64>(a, st);
        return dv == 128 ? launch_prefill_affine_t<OP, 64, 128>(a, st) : launch_prefill_affine_t<OP, 64, 64>(a, st);
    };
    return bf16 ? go(__bf16{}) : go(0.f);
}

hipError_t launch_prefill(const PrefillArgs& a, bool bf16, int dk, int dv, hipStream_t st, bool raw) {
    if (a.num_seqs == 0) return hipSuccess;
    if (raw) return bf16 ? launch_prefill_dt<__bf16, true>(a, dk, dv, st) : launch_prefill_dt<float, true>(a, dk, dv, st);
    return bf16 ? launch_prefill_dt<__bf16, false>(a, dk, dv, st) : launch_prefill_dt<float, false>(a, dk, dv, st);
}

}  // namespace gdn
