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
//    parallel: stages K and Q in LDS, the gate cumsum (fp64), Gamma-weighted
//    K K^T and Q K^T on bf16 (or fp32) matrix cores, the unit-lower-triangular
//    inverse in LDS (16x16 diagonal blocks by forward substitution,
//    off-diagonal blocks by fp32 MFMA block products), and writes T~, P (in
//    the order the scan's operand fragments use) and the chunk's gates to a
//    workspace.
//  * gdn_scan_kernel  -- sequential over the chunks of one sequence, parallel
//    over (sequence, value head, 16-column block of d_v); the d_k rows of the
//    state block are split over the workgroup's waves and stay in fp32
//    matrix-core accumulators for the whole sequence (details above the
//    kernel).
//
// Exponentials use exp2 of log2-scaled cumulative gates (G2 = G log2 e).
// Padding: a final partial chunk is padded with k = q = 0, g = 0, beta = 0 in
// the prep kernel; padded rows then carry u = 0 (their rows and columns of
// T~ vanish), so they leave S and the real rows untouched whatever the scan
// reads for them, and gamma_n = e^{G2_63} equals the decay up to the last
// real token.
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

// ===========================================================================
// workspace layout shared by the two kernels
// ===========================================================================
// Every matrix the scan reads as matrix-core operands is stored
// fragment-major: 16-byte unit e = (f * FU + u) * 64 + lane holds unit u of
// operand fragment f for that lane, so a wave reads a fragment as one
// contiguous 1 KB block.  A fragment holds, for lane (r, gq) =
// (lane & 15, lane >> 4), eight elements of row r of a 16-row tile, columns
// c0 + 8 gq .. c0 + 8 gq + 7 (u = 0, 1 split them for fp32).
//  * T~ and P of a (chunk, value head): f = tw * 2 + kk, rows 16 tw + r,
//    c0 = 32 kk (64 x 64);
//  * K and Q of a (chunk, q/k head): f = w * 4 + tm, rows 16 tm + r (tokens),
//    c0 = 32 w (64 x d_k; the scan's wave w owns d_k columns 32 w .. 32 w + 31).
// The gates of a chunk are 64 float pairs (G2_t, G2_last - G2_t), the
// difference taken in fp64; zeros (what a read past the end returns) stand
// for a chunk without decay.
template <typename OP> struct FragMajor {
    static constexpr int VE = 16 / (int)sizeof(OP);      // elements per 16-byte unit
    static constexpr int FU = 8 / VE;                    // units per operand fragment
    static constexpr int UNITS = kChunk * kChunk / VE;   // of a 64 x 64 matrix
    __device__ __forceinline__ static int frag_of(int e) { return (e >> 6) / FU; }
    __device__ __forceinline__ static int col_in(int e) { return 8 * ((e >> 4) & 3) + VE * ((e >> 6) % FU); }
    // 64 x 64 (T~, P)
    __device__ __forceinline__ static int row(int e) { return 16 * (frag_of(e) >> 1) + (e & 15); }
    __device__ __forceinline__ static int col(int e) { return 32 * (frag_of(e) & 1) + col_in(e); }
    // 64 x d_k (K, Q)
    __device__ __forceinline__ static int kq_row(int e) { return 16 * (frag_of(e) & 3) + (e & 15); }
    __device__ __forceinline__ static int kq_col(int e) { return 32 * (frag_of(e) >> 2) + col_in(e); }
};
constexpr int kGateFloats = 2 * kChunk;   // floats per (chunk, value head)

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
        const double G = wave_cumsum_f64((double)gv * 1.4426950408889634);
        sm.G[l] = G;
        sm.B[l] = bv;
        const double Gl = lane63_f64(G);
        reinterpret_cast<f32x2*>(a.ws_g + ((size_t)slot * a.hv + h) * kGateFloats)[l] =
            f32x2{(float)G, (float)(Gl - G)};
    }
    __syncthreads();

    // ---- fragment-major copies of K and Q for the scan (padded rows are
    // zero); one writer per q/k head
    if ((h * a.hqk) % a.hv == 0) {
        using FM = FragMajor<OP>;
        OP* Kw = static_cast<OP*>(a.ws_k) + ((size_t)slot * a.hqk + hq) * (kChunk * DK);
        OP* Qw = static_cast<OP*>(a.ws_q) + ((size_t)slot * a.hqk + hq) * (kChunk * DK);
        for (int e = tid; e < kChunk * DK / VE; e += kPrepThreads) {
            const int row = FM::kq_row(e), col = FM::kq_col(e);
            *reinterpret_cast<u32x4*>(Kw + e * VE) = ld16(sm.K + row * LD + col);
            *reinterpret_cast<u32x4*>(Qw + e * VE) = ld16(sm.Q + row * LD + col);
        }
    }

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

    // ---- T~ and P to the workspace, fragment-major, consecutive lanes on
    // consecutive 16-byte units
    using FM = FragMajor<OP>;
    OP* Pw = static_cast<OP*>(a.ws_p) + ((size_t)slot * a.hv + h) * (kChunk * kChunk);
    OP* Tw = static_cast<OP*>(a.ws_t) + ((size_t)slot * a.hv + h) * (kChunk * kChunk);
    for (int e = tid; e < FM::UNITS; e += kPrepThreads) {
        const int row = FM::row(e), col = FM::col(e);
        *reinterpret_cast<u32x4*>(Tw + e * VE) = ld16(Tl + row * LDP + col);
        *reinterpret_cast<u32x4*>(Pw + e * VE) = ld16(Pl + row * LDP + col);
    }
}

// ===========================================================================
// scan: sequential over the chunks of one sequence
// ===========================================================================
// One workgroup per (sequence, value head, 16-column block of d_v).  Its
// NWS = DK / 32 waves split d_k: wave w owns state rows S[:, 32w .. 32w+32)
// as two fp32 accumulator tiles (d_k x 16).  Inside the slice the d_k order of
// the tiles is permuted (tile `sub`, row 4 gq + i  <->  d_k 8 gq + 4 sub + i)
// so that an operand fragment of K or Q pairs with the state tiles directly.
// Wave w also owns token tiles tw = w + NWS jt (jt < TPW = 4 / NWS).  Per chunk:
//   wave w:  X_w^T = S_w K_w^T,  Y_w^T = S_w Q_w^T          (partial over d_k)
//   E1 (LDS): X partials -> the owner of token tile tw sums X^T there
//   owner:   R^T = V^T - X^T diag(gamma)
//            K_w^T in operand layout via an exact identity product
//   E2 (LDS): R for all tokens to every wave, Y partials to the owners
//   owner:   U = T~_tw R,  D o U  (D = e^{G_last - G_t} per token)
//   E3 (LDS): U and D o U for all tokens to every wave
//   wave w:  S_w^T <- gamma_n S_w^T + K_w^T (D o U)
//   owner:   O^T = Y^T diag(gamma) + U^T P_tw^T
// A wave keeps its own partial tiles in registers and writes only the tiles
// other waves own.
//
// Global memory.  The vector memory path serves a wave request four lanes at
// a time, and four lanes on four different rows cost four times as much as
// four lanes on one 64-byte piece, so every access keeps consecutive lanes on
// consecutive bytes: K, Q, T~ and P come fragment-major from the prep
// kernel's workspace (one 1 KB block per fragment), the gates as one
// 512-byte record per chunk, and V and O pass through a small wave-private
// LDS area between their row-wise global form and the lanes' tile layout.
// Operands are fetched two chunks ahead into registers.  All loads go
// through buffer resources (reads past the end of a resource return 0, writes
// past it are dropped), and no load, store or use of a loaded value sits
// behind a branch, so the compiler's memory-counter waits stay exact.
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

// A/B fragment of a row-major LDS matrix in natural K order: k0 + 8 gq + (0..7).
template <typename T>
__device__ __forceinline__ typename Op<T>::frag frag_nat(const T* M, int ld, int row, int k0) {
    using frag = typename Op<T>::frag;
    return *reinterpret_cast<const frag*>(M + (size_t)row * ld + k0 + 8 * (lane_id() >> 4));
}

// XOR swizzle of the V/O staging tiles (16 rows of four 4-element quads): the
// quad index is XORed with a function of the row so that both the row-wise
// side (four lanes per row) and the tile side (one row per lane) spread over
// the LDS banks.
__device__ __forceinline__ int swz_vo(int row, int elem) {
    return elem == 2 ? ((row >> 2) & 3) : (((row >> 1) ^ (row >> 3)) & 3);
}

// Orders this wave's LDS writes before its later LDS reads of the same area.
// LDS executes one wave's operations in issue order; the fence only keeps the
// compiler from moving them.
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront"); }

template <typename OP, int DK>
struct ScanGeom {
    static constexpr int NWS = DK / 32;                 // waves per workgroup (d_k split)
    static constexpr int TPW = 4 / NWS;                 // token tiles per wave
    static constexpr int E = (int)sizeof(OP);
    static constexpr int FU = 8 * E / 16;               // 16-byte units per operand fragment
    static constexpr int QE = 4 * E;                    // bytes per V/O quad
    static constexpr int VROWB = 16 * E;                // bytes per V/O tile row
    static constexpr int VB = 16 * VROWB;               // bytes per V/O tile
    static constexpr int RLD = kChunk + (E == 2 ? 8 : 4);   // 16-byte rows, staggered banks
};

template <typename OP, int DK>
struct ScanSmem {
    using G = ScanGeom<OP, DK>;
    f32x4 part[G::NWS][8][kWave];        // X^T partials (0..3) and Y^T partials (4..7)
    alignas(16) OP Rt[16 * G::RLD];      // R as [column][token]
    alignas(16) OP Ut[16 * G::RLD];      // U as [column][token]
    alignas(16) OP Dt[16 * G::RLD];      // D o U as [column][token]
    alignas(16) float gam[2][kChunk];    // by chunk parity: e^{G_t}
    alignas(16) float dec[2][kChunk];    //                  e^{G_last - G_t}
    alignas(16) char vst[G::NWS][G::TPW][G::VB];   // wave-private V / O tiles
};

template <typename OP, int DK>
struct ScanCtx {
    using G = ScanGeom<OP, DK>;
    using B = Buf<OP>;
    using frag = typename Op<OP>::frag;
    using quad = typename Op<OP>::quad;
    static constexpr int NWS = G::NWS, TPW = G::TPW, E = G::E, FU = G::FU;
    // One chunk's operands for one wave, in the order the chunk uses them.
    struct Stage {
        f32x2 gate;          // (G2_l, G2_last - G2_l) of token `lane`
        frag kf[4];          // K[16 tm + r][32 w + 8 gq + (0..7)]
        frag qf[4];          // Q, same positions
        quad v[TPW];         // V[16 tw + (l >> 2)][16 blk + 4 (l & 3) + (0..3)]
        frag t[TPW][2];      // T~[16 tw + r][32 kk + 8 gq + (0..7)]
        frag p[TPW][2];      // P, same positions
    };

    // per-sequence: byte address of the sequence's first chunk in each tensor
    const char* kb; const char* qb; const char* gb;
    const char* tb; const char* pb;
    const char* vb; int64_t vn;                 // V: and the bytes to its end
    int64_t kq_step, g_step, w_step, v_step;    // bytes per chunk step
    int v_row;                                  // bytes per token row of V and O
    int w;
    // Loop-invariant per-lane byte offsets.  Row offsets that a bounds check
    // must see stay in the per-lane offset; the scalar offset only carries
    // fragment offsets inside a fully valid block.
    unsigned v_voff[TPW];   // row-wise V/O of tile tw: row 16 tw + (l >> 2), quad l & 3
    unsigned f_voff;        // fragment-major blocks: unit `lane`
    unsigned g_voff;        // gate pair of token `lane`

    __device__ __forceinline__ void init(const PrefillArgs& a, int64_t s0, int64_t base, int h, int blk,
                                         int wave) {
        const int l = lane_id();
        const int hq = (h * a.hqk) / a.hv;
        w = wave;
        const size_t kq0 = ((size_t)base * a.hqk + hq) * (kChunk * DK);
        kb = reinterpret_cast<const char*>(static_cast<const OP*>(a.ws_k) + kq0);
        qb = reinterpret_cast<const char*>(static_cast<const OP*>(a.ws_q) + kq0);
        const size_t w0 = ((size_t)base * a.hv + h) * (kChunk * kChunk);
        tb = reinterpret_cast<const char*>(static_cast<const OP*>(a.ws_t) + w0);
        pb = reinterpret_cast<const char*>(static_cast<const OP*>(a.ws_p) + w0);
        gb = reinterpret_cast<const char*>(a.ws_g + ((size_t)base * a.hv + h) * kGateFloats);
        const size_t v0 = ((size_t)s0 * a.hv + h) * a.dv + blk * 16;
        vb = reinterpret_cast<const char*>(static_cast<const OP*>(a.v) + v0);
        vn = ((int64_t)a.num_tokens * a.hv * a.dv - (int64_t)v0) * E;
        v_row = a.hv * a.dv * E;
        kq_step = (int64_t)a.hqk * kChunk * DK * E;
        g_step = (int64_t)a.hv * kGateFloats * 4;
        w_step = (int64_t)a.hv * kChunk * kChunk * E;
        v_step = (int64_t)kChunk * v_row;
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt)
            v_voff[jt] = (unsigned)((16 * (w + NWS * jt) + (l >> 2)) * v_row + (l & 3) * G::QE);
        f_voff = (unsigned)(l * 16);
        g_voff = (unsigned)(l * 8);
    }

    // Fetch the operands of the sequence's chunk j (zeros when !valid), in
    // four groups issued at different points of a chunk, each as soon as the
    // registers it refills are free: Q and V, then K and the gates, then T~,
    // then P.
    __device__ __forceinline__ int64_t cj(int64_t j, bool valid) const { return valid ? j : 0; }
    __device__ __forceinline__ void load_qv(Stage& s, int64_t j, bool valid) const {
        const int64_t jc = cj(j, valid);
        const auto rq = make_rsrc(qb + jc * kq_step, valid ? (int64_t)kChunk * DK * E : 0);
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) s.qf[tm] = B::frag(rq, f_voff, (unsigned)((w * 4 + tm) * FU * 1024));
        const int64_t vo = jc * v_step;
        const auto rv = make_rsrc(vb + vo, valid ? vn - vo : 0);
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) s.v[jt] = B::quad(rv, v_voff[jt]);
    }
    __device__ __forceinline__ void load_kg(Stage& s, int64_t j, bool valid) const {
        const int64_t jc = cj(j, valid);
        const auto rk = make_rsrc(kb + jc * kq_step, valid ? (int64_t)kChunk * DK * E : 0);
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) s.kf[tm] = B::frag(rk, f_voff, (unsigned)((w * 4 + tm) * FU * 1024));
        const auto rg = make_rsrc(gb + jc * g_step, valid ? kGateFloats * 4 : 0);
        s.gate = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, g_voff, 0, 0));
    }
    __device__ __forceinline__ void load_t(Stage& s, int64_t j, bool valid) const {
        const auto rt = make_rsrc(tb + cj(j, valid) * w_step, valid ? kChunk * kChunk * E : 0);
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                s.t[jt][kk] = B::frag(rt, f_voff, (unsigned)(((w + NWS * jt) * 2 + kk) * FU * 1024));
    }
    __device__ __forceinline__ void load_p(Stage& s, int64_t j, bool valid) const {
        const auto rp = make_rsrc(pb + cj(j, valid) * w_step, valid ? kChunk * kChunk * E : 0);
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
                s.p[jt][kk] = B::frag(rp, f_voff, (unsigned)(((w + NWS * jt) * 2 + kk) * FU * 1024));
    }
    __device__ __forceinline__ void load(Stage& s, int64_t j, bool valid) const {
        load_qv(s, j, valid);
        load_kg(s, j, valid);
        load_t(s, j, valid);
        load_p(s, j, valid);
    }
};

// The work of wave W of a scan workgroup (W is a compile-time constant, so
// every tile index below is static).
template <typename OP, int DK, int W>
__device__ __forceinline__ void scan_wave(const PrefillArgs& a, ScanSmem<OP, DK>& sm, int chain, int blk) {
    using Ops = Op<OP>;
    using frag = typename Ops::frag;
    using quad = typename Ops::quad;
    using G = ScanGeom<OP, DK>;
    using Ctx = ScanCtx<OP, DK>;
    using St = typename Ctx::Stage;
    using B = Buf<OP>;
    constexpr int NWS = G::NWS, TPW = G::TPW, RLD = G::RLD, E = G::E;
    constexpr int w = W;
    const int n = chain / a.hv;
    const int h = chain - n * a.hv;
    const int l = lane_id(), r = l & 15, gq = l >> 4;
    const int c = blk * 16 + r;

    const SeqIndex si{a.cu, a.seqlen};
    const int64_t s0 = si.start(n), s1 = si.start(n + 1);
    const int64_t base = slot_base(s0, n);
    Ctx ctx;
    ctx.init(a, s0, base, h, blk, w);

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

    // V/O staging: row-wise side (row l >> 2, quad l & 3) and tile side
    // (row r, quad gq), byte offsets inside a tile
    const unsigned v_wr = (unsigned)((l >> 2) * G::VROWB + G::QE * ((l & 3) ^ swz_vo(l >> 2, E)));
    const unsigned v_rd = (unsigned)(r * G::VROWB + G::QE * (gq ^ swz_vo(r, E)));
    auto gates = [&](const St& s, int par) {
        sm.gam[par][l] = fast_exp2(s.gate[0]);
        sm.dec[par][l] = fast_exp2(s.gate[1]);
    };

    const int64_t nchunks = (s1 - s0 + kChunk - 1) / kChunk;
    // One chunk j: `cur` holds its operands, `nxt` those of chunk j+1, whose
    // gates are moved into LDS here (read after the next chunk's first barrier).
    auto chunk = [&](St& cur, const St& nxt, int64_t j, int par) {
        const int64_t t0 = s0 + j * kChunk;
        // V tiles into lane layout (read back after E1)
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) *reinterpret_cast<quad*>(sm.vst[w][jt] + v_wr) = cur.v[jt];
        // ---- partial products over the d_k slice; other waves' X tiles to LDS
        const frag Sb = Ops::pack(S[0], S[1]);
        f32x4 Xp[4], Yp[4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) Xp[tm] = Ops::mma(Sb, cur.kf[tm], zero4());
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
            if (tm % NWS != w) sm.part[w][tm][l] = Xp[tm];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) Yp[tm] = Ops::mma(Sb, cur.qf[tm], zero4());
        __syncthreads();                                                        // E1
        gates(nxt, par ^ 1);
        // Q and V of this chunk are consumed: fetch those of chunk j+2
        const bool pre = j + 2 < nchunks;
        __builtin_amdgcn_sched_barrier(0);
        ctx.load_qv(cur, j + 2, pre);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
            if (tm % NWS != w) sm.part[w][4 + tm][l] = Yp[tm];
        // owner: R^T = V^T - X^T diag(gamma)
        float gt[TPW];
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
            const int tw = w + NWS * jt;
            f32x4 X = Xp[tw];
#pragma unroll
            for (int v2 = 0; v2 < NWS; ++v2)
                if (v2 != w) X += sm.part[v2][tw][l];
            gt[jt] = sm.gam[par][16 * tw + r];
            const quad vq = *reinterpret_cast<const quad*>(sm.vst[w][jt] + v_rd);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sm.Rt[(4 * gq + i) * RLD + 16 * tw + r] = from_f32<OP>(to_f32(vq[i]) - gt[jt] * X[i]);
        }
        const float gn = sm.gam[par][kChunk - 1];
        // K^T in operand layout (exact identity product)
        frag Ktf[2][2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
                Ktf[sub][kk] = Ops::pack(Ops::mma(cur.kf[2 * kk], Iden[sub], zero4()),
                                         Ops::mma(cur.kf[2 * kk + 1], Iden[sub], zero4()));
        __builtin_amdgcn_sched_barrier(0);
        ctx.load_kg(cur, j + 2, pre);
        __builtin_amdgcn_sched_barrier(0);
        __syncthreads();                                                        // E2
        const frag Rb0 = frag_nat(sm.Rt, RLD, r, 0), Rb1 = frag_nat(sm.Rt, RLD, r, 32);
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
            const int tw = w + NWS * jt;
            const f32x4 U = Ops::mma(cur.t[jt][1], Rb1, Ops::mma(cur.t[jt][0], Rb0, zero4()));
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
        __builtin_amdgcn_sched_barrier(0);
        ctx.load_t(cur, j + 2, pre);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 Y[TPW];
#pragma unroll
        for (int jt = 0; jt < TPW; ++jt) {
            const int tw = w + NWS * jt;
            Y[jt] = Yp[tw];
#pragma unroll
            for (int v2 = 0; v2 < NWS; ++v2)
                if (v2 != w) Y[jt] += sm.part[v2][4 + tw][l];
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
            Ot[jt] = Ops::mma(Ub1, cur.p[jt][1], Ops::mma(Ub0, cur.p[jt][0], gt[jt] * Y[jt]));
        __builtin_amdgcn_sched_barrier(0);
        ctx.load_p(cur, j + 2, pre);
        __builtin_amdgcn_sched_barrier(0);
        // O through the wave's V/O area to row-wise stores; rows past the end
        // of the sequence fall outside the resource
        {
            const int64_t ntl = s1 - t0;
            const auto ro = make_rsrc(static_cast<OP*>(a.out) + ((size_t)t0 * a.hv + h) * a.dv + blk * 16,
                                      ntl > 0 ? (ntl - 1) * ctx.v_row + 16 * E : 0);
#pragma unroll
            for (int jt = 0; jt < TPW; ++jt) {
                quad oq;
#pragma unroll
                for (int i = 0; i < 4; ++i) oq[i] = from_f32<OP>(Ot[jt][i]);
                *reinterpret_cast<quad*>(sm.vst[w][jt] + v_rd) = oq;
            }
            wave_lds_fence();
#pragma unroll
            for (int jt = 0; jt < TPW; ++jt)
                B::store4(*reinterpret_cast<const quad*>(sm.vst[w][jt] + v_wr), ro, ctx.v_voff[jt]);
        }
    };

    // Chunks are processed in pairs (stages A, B).  An odd count gets one
    // trailing empty chunk, which is an exact no-op: its loads read zeros
    // (gates 0, so gamma_n = 1 and S is unchanged) and its stores are dropped.
    // Keeping the loop free of an early exit keeps the load order identical on
    // every path into the loop, so the memory-counter waits stay exact.
    St A, Bs;
    ctx.load(A, 0, nchunks > 0);
    ctx.load(Bs, 1, nchunks > 1);
    gates(A, 0);
    __syncthreads();   // gates of chunk 0
    for (int64_t j = 0; j < nchunks; j += 2) {
        chunk(A, Bs, j, 0);
        chunk(Bs, A, j + 1, 1);
    }
    if (a.final_state) {
        *reinterpret_cast<f32x4*>(a.final_state + srow) = S[0];
        *reinterpret_cast<f32x4*>(a.final_state + srow + 4) = S[1];
    }
}

template <typename OP, int DK>
__global__ __launch_bounds__(DK / 32 * kWave) void gdn_scan_kernel(PrefillArgs a, int xcd_map) {
    __shared__ ScanSmem<OP, DK> sm;
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
    switch (wave_id()) {
        case 0: scan_wave<OP, DK, 0>(a, sm, chain, blk); break;
        case 1: scan_wave<OP, DK, 1>(a, sm, chain, blk); break;
        case 2: if constexpr (DK / 32 > 2) scan_wave<OP, DK, 2>(a, sm, chain, blk); break;
        default: if constexpr (DK / 32 > 3) scan_wave<OP, DK, 3>(a, sm, chain, blk); break;
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
    const int64_t chains = (int64_t)a.num_seqs * a.hv;
    const int nblk = a.dv / 16;
    const int xcd = (nblk == 8 && chains % 8 == 0) ? 1 : 0;
    dim3 grid((unsigned)(chains * nblk)), block(DK / 32 * kWave);
    hipLaunchKernelGGL((gdn_scan_kernel<OP, DK>), grid, block, 0, st, a, xcd);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, bool bf16, int dk, hipStream_t st) {
    if (a.num_seqs == 0) return hipSuccess;
    if (bf16) return dk == 128 ? launch_prefill_t<__bf16, 128>(a, st) : launch_prefill_t<__bf16, 64>(a, st);
    return dk == 128 ? launch_prefill_t<float, 128>(a, st) : launch_prefill_t<float, 64>(a, st);
}

}  // namespace gdn
