// gdn_device.h -- device-side building blocks shared by the GDN kernels (gfx950).
//
// Matrix-core fragments.  Every product on the chunk path is written as a
// sequence of 16x16 output tiles with a K step of 32, in one of two
// element types:
//   * bf16 operands: one v_mfma_f32_16x16x32_bf16 per K step;
//   * fp32 operands: eight v_mfma_f32_16x16x4_f32 per K step (fp32 path).
// Lane l of a 64-wide wave works on row/column (l & 15) and lane group
// gq = l >> 4.  Accumulators (16x16 fp32) hold rows 4*gq + {0..3} of column
// (l & 15).  Operand fragments hold 8 K values per lane; we fix the K order
// inside a 32-wide step to the "paired" order
//     slot 8*gq + i      <->  k = 4*gq + i        (i = 0..3)
//     slot 8*gq + 4 + i  <->  k = 16 + 4*gq + i   (i = 0..3)
// so that two stacked accumulator tiles (rows 0..15 and 16..31 of a K range)
// are directly an operand fragment of the next product after conversion,
// without a trip through LDS.  A and B fragments of one product always use the
// same order, so the order itself never changes a result.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kChunk = 64;   // tokens per chunk
constexpr int kWave = 64;    // lanes per wavefront

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
// Wave index, marked wave-uniform so that branches on it stay scalar.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ---------------------------------------------------------------------------
// operand traits
// ---------------------------------------------------------------------------
template <typename T> struct Op;

template <> struct Op<__bf16> {
    using frag = bf16x8;
    using quad = bf16x4;
    __device__ __forceinline__ static frag pack(f32x4 lo, f32x4 hi) {
        frag r;
        r[0] = (__bf16)lo[0]; r[1] = (__bf16)lo[1]; r[2] = (__bf16)lo[2]; r[3] = (__bf16)lo[3];
        r[4] = (__bf16)hi[0]; r[5] = (__bf16)hi[1]; r[6] = (__bf16)hi[2]; r[7] = (__bf16)hi[3];
        return r;
    }
    __device__ __forceinline__ static frag join(quad lo, quad hi) {
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

template <> struct Op<float> {
    using frag = f32x8;
    using quad = f32x4;
    __device__ __forceinline__ static frag pack(f32x4 lo, f32x4 hi) {
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    __device__ __forceinline__ static frag join(quad lo, quad hi) { return pack(lo, hi); }
    __device__ __forceinline__ static f32x4 mma(frag a, frag b, f32x4 c) {
#pragma unroll
        for (int s = 0; s < 8; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
        return c;
    }
};

// A/B fragment of a row-major matrix M (leading dimension ld, in elements):
// row `row`, K step starting at column k0, paired order.
template <typename T>
__device__ __forceinline__ typename Op<T>::frag frag_rows(const T* M, int ld, int row, int k0) {
    using quad = typename Op<T>::quad;
    const int gq = lane_id() >> 4;
    const T* p = M + (size_t)row * ld + k0 + 4 * gq;
    quad lo = *reinterpret_cast<const quad*>(p);
    quad hi = *reinterpret_cast<const quad*>(p + 16);
    return Op<T>::join(lo, hi);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// fp32 16x16x16 block product on the matrix cores, for small fp32 solves:
//   c += A * B   where A is given as the lane's 4 K values A[l&15][4*gq + 0..3]
//   and B in accumulator layout (lane holds B[4*gq + i][l&15], i = 0..3).
__device__ __forceinline__ f32x4 mm16_f32(f32x4 a, f32x4 b, f32x4 c) {
#pragma unroll
    for (int s = 0; s < 4; ++s) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[s], b[s], c, 0, 0, 0);
    return c;
}

// ---------------------------------------------------------------------------
// raw projections
// ---------------------------------------------------------------------------
// The *_raw entry points take q and k unnormalised and the gates as logits a
// (decay) and b (write strength), and apply per (token, head)
//     q <- q / sqrt(|q|^2 + kNormEps),  k likewise,
//     g = -softplus(a),  beta = sigmoid(b)
// -- the steps that precede the recurrence in the layer; the resulting
// distributions are those of the synthetic inputs (unit q, k; g < 0; beta in
// (0, 1)).
constexpr float kNormEps = 1e-6f;
__device__ __forceinline__ float gate_from_logit(float a) {
    return -(fmaxf(a, 0.f) + log1pf(expf(-fabsf(a))));
}
__device__ __forceinline__ float beta_from_logit(float b) { return 1.f / (1.f + expf(-b)); }

// ---------------------------------------------------------------------------
// element I/O
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// 16-byte vector of elements (8 bf16 or 4 fp32)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// sequence bookkeeping (packed varlen)
// ---------------------------------------------------------------------------
// Token range of sequence n: from cu_seqlens if given, else equal lengths.
struct SeqIndex {
    const int32_t* cu;   // device offsets [N+1] or nullptr
    int64_t seqlen;      // equal length when cu == nullptr
    __device__ __forceinline__ int64_t start(int n) const { return cu ? (int64_t)cu[n] : (int64_t)n * seqlen; }
};

// Chunk slots: chunk j of sequence n (first token t0 = start(n) + 64 j) gets
// slot floor(t0 / 64) + n.  Slots are distinct, increase with (n, j), and the
// slots of sequence n form the range [base(n), base(n) + ceil(len / 64)),
// so at most ceil(tokens / 64) + N slots exist.
__device__ __forceinline__ int64_t slot_base(int64_t start, int n) { return start / kChunk + n; }

}  // namespace gdn
