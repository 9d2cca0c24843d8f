/*
 * gdn_oracle.c -- plain fp64 sequential reference for the Gated DeltaNet
 * (GDN) token mixer.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  It shares no code, header or
 * constant with the HIP library and must never serve a product call.
 *
 * What it computes.  The pages (flozi.net, "Qwen3.8-Flash-Next architecture",
 * section "Der Weg eines Tokens durch das Modell", item 1, and the stack
 * table) say that each GDN layer keeps a fixed-size recurrent state per head
 * instead of a per-token KV entry; they print no formula.  The recurrence
 * used is the gated delta rule, per value head with state S (d_v x d_k):
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,            alpha_t = exp(g_t).
 *
 * Expanding the product by distributivity gives the rank-1 form evaluated
 * here, step by step and in token order:
 *
 *     s   = S k_t                       (read the state at the key)
 *     u   = beta_t (v_t - alpha_t s)    (delta: new value minus decayed recall)
 *     S  <- alpha_t S + u k_t^T         (decay, then rank-1 write)
 *     o_t = S q_t                       (read after this token's write)
 *
 * Everything is fp64.  Inputs are the exact values the GPU receives: bf16
 * bit patterns or fp32 are widened exactly before use.
 *
 * Layouts (row-major, contiguous):
 *   q, k        [tokens, Hqk, dk]       element type `elem` (0 = fp32, 1 = bf16 bits)
 *   v           [tokens, Hv,  dv]       element type `elem`
 *   g, beta     [tokens, Hv]            fp32
 *   init_state  [N, Hv, dv, dk]         fp32, may be NULL (zero state)
 *   out         [tokens, Hv, dv]        fp64
 *   final_state [N, Hv, dv, dk]         fp64, may be NULL
 * Value head h reads q/k head floor(h * Hqk / Hv) (contiguous groups).
 * Sequence n covers tokens [cu[n], cu[n+1]).
 *
 * Parallelism: independent chains (sequence, value head) only; the token loop
 * of a chain is strictly sequential.
 *
 * Raw-projection variants (..._raw): the steps just before the recurrence are
 * applied per token, in fp64, before the same token step:
 *     q <- q / sqrt(|q|^2 + 1e-6),   k <- k / sqrt(|k|^2 + 1e-6),
 *     g  = -softplus(a) = -(max(a, 0) + log1p(exp(-|a|))),
 *     beta = 1 / (1 + exp(-b)),
 * where a and b are the per-(token, value head) gate and write-strength
 * logits passed in place of g and beta.  (The pages give the model's layer
 * layout but none of these formulas; these are the usual forms, matching the
 * value distributions of the synthetic inputs.)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double widen(const void* p, int64_t i, int elem) {
    if (elem == 1) {
        uint32_t u = ((uint32_t)((const uint16_t*)p)[i]) << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float*)p)[i];
}

/* One token of the recurrence on state S (dv x dk, row-major). */
static void gdn_token(double* S, int dk, int dv, const double* kt, const double* qt,
                      const double* vt, double alpha, double beta, double* s, double* u,
                      double* ot) {
    for (int i = 0; i < dv; ++i) {           /* s = S k */
        double acc = 0.0;
        for (int j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * kt[j];
        s[i] = acc;
    }
    for (int i = 0; i < dv; ++i) u[i] = beta * (vt[i] - alpha * s[i]);
    for (int i = 0; i < dv; ++i)             /* S = alpha S + u k^T */
        for (int j = 0; j < dk; ++j)
            S[(int64_t)i * dk + j] = alpha * S[(int64_t)i * dk + j] + u[i] * kt[j];
    for (int i = 0; i < dv; ++i) {           /* o = S q */
        double acc = 0.0;
        for (int j = 0; j < dk; ++j) acc += S[(int64_t)i * dk + j] * qt[j];
        ot[i] = acc;
    }
}

static const double kNormEps = 1e-6;

/* The prologue of the raw-projection variants, in place. */
static void normalise(double* x, int d) {
    double s2 = 0.0;
    for (int j = 0; j < d; ++j) s2 += x[j] * x[j];
    const double inv = 1.0 / sqrt(s2 + kNormEps);
    for (int j = 0; j < d; ++j) x[j] *= inv;
}
static double gate_from_logit(double a) { return -((a > 0.0 ? a : 0.0) + log1p(exp(-fabs(a)))); }
static double beta_from_logit(double b) { return 1.0 / (1.0 + exp(-b)); }

static int max_threads(int nthreads) {
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

int gdn_oracle_threads(int nthreads) { return max_threads(nthreads); }

/* Prefill: every sequence from its initial state, outputs for every token. */
static int prefill(int raw, int64_t nseq, const int64_t* cu, int hqk, int hv, int dk, int dv,
                   int elem, const void* q, const void* k, const void* v, const float* g,
                   const float* beta, const float* init_state, double* out,
                   double* final_state, int nthreads) {
    if (nseq < 0 || hqk <= 0 || hv <= 0 || dk <= 0 || dv <= 0 || hv % hqk != 0) return 1;
    int64_t nchain = nseq * hv;
    int err = 0;
    int nt = max_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t c = 0; c < nchain; ++c) {
        int64_t n = c / hv;
        int h = (int)(c % hv);
        int hq = (int)(((int64_t)h * hqk) / hv);
        double* S = (double*)malloc(sizeof(double) * (size_t)dv * dk);
        double* buf = (double*)malloc(sizeof(double) * (size_t)(2 * dk + 4 * dv));
        if (!S || !buf) {
            free(S);
            free(buf);
#pragma omp atomic write
            err = 2;
            continue;
        }
        double *kt = buf, *qt = buf + dk, *vt = buf + 2 * dk, *s = vt + dv, *u = s + dv,
               *ot = u + dv;
        const int64_t sbase = (n * hv + h) * (int64_t)dv * dk;
        for (int64_t e = 0; e < (int64_t)dv * dk; ++e)
            S[e] = init_state ? (double)init_state[sbase + e] : 0.0;
        for (int64_t t = cu[n]; t < cu[n + 1]; ++t) {
            for (int j = 0; j < dk; ++j) {
                kt[j] = widen(k, (t * hqk + hq) * dk + j, elem);
                qt[j] = widen(q, (t * hqk + hq) * dk + j, elem);
            }
            for (int i = 0; i < dv; ++i) vt[i] = widen(v, (t * hv + h) * dv + i, elem);
            double gt = (double)g[t * hv + h], bt = (double)beta[t * hv + h];
            if (raw) {
                normalise(kt, dk);
                normalise(qt, dk);
                gt = gate_from_logit(gt);
                bt = beta_from_logit(bt);
            }
            gdn_token(S, dk, dv, kt, qt, vt, exp(gt), bt, s, u, ot);
            memcpy(out + (t * hv + h) * dv, ot, sizeof(double) * dv);
        }
        if (final_state) memcpy(final_state + sbase, S, sizeof(double) * (size_t)dv * dk);
        free(S);
        free(buf);
    }
    return err;
}

/* Decode: one token per sequence, fp64 state [N, Hv, dv, dk] updated in place. */
static int decode_step(int raw, int64_t nseq, int hqk, int hv, int dk, int dv, int elem,
                       const void* q, const void* k, const void* v, const float* g,
                       const float* beta, double* state, double* out, int nthreads) {
    if (nseq < 0 || hqk <= 0 || hv <= 0 || dk <= 0 || dv <= 0 || hv % hqk != 0) return 1;
    int64_t nchain = nseq * hv;
    int err = 0;
    int nt = max_threads(nthreads);
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t c = 0; c < nchain; ++c) {
        int64_t n = c / hv;
        int h = (int)(c % hv);
        int hq = (int)(((int64_t)h * hqk) / hv);
        double* buf = (double*)malloc(sizeof(double) * (size_t)(2 * dk + 4 * dv));
        if (!buf) {
#pragma omp atomic write
            err = 2;
            continue;
        }
        double *kt = buf, *qt = buf + dk, *vt = buf + 2 * dk, *s = vt + dv, *u = s + dv,
               *ot = u + dv;
        for (int j = 0; j < dk; ++j) {
            kt[j] = widen(k, (n * hqk + hq) * dk + j, elem);
            qt[j] = widen(q, (n * hqk + hq) * dk + j, elem);
        }
        for (int i = 0; i < dv; ++i) vt[i] = widen(v, (n * hv + h) * dv + i, elem);
        double gt = (double)g[n * hv + h], bt = (double)beta[n * hv + h];
        if (raw) {
            normalise(kt, dk);
            normalise(qt, dk);
            gt = gate_from_logit(gt);
            bt = beta_from_logit(bt);
        }
        gdn_token(state + c * (int64_t)dv * dk, dk, dv, kt, qt, vt, exp(gt), bt, s, u, ot);
        memcpy(out + c * dv, ot, sizeof(double) * dv);
        free(buf);
    }
    return err;
}

int gdn_oracle_prefill(int64_t nseq, const int64_t* cu, int hqk, int hv, int dk, int dv,
                       int elem, const void* q, const void* k, const void* v, const float* g,
                       const float* beta, const float* init_state, double* out,
                       double* final_state, int nthreads) {
    return prefill(0, nseq, cu, hqk, hv, dk, dv, elem, q, k, v, g, beta, init_state, out,
                   final_state, nthreads);
}

/* a, b: gate and write-strength logits in place of g, beta; q, k unnormalised. */
int gdn_oracle_prefill_raw(int64_t nseq, const int64_t* cu, int hqk, int hv, int dk, int dv,
                           int elem, const void* q, const void* k, const void* v, const float* a,
                           const float* b, const float* init_state, double* out,
                           double* final_state, int nthreads) {
    return prefill(1, nseq, cu, hqk, hv, dk, dv, elem, q, k, v, a, b, init_state, out,
                   final_state, nthreads);
}

int gdn_oracle_decode_step(int64_t nseq, int hqk, int hv, int dk, int dv, int elem,
                           const void* q, const void* k, const void* v, const float* g,
                           const float* beta, double* state, double* out, int nthreads) {
    return decode_step(0, nseq, hqk, hv, dk, dv, elem, q, k, v, g, beta, state, out, nthreads);
}

int gdn_oracle_decode_step_raw(int64_t nseq, int hqk, int hv, int dk, int dv, int elem,
                               const void* q, const void* k, const void* v, const float* a,
                               const float* b, double* state, double* out, int nthreads) {
    return decode_step(1, nseq, hqk, hv, dk, dv, elem, q, k, v, a, b, state, out, nthreads);
}
