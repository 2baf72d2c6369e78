/*
 * fp64 token-by-token Gated DeltaNet recurrence: the ORACLE.
 *
 * Test infrastructure only. The product library never links, loads or calls
 * this file; only the tests, the smoke check and the benchmark's CPU-baseline
 * leg do. It shares no code with the GPU path.
 *
 * What it computes (page "Qwen3-Next-80B-A3B-Instruct" model card, section
 * "Model Overview": Gated DeltaNet with 32 V heads sharing 16 QK heads, head
 * dimension 128; page "Qwen3-Next and vLLM", section "Hybrid Attention": Gated
 * DeltaNet is a linear-attention mixer). The pages give the rule only in
 * words; the plainest reading, used here, is for every packed sequence n,
 * every V head h and its QK head h' = h / (Hv / Hqk):
 *
 *     S = initial_state[n, h]          (dv x dk; zeros when absent)
 *     for each token t of the sequence, in order:
 *         alpha = exp(g[t, h]),  b = beta[t, h]
 *         S = alpha * S                                  decay
 *         S = S + b * (v[t, h] - S k[t, h']) k[t, h']^T   delta-rule write along k
 *         out[t, h] = scale * S q[t, h']                 read-out after the write
 *     final_state[n, h] = S
 *
 * Element S[i][j]: i is the value index, j the key index. All arithmetic is
 * in double precision on the exact widening of the stored inputs (bf16, fp32
 * or fp64); nothing is blocked, fused or reordered.
 *
 * `mutant` exists only so the tests can show that their pins detect plausible
 * mistakes; 0 is the rule above and the only value anything else passes.
 *   1: no decay        2: read-out before the write   3: state used transposed
 *   4: V head mapped to QK head h % Hqk               5: sign of the correction flipped
 *   6: decay applied after the write
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_BF16 = 0, ORC_FP32 = 1, ORC_FP64 = 2 };

static double load_elem(const void* p, int dt, int64_t i) {
    if (dt == ORC_FP64) return ((const double*)p)[i];
    if (dt == ORC_FP32) return (double)((const float*)p)[i];
    uint32_t bits = ((uint32_t)((const uint16_t*)p)[i]) << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* One (sequence, V head) pair over its tokens. */
static void run_pair(const void* q, const void* k, const void* v, int qkv_dt,
                     const void* g, const void* beta, const void* s0, int aux_dt,
                     int64_t t_begin, int64_t t_end, int32_t n, int32_t h, int32_t h_out,
                     int32_t Hqk, int32_t Hv, int32_t n_out_heads, int32_t dk, int32_t dv,
                     double scale, double* out, double* sT, int mutant,
                     double* S, double* kk, double* qq, double* vv, double* a) {
    const int32_t group = Hv / Hqk;
    const int32_t hq = (mutant == 4) ? (h % Hqk) : (h / group);
    const int64_t sz = (int64_t)dv * dk;
    if (s0) {
        const int64_t base = ((int64_t)n * Hv + h) * sz;
        for (int64_t e = 0; e < sz; ++e) S[e] = load_elem(s0, aux_dt, base + e);
    } else {
        for (int64_t e = 0; e < sz; ++e) S[e] = 0.0;
    }
    for (int64_t t = t_begin; t < t_end; ++t) {
        const double alpha = exp(load_elem(g, aux_dt, t * Hv + h));
        const double b = load_elem(beta, aux_dt, t * Hv + h);
        for (int32_t j = 0; j < dk; ++j) {
            kk[j] = load_elem(k, qkv_dt, (t * Hqk + hq) * dk + j);
            qq[j] = load_elem(q, qkv_dt, (t * Hqk + hq) * dk + j);
        }
        for (int32_t i = 0; i < dv; ++i) vv[i] = load_elem(v, qkv_dt, (t * Hv + h) * dv + i);

        double* o = out + (t * n_out_heads + h_out) * dv;
        if (mutant == 2) { /* read-out before the write */
            for (int32_t i = 0; i < dv; ++i) {
                double acc = 0.0;
                for (int32_t j = 0; j < dk; ++j) acc += S[i * dk + j] * qq[j];
                o[i] = scale * acc;
            }
        }
        if (mutant != 1 && mutant != 6)
            for (int64_t e = 0; e < sz; ++e) S[e] *= alpha;
        /* a = S k (mutant 3 uses S^T k; only meaningful when dk == dv) */
        for (int32_t i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int32_t j = 0; j < dk; ++j)
                acc += (mutant == 3 ? S[j * dk + i] : S[i * dk + j]) * kk[j];
            a[i] = acc;
        }
        for (int32_t i = 0; i < dv; ++i) {
            const double c = (mutant == 5) ? b * (vv[i] + a[i]) : b * (vv[i] - a[i]);
            for (int32_t j = 0; j < dk; ++j) S[i * dk + j] += c * kk[j];
        }
        if (mutant == 6)
            for (int64_t e = 0; e < sz; ++e) S[e] *= alpha;
        if (mutant != 2) {
            for (int32_t i = 0; i < dv; ++i) {
                double acc = 0.0;
                for (int32_t j = 0; j < dk; ++j) acc += S[i * dk + j] * qq[j];
                o[i] = scale * acc;
            }
        }
    }
    if (sT) {
        const int64_t base = ((int64_t)n * n_out_heads + h_out) * sz;
        for (int64_t e = 0; e < sz; ++e) sT[base + e] = S[e];
    }
}

/*
 * q, k  [T, Hqk, dk], v [T, Hv, dv] in qkv_dt; g, beta [T, Hv] and s0
 * [N, Hv, dv, dk] (may be NULL) in aux_dt; cu [N + 1] int64 offsets.
 * Only V heads h_begin <= h < h_end are computed; out is [T, h_end - h_begin, dv]
 * and sT (may be NULL) is [N, h_end - h_begin, dv, dk], both fp64.
 * Returns the number of threads used, or a negative value on bad arguments.
 */
int gdn_oracle_recurrent(const void* q, const void* k, const void* v, int qkv_dt,
                         const void* g, const void* beta, const void* s0, int aux_dt,
                         const int64_t* cu, int32_t N, int32_t Hqk, int32_t Hv,
                         int32_t dk, int32_t dv, double scale,
                         int32_t h_begin, int32_t h_end,
                         double* out, double* sT, int32_t nthreads, int32_t mutant) {
    if (N < 0 || Hqk <= 0 || Hv <= 0 || Hv % Hqk != 0 || dk <= 0 || dv <= 0) return -1;
    if (h_begin < 0 || h_end > Hv || h_begin > h_end) return -1;
    const int32_t nh = h_end - h_begin;
    const int64_t npairs = (int64_t)N * nh;
    int used = 1;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    if (nthreads > npairs && npairs > 0) nthreads = (int32_t)npairs;
    used = nthreads > 0 ? nthreads : 1;
#pragma omp parallel num_threads(used)
#endif
    {
        const int64_t sz = (int64_t)dv * dk;
        double* S = (double*)malloc(sizeof(double) * (size_t)(sz + 2 * dk + 2 * dv));
        double* kk = S + sz;
        double* qq = kk + dk;
        double* vv = qq + dk;
        double* a = vv + dv;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (int64_t p = 0; p < npairs; ++p) {
            const int32_t n = (int32_t)(p / nh);
            const int32_t ho = (int32_t)(p % nh);
            run_pair(q, k, v, qkv_dt, g, beta, s0, aux_dt, cu[n], cu[n + 1], n, h_begin + ho, ho,
                     Hqk, Hv, nh, dk, dv, scale, out, sT, mutant, S, kk, qq, vv, a);
        }
        free(S);
    }
    return used;
}
