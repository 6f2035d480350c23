/*
 * cap_oracle.c -- CPU fp64 oracle for decode attention over a paged radix
 * tree.  TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and
 * the cpu_baseline leg of bench.py may load it.  It shares no code, header
 * or table with the HIP library.
 *
 * What it computes (Capillary Kernels project page, abstract: attention for
 * long-context decoding over a radix-tree KV cache in which requests reuse
 * common context prefixes).  The page gives no formula; the plain reading,
 * used here, is standard scaled-dot-product softmax attention of each
 * request's single decode query over its whole context:
 *
 *   C_r    = tokens of the nodes on r's path, root first, each node's tokens
 *            in order (token t of node n lives in page
 *            page_ids[page_offsets[n] + t / P], slot t % P);
 *   s_t    = sm_scale * sum_d q[r][h][d] * K[t][g][d],  g = h / (Hq / Hkv);
 *   out    = sum_t exp(s_t - max s) V[t][g] / sum_t exp(s_t - max s).
 *
 * No sharing, no chunking, no base-2 exponent: each (request, head) is done
 * on its own over the flattened context, in double precision, with the bf16
 * inputs widened exactly.  Pool layouts (bf16 bit patterns):
 *   K: [pool_pages][Hkv][D/8][P][8]   element (t, d) at ((d/8)*P + t)*8 + d%8
 *   V: [pool_pages][Hkv][D][P]        element (t, d) at d*P + t
 *   q: [R][Hq][D]; out: double [R][Hq][D].
 * Returns 0 on success, a negative code for inputs it cannot interpret.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int cap_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

int cap_oracle_decode(int R, int Hq, int Hkv, int D, int P, double sm_scale,
                      int num_nodes, const int32_t *num_tokens,
                      const int64_t *page_offsets, const int32_t *page_ids,
                      const int32_t *path_offsets, const int32_t *path_nodes,
                      const uint16_t *q, const uint16_t *k_pool,
                      const uint16_t *v_pool, int nthreads, double *out)
{
    if (R < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || D % 8 != 0 || P <= 0)
        return -1;
    const int G = Hq / Hkv;
    const int64_t blk = (int64_t)P * D;          /* elements per (page, KV head) */
    int bad = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int64_t task = 0; task < (int64_t)R * Hkv; ++task) {
        const int r = (int)(task / Hkv), g = (int)(task % Hkv);
        /* context length */
        int64_t ctx = 0;
        for (int j = path_offsets[r]; j < path_offsets[r + 1]; ++j) {
            int n = path_nodes[j];
            if (n < 0 || n >= num_nodes) { bad |= 1; break; }
            ctx += num_tokens[n];
        }
        if (bad || ctx == 0) { bad |= 1; continue; }
        double *s = (double *)malloc(sizeof(double) * (size_t)ctx * G);
        double *qd = (double *)malloc(sizeof(double) * (size_t)G * D);
        double *acc = (double *)calloc((size_t)G * D, sizeof(double));
        double *vrow = (double *)malloc(sizeof(double) * (size_t)D);
        for (int i = 0; i < G; ++i)
            for (int d = 0; d < D; ++d)
                qd[i * D + d] = bf16_to_double(q[((int64_t)r * Hq + g * G + i) * D + d]);

        /* pass 1: scores for every context token and the G heads of KV head g */
        int64_t t_ctx = 0;
        for (int j = path_offsets[r]; j < path_offsets[r + 1]; ++j) {
            const int n = path_nodes[j];
            for (int t = 0; t < num_tokens[n]; ++t, ++t_ctx) {
                const int64_t page = page_ids[page_offsets[n] + t / P];
                const int slot = t % P;
                const uint16_t *kb = k_pool + (page * Hkv + g) * blk;
                for (int i = 0; i < G; ++i) {
                    double dot = 0.0;
                    for (int d = 0; d < D; ++d)
                        dot += qd[i * D + d] *
                               bf16_to_double(kb[((int64_t)(d / 8) * P + slot) * 8 + d % 8]);
                    s[t_ctx * G + i] = sm_scale * dot;
                }
            }
        }
        /* pass 2: softmax weights and the weighted sum of V */
        for (int i = 0; i < G; ++i) {
            double mx = -INFINITY;
            for (int64_t t = 0; t < ctx; ++t)
                if (s[t * G + i] > mx) mx = s[t * G + i];
            for (int64_t t = 0; t < ctx; ++t)
                s[t * G + i] = exp(s[t * G + i] - mx);
        }
        double *den = (double *)calloc((size_t)G, sizeof(double));
        t_ctx = 0;
        for (int j = path_offsets[r]; j < path_offsets[r + 1]; ++j) {
            const int n = path_nodes[j];
            for (int t = 0; t < num_tokens[n]; ++t, ++t_ctx) {
                const int64_t page = page_ids[page_offsets[n] + t / P];
                const int slot = t % P;
                const uint16_t *vb = v_pool + (page * Hkv + g) * blk;
                for (int d = 0; d < D; ++d)
                    vrow[d] = bf16_to_double(vb[(int64_t)d * P + slot]);
                for (int i = 0; i < G; ++i) {
                    const double w = s[t_ctx * G + i];
                    den[i] += w;
                    for (int d = 0; d < D; ++d)
                        acc[i * D + d] += w * vrow[d];
                }
            }
        }
        for (int i = 0; i < G; ++i)
            for (int d = 0; d < D; ++d)
                out[((int64_t)r * Hq + g * G + i) * D + d] = acc[i * D + d] / den[i];
        free(den); free(vrow); free(acc); free(qd); free(s);
    }
    return bad ? -2 : 0;
}
