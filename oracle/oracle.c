/*
 * oracle.c - plain, slow, fp64 CPU oracle for query-driven key-cache channel
 * pruning (ThinK).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, includes
 * or calls this file; only the test-suite, the smoke check and the CPU
 * baseline leg of the benchmark load it.  It shares no code, header, table or
 * constant with the HIP path.
 *
 * Method source (the pages name no formula, layout or API; readings below):
 *   "ThinK: Thinner Key Cache by Query-Driven Pruning", Method details ->
 *   Technical framework: for the queries, measure how relevant each key-cache
 *   channel is; order the channels by that relevance and drop the weakest;
 *   then run inference on the pruned key cache.
 *   Same page, Method details -> Key design (1)-(2) and the original
 *   abstract: relevance is measured through the attention weights, and the
 *   pruning is chosen to keep the loss of attention weight small.
 *
 * Reading of the score (the plainest one the pages support): the logits
 * Q_w K^T of an observation window Q_w decompose over channels as
 * sum_c Q_w[:,c] K[:,c]^T; channel c's relevance is the Frobenius norm of its
 * rank-1 term, which equals ||Q_w[:,c]||_2 * ||K[:,c]||_2.  For grouped-query
 * attention the per-query-head norms of one key/value group are summed.
 *
 * Everything is computed in fp64.  Inputs are widened exactly (fp32 -> fp64,
 * bf16 -> fp32 -> fp64).  All sums run in ascending index order.  OpenMP
 * splits work over (batch, head) pairs only, so results never depend on the
 * thread count.
 *
 * Status codes: 0 ok, -1 bad argument, -2 non-finite input.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_BF16 = 1 };

/* Exact widening of one stored element to fp64. */
static double widen(const void *base, int dtype, size_t i) {
    if (dtype == OR_F32) return (double)((const float *)base)[i];
    uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static size_t elem_size(int dtype) { return dtype == OR_F32 ? 4 : 2; }

static int dims_ok(int B, int S_cap, int Hq, int Hkv, int D, int dtype) {
    if (B < 1 || S_cap < 1 || Hkv < 1 || Hq < Hkv || D < 1) return 0;
    if (Hq % Hkv != 0) return 0;
    if (dtype != OR_F32 && dtype != OR_BF16) return 0;
    return 1;
}

static int lens_ok(int B, int S_cap, const int32_t *lens) {
    for (int b = 0; b < B; ++b)
        if (lens[b] < 1 || lens[b] > S_cap) return 0;
    return 1;
}

/* the append alone also takes empty sequences: their first row is row 0 */
static int lens_ok_or_empty(int B, int S_cap, const int32_t *lens) {
    for (int b = 0; b < B; ++b)
        if (lens[b] < 0 || lens[b] > S_cap) return 0;
    return 1;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------------------
 * Stage (a): per-channel relevance score.
 *   K2[b,kv,c]  = sum_{t < len_b} K[b,t,kv,c]^2
 *   Q2[b,h,c]   = sum_{i < W}     Q_w[b,i,h,c]^2
 *   s[b,kv,c]   = sqrt(K2) * sum_{g < G} sqrt(Q2[b, kv*G+g, c])
 * Layouts: K [B,S_cap,Hkv,D], Q_w [B,W,Hq,D], scores [B,Hkv,D] (fp64).
 * ------------------------------------------------------------------------- */
int oracle_score(int B, int S_cap, int Hq, int Hkv, int D, int dtype,
                 const void *k_cache, const int32_t *seq_lens, const void *q_obs,
                 int W, double *scores) {
    if (!dims_ok(B, S_cap, Hq, Hkv, D, dtype) || W < 1) return -1;
    if (!k_cache || !seq_lens || !q_obs || !scores) return -1;
    if (!lens_ok(B, S_cap, seq_lens)) return -1;
    const int G = Hq / Hkv;
    int bad = 0;
#pragma omp parallel for collapse(2) schedule(static) reduction(| : bad)
    for (int b = 0; b < B; ++b) {
        for (int kv = 0; kv < Hkv; ++kv) {
            double *K2 = (double *)calloc((size_t)D, sizeof(double));
            const int len = seq_lens[b];
            /* token loop outside the channel loop: each channel's sum still
               runs in ascending t, this order only reads K row by row */
            for (int t = 0; t < len; ++t) {
                const size_t row = (((size_t)b * S_cap + t) * Hkv + kv) * D;
                for (int c = 0; c < D; ++c) {
                    const double x = widen(k_cache, dtype, row + c);
                    if (!isfinite(x)) bad = 1;
                    K2[c] += x * x;
                }
            }
            for (int c = 0; c < D; ++c) {
                double qsum = 0.0;
                for (int g = 0; g < G; ++g) {
                    const int h = kv * G + g;
                    double Q2 = 0.0;
                    for (int i = 0; i < W; ++i) {
                        const double q = widen(q_obs, dtype, (((size_t)b * W + i) * Hq + h) * D + c);
                        if (!isfinite(q)) bad = 1;
                        Q2 += q * q;
                    }
                    qsum += sqrt(Q2);
                }
                scores[((size_t)b * Hkv + kv) * D + c] = sqrt(K2[c]) * qsum;
            }
            free(K2);
        }
    }
    return bad ? -2 : 0;
}

/* ---------------------------------------------------------------------------
 * Prefill-fused scoring (the step before the path).  Stage (a) needs the
 * keys only through K2[b,kv,c] = sum_t K[b,t,kv,c]^2, so the sums can be
 * gathered while the prompt's keys are written to the cache, chunk by chunk,
 * and the score later needs no key read.
 *
 * Write: a chunk of n_rows new rows per sequence at positions t0 .. t0+n_rows-1:
 *   K[b,t0+t,kv,:] = k_rows[b,t,kv,:],  V[b,t0+t,kv,:] = v_rows[b,t,kv,:]
 *   K2[b,kv,c]   += k_rows[b,t,kv,c]^2
 * for every t with t0+t < min(len_b, S_cap) (seq_lens = the prompts' lengths);
 * other rows are neither written nor counted.  Rows in ascending t.
 * Layouts: k_rows, v_rows [B,n_rows,Hkv,D]; K2 fp64 [B,Hkv,D].
 * ------------------------------------------------------------------------- */
int oracle_prefill_write(int B, int S_cap, int Hkv, int D, int dtype, const void *k_rows,
                         const void *v_rows, int t0, int n_rows, const int32_t *seq_lens,
                         void *k_cache, void *v_cache, double *k2) {
    if (!dims_ok(B, S_cap, Hkv, Hkv, D, dtype) || t0 < 0 || n_rows < 0) return -1;
    if (!k_rows || !v_rows || !seq_lens || !k_cache || !v_cache || !k2) return -1;
    if (!lens_ok(B, S_cap, seq_lens)) return -1;
    const size_t es = elem_size(dtype), row = (size_t)Hkv * D;
    int bad = 0;
    for (int b = 0; b < B; ++b) {
        for (int t = 0; t < n_rows; ++t) {
            const int pos = t0 + t;
            if (pos >= seq_lens[b]) break;
            const size_t src = ((size_t)b * n_rows + t) * row;
            const size_t dst = ((size_t)b * S_cap + pos) * row;
            memcpy((unsigned char *)k_cache + dst * es, (const unsigned char *)k_rows + src * es,
                   row * es);
            memcpy((unsigned char *)v_cache + dst * es, (const unsigned char *)v_rows + src * es,
                   row * es);
            for (size_t i = 0; i < row; ++i) {
                const double x = widen(k_rows, dtype, src + i);
                if (!isfinite(x)) bad = 1;
                k2[(size_t)b * row + i] += x * x;
            }
        }
    }
    return bad ? -2 : 0;
}

/* Score from the gathered sums: s[b,kv,c] = sqrt(K2[b,kv,c]) *
 * sum_g sqrt(sum_i Q_w[b,i,kv*G+g,c]^2), the stage (a) formula with K2 given. */
int oracle_score_from_k2(int B, int Hq, int Hkv, int D, int dtype, const double *k2,
                         const void *q_obs, int W, double *scores) {
    if (!dims_ok(B, 1, Hq, Hkv, D, dtype) || W < 1) return -1;
    if (!k2 || !q_obs || !scores) return -1;
    const int G = Hq / Hkv;
    int bad = 0;
    for (int b = 0; b < B; ++b)
        for (int kv = 0; kv < Hkv; ++kv)
            for (int c = 0; c < D; ++c) {
                const double K2 = k2[((size_t)b * Hkv + kv) * D + c];
                if (!isfinite(K2) || K2 < 0.0) bad = 1;
                double qsum = 0.0;
                for (int g = 0; g < G; ++g) {
                    double Q2 = 0.0;
                    for (int i = 0; i < W; ++i) {
                        const double q =
                            widen(q_obs, dtype, (((size_t)b * W + i) * Hq + kv * G + g) * D + c);
                        if (!isfinite(q)) bad = 1;
                        Q2 += q * q;
                    }
                    qsum += sqrt(Q2);
                }
                scores[((size_t)b * Hkv + kv) * D + c] = sqrt(K2) * qsum;
            }
    return bad ? -2 : 0;
}

/* The other reading of the grouped-query aggregation, kept for reports only:
 * the Frobenius norm of the stacked (G*W) x len block, i.e.
 * sqrt(K2) * sqrt(sum_g Q2[g]).  Not used by the pruning path. */
int oracle_score_rss(int B, int S_cap, int Hq, int Hkv, int D, int dtype,
                     const void *k_cache, const int32_t *seq_lens, const void *q_obs,
                     int W, double *scores) {
    if (!dims_ok(B, S_cap, Hq, Hkv, D, dtype) || W < 1) return -1;
    if (!k_cache || !seq_lens || !q_obs || !scores) return -1;
    if (!lens_ok(B, S_cap, seq_lens)) return -1;
    const int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int kv = 0; kv < Hkv; ++kv) {
            for (int c = 0; c < D; ++c) {
                double K2 = 0.0;
                for (int t = 0; t < seq_lens[b]; ++t) {
                    const double x = widen(k_cache, dtype, (((size_t)b * S_cap + t) * Hkv + kv) * D + c);
                    K2 += x * x;
                }
                double Q2 = 0.0;
                for (int g = 0; g < G; ++g)
                    for (int i = 0; i < W; ++i) {
                        const double q = widen(q_obs, dtype, (((size_t)b * W + i) * Hq + kv * G + g) * D + c);
                        Q2 += q * q;
                    }
                scores[((size_t)b * Hkv + kv) * D + c] = sqrt(K2) * sqrt(Q2);
            }
        }
    }
    return 0;
}

/* Stage (a) by its definition, for small inputs: materialise, per channel and
 * query head, the W x len matrix M = Q_w[:,c] K[:,c]^T and take ||M||_F; sum
 * over the query heads of the group.  No closed form is used here. */
int oracle_score_materialised(int B, int S_cap, int Hq, int Hkv, int D, int dtype,
                              const void *k_cache, const int32_t *seq_lens,
                              const void *q_obs, int W, double *scores) {
    if (!dims_ok(B, S_cap, Hq, Hkv, D, dtype) || W < 1) return -1;
    if (!k_cache || !seq_lens || !q_obs || !scores) return -1;
    if (!lens_ok(B, S_cap, seq_lens)) return -1;
    const int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int kv = 0; kv < Hkv; ++kv) {
            const int len = seq_lens[b];
            double *M = (double *)malloc((size_t)W * len * sizeof(double));
            for (int c = 0; c < D; ++c) {
                double total = 0.0;
                for (int g = 0; g < G; ++g) {
                    const int h = kv * G + g;
                    for (int i = 0; i < W; ++i)
                        for (int t = 0; t < len; ++t)
                            M[(size_t)i * len + t] =
                                widen(q_obs, dtype, (((size_t)b * W + i) * Hq + h) * D + c) *
                                widen(k_cache, dtype, (((size_t)b * S_cap + t) * Hkv + kv) * D + c);
                    double fro2 = 0.0;
                    for (size_t e = 0; e < (size_t)W * len; ++e) fro2 += M[e] * M[e];
                    total += sqrt(fro2);
                }
                scores[((size_t)b * Hkv + kv) * D + c] = total;
            }
            free(M);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Stage (b): keep the `keep` most relevant channels per (b, kv head).
 * Order: score descending, then channel index ascending (a total order, so
 * ties at the cutoff are resolved towards the lower channel).  The kept
 * channels are written in ascending channel order.
 * near_tie[b,kv] = keep < D and s_(keep) - s_(keep+1) <= 1e-5 * s_(keep),
 * where s_(r) is the r-th score in that order (1-based).
 * ------------------------------------------------------------------------- */
typedef struct {
    double s;
    int c;
} scored_channel;

static int by_score_desc_then_channel(const void *pa, const void *pb) {
    const scored_channel *a = (const scored_channel *)pa;
    const scored_channel *b = (const scored_channel *)pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->c > b->c) - (a->c < b->c);
}

int oracle_select(int B, int Hkv, int D, const double *scores, int keep,
                  int32_t *kept_idx, int32_t *near_tie) {
    if (B < 1 || Hkv < 1 || D < 1 || keep < 1 || keep > D) return -1;
    if (!scores || !kept_idx) return -1;
    for (size_t i = 0; i < (size_t)B * Hkv * D; ++i)
        if (!isfinite(scores[i])) return -2;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int kv = 0; kv < Hkv; ++kv) {
            const double *s = scores + ((size_t)b * Hkv + kv) * D;
            scored_channel *order = (scored_channel *)malloc((size_t)D * sizeof *order);
            unsigned char *kept = (unsigned char *)calloc((size_t)D, 1);
            for (int c = 0; c < D; ++c) {
                order[c].s = s[c];
                order[c].c = c;
            }
            qsort(order, (size_t)D, sizeof *order, by_score_desc_then_channel);
            for (int r = 0; r < keep; ++r) kept[order[r].c] = 1;
            int32_t *out = kept_idx + ((size_t)b * Hkv + kv) * keep;
            int j = 0;
            for (int c = 0; c < D; ++c)
                if (kept[c]) out[j++] = c;
            if (near_tie) {
                int flag = 0;
                if (keep < D) {
                    const double hi = order[keep - 1].s, lo = order[keep].s;
                    flag = (hi - lo) <= 1e-5 * hi;
                }
                near_tie[(size_t)b * Hkv + kv] = flag;
            }
            free(kept);
            free(order);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Stage (c): the thinner key cache.
 *   K_thin[b,t,kv,j] = K[b,t,kv, kept_idx[b,kv,j]]   for t < len_b
 * A copy of the stored bytes; rows t >= len_b of K_thin are left untouched.
 * Layout: K_thin [B,S_cap,Hkv,keep], dense.
 * ------------------------------------------------------------------------- */
int oracle_compact(int B, int S_cap, int Hkv, int D, int dtype, const void *k_cache,
                   const int32_t *seq_lens, const int32_t *kept_idx, int keep,
                   void *k_thin) {
    if (!dims_ok(B, S_cap, Hkv, Hkv, D, dtype) || keep < 1 || keep > D) return -1;
    if (!k_cache || !seq_lens || !kept_idx || !k_thin) return -1;
    if (!lens_ok(B, S_cap, seq_lens)) return -1;
    for (size_t i = 0; i < (size_t)B * Hkv * keep; ++i)
        if (kept_idx[i] < 0 || kept_idx[i] >= D) return -1;
    const size_t es = elem_size(dtype);
    const unsigned char *src = (const unsigned char *)k_cache;
    unsigned char *dst = (unsigned char *)k_thin;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int kv = 0; kv < Hkv; ++kv) {
            const int32_t *idx = kept_idx + ((size_t)b * Hkv + kv) * keep;
            for (int t = 0; t < seq_lens[b]; ++t) {
                const size_t srow = (((size_t)b * S_cap + t) * Hkv + kv) * D;
                const size_t drow = (((size_t)b * S_cap + t) * Hkv + kv) * keep;
                for (int j = 0; j < keep; ++j)
                    memcpy(dst + (drow + j) * es, src + (srow + idx[j]) * es, es);
            }
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Decode-time append (the step after the path): inference continues on the
 * pruned cache ("ThinK: Thinner Key Cache by Query-Driven Pruning", Method
 * details -> Technical framework, last step), so a generated token's key is
 * stored pruned with the same kept set as the cached keys, and its value in
 * full.  For every b with len_b < S_cap:
 *   K_thin[b,len_b,kv,j] = k_new[b,kv,kept_idx[b,kv,j]]
 *   V[b,len_b,kv,:]      = v_new[b,kv,:]
 *   len_b               += 1
 * A sequence already at capacity is left as it is; an empty one (len_b = 0)
 * gets row 0.  Byte copies.
 * Layouts: k_new, v_new [B,Hkv,D]; K_thin [B,S_cap,Hkv,keep]; V [B,S_cap,Hkv,D].
 * ------------------------------------------------------------------------- */
int oracle_append(int B, int S_cap, int Hkv, int D, int dtype, const void *k_new,
                  const void *v_new, int32_t *seq_lens, const int32_t *kept_idx, int keep,
                  void *k_thin, void *v_cache) {
    if (!dims_ok(B, S_cap, Hkv, Hkv, D, dtype) || keep < 1 || keep > D) return -1;
    if (!k_new || !v_new || !seq_lens || !kept_idx || !k_thin || !v_cache) return -1;
    if (!lens_ok_or_empty(B, S_cap, seq_lens)) return -1;
    for (size_t i = 0; i < (size_t)B * Hkv * keep; ++i)
        if (kept_idx[i] < 0 || kept_idx[i] >= D) return -1;
    const size_t es = elem_size(dtype);
    const unsigned char *kn = (const unsigned char *)k_new;
    const unsigned char *vn = (const unsigned char *)v_new;
    unsigned char *kt = (unsigned char *)k_thin;
    unsigned char *vc = (unsigned char *)v_cache;
    for (int b = 0; b < B; ++b) {
        const int t = seq_lens[b];
        if (t >= S_cap) continue;
        for (int kv = 0; kv < Hkv; ++kv) {
            const int32_t *idx = kept_idx + ((size_t)b * Hkv + kv) * keep;
            const size_t src = ((size_t)b * Hkv + kv) * D;
            const size_t krow = (((size_t)b * S_cap + t) * Hkv + kv) * keep;
            const size_t vrow = (((size_t)b * S_cap + t) * Hkv + kv) * D;
            for (int j = 0; j < keep; ++j)
                memcpy(kt + (krow + j) * es, kn + (src + idx[j]) * es, es);
            memcpy(vc + vrow * es, vn + src * es, (size_t)D * es);
        }
        seq_lens[b] = t + 1;
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Stage (d): decode attention on the pruned key cache, per (b, q head h),
 * with kv = h / G:
 *   qS[j] = q[b,h,kept_idx[b,kv,j]]
 *   l_t   = scale * sum_j qS[j] * K_thin[b,t,kv,j]      (t < len_b)
 *   p     = softmax(l)   (max-subtracted)
 *   o     = sum_t p_t V[b,t,kv,:]
 * V is not pruned.  Output fp64 [B,Hq,D].
 * ------------------------------------------------------------------------- */
static void attend_one(const double *qsel, const void *keys, size_t key_row0, size_t key_stride,
                       int kdim, const void *v_cache, size_t v_row0, size_t v_stride, int D,
                       int dtype, int len, double scale, double *logits, double *out) {
    for (int t = 0; t < len; ++t) {
        double acc = 0.0;
        const size_t kr = key_row0 + (size_t)t * key_stride;
        for (int j = 0; j < kdim; ++j) acc += qsel[j] * widen(keys, dtype, kr + j);
        logits[t] = scale * acc;
    }
    double m = logits[0];
    for (int t = 1; t < len; ++t)
        if (logits[t] > m) m = logits[t];
    double denom = 0.0;
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    for (int t = 0; t < len; ++t) {
        const double p = exp(logits[t] - m);
        denom += p;
        const size_t vr = v_row0 + (size_t)t * v_stride;
        for (int d = 0; d < D; ++d) out[d] += p * widen(v_cache, dtype, vr + d);
    }
    for (int d = 0; d < D; ++d) out[d] /= denom;
}

int oracle_decode(int B, int S_cap, int Hq, int Hkv, int D, int dtype, const void *q,
                  const void *k_thin, const void *v_cache, const int32_t *seq_lens,
                  const int32_t *kept_idx, int keep, double scale, double *out) {
    if (!dims_ok(B, S_cap, Hq, Hkv, D, dtype) || keep < 1 || keep > D) return -1;
    if (!q || !k_thin || !v_cache || !seq_lens || !kept_idx || !out) return -1;
    if (!lens_ok(B, S_cap, seq_lens)) return -1;
    for (size_t i = 0; i < (size_t)B * Hkv * keep; ++i)
        if (kept_idx[i] < 0 || kept_idx[i] >= D) return -1;
    const int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hq; ++h) {
            const int kv = h / G;
            const int len = seq_lens[b];
            const int32_t *idx = kept_idx + ((size_t)b * Hkv + kv) * keep;
            double *qsel = (double *)malloc((size_t)keep * sizeof(double));
            double *logits = (double *)malloc((size_t)len * sizeof(double));
            for (int j = 0; j < keep; ++j) qsel[j] = widen(q, dtype, ((size_t)b * Hq + h) * D + idx[j]);
            attend_one(qsel, k_thin, (((size_t)b * S_cap) * Hkv + kv) * keep, (size_t)Hkv * keep, keep,
                       v_cache, (((size_t)b * S_cap) * Hkv + kv) * D, (size_t)Hkv * D, D, dtype, len,
                       scale, logits, out + ((size_t)b * Hq + h) * D);
            free(logits);
            free(qsel);
        }
    }
    return 0;
}

/* Unpruned decode attention over the original key cache: the same loops with
 * every channel kept, so at keep == D the pruned path must agree bit for bit. */
int oracle_full_attn(int B, int S_cap, int Hq, int Hkv, int D, int dtype, const void *q,
                     const void *k_cache, const void *v_cache, const int32_t *seq_lens,
                     double scale, double *out) {
    if (!dims_ok(B, S_cap, Hq, Hkv, D, dtype)) return -1;
    if (!q || !k_cache || !v_cache || !seq_lens || !out) return -1;
    if (!lens_ok(B, S_cap, seq_lens)) return -1;
    const int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(static)
    for (int b = 0; b < B; ++b) {
        for (int h = 0; h < Hq; ++h) {
            const int kv = h / G;
            const int len = seq_lens[b];
            double *qsel = (double *)malloc((size_t)D * sizeof(double));
            double *logits = (double *)malloc((size_t)len * sizeof(double));
            for (int c = 0; c < D; ++c) qsel[c] = widen(q, dtype, ((size_t)b * Hq + h) * D + c);
            attend_one(qsel, k_cache, (((size_t)b * S_cap) * Hkv + kv) * D, (size_t)Hkv * D, D,
                       v_cache, (((size_t)b * S_cap) * Hkv + kv) * D, (size_t)Hkv * D, D, dtype, len,
                       scale, logits, out + ((size_t)b * Hq + h) * D);
            free(logits);
            free(qsel);
        }
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * The pruning objective (original abstract: keep the loss of attention weight
 * small), for one head, fp64 inputs Qw [W,D] and K [L,D] row-major:
 *   R(S) = || Qw K^T - Qw[:,S] K[:,S]^T ||_F = || sum_{c not in S} Qw[:,c] K[:,c]^T ||_F
 * `in_set[c]` is 1 for kept channels.
 * ------------------------------------------------------------------------- */
double oracle_residual_materialised(int W, int L, int D, const double *Qw, const double *K,
                                    const int32_t *in_set) {
    double fro2 = 0.0;
    for (int i = 0; i < W; ++i)
        for (int t = 0; t < L; ++t) {
            double e = 0.0;
            for (int c = 0; c < D; ++c)
                if (!in_set[c]) e += Qw[(size_t)i * D + c] * K[(size_t)t * D + c];
            fro2 += e * e;
        }
    return sqrt(fro2);
}

/* The same residual through the Gram matrices:
 *   R(S)^2 = sum_{a,b not in S} (q_a . q_b) (k_a . k_b)                       */
double oracle_residual_gram(int W, int L, int D, const double *Qw, const double *K,
                            const int32_t *in_set) {
    double r2 = 0.0;
    for (int a = 0; a < D; ++a) {
        if (in_set[a]) continue;
        for (int b = 0; b < D; ++b) {
            if (in_set[b]) continue;
            double qq = 0.0, kk = 0.0;
            for (int i = 0; i < W; ++i) qq += Qw[(size_t)i * D + a] * Qw[(size_t)i * D + b];
            for (int t = 0; t < L; ++t) kk += K[(size_t)t * D + a] * K[(size_t)t * D + b];
            r2 += qq * kk;
        }
    }
    return r2 > 0.0 ? sqrt(r2) : 0.0;
}

/* Exhaustive search over every keep-subset of D <= 20 channels for the
 * smallest residual.  Writes the optimum R_opt and its set (flags), and, for
 * a given candidate set, how many subsets have a strictly smaller residual
 * (its 0-based rank).  Returns the number of subsets visited, or -1. */
long oracle_bruteforce(int W, int L, int D, const double *Qw, const double *K, int keep,
                       const int32_t *candidate, double *r_opt, int32_t *opt_set,
                       double *r_candidate, long *candidate_rank) {
    if (D < 1 || D > 20 || keep < 0 || keep > D || W < 1 || L < 1) return -1;
    double *H = (double *)malloc((size_t)D * D * sizeof(double));
    for (int a = 0; a < D; ++a)
        for (int b = 0; b < D; ++b) {
            double qq = 0.0, kk = 0.0;
            for (int i = 0; i < W; ++i) qq += Qw[(size_t)i * D + a] * Qw[(size_t)i * D + b];
            for (int t = 0; t < L; ++t) kk += K[(size_t)t * D + a] * K[(size_t)t * D + b];
            H[(size_t)a * D + b] = qq * kk;
        }
    /* residual of a kept-set bitmask through H */
#define RESID2(mask, out)                                                      \
    do {                                                                       \
        double r2_ = 0.0;                                                      \
        for (int a_ = 0; a_ < D; ++a_) {                                       \
            if ((mask) >> a_ & 1u) continue;                                   \
            for (int b_ = 0; b_ < D; ++b_)                                     \
                if (!((mask) >> b_ & 1u)) r2_ += H[(size_t)a_ * D + b_];       \
        }                                                                      \
        (out) = r2_ > 0.0 ? sqrt(r2_) : 0.0;                                   \
    } while (0)
    unsigned cand_mask = 0;
    if (candidate)
        for (int c = 0; c < D; ++c)
            if (candidate[c]) cand_mask |= 1u << c;
    double cand_r = 0.0;
    if (candidate) RESID2(cand_mask, cand_r);
    double best = INFINITY;
    unsigned best_mask = 0;
    long visited = 0, below = 0;
    for (unsigned mask = 0; mask < (1u << D); ++mask) {
        if (__builtin_popcount(mask) != keep) continue;
        double r;
        RESID2(mask, r);
        ++visited;
        if (r < best) {
            best = r;
            best_mask = mask;
        }
        if (candidate && r < cand_r) ++below;
    }
#undef RESID2
    free(H);
    if (r_opt) *r_opt = best;
    if (opt_set)
        for (int c = 0; c < D; ++c) opt_set[c] = (int32_t)(best_mask >> c & 1u);
    if (r_candidate) *r_candidate = cand_r;
    if (candidate_rank) *candidate_rank = below;
    return visited;
}
