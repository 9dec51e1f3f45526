/*
 * Graph Machine sparse-layer oracle: plain, slow, single-threaded C in double.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker the GPU path is held
 * against.  Only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark load it; the product library never links, calls or includes it,
 * and it includes nothing of the product library.
 *
 * Sources (the pages on the Graph Machine, arXiv 2609.02881):
 *   [ai.info]  "Graph Machine: Towards Better Pretraining via Edges",
 *              ai.info AI summary: Key Contributions 2-3, Methodology in
 *              Plain English, Main Findings ("KV access reduction").
 *   [rit.work] "Graph Machine" news article, section "Что сделали"
 *              (what was done): edges, referral, hard selection, gradients.
 *
 * What is computed (readings of the pages are named where they are taken):
 *   SER  A' = Sparsify_s1(A1 A2): two-hop paths i -> j -> m through leg 1
 *        (row i of A1) and leg 2 (row j of A2), path weight w1*w2, paths to
 *        the same target merged by summing, top-s1 kept ([ai.info] Key
 *        Contributions 3; Methodology, referral paragraph).
 *   SEA  softmax over the edge slots of scale*q.k + ln w, a product of a node
 *        expert and an edge expert, then the weighted sum of the gathered
 *        values ([ai.info] Key Contributions 3; Methodology, second job).
 *   Backward of both through the soft weights only: indices carry no
 *        gradient, and only retained edges receive one ([rit.work] what was
 *        done; [ai.info] Methodology: gradients reach the kept weights alone).
 *   Leg construction: a token's stored edges mixed into a leg and
 *        sparsified ([ai.info] Methodology, referral paragraph; the mixing
 *        itself is a reading, stated at the function), forward and backward.
 *   Refresh edges: the top positions of a dense attention layer
 *        ([ai.info] Methodology, referral paragraph; the ranking is a
 *        reading, stated at the function).
 *
 * Layouts (row-major): q, o, dout, dq [B,n,hq,d]; k, v, dk, dv [B,n,hkv,d];
 * edges idx [B,n,hkv,s] int32 and w [B,n,hkv,s].  Query head hq reads KV head
 * hq / (hq_count / hkv) (grouped heads, reading: edges are per KV head, since
 * the pages count retrieved tokens for each KV head).  Every floating value is double here;
 * fp32 and bf16 inputs are exact in double.
 *
 * Return value of every function: 0, or a negative code when an input breaks
 * the edge contract (index outside [0, i]), which is a caller error.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_ERR_INDEX (-1)
#define ORACLE_ERR_ARGS  (-2)
#define ORACLE_MAX_CAND  4096

static size_t row(int b, int i, int h, int n, int hkv) {
    return ((size_t)b * n + i) * hkv + h;
}

/*
 * SER forward ([ai.info] Key Contributions 3: A' = Sparsify_s1(A1 A2), the
 * s2*s3 candidates at most cut back to s1; Methodology: the first leg's
 * indices select rows of the second leg, whose indices and weights turn each
 * two-hop path into a one-hop edge, and a hard top-s keeps the budget;
 * [rit.work]: paths are merged and the heaviest addresses kept).
 *
 * For each unit (b, i, h):
 *   for a in leg-1 slots (order a = 0..s2-1), j = idx1[i,a], x = w1[i,a]
 *     for c in leg-2 slots (order c = 0..s3-1), m = idx2[j,c], y = w2[j,c]
 *       acc[m] += x * y                   (merge duplicate targets by sum)
 *   key[m] = acc[m] rounded to fp32 (the stored edge-weight type)
 *   keep the s1 targets of largest positive key; equal keys: lower index
 *   first.  Output slot r holds the r-th kept (m, key); unused slots hold
 *   (0, 0): position 0 is the padding token that absorbs missing edges
 *   ([ai.info] Methodology, padding token at the start of each sequence).
 * Zero-weight candidates are not edges (a sparse matrix has no zero
 * entries), so they never fill a slot.
 * w_out_exact (may be NULL) receives the unrounded double sum of each kept
 * target, 0 for padding.
 */
int oracle_ser_forward(int B, int n, int hkv,
                       const int32_t* idx1, const double* w1, int s2,
                       const int32_t* idx2, const double* w2, int s3,
                       int s1, int32_t* idx_out, float* w_out,
                       double* w_out_exact) {
    if (B < 0 || n < 0 || hkv < 0 || s1 < 1 || s2 < 1 || s3 < 1 ||
        s2 * s3 > ORACLE_MAX_CAND)
        return ORACLE_ERR_ARGS;
    int32_t cand_m[ORACLE_MAX_CAND];
    double cand_acc[ORACLE_MAX_CAND];
    float cand_key[ORACLE_MAX_CAND];
    int taken[ORACLE_MAX_CAND];
    for (int b = 0; b < B; ++b)
    for (int i = 0; i < n; ++i)
    for (int h = 0; h < hkv; ++h) {
        size_t r1 = row(b, i, h, n, hkv);
        int ncand = 0;
        for (int a = 0; a < s2; ++a) {
            int j = idx1[r1 * s2 + a];
            double x = w1[r1 * s2 + a];
            if (j < 0 || j > i) return ORACLE_ERR_INDEX;
            size_t r2 = row(b, j, h, n, hkv);
            for (int c = 0; c < s3; ++c) {
                int m = idx2[r2 * s3 + c];
                double y = w2[r2 * s3 + c];
                if (m < 0 || m > j) return ORACLE_ERR_INDEX;
                int found = -1;
                for (int e = 0; e < ncand; ++e)
                    if (cand_m[e] == m) { found = e; break; }
                if (found < 0) {
                    found = ncand++;
                    cand_m[found] = m;
                    cand_acc[found] = 0.0;
                }
                cand_acc[found] += x * y;
            }
        }
        for (int e = 0; e < ncand; ++e) {
            cand_key[e] = (float)cand_acc[e];
            taken[e] = 0;
        }
        for (int slot = 0; slot < s1; ++slot) {
            int best = -1;
            for (int e = 0; e < ncand; ++e) {
                if (taken[e] || !(cand_key[e] > 0.0f)) continue;
                if (best < 0 || cand_key[e] > cand_key[best] ||
                    (cand_key[e] == cand_key[best] && cand_m[e] < cand_m[best]))
                    best = e;
            }
            size_t o = r1 * s1 + slot;
            if (best < 0) {
                idx_out[o] = 0;
                w_out[o] = 0.0f;
                if (w_out_exact) w_out_exact[o] = 0.0;
            } else {
                taken[best] = 1;
                idx_out[o] = cand_m[best];
                w_out[o] = cand_key[best];
                if (w_out_exact) w_out_exact[o] = cand_acc[best];
            }
        }
    }
    return 0;
}

/*
 * SEA forward ([ai.info] Key Contributions 3: edge indices select which
 * positions supply keys and values; node factor = scaled query-key score,
 * edge factor = log edge weight, combined as a product of experts;
 * Methodology: RoPE is omitted; [rit.work]: the query-key match is combined
 * with the edge weight).
 *
 * For each unit (b, i, h) and each query head hq of KV head h, over the slots
 * t with w_t > 0 (a zero weight is log 0 = -inf, i.e. no expert mass):
 *   l_t = scale * sum_c q[hq,c] k[idx_t,h,c] + ln w_t
 *   p_t = exp(l_t - max l) / sum_u exp(l_u - max l)
 *   o[hq,c] = sum_t p_t v[idx_t,h,c]
 * A unit with no live slot outputs 0.  p_out (may be NULL) receives p_t per
 * (b, i, query head, slot), 0 for dead slots.  kv_rows (may be NULL)
 * receives the number of (unit, slot) key/value rows read, the access count
 * behind the "KV access reduction" finding.
 */
int oracle_sea_forward(int B, int n, int hq, int hkv, int d, double scale,
                       const double* q, const double* k, const double* v,
                       const int32_t* idx, const double* w, int s,
                       double* o, double* p_out, long long* kv_rows) {
    if (hkv <= 0 || hq % hkv != 0 || s < 1 || d < 1) return ORACLE_ERR_ARGS;
    int G = hq / hkv;
    long long rows_read = 0;
    double l[ORACLE_MAX_CAND];
    if (s > ORACLE_MAX_CAND) return ORACLE_ERR_ARGS;
    for (int b = 0; b < B; ++b)
    for (int i = 0; i < n; ++i)
    for (int h = 0; h < hkv; ++h) {
        size_t r = row(b, i, h, n, hkv);
        for (int t = 0; t < s; ++t) {
            int j = idx[r * s + t];
            if (j < 0 || j > i) return ORACLE_ERR_INDEX;
            if (w[r * s + t] > 0.0) rows_read++;
        }
        for (int g = 0; g < G; ++g) {
            int head = h * G + g;
            const double* qv = q + (((size_t)b * n + i) * hq + head) * d;
            double* ov = o + (((size_t)b * n + i) * hq + head) * d;
            double* pv = p_out ? p_out + (((size_t)b * n + i) * hq + head) * s : NULL;
            for (int c = 0; c < d; ++c) ov[c] = 0.0;
            if (pv)
                for (int t = 0; t < s; ++t) pv[t] = 0.0;
            double mx = -INFINITY;
            int live = 0;
            for (int t = 0; t < s; ++t) {
                double wt = w[r * s + t];
                if (!(wt > 0.0)) continue;
                const double* kv = k + row(b, idx[r * s + t], h, n, hkv) * d;
                double dot = 0.0;
                for (int c = 0; c < d; ++c) dot += qv[c] * kv[c];
                l[t] = scale * dot + log(wt);
                if (l[t] > mx) mx = l[t];
                live++;
            }
            if (!live) continue;
            double z = 0.0;
            for (int t = 0; t < s; ++t)
                if (w[r * s + t] > 0.0) z += exp(l[t] - mx);
            for (int t = 0; t < s; ++t) {
                if (!(w[r * s + t] > 0.0)) continue;
                double p = exp(l[t] - mx) / z;
                if (pv) pv[t] = p;
                const double* vv = v + row(b, idx[r * s + t], h, n, hkv) * d;
                for (int c = 0; c < d; ++c) ov[c] += p * vv[c];
            }
        }
    }
    if (kv_rows) *kv_rows = rows_read;
    return 0;
}

/*
 * SEA backward: the chain rule through the forward above, with indices held
 * fixed ([rit.work]: indices are discrete and get no gradient, training goes
 * through the soft edge weights).
 *   g_t   = dout[hq] . v[idx_t]            gbar = sum_t p_t g_t
 *   dl_t  = p_t (g_t - gbar)               (softmax backward)
 *   dq[hq]      = scale sum_t dl_t k[idx_t]
 *   dk[idx_t]  += scale dl_t q[hq]          (scatter to the source row)
 *   dv[idx_t]  += p_t dout[hq]
 *   dw_t       += dl_t / w_t                (d ln w / d w), summed over the
 *                                           query heads that share the edge
 * Slots with w_t = 0 are padding: they neither receive nor pass gradient.
 * All outputs are overwritten.
 */
int oracle_sea_backward(int B, int n, int hq, int hkv, int d, double scale,
                        const double* q, const double* k, const double* v,
                        const int32_t* idx, const double* w, int s,
                        const double* dout, double* dq, double* dk, double* dv,
                        double* dw) {
    if (hkv <= 0 || hq % hkv != 0 || s < 1 || d < 1 || s > ORACLE_MAX_CAND)
        return ORACLE_ERR_ARGS;
    int G = hq / hkv;
    size_t nq = (size_t)B * n * hq * d, nk = (size_t)B * n * hkv * d;
    size_t ne = (size_t)B * n * hkv * s;
    memset(dq, 0, nq * sizeof(double));
    memset(dk, 0, nk * sizeof(double));
    memset(dv, 0, nk * sizeof(double));
    memset(dw, 0, ne * sizeof(double));
    double l[ORACLE_MAX_CAND], p[ORACLE_MAX_CAND], gt[ORACLE_MAX_CAND];
    for (int b = 0; b < B; ++b)
    for (int i = 0; i < n; ++i)
    for (int h = 0; h < hkv; ++h) {
        size_t r = row(b, i, h, n, hkv);
        for (int t = 0; t < s; ++t) {
            int j = idx[r * s + t];
            if (j < 0 || j > i) return ORACLE_ERR_INDEX;
        }
        for (int g = 0; g < G; ++g) {
            int head = h * G + g;
            size_t qoff = (((size_t)b * n + i) * hq + head) * d;
            const double* qv = q + qoff;
            const double* dov = dout + qoff;
            double* dqv = dq + qoff;
            double mx = -INFINITY;
            int live = 0;
            for (int t = 0; t < s; ++t) {
                double wt = w[r * s + t];
                if (!(wt > 0.0)) continue;
                const double* kv = k + row(b, idx[r * s + t], h, n, hkv) * d;
                double dot = 0.0;
                for (int c = 0; c < d; ++c) dot += qv[c] * kv[c];
                l[t] = scale * dot + log(wt);
                if (l[t] > mx) mx = l[t];
                live++;
            }
            if (!live) continue;
            double z = 0.0;
            for (int t = 0; t < s; ++t)
                if (w[r * s + t] > 0.0) z += exp(l[t] - mx);
            double gbar = 0.0;
            for (int t = 0; t < s; ++t) {
                if (!(w[r * s + t] > 0.0)) continue;
                p[t] = exp(l[t] - mx) / z;
                const double* vv = v + row(b, idx[r * s + t], h, n, hkv) * d;
                double dot = 0.0;
                for (int c = 0; c < d; ++c) dot += dov[c] * vv[c];
                gt[t] = dot;
                gbar += p[t] * gt[t];
            }
            for (int t = 0; t < s; ++t) {
                double wt = w[r * s + t];
                if (!(wt > 0.0)) continue;
                double dl = p[t] * (gt[t] - gbar);
                size_t src = row(b, idx[r * s + t], h, n, hkv) * d;
                const double* kv = k + src;
                for (int c = 0; c < d; ++c) {
                    dqv[c] += scale * dl * kv[c];
                    dk[src + c] += scale * dl * qv[c];
                    dv[src + c] += p[t] * dov[c];
                }
                dw[r * s + t] += dl / wt;
            }
        }
    }
    return 0;
}

/*
 * SER backward: the chain rule through the forward's merge, with the
 * selection (the retained slots of A') held fixed ([ai.info] Methodology:
 * gradients reach the kept weights alone; [rit.work]: hard selection keeps
 * sparsity, only the kept variants get gradients).
 * For each unit (b, i, h), each path (a, c) with x = w1[i,a] > 0 and
 * y = w2[j,c] > 0 (j = idx1[i,a], m = idx2[j,c]) and each retained slot t of
 * A'[i] (w_out_t > 0) whose index equals m:
 *   dw1[i,a] += dw_out_t * y       dw2[j,c] += dw_out_t * x
 * (d(x y)/dx = y, d(x y)/dy = x; the merged weight is a plain sum.)
 * dw1 and dw2 may be the same array (A' = Sparsify(A A)): both
 * contributions then land in it.  Both outputs are overwritten first.
 */
int oracle_ser_backward(int B, int n, int hkv,
                        const int32_t* idx1, const double* w1, int s2,
                        const int32_t* idx2, const double* w2, int s3,
                        const int32_t* idx_out, const double* w_out, int s1,
                        const double* dw_out, double* dw1, double* dw2) {
    if (B < 0 || n < 0 || hkv < 0 || s1 < 1 || s2 < 1 || s3 < 1)
        return ORACLE_ERR_ARGS;
    memset(dw1, 0, (size_t)B * n * hkv * s2 * sizeof(double));
    memset(dw2, 0, (size_t)B * n * hkv * s3 * sizeof(double));
    for (int b = 0; b < B; ++b)
    for (int i = 0; i < n; ++i)
    for (int h = 0; h < hkv; ++h) {
        size_t r1 = row(b, i, h, n, hkv);
        for (int a = 0; a < s2; ++a) {
            int j = idx1[r1 * s2 + a];
            double x = w1[r1 * s2 + a];
            if (j < 0 || j > i) return ORACLE_ERR_INDEX;
            if (!(x > 0.0)) continue;
            size_t r2 = row(b, j, h, n, hkv);
            for (int c = 0; c < s3; ++c) {
                int m = idx2[r2 * s3 + c];
                double y = w2[r2 * s3 + c];
                if (m < 0 || m > j) return ORACLE_ERR_INDEX;
                if (!(y > 0.0)) continue;
                for (int t = 0; t < s1; ++t) {
                    if (!(w_out[r1 * s1 + t] > 0.0)) continue;
                    if (idx_out[r1 * s1 + t] != m) continue;
                    double gt = dw_out[r1 * s1 + t];
                    dw1[r1 * s2 + a] += gt * y;
                    dw2[r2 * s3 + c] += gt * x;
                }
            }
        }
    }
    return 0;
}

/*
 * Leg construction ([ai.info] Methodology, referral paragraph: referral
 * first mixes the stored edges into pairs and sparsifies each leg, and only
 * then composes the legs).  The pages give no mixing formula; reading: a leg
 * is a non-negative mixture of a token's K stored edges with one mixing
 * weight per (KV head, stored slot), then the same sparsification as SER:
 * For each unit (b, i, h), over the stored slots k = 0..K-1 in order:
 *   m = idx[i,k];  acc[m] += alpha[h,k] * w[i,k]      (duplicates merged)
 *   key[m] = acc[m] rounded to fp32; keep the s largest positive keys, equal
 *   keys to the lower index; unused slots (0, 0).
 * Indices are copied, never read through, so only 0 <= idx <= i is asked.
 */
int oracle_leg_mix_forward(int B, int n, int hkv, const int32_t* idx, const double* w, int K,
                           const double* alpha, int s, int32_t* idx_out, float* w_out) {
    if (B < 0 || n < 0 || hkv < 0 || K < 1 || s < 1 || K > ORACLE_MAX_CAND)
        return ORACLE_ERR_ARGS;
    int32_t cand_m[ORACLE_MAX_CAND];
    double cand_acc[ORACLE_MAX_CAND];
    float cand_key[ORACLE_MAX_CAND];
    int taken[ORACLE_MAX_CAND];
    for (int b = 0; b < B; ++b)
    for (int i = 0; i < n; ++i)
    for (int h = 0; h < hkv; ++h) {
        size_t r = row(b, i, h, n, hkv);
        int ncand = 0;
        for (int k = 0; k < K; ++k) {
            int m = idx[r * K + k];
            if (m < 0 || m > i) return ORACLE_ERR_INDEX;
            int found = -1;
            for (int e = 0; e < ncand; ++e)
                if (cand_m[e] == m) { found = e; break; }
            if (found < 0) {
                found = ncand++;
                cand_m[found] = m;
                cand_acc[found] = 0.0;
            }
            cand_acc[found] += alpha[(size_t)h * K + k] * w[r * K + k];
        }
        for (int e = 0; e < ncand; ++e) {
            cand_key[e] = (float)cand_acc[e];
            taken[e] = 0;
        }
        for (int slot = 0; slot < s; ++slot) {
            int best = -1;
            for (int e = 0; e < ncand; ++e) {
                if (taken[e] || !(cand_key[e] > 0.0f)) continue;
                if (best < 0 || cand_key[e] > cand_key[best] ||
                    (cand_key[e] == cand_key[best] && cand_m[e] < cand_m[best]))
                    best = e;
            }
            size_t o = r * s + slot;
            if (best < 0) {
                idx_out[o] = 0;
                w_out[o] = 0.0f;
            } else {
                taken[best] = 1;
                idx_out[o] = cand_m[best];
                w_out[o] = cand_key[best];
            }
        }
    }
    return 0;
}

/*
 * Leg construction backward, with the selection (the retained leg slots)
 * held fixed, as for SER: for each unit and stored slot k with
 * alpha[h,k] > 0 and w[i,k] > 0, and each retained slot t of the leg
 * (w_out_t > 0) whose index equals idx[i,k]:
 *   dw[i,k] += dleg_t * alpha[h,k]        dalpha[h,k] += dleg_t * w[i,k]
 * (dalpha sums over every unit of the KV head).  Both outputs are
 * overwritten first.
 */
int oracle_leg_mix_backward(int B, int n, int hkv, const int32_t* idx, const double* w, int K,
                            const double* alpha, const int32_t* idx_out, const double* w_out,
                            int s, const double* dleg, double* dw, double* dalpha) {
    if (B < 0 || n < 0 || hkv < 0 || K < 1 || s < 1) return ORACLE_ERR_ARGS;
    memset(dw, 0, (size_t)B * n * hkv * K * sizeof(double));
    memset(dalpha, 0, (size_t)hkv * K * sizeof(double));
    for (int b = 0; b < B; ++b)
    for (int i = 0; i < n; ++i)
    for (int h = 0; h < hkv; ++h) {
        size_t r = row(b, i, h, n, hkv);
        for (int k = 0; k < K; ++k) {
            int m = idx[r * K + k];
            double a = alpha[(size_t)h * K + k], x = w[r * K + k];
            if (m < 0 || m > i) return ORACLE_ERR_INDEX;
            if (!(a > 0.0) || !(x > 0.0)) continue;
            for (int t = 0; t < s; ++t) {
                if (!(w_out[r * s + t] > 0.0) || idx_out[r * s + t] != m) continue;
                double g = dleg[r * s + t];
                dw[r * K + k] += g * a;
                dalpha[(size_t)h * K + k] += g * x;
            }
        }
    }
    return 0;
}

/*
 * Refresh edges from a dense attention layer ([ai.info] Methodology,
 * referral paragraph: optional refresh edges pull in the top-k positions of
 * the most recent dense-attention layer; Main Findings: refresh helps).  The
 * pages do not define the ranking; reading: per unit (b, i, h) over the
 * causal positions j <= i, the group-mean attention probability
 *   pbar_j = (1/G) sum_g softmax_j(scale * q[i, h*G+g] . k[j, h])
 * ranks the positions; keep the s largest (equal values to the lower index),
 * weight = pbar_j rounded to fp32; unused slots (0, 0).  lse[b, i, hq]
 * receives each query head's log-sum-exp of its scaled scores.
 */
int oracle_dense_refresh(int B, int n, int hq, int hkv, int d, double scale,
                         const double* q, const double* k, int s,
                         int32_t* idx_out, float* w_out, double* lse) {
    if (B < 0 || n < 0 || hkv <= 0 || hq % hkv != 0 || d < 1 || s < 1) return ORACLE_ERR_ARGS;
    int G = hq / hkv;
    double* sc = (double*)malloc((size_t)n * sizeof(double));
    double* pbar = (double*)malloc((size_t)n * sizeof(double));
    int* taken = (int*)malloc((size_t)n * sizeof(int));
    if (!sc || !pbar || !taken) { free(sc); free(pbar); free(taken); return ORACLE_ERR_ARGS; }
    for (int b = 0; b < B; ++b)
    for (int i = 0; i < n; ++i)
    for (int h = 0; h < hkv; ++h) {
        for (int j = 0; j <= i; ++j) pbar[j] = 0.0;
        for (int g = 0; g < G; ++g) {
            int head = h * G + g;
            const double* qv = q + (((size_t)b * n + i) * hq + head) * d;
            double mx = -INFINITY;
            for (int j = 0; j <= i; ++j) {
                const double* kv = k + row(b, j, h, n, hkv) * d;
                double dot = 0.0;
                for (int c = 0; c < d; ++c) dot += qv[c] * kv[c];
                sc[j] = scale * dot;
                if (sc[j] > mx) mx = sc[j];
            }
            double z = 0.0;
            for (int j = 0; j <= i; ++j) z += exp(sc[j] - mx);
            lse[((size_t)b * n + i) * hq + head] = mx + log(z);
            for (int j = 0; j <= i; ++j) pbar[j] += exp(sc[j] - mx) / z / G;
        }
        size_t r = row(b, i, h, n, hkv);
        for (int j = 0; j <= i; ++j) taken[j] = 0;
        for (int slot = 0; slot < s; ++slot) {
            int best = -1;
            for (int j = 0; j <= i; ++j) {
                if (taken[j] || !(pbar[j] > 0.0)) continue;
                if (best < 0 || pbar[j] > pbar[best]) best = j;   /* j ascending: ties keep the lower */
            }
            if (best < 0) {
                idx_out[r * s + slot] = 0;
                w_out[r * s + slot] = 0.0f;
            } else {
                taken[best] = 1;
                idx_out[r * s + slot] = best;
                w_out[r * s + slot] = (float)pbar[best];
            }
        }
    }
    free(sc); free(pbar); free(taken);
    return 0;
}
