/*
 * attn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU reference for causal scaled-dot-product
 * attention, its vector-Jacobian product and single-token decode, written in
 * double precision.  Only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg may load this library.  The product (the HIP library under
 * causal_self_attention_amd/) never links, loads or calls it, and the two share
 * no source.
 *
 * What is computed follows the riftco-transformer documentation pages:
 *   - "Architecture", section "Tensor conventions": contiguous row-major storage,
 *     scores laid out [B,H,Tq,Tk], key position t_k excluded when t_k > t_q
 *     (so the diagonal key is kept).
 *   - learn/neural_network page, section "Stable softmax and cross-entropy":
 *     softmax subtracts the row maximum before exponentiating; masked entries
 *     take no part in the row.
 *   - learn/neural_network page, section "Where attention is": the per-head
 *     operation is "scaled causal attention"; the scale is an explicit argument
 *     here (the usual value is 1/sqrt(d_head)).
 *   - "Execution Backends and the Python ABI", section "What the Metal slice
 *     does": the default path materialises the [T,T] probabilities and runs the
 *     VJP through them -- that is exactly what this file does, one head at a time.
 *   - same page, section "Incremental attention": paged decode resolves each
 *     logical position's K/V address through a per-request page table, with
 *     pools laid out [physical_page, H, page_offset, d_h].
 *   - ARCHITECTURE.md of the algo-v1-codepoint project, "config.py": grouped
 *     query attention needs num_query_heads % num_kv_heads == 0.  Query head h
 *     reads key/value head h / (Hq/Hkv) (contiguous groups); the pages only say
 *     "broadcast", so this grouping is a stated reading.
 *
 * All arithmetic is in double; inputs are double arrays (fp32 data converts
 * exactly).  No blocking, no online softmax, no fusion: the probability matrix
 * of one head is formed in full, then used.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Probabilities of one head: P[i*T + j] for j <= i, zero for j > i.
 * Also writes lse[i] = m_i + ln sum_j exp(s_ij - m_i) when lse != NULL.
 *   s_ij = scale * <q_i, k_j>     (j <= i only; j > i is excluded)
 *   m_i  = max_j s_ij
 *   P_ij = exp(s_ij - m_i) / sum_{j'<=i} exp(s_ij' - m_i)                     */
static void head_probabilities(const double* q, const double* k, int64_t T, int64_t D,
                               double scale, double* P, double* lse) {
    for (int64_t i = 0; i < T; ++i) {
        double* row = P + i * T;
        double m = -INFINITY;
        for (int64_t j = 0; j <= i; ++j) {
            double s = 0.0;
            for (int64_t c = 0; c < D; ++c) s += q[i * D + c] * k[j * D + c];
            s *= scale;
            row[j] = s;
            if (s > m) m = s;
        }
        double z = 0.0;
        for (int64_t j = 0; j <= i; ++j) {
            row[j] = exp(row[j] - m);
            z += row[j];
        }
        for (int64_t j = 0; j <= i; ++j) row[j] /= z;
        for (int64_t j = i + 1; j < T; ++j) row[j] = 0.0;
        if (lse) lse[i] = m + log(z);
    }
}

/* Forward.  q,o: [B,Hq,T,D]; k,v: [B,Hkv,T,D]; lse: [B,Hq,T] (natural log).
 * p_out, if not NULL, receives the full [B,Hq,T,T] probability tensor.
 * Returns 0, or -1 on an invalid shape or allocation failure.              */
int oracle_causal_fwd(const double* q, const double* k, const double* v,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t D, double scale,
                      double* o, double* lse, double* p_out) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || T <= 0 || D <= 0 || Hq % Hkv != 0) return -1;
    const int64_t G = Hq / Hkv;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * Hq; ++bh) {
        const int64_t b = bh / Hq, h = bh % Hq, g = h / G;
        const double* qh = q + (b * Hq + h) * T * D;
        const double* kg = k + (b * Hkv + g) * T * D;
        const double* vg = v + (b * Hkv + g) * T * D;
        double* oh = o + (b * Hq + h) * T * D;
        double* P = p_out ? p_out + (b * Hq + h) * T * T : (double*)malloc((size_t)(T * T) * sizeof(double));
        if (!P) { failed = 1; continue; }
        head_probabilities(qh, kg, T, D, scale, P, lse ? lse + (b * Hq + h) * T : NULL);
        /* O_i = sum_{j<=i} P_ij v_j */
        for (int64_t i = 0; i < T; ++i) {
            for (int64_t c = 0; c < D; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j <= i; ++j) acc += P[i * T + j] * vg[j * D + c];
                oh[i * D + c] = acc;
            }
        }
        if (!p_out) free(P);
    }
    return failed ? -1 : 0;
}

/* Vector-Jacobian product of the forward for the loss L = sum(dout * O).
 * dq: [B,Hq,T,D]; dk, dv: [B,Hkv,T,D] (summed over the query heads that share
 * each key/value head -- a broadcast input's gradient is reduced back to its own
 * shape).  With dS_ij = P_ij (dP_ij - Delta_i), dP_ij = <dO_i, v_j>,
 * Delta_i = sum_j P_ij dP_ij (the chain rule through the row normalisation):
 *   dQ_i = scale * sum_{j<=i} dS_ij k_j
 *   dK_j = scale * sum_h sum_{i>=j} dS_ij q_i
 *   dV_j =         sum_h sum_{i>=j} P_ij dO_i
 * One query head at a time (in parallel over heads): its P and dS [T,T], its dQ,
 * and its own share of dK and dV; the shares of a key/value head's query heads
 * are then added in head order.  Every sum takes its terms in ascending index
 * order (j for dQ, i for the shares, h for the group sum).                  */
int oracle_causal_bwd(const double* q, const double* k, const double* v, const double* dout,
                      int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t D, double scale,
                      double* dq, double* dk, double* dv) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || T <= 0 || D <= 0 || Hq % Hkv != 0) return -1;
    const int64_t G = Hq / Hkv;
    /* each query head's share of dK and dV: [B,Hq,T,D] */
    double* dk_share = (double*)malloc((size_t)(B * Hq * T * D) * sizeof(double));
    double* dv_share = (double*)malloc((size_t)(B * Hq * T * D) * sizeof(double));
    if (!dk_share || !dv_share) { free(dk_share); free(dv_share); return -1; }
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < B * Hq; ++bh) {
        const int64_t b = bh / Hq, h = bh % Hq, kvh = h / G;
        const double* qh = q + bh * T * D;
        const double* doh = dout + bh * T * D;
        const double* kg = k + (b * Hkv + kvh) * T * D;
        const double* vg = v + (b * Hkv + kvh) * T * D;
        double* dqh = dq + bh * T * D;
        double* dkh = dk_share + bh * T * D;
        double* dvh = dv_share + bh * T * D;
        double* P = (double*)malloc((size_t)(T * T) * sizeof(double));
        double* dS = (double*)calloc((size_t)(T * T), sizeof(double));
        if (!P || !dS) { free(P); free(dS); failed = 1; continue; }
        head_probabilities(qh, kg, T, D, scale, P, NULL);
        for (int64_t i = 0; i < T; ++i) {
            double delta = 0.0;
            for (int64_t j = 0; j <= i; ++j) {
                double dp = 0.0;
                for (int64_t c = 0; c < D; ++c) dp += doh[i * D + c] * vg[j * D + c];
                dS[i * T + j] = dp;               /* dP for now */
                delta += P[i * T + j] * dp;
            }
            for (int64_t j = 0; j <= i; ++j) dS[i * T + j] = P[i * T + j] * (dS[i * T + j] - delta);
        }
        /* dQ_i = scale * sum_{j<=i} dS_ij k_j */
        for (int64_t i = 0; i < T; ++i) {
            for (int64_t c = 0; c < D; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j <= i; ++j) acc += dS[i * T + j] * kg[j * D + c];
                dqh[i * D + c] = scale * acc;
            }
        }
        /* this head's share: sum_{i>=j} dS_ij q_i (times scale) and sum_{i>=j} P_ij dO_i,
         * row i of dS and P adding its terms to every key j <= i, i ascending */
        memset(dkh, 0, (size_t)(T * D) * sizeof(double));
        memset(dvh, 0, (size_t)(T * D) * sizeof(double));
        for (int64_t i = 0; i < T; ++i) {
            for (int64_t j = 0; j <= i; ++j) {
                const double dsij = dS[i * T + j], pij = P[i * T + j];
                for (int64_t c = 0; c < D; ++c) {
                    dkh[j * D + c] += dsij * qh[i * D + c];
                    dvh[j * D + c] += pij * doh[i * D + c];
                }
            }
        }
        for (int64_t e = 0; e < T * D; ++e) dkh[e] = scale * dkh[e];
        free(P);
        free(dS);
    }
    /* dK, dV of key/value head g: the shares of its query heads g*G .. g*G+G-1 */
    if (!failed) {
#pragma omp parallel for schedule(static)
        for (int64_t bg = 0; bg < B * Hkv; ++bg) {
            const int64_t b = bg / Hkv, g = bg % Hkv;
            double* dkg = dk + bg * T * D;
            double* dvg = dv + bg * T * D;
            memset(dkg, 0, (size_t)(T * D) * sizeof(double));
            memset(dvg, 0, (size_t)(T * D) * sizeof(double));
            for (int64_t h = g * G; h < (g + 1) * G; ++h) {
                const double* dkh = dk_share + (b * Hq + h) * T * D;
                const double* dvh = dv_share + (b * Hq + h) * T * D;
                for (int64_t e = 0; e < T * D; ++e) {
                    dkg[e] += dkh[e];
                    dvg[e] += dvh[e];
                }
            }
        }
    }
    free(dk_share);
    free(dv_share);
    return failed ? -1 : 0;
}

/* Dense single-token decode of one sequence: the query is the newest position,
 * so it attends to every one of the n cached positions (no mask inside the
 * context).  q, o: [Hq,D]; kseq, vseq: [n,Hkv,D]; lse: [Hq] or NULL.         */
int oracle_decode_dense(const double* q, const double* kseq, const double* vseq, int64_t n,
                        int64_t Hq, int64_t Hkv, int64_t D, double scale, double* o, double* lse) {
    if (n <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0) return -1;
    const int64_t G = Hq / Hkv;
    double* p = (double*)malloc((size_t)n * sizeof(double));
    if (!p) return -1;
    for (int64_t h = 0; h < Hq; ++h) {
        const int64_t g = h / G;
        double m = -INFINITY;
        for (int64_t t = 0; t < n; ++t) {
            double s = 0.0;
            for (int64_t c = 0; c < D; ++c) s += q[h * D + c] * kseq[(t * Hkv + g) * D + c];
            p[t] = scale * s;
            if (p[t] > m) m = p[t];
        }
        double z = 0.0;
        for (int64_t t = 0; t < n; ++t) { p[t] = exp(p[t] - m); z += p[t]; }
        for (int64_t c = 0; c < D; ++c) {
            double acc = 0.0;
            for (int64_t t = 0; t < n; ++t) acc += (p[t] / z) * vseq[(t * Hkv + g) * D + c];
            o[h * D + c] = acc;
        }
        if (lse) lse[h] = m + log(z);
    }
    free(p);
    return 0;
}

/* Sequence s's first n positions, resolved position by position through its page
 * table into contiguous kseq, vseq [n,Hkv,D]: position t of the sequence lives at
 *   pool[block_table[s, t / page_size], g, t % page_size, :].
 * Returns -1 on a page index outside the pool.  */
static int gather_paged(const double* k_pool, const double* v_pool, const int32_t* block_table, int64_t s,
                        int64_t n, int64_t Hkv, int64_t D, int64_t page_size, int64_t max_pages,
                        int64_t num_pages, double* kseq, double* vseq) {
    for (int64_t t = 0; t < n; ++t) {
        const int64_t phys = block_table[s * max_pages + t / page_size];
        if (phys < 0 || phys >= num_pages) return -1;
        for (int64_t g = 0; g < Hkv; ++g) {
            const int64_t src = ((phys * Hkv + g) * page_size + t % page_size) * D;
            memcpy(kseq + (t * Hkv + g) * D, k_pool + src, (size_t)D * sizeof(double));
            memcpy(vseq + (t * Hkv + g) * D, v_pool + src, (size_t)D * sizeof(double));
        }
    }
    return 0;
}

/* Paged single-token decode over S independent sequences sharing one pool.
 * q, o: [S,Hq,D]; k_pool, v_pool: [num_pages,Hkv,page_size,D];
 * block_table: [S,max_pages] (logical page -> physical page); ctx: [S];
 * lse: [S,Hq] or NULL.  Position t of sequence s lives at
 *   pool[block_table[s, t / page_size], g, t % page_size, :].
 * Each sequence is resolved position by position into a contiguous copy and
 * handed to oracle_decode_dense.  Returns -1 on a bad length or page index.  */
int oracle_paged_decode(const double* q, const double* k_pool, const double* v_pool,
                        const int32_t* block_table, const int32_t* ctx,
                        int64_t S, int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size,
                        int64_t max_pages, int64_t num_pages, double scale,
                        double* o, double* lse) {
    if (S <= 0 || page_size <= 0 || max_pages <= 0) return -1;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t s = 0; s < S; ++s) {
        const int64_t n = ctx[s];
        if (n <= 0 || n > max_pages * page_size) { failed = 1; continue; }
        double* kseq = (double*)malloc((size_t)(n * Hkv * D) * sizeof(double));
        double* vseq = (double*)malloc((size_t)(n * Hkv * D) * sizeof(double));
        if (!kseq || !vseq) { free(kseq); free(vseq); failed = 1; continue; }
        const int bad = gather_paged(k_pool, v_pool, block_table, s, n, Hkv, D, page_size, max_pages, num_pages,
                                     kseq, vseq);
        if (bad || oracle_decode_dense(q + s * Hq * D, kseq, vseq, n, Hq, Hkv, D, scale,
                                       o + s * Hq * D, lse ? lse + s * Hq : NULL) != 0)
            failed = 1;
        free(kseq);
        free(vseq);
    }
    return failed ? -1 : 0;
}

/* Batched prefill over S sequences sharing one pool ("Architecture", "Serving
 * boundary"; "Execution Backends and the Python ABI", "Incremental attention":
 * K/V read through the sequence's page table; "Tensor conventions": a key after
 * the query is excluded).  Sequence s has n_s = token_start[s+1] - token_start[s]
 * new tokens, whose queries are rows token_start[s] + j of q [N,Hq,D]; its cache
 * holds ctx[s] >= n_s positions, so token j sits at position t = ctx[s] - n_s + j.
 * Each row is the plain definition: softmax over the scores of positions 0..t,
 * then the weighted sum of their values -- i.e. the dense decode definition over
 * the first t + 1 gathered positions.  o: [N,Hq,D]; lse: [N,Hq] or NULL.
 * Returns -1 on a bad table, length or page index.  */
int oracle_paged_prefill(const double* q, const double* k_pool, const double* v_pool,
                         const int32_t* block_table, const int32_t* ctx, const int32_t* token_start,
                         int64_t S, int64_t N, int64_t Hq, int64_t Hkv, int64_t D, int64_t page_size,
                         int64_t max_pages, int64_t num_pages, double scale, double* o, double* lse) {
    if (S <= 0 || N < 0 || page_size <= 0 || max_pages <= 0 || token_start[0] != 0 || token_start[S] != N)
        return -1;
    for (int64_t s = 0; s < S; ++s)
        if (token_start[s + 1] < token_start[s]) return -1;
    int failed = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t s = 0; s < S; ++s) {
        const int64_t n_new = token_start[s + 1] - token_start[s];
        const int64_t n = ctx[s];
        if (n_new == 0) continue;
        if (n < n_new || n > max_pages * page_size) { failed = 1; continue; }
        double* kseq = (double*)malloc((size_t)(n * Hkv * D) * sizeof(double));
        double* vseq = (double*)malloc((size_t)(n * Hkv * D) * sizeof(double));
        if (!kseq || !vseq) { free(kseq); free(vseq); failed = 1; continue; }
        int bad = gather_paged(k_pool, v_pool, block_table, s, n, Hkv, D, page_size, max_pages, num_pages, kseq,
                               vseq);
        for (int64_t j = 0; j < n_new && !bad; ++j) {
            const int64_t row = token_start[s] + j;
            const int64_t pos = n - n_new + j;
            if (oracle_decode_dense(q + row * Hq * D, kseq, vseq, pos + 1, Hq, Hkv, D, scale, o + row * Hq * D,
                                    lse ? lse + row * Hq : NULL) != 0)
                bad = 1;
        }
        if (bad) failed = 1;
        free(kseq);
        free(vseq);
    }
    return failed ? -1 : 0;
}
