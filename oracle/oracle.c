/*
 * FP64 CPU oracle for deterministic grouped-query attention (forward).
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * statement of what the attention path computes.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load it.  It
 * shares no code, header, table or helper with the HIP library, and it never
 * reads anything the GPU produced.
 *
 * Sources (the web pages this project is specified by):
 *   [P1] "WS2 Attention PR5 Drift Benchmark" (design doc), sections "Scope",
 *        "Transformer Engine Reuse" and "Report Contract".
 *   [P3] "[WS2][Attention] H100 validation and reproduction guide for #235
 *        PR1-PR8", sections "Status" and "Acceptance".
 *
 * Every function evaluates the plain mathematical definition in double
 * precision; bf16 inputs are widened exactly.  No blocking, tiling or online
 * rescaling is used: where a maximum is subtracted before exp() it is only the
 * textbook guard against overflow and does not change the value.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC oracle.c -o liboracle.so -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* bf16 bit pattern -> double, exact (bf16 is the top half of an IEEE binary32). */
static double bf16_to_double(uint16_t h) {
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Attention over an explicit key set, for a list of query rows.
 *
 * Definition ([P1] "Scope": Qwen3-8B GQA attention with Hq query heads sharing
 * Hkv key/value heads; queries consume post-RoPE Q/K; [P3] "Acceptance":
 * outputs are Out and the attention-domain LSE):
 *   kv head of q head h is h / (Hq / Hkv)         (contiguous GQA groups)
 *   key set J(row) = { j : key_lo <= j < key_hi, j < kv_len, and j <= pos if causal }
 *   s_j   = scale * sum_d Q[row,h,d] * K[j,hk,d]
 *   LSE   = ln sum_{j in J} exp(s_j)               (natural log)
 *   Out_d = sum_{j in J} exp(s_j - LSE) * V[j,hk,d]
 *   J empty -> Out = 0, LSE = -inf.
 *
 * With key_lo = 0 and key_hi = kv_len this is full attention.  With
 * [key_lo, key_hi) = [i*Bk, (i+1)*Bk) it is the partial state of KV block i
 * ([P1] "Transformer Engine Reuse": one partial state per logical KV block,
 * tagged with its global block index; out_i is normalised by the block's own
 * sum and lse_i is that block's log-sum-exp).
 *
 * Layouts (token-major): q [B][Sq][Hq][D], k and v [B][Skv][Hkv][D], all bf16
 * bit patterns.  Query t of batch b sits at absolute position pos0 + t, which
 * is how chunked-prefill replay is evaluated: a chunk is the same definition
 * at shifted positions over the cached keys.
 *
 * rows: flat indices b*Sq + t to evaluate (NULL = all B*Sq rows in order).
 * out [n_rows][Hq][D], lse [n_rows][Hq] in double.
 * Returns 0, or -1 on bad arguments.
 */
int orc_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                  int B, int Sq, int Skv, int Hq, int Hkv, int D,
                  int64_t pos0, int causal, int64_t kv_len, double scale,
                  int64_t key_lo, int64_t key_hi,
                  const int64_t* rows, int64_t n_rows,
                  double* out, double* lse) {
    if (B <= 0 || Sq < 0 || Skv < 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return -1;
    if (Hq % Hkv != 0) return -1;
    if (kv_len > Skv) return -1;
    if (rows == NULL) n_rows = (int64_t)B * Sq;
    const int group = Hq / Hkv;
    const int64_t n_items = n_rows * Hq;
    int bad = 0;

#pragma omp parallel
    {
        double* s = (double*)malloc(sizeof(double) * (size_t)(Skv > 0 ? Skv : 1));
        double* acc = (double*)malloc(sizeof(double) * (size_t)D);
        if (s == NULL || acc == NULL) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 8)
        for (int64_t it = 0; it < n_items; ++it) {
            if (s == NULL || acc == NULL) continue;
            const int64_t r = it / Hq;
            const int h = (int)(it % Hq);
            const int64_t flat = rows ? rows[r] : r;
            if (flat < 0 || flat >= (int64_t)B * Sq) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            const int64_t b = flat / Sq, t = flat % Sq;
            const int64_t pos = pos0 + t;
            const int hk = h / group;
            const uint16_t* qrow = q + ((b * Sq + t) * Hq + h) * (int64_t)D;

            int64_t lo = key_lo < 0 ? 0 : key_lo;
            int64_t hi = key_hi < kv_len ? key_hi : kv_len;
            if (causal && hi > pos + 1) hi = pos + 1;

            double* o = out + (r * Hq + h) * (int64_t)D;
            if (hi <= lo) { /* no key: empty state */
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                lse[r * Hq + h] = -INFINITY;
                continue;
            }
            double m = -INFINITY;
            for (int64_t j = lo; j < hi; ++j) {
                const uint16_t* krow = k + ((b * Skv + j) * Hkv + hk) * (int64_t)D;
                double dot = 0.0;
                for (int d = 0; d < D; ++d) dot += bf16_to_double(qrow[d]) * bf16_to_double(krow[d]);
                s[j - lo] = scale * dot;
                if (s[j - lo] > m) m = s[j - lo];
            }
            double sum = 0.0;
            for (int64_t j = lo; j < hi; ++j) sum += exp(s[j - lo] - m);
            const double L = m + log(sum);
            for (int d = 0; d < D; ++d) acc[d] = 0.0;
            for (int64_t j = lo; j < hi; ++j) {
                const double w = exp(s[j - lo] - L);
                const uint16_t* vrow = v + ((b * Skv + j) * Hkv + hk) * (int64_t)D;
                for (int d = 0; d < D; ++d) acc[d] += w * bf16_to_double(vrow[d]);
            }
            for (int d = 0; d < D; ++d) o[d] = acc[d];
            lse[r * Hq + h] = L;
        }
        free(s);
        free(acc);
    }
    return bad ? -1 : 0;
}

/*
 * Merge of partial states ([P1] "Transformer Engine Reuse" and "Scope",
 * merge_order_probe; [P1] "Report Contract": the merge order is always
 * global_block_index).
 *
 * Each part i holds (out_i, lse_i) for every row and head, plus its
 * global_block_index.  The parts are first put in ascending
 * global_block_index order (arrival order is discarded; a repeated index is
 * an error), then combined by the log-sum-exp rule:
 *   L   = M + ln sum_i exp(L_i - M),   M = max_i L_i
 *   Out = sum_i exp(L_i - L) * out_i
 * Parts with L_i = -inf carry no mass.  All parts empty -> Out = 0, L = -inf.
 *
 * out_parts [n_parts][rows][Hq][D], lse_parts [n_parts][rows][Hq] (double),
 * gbi [n_parts] in arrival order.  Returns 0, -1 on bad arguments, -2 on a
 * duplicate global_block_index.
 */
typedef struct { int64_t key; int idx; } orc_order_item;

static int orc_cmp_items(const void* a, const void* b) {
    const orc_order_item* x = (const orc_order_item*)a;
    const orc_order_item* y = (const orc_order_item*)b;
    if (x->key != y->key) return x->key < y->key ? -1 : 1;
    return x->idx < y->idx ? -1 : (x->idx > y->idx);
}

int orc_merge(const double* out_parts, const double* lse_parts, const int64_t* gbi,
              int n_parts, int64_t rows, int Hq, int D, double* out, double* lse) {
    if (n_parts < 0 || rows < 0 || Hq <= 0 || D <= 0) return -1;
    orc_order_item* order = (orc_order_item*)malloc(sizeof(orc_order_item) * (size_t)(n_parts > 0 ? n_parts : 1));
    if (order == NULL) return -1;
    for (int i = 0; i < n_parts; ++i) { order[i].key = gbi[i]; order[i].idx = i; }
    qsort(order, (size_t)n_parts, sizeof(orc_order_item), orc_cmp_items);
    for (int i = 1; i < n_parts; ++i) {
        if (order[i].key == order[i - 1].key) { free(order); return -2; }
    }
    const int64_t n_items = rows * Hq;
#pragma omp parallel for schedule(static)
    for (int64_t it = 0; it < n_items; ++it) {
        double M = -INFINITY;
        for (int i = 0; i < n_parts; ++i) {
            const double Li = lse_parts[(int64_t)order[i].idx * n_items + it];
            if (Li > M) M = Li;
        }
        double* o = out + it * D;
        if (M == -INFINITY) {
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            lse[it] = -INFINITY;
            continue;
        }
        double sum = 0.0;
        for (int i = 0; i < n_parts; ++i) {
            const double Li = lse_parts[(int64_t)order[i].idx * n_items + it];
            if (Li != -INFINITY) sum += exp(Li - M);
        }
        const double L = M + log(sum);
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        for (int i = 0; i < n_parts; ++i) {
            const int64_t base = (int64_t)order[i].idx * n_items + it;
            const double Li = lse_parts[base];
            if (Li == -INFINITY) continue;
            const double w = exp(Li - L);
            const double* oi = out_parts + base * D;
            for (int d = 0; d < D; ++d) o[d] += w * oi[d];
        }
        lse[it] = L;
    }
    free(order);
    return 0;
}

/*
 * Paged-KV decode ([P1] "Commands": paged prefill/decode with batch- and
 * page-layout invariance; [P3] "Status": strict decode/prefill gate).
 *
 * One query token per sequence.  Key j of sequence s lives in page
 * page_table[s][j / P] at slot j % P of the pool, which is laid out
 * [num_pages][Hkv][P][D].  The query attends to every cached key j < len_s
 * (the cache already holds the current token).  The value is the plain
 * definition of orc_attention over that gathered key list.
 *
 * q [Bd][Hq][D]; out [n_seq][Hq][D], lse [n_seq][Hq] for the sequences listed
 * in seqs (NULL = all Bd).  Returns 0, -1 on bad arguments or a page index
 * outside the pool.
 */
int orc_decode_paged(const uint16_t* q, const uint16_t* k_pool, const uint16_t* v_pool,
                     int64_t num_pages, int P, const int32_t* page_table, int max_pages,
                     const int32_t* ctx_lens, int Bd, int Hq, int Hkv, int D, double scale,
                     const int64_t* seqs, int64_t n_seq, double* out, double* lse) {
    if (Bd < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || P <= 0 || Hq % Hkv != 0) return -1;
    if (seqs == NULL) n_seq = Bd;
    const int group = Hq / Hkv;
    const int64_t n_items = n_seq * Hq;
    int bad = 0;
#pragma omp parallel
    {
        int64_t cap = (int64_t)max_pages * P;
        double* s = (double*)malloc(sizeof(double) * (size_t)(cap > 0 ? cap : 1));
        double* acc = (double*)malloc(sizeof(double) * (size_t)D);
#pragma omp for schedule(dynamic, 1)
        for (int64_t it = 0; it < n_items; ++it) {
            const int64_t r = it / Hq;
            const int h = (int)(it % Hq);
            const int64_t sq = seqs ? seqs[r] : r;
            double* o = out + it * D;
            if (s == NULL || acc == NULL || sq < 0 || sq >= Bd) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            const int64_t len = ctx_lens[sq];
            if (len < 0 || len > cap) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            const int hk = h / group;
            const uint16_t* qrow = q + (sq * Hq + h) * (int64_t)D;
            if (len == 0) {
                for (int d = 0; d < D; ++d) o[d] = 0.0;
                lse[it] = -INFINITY;
                continue;
            }
            double m = -INFINITY;
            int page_bad = 0;
            for (int64_t j = 0; j < len; ++j) {
                const int64_t page = page_table[sq * (int64_t)max_pages + j / P];
                if (page < 0 || page >= num_pages) { page_bad = 1; break; }
                const uint16_t* krow = k_pool + ((page * Hkv + hk) * P + j % P) * (int64_t)D;
                double dot = 0.0;
                for (int d = 0; d < D; ++d) dot += bf16_to_double(qrow[d]) * bf16_to_double(krow[d]);
                s[j] = scale * dot;
                if (s[j] > m) m = s[j];
            }
            if (page_bad) {
#pragma omp atomic write
                bad = 1;
                continue;
            }
            double sum = 0.0;
            for (int64_t j = 0; j < len; ++j) sum += exp(s[j] - m);
            const double L = m + log(sum);
            for (int d = 0; d < D; ++d) acc[d] = 0.0;
            for (int64_t j = 0; j < len; ++j) {
                const int64_t page = page_table[sq * (int64_t)max_pages + j / P];
                const double w = exp(s[j] - L);
                const uint16_t* vrow = v_pool + ((page * Hkv + hk) * P + j % P) * (int64_t)D;
                for (int d = 0; d < D; ++d) acc[d] += w * bf16_to_double(vrow[d]);
            }
            for (int d = 0; d < D; ++d) o[d] = acc[d];
            lse[it] = L;
        }
        free(s);
        free(acc);
    }
    return bad ? -1 : 0;
}

/*
 * Gradient of attention (the backward pass: [P3] "PR stack", the
 * prefill/chunked-prefill backward reference for dQ/dK/dV; [P3] "Status" and
 * "Acceptance": dQ, dK and dV are strict outputs alongside Out and LSE).
 *
 * Definition.  For the forward of orc_attention (full key range) and an
 * upstream gradient dOut of Out (the LSE output receives no gradient), the
 * exact partial derivatives of  Lsum = sum_{rows, h, d} Out * dOut  are, per
 * query row i of q head h with key set J(i) and probabilities
 * P_ij = exp(s_ij - LSE_i):
 *   dP_ij   = sum_d dOut[i,h,d] * V[j,hk,d]
 *   Delta_i = sum_{j in J(i)} P_ij * dP_ij
 *   dS_ij   = P_ij * (dP_ij - Delta_i)             (softmax Jacobian)
 *   dQ[i,h] = scale * sum_j dS_ij * K[j,hk]
 *   dK[j,hk] += scale * dS_ij * Q[i,h]             (summed over the group's q heads)
 *   dV[j,hk] += P_ij * dOut[i,h]
 * Keys outside every row's key set get dK = dV = 0; a row with no key gets
 * dQ = 0.  The sums run in plain row and key order in double precision.
 *
 * Optional error-bound magnitudes (any may be NULL): with
 *   |dP|_ij = sum_d |dOut[i,h,d]| |V[j,hk,d]|,   delta_i = sum_j P_ij |dP|_ij,
 *   G_ij    = scale * (|P_ij (dP_ij - Delta_i)| + P_ij (delta_i + |dP|_ij)),
 * mag_dq[i,h,d] = sum_j G_ij |K[j,hk,d]|, mag_dk[j,hk,d] = sum_{i,h} G_ij |Q[i,h,d]|
 * and mag_dv[j,hk,d] = sum_{i,h} P_ij |dOut[i,h,d]|.  They are the sums of
 * absolute values that a bound on a finite-precision evaluation scales: G_ij
 * bounds |dS_ij| plus the part of dS_ij that an error in Delta_i (relative to
 * delta_i) or in dP_ij (relative to |dP|_ij) can move.
 *
 * Layouts: q, dout [B][Sq][Hq][D]; k, v [B][Skv][Hkv][D] (bf16 bits);
 * dq and mag_dq [B][Sq][Hq][D], dk, dv, mag_dk, mag_dv [B][Skv][Hkv][D]
 * (double).  Query t sits at position pos0 + t.
 * rows: ascending flat indices b*Sq + t of the query rows to take (NULL = all
 * rows).  dQ of the listed rows is complete; dK and dV then hold only the
 * listed rows' terms (a sample, for checking dQ of a few rows of a large
 * problem).  Returns 0, or -1 on bad arguments.
 */
int orc_attention_backward(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const uint16_t* dout, int B, int Sq, int Skv, int Hq, int Hkv, int D,
                           int64_t pos0, int causal, int64_t kv_len, double scale,
                           const int64_t* rows, int64_t n_rows,
                           double* dq, double* dk, double* dv,
                           double* mag_dq, double* mag_dk, double* mag_dv) {
    if (B <= 0 || Sq < 0 || Skv < 0 || Hq <= 0 || Hkv <= 0 || D <= 0) return -1;
    if (Hq % Hkv != 0 || kv_len > Skv || kv_len < 0) return -1;
    if (rows != NULL) {
        for (int64_t r = 0; r < n_rows; ++r) {
            if (rows[r] < 0 || rows[r] >= (int64_t)B * Sq || (r > 0 && rows[r] <= rows[r - 1])) return -1;
        }
    }
    const int group = Hq / Hkv;
    int bad = 0;
    memset(dq, 0, sizeof(double) * (size_t)B * Sq * Hq * D);
    memset(dk, 0, sizeof(double) * (size_t)B * Skv * Hkv * D);
    memset(dv, 0, sizeof(double) * (size_t)B * Skv * Hkv * D);
    if (mag_dq) memset(mag_dq, 0, sizeof(double) * (size_t)B * Sq * Hq * D);
    if (mag_dk) memset(mag_dk, 0, sizeof(double) * (size_t)B * Skv * Hkv * D);
    if (mag_dv) memset(mag_dv, 0, sizeof(double) * (size_t)B * Skv * Hkv * D);

    /* One (batch, kv head) per iteration: every write below lands in that
     * pair's rows, so iterations never touch the same memory. */
#pragma omp parallel
    {
        const size_t n = (size_t)(Skv > 0 ? Skv : 1);
        double* s = (double*)malloc(sizeof(double) * n);
        double* dp = (double*)malloc(sizeof(double) * n);
        double* adp = (double*)malloc(sizeof(double) * n);
        if (s == NULL || dp == NULL || adp == NULL) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t pair = 0; pair < (int64_t)B * Hkv; ++pair) {
            if (s == NULL || dp == NULL || adp == NULL) continue;
            const int64_t b = pair / Hkv;
            const int hk = (int)(pair % Hkv);
            /* this batch row's span of the row list */
            int64_t r_lo = 0, r_hi = Sq;
            if (rows != NULL) {
                r_lo = 0;
                while (r_lo < n_rows && rows[r_lo] < b * Sq) ++r_lo;
                r_hi = r_lo;
                while (r_hi < n_rows && rows[r_hi] < (b + 1) * Sq) ++r_hi;
            }
            for (int h = hk * group; h < (hk + 1) * group; ++h) {
                for (int64_t r = r_lo; r < r_hi; ++r) {
                    const int64_t t = rows != NULL ? rows[r] - b * Sq : r;
                    const int64_t pos = pos0 + t;
                    int64_t hi = kv_len;
                    if (causal && hi > pos + 1) hi = pos + 1;
                    if (hi <= 0) continue;
                    const int64_t qoff = ((b * Sq + t) * Hq + h) * (int64_t)D;
                    const uint16_t* qrow = q + qoff;
                    const uint16_t* grow = dout + qoff;
                    double m = -INFINITY;
                    for (int64_t j = 0; j < hi; ++j) {
                        const int64_t koff = ((b * Skv + j) * Hkv + hk) * (int64_t)D;
                        double dot = 0.0, g = 0.0, ag = 0.0;
                        for (int d = 0; d < D; ++d) {
                            dot += bf16_to_double(qrow[d]) * bf16_to_double(k[koff + d]);
                            g += bf16_to_double(grow[d]) * bf16_to_double(v[koff + d]);
                            ag += fabs(bf16_to_double(grow[d])) * fabs(bf16_to_double(v[koff + d]));
                        }
                        s[j] = scale * dot;
                        dp[j] = g;
                        adp[j] = ag;
                        if (s[j] > m) m = s[j];
                    }
                    double sum = 0.0;
                    for (int64_t j = 0; j < hi; ++j) sum += exp(s[j] - m);
                    const double L = m + log(sum);
                    /* s[j] becomes P_ij from here on. */
                    double delta = 0.0, adelta = 0.0;
                    for (int64_t j = 0; j < hi; ++j) {
                        s[j] = exp(s[j] - L);
                        delta += s[j] * dp[j];
                        adelta += s[j] * adp[j];
                    }
                    double* dqrow = dq + qoff;
                    for (int64_t j = 0; j < hi; ++j) {
                        const double p = s[j];
                        const double ds = p * (dp[j] - delta);
                        const double gmag = scale * (fabs(ds) + p * (adelta + adp[j]));
                        const int64_t koff = ((b * Skv + j) * Hkv + hk) * (int64_t)D;
                        for (int d = 0; d < D; ++d) {
                            const double kd = bf16_to_double(k[koff + d]);
                            const double qd = bf16_to_double(qrow[d]);
                            const double gd = bf16_to_double(grow[d]);
                            dqrow[d] += scale * ds * kd;
                            dk[koff + d] += scale * ds * qd;
                            dv[koff + d] += p * gd;
                            if (mag_dq) mag_dq[qoff + d] += gmag * fabs(kd);
                            if (mag_dk) mag_dk[koff + d] += gmag * fabs(qd);
                            if (mag_dv) mag_dv[koff + d] += p * fabs(gd);
                        }
                    }
                }
            }
        }
        free(s);
        free(dp);
        free(adp);
    }
    return bad ? -1 : 0;
}

/*
 * Selected log-probability through a synthetic FP32 lm_head ([P1] "Scope":
 * both attention outputs are projected through the same deterministic
 * synthetic FP32 lm_head and the active-token selected log-prob drift is
 * reported; [P3] "Status": decode/prefill dlogp max abs 0.0).
 *
 * Definition, per active token t with attention output x_t (the Out row of
 * the token, all q heads side by side: H = Hq * D values) and token id y_t:
 *   z_tv   = sum_h x_th * W_vh              (logits, v < V)
 *   logZ_t = ln sum_v exp(z_tv)
 *   logp_t = z_{t, y_t} - logZ_t
 * x is given as bf16 bits (x_f32 == NULL) or as fp32 (x_bf16 == NULL), W as
 * fp32 [V][H]; everything is widened exactly and evaluated in double.
 * Optional mag [T] (may be NULL): max_v sum_h |x_th| |W_vh|, the magnitude a
 * bound on a finite-precision evaluation of the logits scales.
 * Returns 0, or -1 on bad arguments (including a token id outside [0, V)).
 */
int orc_lm_head_logprobs(const uint16_t* x_bf16, const float* x_f32, const float* w, const int32_t* tokens,
                         int T, int H, int V, double* logp, double* logz, double* mag) {
    if (T < 0 || H <= 0 || V <= 0 || w == NULL || tokens == NULL || logp == NULL) return -1;
    if ((x_bf16 == NULL) == (x_f32 == NULL)) return -1;
    for (int t = 0; t < T; ++t) {
        if (tokens[t] < 0 || tokens[t] >= V) return -1;
    }
    int bad = 0;
#pragma omp parallel
    {
        double* z = (double*)malloc(sizeof(double) * (size_t)V);
        double* xs = (double*)malloc(sizeof(double) * (size_t)H);
        if (z == NULL || xs == NULL) {
#pragma omp atomic write
            bad = 1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int t = 0; t < T; ++t) {
            if (z == NULL || xs == NULL) continue;
            for (int h = 0; h < H; ++h)
                xs[h] = x_bf16 ? bf16_to_double(x_bf16[(int64_t)t * H + h]) : (double)x_f32[(int64_t)t * H + h];
            double m = -INFINITY, big = 0.0;
            for (int v = 0; v < V; ++v) {
                const float* row = w + (int64_t)v * H;
                double acc = 0.0, aabs = 0.0;
                for (int h = 0; h < H; ++h) {
                    acc += xs[h] * (double)row[h];
                    aabs += fabs(xs[h]) * fabs((double)row[h]);
                }
                z[v] = acc;
                if (acc > m) m = acc;
                if (aabs > big) big = aabs;
            }
            double sum = 0.0;
            for (int v = 0; v < V; ++v) sum += exp(z[v] - m);
            const double lz = m + log(sum);
            logp[t] = z[tokens[t]] - lz;
            if (logz) logz[t] = lz;
            if (mag) mag[t] = big;
        }
        free(z);
        free(xs);
    }
    return bad ? -1 : 0;
}
