/*
 * gqa_oracle.c -- plain fp64 CPU reference for the grouped-query attention core.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the oracle that the HIP kernels are
 * checked against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no code, header, table or helper with
 * the GPU library, and it is deliberately slow: no tiling, no online softmax,
 * no fusion, no reordering of the arithmetic beyond what the definition states.
 *
 * What it computes (all in double precision):
 *
 *   Scaled dot-product attention, softmax(Q K^T * scale) V, per query head
 *   ("Modern LLM architecture (1): GQA and RMSNorm", §2.1, the attention
 *   formula), with the grouped-query head map of the same page, §2.3: the
 *   h_kv key/value heads are repeated group_size = h_q / h_kv times along the
 *   head axis with repeat_interleave, so query head h reads key/value head
 *   floor(h / group_size).  The integer-division form of that map is also
 *   stated in "Attention in Qwen, DeepSeek and LLaMA3", §2.2 (cache reuse
 *   structure) and §2.3 (the q_idx // 4 cache index).
 *
 *   The repeat is materialised explicitly (one copied slab per query head),
 *   exactly as the repeat_interleave in the page's module does, so that no
 *   stride trick of the GPU path can hide in here.
 *
 *   Causal masking keeps key j for query i iff j <= i (square alignment; the
 *   masked_fill(mask == 0, -inf) convention of the same page, §2.1-§2.3).
 *
 *   Prefill against existing keys (chunked prefill): L_q new positions whose
 *   keys and values were appended after L_k - L_q earlier ones attend to all
 *   L_k keys of their sequence ("What is Grouped-Query Attention", §3.2:
 *   append to the cache, then attend).  Query row i of the chunk sits at
 *   position L_k - L_q + i, so causally it sees keys 0 .. L_k - L_q + i
 *   (bottom-right alignment; L_q == L_k is the square case above).  Run chunk
 *   by chunk this reproduces one full causal prefill, which processing each
 *   chunk on its own ("Implementing GQA from scratch in PyTorch", §4.3) does
 *   not.
 *
 *   Decode with append: the new token's key and value rows are first written
 *   into cache row seqlens[b] (seqlens[b] < S), then the token attends over
 *   rows [0, seqlens[b] + 1) -- the order of "What is Grouped-Query
 *   Attention", §3.2 (append to the cache, then attend).
 *
 *   Decode: one new query token per sequence attends over the cache rows
 *   [0, seqlens[b]) of a head-major cache [B, h_kv, S, d]
 *   ("What is Grouped-Query Attention", §2.2 step 2 for the cache layout and
 *   §3.2 for appending the new token before attending).  The scale is
 *   1/sqrt(d).  A sequence with seqlens[b] == 0 has no visible key; its output
 *   is defined as zero.
 *
 *   Decode over other cache layouts (the same attention, rows found elsewhere):
 *   - token-major [B, S, h_kv, d], the kv_cache of "Attention in Qwen,
 *     DeepSeek and LLaMA3", §2.2 (shape [bs, max_len, n_kv_heads, head_dim]);
 *   - paged with group-aligned pages, the same page, §4.3: the cache is a
 *     pool of physical blocks [num_pages][h_kv][page_size][d], each block
 *     holding page_size consecutive positions of one sequence with one
 *     contiguous page per group (key/value head), and block_table[b][i] names
 *     the block that holds positions [i * page_size, (i + 1) * page_size) of
 *     sequence b.  Logical row j of (b, g) is block_table[b][j / page_size],
 *     group g, row j % page_size.
 *
 *   Variable-length sequences in a padded batch: the forward pass of
 *   "Implementing GQA from scratch in PyTorch", §3.3 takes an optional mask,
 *   applied as masked_fill(mask == 0, -inf), for sequences of different
 *   lengths.  Read as a key-padding mask given by lengths: key j of sequence b
 *   is visible iff j < kv_lens[b] (and j <= i when causal).  Every query row
 *   is computed, padded ones included; a row with no visible key is zero.
 *
 *   A general keep-mask (the same page's optional mask, and the attn_mask
 *   argument of the GQA module in "Modern LLM architecture (1)", §2.3): key j
 *   is visible to query row i of sequence b iff mask[b][i][j] != 0 (and
 *   j <= L_k - L_q + i when causal).  Each row's visible set is listed
 *   explicitly and the row attends over exactly those keys; an empty set
 *   gives a zero row.
 *
 *   Rotary position embedding before the scores ("Attention in Qwen,
 *   DeepSeek and LLaMA3", §1, apply_rotary_pos_emb; the model-family table
 *   of "Modern LLM architecture (1)", §1 lists RoPE for every GQA family).
 *   For a vector x of even length d at position p, with tables cos, sin
 *   [L][d/2] indexed by position:
 *     out[i]       = x[2i] cos[p][i] - x[2i+1] sin[p][i]
 *     out[d/2 + i] = x[2i] sin[p][i] + x[2i+1] cos[p][i]      (0 <= i < d/2)
 *   -- the even/odd pairs rotated, the two results concatenated along the
 *   last axis as the page writes it.  q and k are rotated, v is not; then the
 *   attention above.  In a decode step the new token sits at position
 *   seqlens[b]: its q and k are rotated with row seqlens[b] of the tables,
 *   the rotated key is appended, then the token attends (decode with append).
 *
 * Every entry point returns 0 on success and a negative number for a bad
 * argument (it never aborts).  Arrays are dense, row-major, caller-owned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_ERR_ARG (-1)
#define ORACLE_ERR_NOMEM (-2)

/* Number of threads the parallel loops below will use. */
int gqa_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Query head h reads key/value head floor(h / group_size). */
static int kv_head_of(int h, int h_q, int h_kv) {
    int group_size = h_q / h_kv;
    return h / group_size;
}

/*
 * Explicit repeat: copy the n_keys rows of key/value head kvh of sequence b out
 * of a strided source into a dense [n_keys][d] slab.  The source element
 * (b, j, kvh, c) sits at b*sb + j*sj + kvh*sh + c.
 */
static void repeat_kv_slab(const double *src, long sb, long sj, long sh, int b,
                           int kvh, int n_keys, int d, double *dst) {
    for (int j = 0; j < n_keys; ++j) {
        const double *row = src + (long)b * sb + (long)j * sj + (long)kvh * sh;
        memcpy(dst + (long)j * d, row, sizeof(double) * (size_t)d);
    }
}

/*
 * One query row against n_vis keys of its (already repeated) head:
 *   s_j   = scale * sum_c q[c] * krep[j][c]          (c ascending)
 *   m     = max_j s_j
 *   e_j   = exp(s_j - m),  Z = sum_j e_j
 *   out   = sum_j (e_j / Z) * vrep[j]
 * The max subtraction does not change the result in real arithmetic; it keeps
 * exp() finite.  n_vis == 0 gives a zero row.  `scores` is scratch of n_vis
 * doubles; `probs`, when not NULL, receives e_j / Z.
 */
static void attend_one_row(const double *q, const double *krep, const double *vrep,
                           int n_vis, int d, double scale, double *scores,
                           double *out, double *probs) {
    for (int c = 0; c < d; ++c) out[c] = 0.0;
    if (n_vis <= 0) return;

    double m = -INFINITY;
    for (int j = 0; j < n_vis; ++j) {
        double dot = 0.0;
        for (int c = 0; c < d; ++c) dot += q[c] * krep[(long)j * d + c];
        scores[j] = scale * dot;
        if (scores[j] > m) m = scores[j];
    }
    double z = 0.0;
    for (int j = 0; j < n_vis; ++j) {
        scores[j] = exp(scores[j] - m);
        z += scores[j];
    }
    for (int j = 0; j < n_vis; ++j) {
        double p = scores[j] / z;
        if (probs) probs[j] = p;
        for (int c = 0; c < d; ++c) out[c] += p * vrep[(long)j * d + c];
    }
}

static int check_heads(int h_q, int h_kv) {
    if (h_q <= 0 || h_kv <= 0) return ORACLE_ERR_ARG;
    if (h_q % h_kv != 0) return ORACLE_ERR_ARG; /* group size must be whole */
    return 0;
}

/*
 * Prefill for a list of query rows against L_k keys per sequence.
 *   q_rows  [n_rows][d]   the query vectors of the listed rows
 *   row_bih [n_rows][3]   (b, i, h) of each listed row, 0 <= i < L_q
 *   k, v    [B][L_k][h_kv][d]
 *   out     [n_rows][d]
 *   probs   NULL, or [n_rows][L_k]: the softmax row (zeros beyond the visible keys)
 *   kv_lens NULL, or [B]: only keys j < kv_lens[b] are visible (0 <= kv_lens[b] <= L_k)
 * Query row i sits at position L_k - L_q + i (1 <= L_q <= L_k).  Rows are
 * processed in groups that share (b, h) so the repeated slab of their head is
 * built once per group; rows must be sorted by (b, h) for that to help, but
 * any order is correct.
 */
static int prefill_rows_general(const double *q_rows, const int64_t *row_bih, int64_t n_rows,
                                const double *k, const double *v, int B, int Lq, int Lk,
                                int h_q, int h_kv, int d, int causal, double scale,
                                double *out, double *probs, const int32_t *kv_lens) {
    if (B <= 0 || Lq <= 0 || Lk < Lq || d <= 0 || n_rows < 0) return ORACLE_ERR_ARG;
    if (check_heads(h_q, h_kv)) return ORACLE_ERR_ARG;
    if (kv_lens)
        for (int b = 0; b < B; ++b)
            if (kv_lens[b] < 0 || kv_lens[b] > Lk) return ORACLE_ERR_ARG;
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t b = row_bih[3 * r], i = row_bih[3 * r + 1], h = row_bih[3 * r + 2];
        if (b < 0 || b >= B || i < 0 || i >= Lq || h < 0 || h >= h_q) return ORACLE_ERR_ARG;
    }
    const long sh = d, sj = (long)h_kv * d, sb = (long)Lk * sj;
    const int first = Lk - Lq; /* position of query row 0 */

    /* Split the row list into runs of equal (b, h). */
    int64_t *run_start = (int64_t *)malloc(sizeof(int64_t) * (size_t)(n_rows + 1));
    if (!run_start) return ORACLE_ERR_NOMEM;
    int64_t n_runs = 0;
    for (int64_t r = 0; r < n_rows; ++r) {
        if (r == 0 || row_bih[3 * r] != row_bih[3 * (r - 1)] ||
            row_bih[3 * r + 2] != row_bih[3 * (r - 1) + 2])
            run_start[n_runs++] = r;
    }
    run_start[n_runs] = n_rows;

    int failed = 0;
#pragma omp parallel
    {
        double *krep = (double *)malloc(sizeof(double) * (size_t)Lk * d);
        double *vrep = (double *)malloc(sizeof(double) * (size_t)Lk * d);
        double *scores = (double *)malloc(sizeof(double) * (size_t)Lk);
        if (!krep || !vrep || !scores) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t run = 0; run < n_runs; ++run) {
                int64_t r0 = run_start[run], r1 = run_start[run + 1];
                int b = (int)row_bih[3 * r0], h = (int)row_bih[3 * r0 + 2];
                int kvh = kv_head_of(h, h_q, h_kv);
                /* explicit repeat of this head's keys and values */
                repeat_kv_slab(k, sb, sj, sh, b, kvh, Lk, d, krep);
                repeat_kv_slab(v, sb, sj, sh, b, kvh, Lk, d, vrep);
                for (int64_t r = r0; r < r1; ++r) {
                    int i = (int)row_bih[3 * r + 1];
                    int n_vis = causal ? first + i + 1 : Lk;
                    if (kv_lens && kv_lens[b] < n_vis) n_vis = kv_lens[b]; /* key padding */
                    double *prow = NULL;
                    if (probs) {
                        prow = probs + r * (int64_t)Lk;
                        for (int j = 0; j < Lk; ++j) prow[j] = 0.0;
                    }
                    attend_one_row(q_rows + r * (int64_t)d, krep, vrep, n_vis, d, scale,
                                   scores, out + r * (int64_t)d, prow);
                }
            }
        }
        free(krep);
        free(vrep);
        free(scores);
    }
    free(run_start);
    return failed ? ORACLE_ERR_NOMEM : 0;
}

/* Square prefill rows: L_q == L_k == L (see prefill_rows_general). */
int gqa_oracle_prefill_rows(const double *q_rows, const int64_t *row_bih, int64_t n_rows,
                            const double *k, const double *v, int B, int L, int h_q,
                            int h_kv, int d, int causal, double scale, double *out,
                            double *probs) {
    return prefill_rows_general(q_rows, row_bih, n_rows, k, v, B, L, L, h_q, h_kv, d, causal,
                                scale, out, probs, NULL);
}

/* Rows of a prefill against L_k keys, L_q new positions (see prefill_rows_general). */
int gqa_oracle_prefill_cached_rows(const double *q_rows, const int64_t *row_bih,
                                   int64_t n_rows, const double *k, const double *v, int B,
                                   int Lq, int Lk, int h_q, int h_kv, int d, int causal,
                                   double scale, double *out) {
    return prefill_rows_general(q_rows, row_bih, n_rows, k, v, B, Lq, Lk, h_q, h_kv, d, causal,
                                scale, out, NULL, NULL);
}

/*
 * Full prefill of L_q positions against L_k keys per sequence:
 *   q, o [B][L_q][h_q][d];  k, v [B][L_k][h_kv][d].
 * probs: NULL, or [B][h_q][L_q][L_k] softmax matrices (zeros where masked).
 */
static int prefill_general(const double *q, const double *k, const double *v, double *o, int B,
                           int Lq, int Lk, int h_q, int h_kv, int d, int causal, double scale,
                           double *probs, const int32_t *kv_lens) {
    if (B <= 0 || Lq <= 0 || Lk < Lq || d <= 0) return ORACLE_ERR_ARG;
    if (check_heads(h_q, h_kv)) return ORACLE_ERR_ARG;
    int64_t n = (int64_t)B * h_q * Lq;
    int64_t *bih = (int64_t *)malloc(sizeof(int64_t) * 3 * (size_t)n);
    double *qr = (double *)malloc(sizeof(double) * (size_t)(n * d));
    double *orow = (double *)malloc(sizeof(double) * (size_t)(n * d));
    if (!bih || !qr || !orow) {
        free(bih);
        free(qr);
        free(orow);
        return ORACLE_ERR_NOMEM;
    }
    /* list rows ordered by (b, h, i); gather their query vectors */
    int64_t r = 0;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < h_q; ++h)
            for (int i = 0; i < Lq; ++i, ++r) {
                bih[3 * r] = b;
                bih[3 * r + 1] = i;
                bih[3 * r + 2] = h;
                memcpy(qr + r * d, q + (((int64_t)b * Lq + i) * h_q + h) * d,
                       sizeof(double) * (size_t)d);
            }
    int rc = prefill_rows_general(qr, bih, n, k, v, B, Lq, Lk, h_q, h_kv, d, causal, scale,
                                  orow, probs, kv_lens);
    if (rc == 0) {
        r = 0;
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < h_q; ++h)
                for (int i = 0; i < Lq; ++i, ++r)
                    memcpy(o + (((int64_t)b * Lq + i) * h_q + h) * d, orow + r * d,
                           sizeof(double) * (size_t)d);
    }
    free(bih);
    free(qr);
    free(orow);
    return rc;
}

/*
 * Full prefill:  q, o [B][L][h_q][d];  k, v [B][L][h_kv][d].
 * probs: NULL, or [B][h_q][L][L] softmax matrices (zeros where masked).
 */
int gqa_oracle_prefill(const double *q, const double *k, const double *v, double *o, int B,
                       int L, int h_q, int h_kv, int d, int causal, double scale,
                       double *probs) {
    return prefill_general(q, k, v, o, B, L, L, h_q, h_kv, d, causal, scale, probs, NULL);
}

/*
 * Prefill of a padded batch of variable-length sequences: q, o [B][L][h_q][d],
 * k, v [B][L][h_kv][d], kv_lens [B] in [0, L]; key j of sequence b is visible
 * iff j < kv_lens[b] (and j <= i when causal).
 */
int gqa_oracle_prefill_varlen(const double *q, const double *k, const double *v,
                              const int32_t *kv_lens, double *o, int B, int L, int h_q, int h_kv,
                              int d, int causal, double scale) {
    if (!kv_lens) return ORACLE_ERR_ARG;
    return prefill_general(q, k, v, o, B, L, L, h_q, h_kv, d, causal, scale, NULL, kv_lens);
}

/* Selected rows of the padded variable-length prefill (see prefill_rows_general). */
int gqa_oracle_prefill_varlen_rows(const double *q_rows, const int64_t *row_bih, int64_t n_rows,
                                   const double *k, const double *v, const int32_t *kv_lens,
                                   int B, int L, int h_q, int h_kv, int d, int causal,
                                   double scale, double *out) {
    if (!kv_lens) return ORACLE_ERR_ARG;
    return prefill_rows_general(q_rows, row_bih, n_rows, k, v, B, L, L, h_q, h_kv, d, causal,
                                scale, out, NULL, kv_lens);
}

/*
 * Prefill with a keep-mask, for a list of query rows.
 *   q_rows  [n_rows][d], row_bih [n_rows][3] (b, i, h), 0 <= i < L_q
 *   k, v    [B][L_k][h_kv][d]
 *   mask    [B][L_q][L_k] bytes: key j is visible to row (b, i) iff
 *           mask[b][i][j] != 0, and also j <= L_k - L_q + i when causal
 *   out     [n_rows][d]
 *   probs   NULL, or [n_rows][L_k]: the softmax row (zeros at hidden keys)
 * The row's head is repeated into a slab, its visible keys and values are
 * gathered in ascending j, and attend_one_row evaluates the softmax over
 * exactly that set.  No visible key gives a zero row.
 */
int gqa_oracle_prefill_mask_rows(const double *q_rows, const int64_t *row_bih, int64_t n_rows,
                                 const double *k, const double *v, const uint8_t *mask, int B,
                                 int Lq, int Lk, int h_q, int h_kv, int d, int causal,
                                 double scale, double *out, double *probs) {
    if (!mask || B <= 0 || Lq <= 0 || Lk < Lq || d <= 0 || n_rows < 0) return ORACLE_ERR_ARG;
    if (check_heads(h_q, h_kv)) return ORACLE_ERR_ARG;
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t b = row_bih[3 * r], i = row_bih[3 * r + 1], h = row_bih[3 * r + 2];
        if (b < 0 || b >= B || i < 0 || i >= Lq || h < 0 || h >= h_q) return ORACLE_ERR_ARG;
    }
    const long sh = d, sj = (long)h_kv * d, sb = (long)Lk * sj;
    const int first = Lk - Lq; /* position of query row 0 */
    int failed = 0;
#pragma omp parallel
    {
        double *kslab = (double *)malloc(sizeof(double) * (size_t)Lk * d);
        double *vslab = (double *)malloc(sizeof(double) * (size_t)Lk * d);
        double *kvis = (double *)malloc(sizeof(double) * (size_t)Lk * d);
        double *vvis = (double *)malloc(sizeof(double) * (size_t)Lk * d);
        double *scores = (double *)malloc(sizeof(double) * (size_t)Lk);
        double *pvis = (double *)malloc(sizeof(double) * (size_t)Lk);
        int *vis = (int *)malloc(sizeof(int) * (size_t)Lk);
        if (!kslab || !vslab || !kvis || !vvis || !scores || !pvis || !vis) {
#pragma omp atomic write
            failed = 1;
        } else {
            int cur_b = -1, cur_kvh = -1;
#pragma omp for schedule(dynamic, 16)
            for (int64_t r = 0; r < n_rows; ++r) {
                int b = (int)row_bih[3 * r], i = (int)row_bih[3 * r + 1];
                int kvh = kv_head_of((int)row_bih[3 * r + 2], h_q, h_kv);
                if (b != cur_b || kvh != cur_kvh) {
                    /* explicit repeat of this head's keys and values */
                    repeat_kv_slab(k, sb, sj, sh, b, kvh, Lk, d, kslab);
                    repeat_kv_slab(v, sb, sj, sh, b, kvh, Lk, d, vslab);
                    cur_b = b;
                    cur_kvh = kvh;
                }
                /* the visible set of this row */
                const uint8_t *mrow = mask + ((int64_t)b * Lq + i) * (int64_t)Lk;
                int n_vis = 0;
                for (int j = 0; j < Lk; ++j) {
                    if (mrow[j] == 0) continue;
                    if (causal && j > first + i) continue;
                    vis[n_vis++] = j;
                }
                for (int t = 0; t < n_vis; ++t) {
                    memcpy(kvis + (long)t * d, kslab + (long)vis[t] * d, sizeof(double) * (size_t)d);
                    memcpy(vvis + (long)t * d, vslab + (long)vis[t] * d, sizeof(double) * (size_t)d);
                }
                attend_one_row(q_rows + r * (int64_t)d, kvis, vvis, n_vis, d, scale, scores,
                               out + r * (int64_t)d, probs ? pvis : NULL);
                if (probs) {
                    double *prow = probs + r * (int64_t)Lk;
                    for (int j = 0; j < Lk; ++j) prow[j] = 0.0;
                    for (int t = 0; t < n_vis; ++t) prow[vis[t]] = pvis[t];
                }
            }
        }
        free(kslab);
        free(vslab);
        free(kvis);
        free(vvis);
        free(scores);
        free(pvis);
        free(vis);
    }
    return failed ? ORACLE_ERR_NOMEM : 0;
}

/*
 * Full prefill with a keep-mask: q, o [B][L_q][h_q][d], k, v [B][L_k][h_kv][d],
 * mask [B][L_q][L_k] (see gqa_oracle_prefill_mask_rows); probs NULL or
 * [B][h_q][L_q][L_k].
 */
int gqa_oracle_prefill_mask(const double *q, const double *k, const double *v,
                            const uint8_t *mask, double *o, int B, int Lq, int Lk, int h_q,
                            int h_kv, int d, int causal, double scale, double *probs) {
    if (B <= 0 || Lq <= 0 || Lk < Lq || d <= 0) return ORACLE_ERR_ARG;
    if (check_heads(h_q, h_kv)) return ORACLE_ERR_ARG;
    int64_t n = (int64_t)B * h_q * Lq;
    int64_t *bih = (int64_t *)malloc(sizeof(int64_t) * 3 * (size_t)n);
    double *qr = (double *)malloc(sizeof(double) * (size_t)(n * d));
    double *orow = (double *)malloc(sizeof(double) * (size_t)(n * d));
    if (!bih || !qr || !orow) {
        free(bih);
        free(qr);
        free(orow);
        return ORACLE_ERR_NOMEM;
    }
    /* rows ordered by (b, h, i), which is also the order of probs */
    int64_t r = 0;
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < h_q; ++h)
            for (int i = 0; i < Lq; ++i, ++r) {
                bih[3 * r] = b;
                bih[3 * r + 1] = i;
                bih[3 * r + 2] = h;
                memcpy(qr + r * d, q + (((int64_t)b * Lq + i) * h_q + h) * d,
                       sizeof(double) * (size_t)d);
            }
    int rc = gqa_oracle_prefill_mask_rows(qr, bih, n, k, v, mask, B, Lq, Lk, h_q, h_kv, d, causal,
                                          scale, orow, probs);
    if (rc == 0) {
        r = 0;
        for (int b = 0; b < B; ++b)
            for (int h = 0; h < h_q; ++h)
                for (int i = 0; i < Lq; ++i, ++r)
                    memcpy(o + (((int64_t)b * Lq + i) * h_q + h) * d, orow + r * d,
                           sizeof(double) * (size_t)d);
    }
    free(bih);
    free(qr);
    free(orow);
    return rc;
}

/*
 * Rotary embedding of x [B][L][H][d] (d even) with cos, sin [L][d/2] into out
 * (same shape; out must not alias x).
 */
int gqa_oracle_rope(const double *x, const double *cos_t, const double *sin_t, double *out,
                    int B, int L, int H, int d) {
    if (B <= 0 || L <= 0 || H <= 0 || d <= 0 || d % 2 != 0) return ORACLE_ERR_ARG;
    const int half = d / 2;
    for (int b = 0; b < B; ++b)
        for (int p = 0; p < L; ++p)
            for (int h = 0; h < H; ++h) {
                const double *xv = x + (((int64_t)b * L + p) * H + h) * d;
                double *ov = out + (((int64_t)b * L + p) * H + h) * d;
                for (int i = 0; i < half; ++i) {
                    double c = cos_t[(int64_t)p * half + i], sn = sin_t[(int64_t)p * half + i];
                    double x0 = xv[2 * i], x1 = xv[2 * i + 1];
                    ov[i] = x0 * c - x1 * sn;
                    ov[half + i] = x0 * sn + x1 * c;
                }
            }
    return 0;
}

/* One vector: out = rotation of x (length d) by the table rows c, s (length d/2). */
static void rope_vec(const double *x, const double *c, const double *s, double *out, int d) {
    const int half = d / 2;
    for (int i = 0; i < half; ++i) {
        out[i] = x[2 * i] * c[i] - x[2 * i + 1] * s[i];
        out[half + i] = x[2 * i] * s[i] + x[2 * i + 1] * c[i];
    }
}

/*
 * Decode step with rotary embedding: the new token of sequence b sits at
 * position seqlens[b] (0 <= seqlens[b] < S); q [B][h_q][d] and k_new
 * [B][h_kv][d] are rotated with row seqlens[b] of cos, sin [S][d/2], the
 * rotated key and v_new are appended (gqa_oracle_decode_append), then the
 * token attends.
 */
int gqa_oracle_decode_append(const double *q, const double *k_new, const double *v_new,
                             double *k_cache, double *v_cache, const int32_t *seqlens,
                             double *o, int B, int h_q, int h_kv, int S, int d);

int gqa_oracle_decode_append_rope(const double *q, const double *k_new, const double *v_new,
                                  double *k_cache, double *v_cache, const int32_t *seqlens,
                                  const double *cos_t, const double *sin_t, double *o, int B,
                                  int h_q, int h_kv, int S, int d) {
    if (B <= 0 || S <= 0 || d <= 0 || d % 2 != 0) return ORACLE_ERR_ARG;
    if (check_heads(h_q, h_kv)) return ORACLE_ERR_ARG;
    for (int b = 0; b < B; ++b)
        if (seqlens[b] < 0 || seqlens[b] >= S) return ORACLE_ERR_ARG;
    double *qr = (double *)malloc(sizeof(double) * (size_t)B * h_q * d);
    double *kr = (double *)malloc(sizeof(double) * (size_t)B * h_kv * d);
    if (!qr || !kr) {
        free(qr);
        free(kr);
        return ORACLE_ERR_NOMEM;
    }
    const int half = d / 2;
    for (int b = 0; b < B; ++b) {
        const long p = seqlens[b];
        for (int h = 0; h < h_q; ++h)
            rope_vec(q + ((long)b * h_q + h) * d, cos_t + p * half, sin_t + p * half,
                     qr + ((long)b * h_q + h) * d, d);
        for (int g = 0; g < h_kv; ++g)
            rope_vec(k_new + ((long)b * h_kv + g) * d, cos_t + p * half, sin_t + p * half,
                     kr + ((long)b * h_kv + g) * d, d);
    }
    int rc = gqa_oracle_decode_append(qr, kr, v_new, k_cache, v_cache, seqlens, o, B, h_q, h_kv,
                                      S, d);
    free(qr);
    free(kr);
    return rc;
}

/*
 * Prefill with rotary embedding: q, k rotated (gqa_oracle_rope), then the full
 * prefill; k_rot [B][L][h_kv][d] receives the rotated keys.
 */
int gqa_oracle_prefill_rope(const double *q, const double *k, const double *v,
                            const double *cos_t, const double *sin_t, double *o, double *k_rot,
                            int B, int L, int h_q, int h_kv, int d, int causal, double scale) {
    if (B <= 0 || L <= 0 || d <= 0 || d % 2 != 0) return ORACLE_ERR_ARG;
    if (check_heads(h_q, h_kv)) return ORACLE_ERR_ARG;
    double *q_rot = (double *)malloc(sizeof(double) * (size_t)B * L * h_q * d);
    if (!q_rot) return ORACLE_ERR_NOMEM;
    int rc = gqa_oracle_rope(q, cos_t, sin_t, q_rot, B, L, h_q, d);
    if (rc == 0) rc = gqa_oracle_rope(k, cos_t, sin_t, k_rot, B, L, h_kv, d);
    if (rc == 0) rc = prefill_general(q_rot, k_rot, v, o, B, L, L, h_q, h_kv, d, causal, scale,
                                      NULL, NULL);
    free(q_rot);
    return rc;
}

/*
 * Prefill of L_q new positions against L_k keys (chunked prefill):
 *   q, o [B][L_q][h_q][d];  k, v [B][L_k][h_kv][d];  1 <= L_q <= L_k.
 * probs: NULL, or [B][h_q][L_q][L_k].
 */
int gqa_oracle_prefill_cached(const double *q, const double *k, const double *v, double *o,
                              int B, int Lq, int Lk, int h_q, int h_kv, int d, int causal,
                              double scale, double *probs) {
    return prefill_general(q, k, v, o, B, Lq, Lk, h_q, h_kv, d, causal, scale, probs, NULL);
}

/*
 * Decode: q, o [B][h_q][d] (the single new position of each sequence);
 * k_cache, v_cache [B][h_kv][S][d]; seqlens [B] with 0 <= seqlens[b] <= S.
 * scale = 1/sqrt(d).
 */
/*
 * Decode over a cache whose element (b, j, g, c) sits at b*sb + j*sj + g*sh + c.
 */
static int decode_strided(const double *q, const double *k_cache, const double *v_cache,
                          const int32_t *seqlens, double *o, int B, int h_q, int h_kv, int S,
                          int d, long sb, long sj, long sh) {
    if (B <= 0 || S <= 0 || d <= 0) return ORACLE_ERR_ARG;
    if (check_heads(h_q, h_kv)) return ORACLE_ERR_ARG;
    for (int b = 0; b < B; ++b)
        if (seqlens[b] < 0 || seqlens[b] > S) return ORACLE_ERR_ARG;
    const double scale = 1.0 / sqrt((double)d);
    int failed = 0;
#pragma omp parallel
    {
        double *krep = (double *)malloc(sizeof(double) * (size_t)S * d);
        double *vrep = (double *)malloc(sizeof(double) * (size_t)S * d);
        double *scores = (double *)malloc(sizeof(double) * (size_t)S);
        if (!krep || !vrep || !scores) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t bh = 0; bh < (int64_t)B * h_q; ++bh) {
                int b = (int)(bh / h_q), h = (int)(bh % h_q);
                int kvh = kv_head_of(h, h_q, h_kv);
                int n = seqlens[b];
                repeat_kv_slab(k_cache, sb, sj, sh, b, kvh, n, d, krep);
                repeat_kv_slab(v_cache, sb, sj, sh, b, kvh, n, d, vrep);
                attend_one_row(q + bh * d, krep, vrep, n, d, scale, scores, o + bh * d,
                               NULL);
            }
        }
        free(krep);
        free(vrep);
        free(scores);
    }
    return failed ? ORACLE_ERR_NOMEM : 0;
}

/* Decode over a head-major cache [B][h_kv][S][d]. */
int gqa_oracle_decode(const double *q, const double *k_cache, const double *v_cache,
                      const int32_t *seqlens, double *o, int B, int h_q, int h_kv, int S,
                      int d) {
    const long sj = d, sh = (long)S * d, sb = (long)h_kv * sh;
    return decode_strided(q, k_cache, v_cache, seqlens, o, B, h_q, h_kv, S, d, sb, sj, sh);
}

/* Decode over a token-major cache [B][S][h_kv][d]. */
int gqa_oracle_decode_token_major(const double *q, const double *k_cache,
                                  const double *v_cache, const int32_t *seqlens, double *o,
                                  int B, int h_q, int h_kv, int S, int d) {
    const long sh = d, sj = (long)h_kv * d, sb = (long)S * sj;
    return decode_strided(q, k_cache, v_cache, seqlens, o, B, h_q, h_kv, S, d, sb, sj, sh);
}

/*
 * Decode over a paged cache: k_pages, v_pages [num_pages][h_kv][page_size][d],
 * block_table [B][max_blocks].  The logical cache of every sequence is first
 * gathered row by row into a head-major [B][h_kv][S][d] copy,
 * S = max_blocks * page_size, then decoded.  seqlens[b] <= S, and every block
 * that holds a position below seqlens[b] must name a page in [0, num_pages).
 */
int gqa_oracle_decode_paged(const double *q, const double *k_pages, const double *v_pages,
                            const int32_t *block_table, const int32_t *seqlens, double *o,
                            int B, int h_q, int h_kv, int page_size, int max_blocks,
                            int num_pages, int d) {
    if (B <= 0 || page_size <= 0 || max_blocks <= 0 || num_pages <= 0 || d <= 0)
        return ORACLE_ERR_ARG;
    if (check_heads(h_q, h_kv)) return ORACLE_ERR_ARG;
    const long S = (long)max_blocks * page_size;
    if (S > 0x7fffffff) return ORACLE_ERR_ARG;
    for (int b = 0; b < B; ++b) {
        if (seqlens[b] < 0 || seqlens[b] > S) return ORACLE_ERR_ARG;
        for (int i = 0; i * (long)page_size < seqlens[b]; ++i) {
            int page = block_table[(long)b * max_blocks + i];
            if (page < 0 || page >= num_pages) return ORACLE_ERR_ARG;
        }
    }
    size_t n = (size_t)B * h_kv * S * d;
    double *kc = (double *)calloc(n, sizeof(double));
    double *vc = (double *)calloc(n, sizeof(double));
    if (!kc || !vc) {
        free(kc);
        free(vc);
        return ORACLE_ERR_NOMEM;
    }
    for (int b = 0; b < B; ++b)
        for (int g = 0; g < h_kv; ++g)
            for (int j = 0; j < seqlens[b]; ++j) {
                long page = block_table[(long)b * max_blocks + j / page_size];
                long src = ((page * h_kv + g) * page_size + j % page_size) * d;
                long dst = (((long)b * h_kv + g) * S + j) * d;
                memcpy(kc + dst, k_pages + src, sizeof(double) * (size_t)d);
                memcpy(vc + dst, v_pages + src, sizeof(double) * (size_t)d);
            }
    int rc = gqa_oracle_decode(q, kc, vc, seqlens, o, B, h_q, h_kv, (int)S, d);
    free(kc);
    free(vc);
    return rc;
}

/*
 * Decode with append: k_new, v_new [B][h_kv][d] are copied into row
 * seqlens[b] of k_cache, v_cache [B][h_kv][S][d] (modified in place), then
 * q [B][h_q][d] attends over rows [0, seqlens[b] + 1) with scale 1/sqrt(d).
 * Requires 0 <= seqlens[b] < S.
 */
int gqa_oracle_decode_append(const double *q, const double *k_new, const double *v_new,
                             double *k_cache, double *v_cache, const int32_t *seqlens,
                             double *o, int B, int h_q, int h_kv, int S, int d) {
    if (B <= 0 || S <= 0 || d <= 0) return ORACLE_ERR_ARG;
    if (check_heads(h_q, h_kv)) return ORACLE_ERR_ARG;
    for (int b = 0; b < B; ++b)
        if (seqlens[b] < 0 || seqlens[b] >= S) return ORACLE_ERR_ARG;
    int32_t *grown = (int32_t *)malloc(sizeof(int32_t) * (size_t)B);
    if (!grown) return ORACLE_ERR_NOMEM;
    /* append: the new rows become cache row seqlens[b] */
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < h_kv; ++g) {
            long row = (((long)b * h_kv + g) * S + seqlens[b]) * d;
            memcpy(k_cache + row, k_new + ((long)b * h_kv + g) * d, sizeof(double) * (size_t)d);
            memcpy(v_cache + row, v_new + ((long)b * h_kv + g) * d, sizeof(double) * (size_t)d);
        }
        grown[b] = seqlens[b] + 1;
    }
    /* then attend over the grown cache */
    int rc = gqa_oracle_decode(q, k_cache, v_cache, grown, o, B, h_q, h_kv, S, d);
    free(grown);
    return rc;
}
