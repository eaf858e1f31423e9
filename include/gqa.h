/*
 * gqa.h -- C ABI of the MI355X (gfx950) grouped-query attention core.
 *
 * The library computes O = softmax(Q K^T * scale) V per query head, where the
 * h_q query heads are split into h_kv groups of G = h_q / h_kv consecutive
 * heads and every head of a group reads the group's single key/value head:
 * query head h uses key/value head floor(h / G).  The key/value heads are never
 * copied per query head.
 *   - attention formula: "Modern LLM architecture (1): GQA and RMSNorm", §2.1;
 *   - grouping and the floor(h / G) head map: the same page, §2.3, and
 *     "Attention in Qwen, DeepSeek and LLaMA3", §2.2 and §2.3;
 *   - h_q must be a whole multiple of h_kv: "What is Grouped-Query Attention",
 *     §2.2.
 *
 * Conventions shared by every entry point
 *   - Pointers are DEVICE pointers (hipMalloc'd or equivalent), dense and
 *     row-major in the layouts given below, 16-byte aligned.  The caller owns
 *     every buffer, including the decode workspace; the library allocates and
 *     frees nothing and keeps no state between calls, so concurrent calls on
 *     different streams are safe as long as their output/workspace buffers do
 *     not overlap.
 *   - `hip_stream` is a hipStream_t (NULL = the default stream).  Work is
 *     enqueued asynchronously; the caller synchronises.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     non-zero status means nothing was launched.  GQA_ERR_LAUNCH reports a
 *     failure returned by the HIP runtime at launch time.  No entry point
 *     throws or aborts.
 *   - Accumulation and softmax statistics are fp32; outputs have the input
 *     dtype (bf16 outputs are rounded to nearest even).
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o.  A plain int, so that any value a caller
 * passes is defined behaviour and is rejected with GQA_ERR_DTYPE when it is
 * neither constant. */
typedef int gqa_dtype;
enum { GQA_F32 = 0, GQA_BF16 = 1 };

typedef int gqa_status;
enum {
    GQA_OK = 0,
    GQA_ERR_NULL_POINTER = 1,  /* a required pointer is NULL */
    GQA_ERR_ALIGNMENT = 2,     /* a pointer is not 16-byte aligned */
    GQA_ERR_SIZE = 3,          /* a size or split count is out of range, or scale is not > 0 */
    GQA_ERR_HEADS = 4,         /* h_q is not a multiple of h_kv */
    GQA_ERR_HEAD_DIM = 5,      /* d is not 64 or 128 */
    GQA_ERR_DTYPE = 6,         /* dtype not supported by this entry point */
    GQA_ERR_WORKSPACE = 7,     /* workspace NULL, misaligned or smaller than required */
    GQA_ERR_LAUNCH = 8,        /* the HIP runtime reported an error at launch */
    GQA_ERR_DEVICE = 9,        /* the current device is not a gfx950 GPU */
    GQA_ERR_SCRATCH = 10       /* gqa_decode_noalloc: the call needs more than its fixed scratch */
};

/*
 * Prefill: every position attends to the keys of its own sequence.
 *   q, o : [B, L, h_q, d]   (dtype dt)
 *   k, v : [B, L, h_kv, d]  (dtype dt)
 *   causal != 0: position i attends to keys 0..i (square alignment); else to all L.
 *   scale: multiplies Q K^T before the softmax; pass 1/sqrt(d) for the usual form.
 *   dt: GQA_BF16 (bf16 MFMA path) or GQA_F32 (fp32 path).
 * The causal mask follows the masked_fill(mask == 0, -inf) form of
 * "Modern LLM architecture (1): GQA and RMSNorm", §2.1-§2.3.
 * Limits: B * h_q * L and B * h_kv * L must each fit in 2^31 elements of d;
 * for GQA_BF16 also L * h_kv * d * 2 (the bytes spanned by one sequence's
 * key or value rows) must be below 2^32.  Larger calls return GQA_ERR_SIZE.
 * Precision (GQA_BF16): q and k enter the products exactly as given; the
 * scores are accumulated in fp32 and multiplied by scale * log2(e) in fp32
 * (one fused multiply-add with the running max), so a score of any size is
 * exact to fp32 rounding.  When scale * log2(e) is an exact power of two it is
 * folded into q instead (exact in bf16 unless q * scale * log2(e) leaves the
 * normal range).  The probabilities are rounded to bf16 before the product
 * with v, and the row sums are taken over the rounded values; accumulation
 * and the softmax statistics are fp32.
 */
gqa_status gqa_prefill(const void *q, const void *k, const void *v, void *o, int B, int L,
                       int h_q, int h_kv, int d, gqa_dtype dt, int causal, float scale,
                       void *hip_stream);

/*
 * Chunked prefill: the L_q newest positions of each sequence attend to all L_k
 * keys of that sequence (1 <= L_q <= L_k), i.e. a chunk of new tokens whose
 * keys and values were appended after L_k - L_q earlier ones ("What is
 * Grouped-Query Attention", §3.2: append to the cache, then attend).  Run
 * chunk by chunk this reproduces one full causal prefill exactly, unlike
 * processing each chunk on its own ("Implementing GQA from scratch in
 * PyTorch", §4.3).
 *   q, o : [B, L_q, h_q, d]   (dtype dt)
 *   k, v : [B, L_k, h_kv, d]  (dtype dt), positions 0 .. L_k - 1
 *   causal != 0: query row i sits at position L_k - L_q + i and attends to keys
 *          0 .. L_k - L_q + i (bottom-right alignment); else to all L_k keys.
 *   Other arguments, limits and errors as gqa_prefill, with L_k in place of L
 *   for k and v; L_q > L_k returns GQA_ERR_SIZE.  gqa_prefill(..., L, ...) is
 *   gqa_prefill_chunk(..., L, L, ...).
 */
gqa_status gqa_prefill_chunk(const void *q, const void *k, const void *v, void *o, int B,
                             int L_q, int L_k, int h_q, int h_kv, int d, gqa_dtype dt,
                             int causal, float scale, void *hip_stream);

/*
 * Prefill of a padded batch of variable-length sequences.  The attention mask
 * that handles variable-length sequences ("Implementing GQA from scratch in
 * PyTorch", §3.3: masked_fill(mask == 0, -inf)) given as lengths: key j of
 * sequence b is visible iff j < kv_lens[b] (and j <= i when causal).
 *   q, k, v, o, B, L, h_q, h_kv, d, dt, causal, scale: as gqa_prefill (both
 *          dtypes); positions at or beyond kv_lens[b] are padding.
 *   kv_lens : [B] int32 on the device, 4-byte aligned; values are clamped to
 *          [0, L] on the device.  Key/value rows at or beyond kv_lens[b] are
 *          never read into a result (they may hold anything, NaN included).
 * Every query row is computed, padded rows included: a padded row attends to
 * all kv_lens[b] keys.  A row with no visible key (kv_lens[b] == 0) is zero.
 * With every kv_lens[b] == L the result equals gqa_prefill bit for bit.
 */
gqa_status gqa_prefill_varlen(const void *q, const void *k, const void *v, void *o,
                              const int32_t *kv_lens, int B, int L, int h_q, int h_kv, int d,
                              gqa_dtype dt, int causal, float scale, void *hip_stream);

/*
 * Prefill with a keep-mask: key j is visible to query row i of sequence b only
 * if its mask byte is nonzero, the masked_fill(mask == 0, -inf) convention of
 * "Implementing GQA from scratch in PyTorch", §3.3 and of the attn_mask
 * argument in "Modern LLM architecture (1): GQA and RMSNorm", §2.3, combined
 * with the causal mask when causal != 0.  The mask is shared by all heads.
 *   q, o : [B, L_q, h_q, d]; k, v : [B, L_k, h_kv, d] (1 <= L_q <= L_k), as
 *          gqa_prefill_chunk: query row i sits at position L_k - L_q + i, and
 *          causally sees keys 0 .. L_k - L_q + i.
 *   mask : device bytes, 16-byte aligned; the byte of (b, i, j) is
 *          mask[b * mask_batch_stride + i * mask_row_stride + j].
 *   mask_row_stride   : bytes between rows, a multiple of 16 and >= L_k, with
 *          L_q * mask_row_stride below 2^32 (a dense [B, L_q, L_k] mask whose
 *          L_k is not a multiple of 16 is padded per row to one that is).
 *   mask_batch_stride : bytes between sequences, a multiple of 16; 0 shares one
 *          [L_q, L_k] mask across the batch.  The caller's buffer must hold
 *          (B - 1) * mask_batch_stride + L_q * mask_row_stride bytes; the
 *          bytes of a row past L_k are read but ignored.
 *   workspace : device buffer of at least gqa_prefill_mask_workspace_bytes(B,
 *          L_q, L_k) bytes, 16-byte aligned.  The bf16 path writes into it a
 *          summary of the mask (per sequence, query tile and 64 keys: whether
 *          none, some or all of the keys the tile's rows may see are visible)
 *          and the order in which the query tiles are taken (most visible key
 *          tiles first), and reads both back in the same call, so its
 *          contents on entry are ignored; the fp32 path does not touch it.
 *          Calls that overlap in time must not share one.
 * A row with no visible key is zero.  Masked keys receive weight exactly 0, so
 * every key/value row must be finite (0 times a NaN would still be NaN).
 * With every mask byte nonzero the result equals gqa_prefill_chunk.
 * Other arguments, limits and errors as gqa_prefill_chunk (both dtypes); a
 * NULL mask gives GQA_ERR_NULL_POINTER, a misaligned one GQA_ERR_ALIGNMENT,
 * strides breaking the rules above GQA_ERR_SIZE, and a NULL, misaligned or
 * too small workspace GQA_ERR_WORKSPACE.  In bf16 three kernels run on
 * `hip_stream`: the mask's summary, the order of the query tiles, then the
 * prefill.
 */
gqa_status gqa_prefill_mask(const void *q, const void *k, const void *v, const uint8_t *mask,
                            long long mask_row_stride, long long mask_batch_stride, void *o,
                            int B, int L_q, int L_k, int h_q, int h_kv, int d, gqa_dtype dt,
                            int causal, float scale, void *workspace, size_t workspace_bytes,
                            void *hip_stream);

/* Bytes of workspace gqa_prefill_mask needs: B * ceil(L_q / 32) rows of
 * ceil(L_k / 64) bytes rounded up to a multiple of 8, then 4 bytes for each
 * of those B * ceil(L_q / 32) query tiles, each part rounded up to 256, then
 * 256 bytes for the eight per-XCD work counters (0 when B <= 0, L_q <= 0 or
 * L_k < L_q). */
size_t gqa_prefill_mask_workspace_bytes(int B, int L_q, int L_k);

/*
 * Prefill with rotary position embedding: q and k are rotated, then the
 * prefill above runs on the rotated q, k and the unrotated v ("Attention in
 * Qwen, DeepSeek and LLaMA3", §1, apply_rotary_pos_emb).  For a row x at
 * position p and pair i (0 <= i < d/2):
 *   x'[i]       = x[2i] cos[p][i] - x[2i+1] sin[p][i]
 *   x'[d/2 + i] = x[2i] sin[p][i] + x[2i+1] cos[p][i]
 * (the even/odd pairs rotated, the two halves concatenated as the page writes
 * them).
 *   q, k, v, o, B, L, h_q, h_kv, d, causal, scale: as gqa_prefill; dt must be
 *          GQA_BF16 (else GQA_ERR_DTYPE).
 *   cos_table, sin_table : [L, d/2] fp32 device arrays, row p for position p,
 *          16-byte aligned.  Any values: the call does not assume
 *          cos^2 + sin^2 = 1.
 *   k_rot : [B, L, h_kv, d] bf16 output, the rotated keys (what a cache holds);
 *          the attention reads the keys from here.  It must not overlap k
 *          (k_rot == k returns GQA_ERR_SIZE).
 * The keys are rotated by one small kernel (fp32 arithmetic, one rounding to
 * bf16); q is rotated in fp32 as the prefill kernel loads it and rounded to
 * bf16 once; the scores are then scaled in fp32 as in gqa_prefill.  Two
 * kernels run on `hip_stream`.
 */
gqa_status gqa_prefill_rope(const void *q, const void *k, const void *v, const float *cos_table,
                            const float *sin_table, void *o, void *k_rot, int B, int L, int h_q,
                            int h_kv, int d, gqa_dtype dt, int causal, float scale,
                            void *hip_stream);

/*
 * Decode: one new query position per sequence attends to rows [0, seqlens[b])
 * of a head-major key/value cache ("What is Grouped-Query Attention", §2.2 step
 * 2 for the [batch, g, seq_len, d_head] cache and §3.2 for appending the new
 * token's key/value before attending, which the caller has already done).
 *   q, o               : [B, 1, h_q, d]  bf16
 *   k_cache, v_cache   : [B, h_kv, S, d] bf16
 *   seqlens            : [B] int32 on the device, each in [0, S].  The kernels
 *                        clamp a value outside that range into it, so no row
 *                        outside the sequence's cache is ever read.
 *                        seqlens[b] == 0 yields a zero output row.
 *                        Cache rows at or beyond seqlens[b] are never read.
 *   scale is fixed to 1/sqrt(d).
 *   num_splits: how many slices the valid cache blocks are cut into (one wave
 *          of the split pass per slice); 0 picks the library default, else
 *          1 .. 2^20.  The result does not depend on it beyond floating-point
 *          rounding.
 *   workspace: device buffer of at least gqa_decode_workspace_bytes(...) bytes
 *          holding per-slice partial outputs and log-sum-exp values; its
 *          contents on entry are ignored.
 * Two kernels run on `hip_stream`: the split pass (each wave streams one
 * contiguous, equally sized slice of all sequences' valid 32-key blocks) and a
 * log-sum-exp merge pass over (sequence, query head).
 */
gqa_status gqa_decode(const void *q, const void *k_cache, const void *v_cache,
                      const int32_t *seqlens, void *o, int B, int h_q, int h_kv, int S, int d,
                      gqa_dtype dt, int num_splits, void *workspace, size_t workspace_bytes,
                      void *hip_stream);

/*
 * Decode that allocates nothing, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid it): gqa_decode with its workspace in a fixed array in device memory
 * that the library holds, one per GPU, until the process ends.
 *   q, k_cache, v_cache, seqlens, o, B, h_q, h_kv, S, d, dt, num_splits,
 *   hip_stream: as gqa_decode; the caller passes every input and output.
 * The array holds gqa_decode_noalloc_max_bytes() bytes (32 MiB); a call whose
 * gqa_decode_workspace_bytes(...) exceeds that returns GQA_ERR_SCRATCH (after
 * the argument checks gqa_decode makes; nothing is launched).  No call
 * allocates or frees memory; the first call on a GPU looks up the array's
 * address there.
 * Every call on one GPU uses that GPU's one array, so calls that overlap in
 * time on one GPU (on different streams, or from different threads) race;
 * calls in sequence on one stream are safe (the array's contents on entry
 * are ignored).  Results are those of gqa_decode with the same arguments.
 */
gqa_status gqa_decode_noalloc(const void *q, const void *k_cache, const void *v_cache,
                              const int32_t *seqlens, void *o, int B, int h_q, int h_kv, int S,
                              int d, gqa_dtype dt, int num_splits, void *hip_stream);

/* Bytes of the fixed scratch array gqa_decode_noalloc uses on each GPU. */
size_t gqa_decode_noalloc_max_bytes(void);

/*
 * Decode over a token-major cache: as gqa_decode, with the cache laid out
 * [B, S, h_kv, d] (the kv_cache shape of "Attention in Qwen, DeepSeek and
 * LLaMA3", §2.2, and the layout prefill takes its k and v in, so a prefill's
 * keys and values can be attended by later tokens without a transpose).
 *   k_cache, v_cache : [B, S, h_kv, d] bf16; rows of one key/value head are
 *                      h_kv * d elements apart.
 *   Everything else, the workspace and errors as gqa_decode.
 */
gqa_status gqa_decode_token_major(const void *q, const void *k_cache, const void *v_cache,
                                  const int32_t *seqlens, void *o, int B, int h_q, int h_kv, int S,
                                  int d, gqa_dtype dt, int num_splits, void *workspace,
                                  size_t workspace_bytes, void *hip_stream);

/*
 * Decode over a paged cache with group-aligned pages ("Attention in Qwen,
 * DeepSeek and LLaMA3", §4.3: one page per group, so the rows of one
 * key/value head inside a page are contiguous).
 *   k_pages, v_pages : [num_pages, h_kv, page_size, d] bf16: physical block p
 *                      holds page_size consecutive positions of one sequence,
 *                      one contiguous page per key/value head.
 *   block_table      : [B, max_blocks] int32 on the device; block_table[b][i]
 *                      is the physical block holding positions
 *                      [i * page_size, (i + 1) * page_size) of sequence b.
 *                      Entries for blocks at or beyond ceil(seqlens[b] /
 *                      page_size) are never read; the others must name blocks
 *                      of the pool (not checked on the device).  Blocks may be
 *                      shared between sequences (a common prefix).
 *   seqlens          : [B] int32 on the device, each in [0, max_blocks * page_size]
 *                      (clamped into that range on the device, as in gqa_decode).
 *   page_size        : a positive multiple of 32; max_blocks > 0;
 *                      max_blocks * page_size and B * max_blocks below 2^31,
 *                      else GQA_ERR_SIZE.
 *   Everything else, the workspace and errors as gqa_decode; a NULL or
 *   misaligned (4-byte) block_table gives GQA_ERR_NULL_POINTER / GQA_ERR_ALIGNMENT.
 */
gqa_status gqa_decode_paged(const void *q, const void *k_pages, const void *v_pages,
                            const int32_t *block_table, const int32_t *seqlens, void *o, int B,
                            int h_q, int h_kv, int page_size, int max_blocks, int d, gqa_dtype dt,
                            int num_splits, void *workspace, size_t workspace_bytes,
                            void *hip_stream);

/*
 * Decode with append: the new token's key and value rows are written into the
 * cache, then the token attends over the grown cache ("What is Grouped-Query
 * Attention", §3.2: append, then attend), in one call.
 *   q, o             : [B, 1, h_q, d]  bf16
 *   k_new, v_new     : [B, 1, h_kv, d] bf16 (the new token's key and value rows)
 *   k_cache, v_cache : [B, h_kv, S, d] bf16; row seqlens[b] of every key/value
 *                      head is overwritten with k_new / v_new, no other byte of
 *                      the caches is written
 *   seqlens          : [B] int32 on the device, the lengths BEFORE the append,
 *                      each in [0, S - 1]; the token attends over rows
 *                      [0, seqlens[b] + 1).  The caller advances seqlens.
 *                      A value outside [0, S - 1] is clamped into it for the
 *                      attention (the clamped length's rows, then the new row)
 *                      and nothing is written into that sequence's cache.
 *   Other arguments, the workspace and errors as gqa_decode; the workspace size
 *   is gqa_decode_workspace_bytes of the same sizes.  The new rows are read
 *   from k_new / v_new for the attention, so no part of the call depends on
 *   the order of the cache write.
 */
gqa_status gqa_decode_append(const void *q, const void *k_new, const void *v_new, void *k_cache,
                             void *v_cache, const int32_t *seqlens, void *o, int B, int h_q,
                             int h_kv, int S, int d, gqa_dtype dt, int num_splits,
                             void *workspace, size_t workspace_bytes, void *hip_stream);

/*
 * Decode step with rotary position embedding: the new token of sequence b sits
 * at position seqlens[b]; its query and key rows are rotated with row
 * seqlens[b] of the tables (the rotation of gqa_prefill_rope, "Attention in
 * Qwen, DeepSeek and LLaMA3", §1), the rotated key and v_new are appended at
 * cache row seqlens[b], and the token attends over rows [0, seqlens[b] + 1)
 * ("What is Grouped-Query Attention", §3.2).  The cache therefore holds rotated
 * keys, as gqa_prefill_rope's k_rot does.
 *   q, k_new, v_new, k_cache, v_cache, seqlens, o, sizes: as gqa_decode_append.
 *   cos_table, sin_table : [S, d/2] fp32 device arrays, 16-byte aligned; a
 *          position outside [0, S - 1] (a broken precondition) is clamped.
 *   workspace : at least gqa_decode_rope_workspace_bytes(...) bytes (the
 *          decode's part, then the rotated q and k_new rows).
 * Everything is validated before anything is enqueued; errors as
 * gqa_decode_append.  Three kernels run on `hip_stream`: the rotation of the
 * new token's q and k rows (one launch), then the split and merge passes.
 */
gqa_status gqa_decode_append_rope(const void *q, const void *k_new, const void *v_new,
                                  void *k_cache, void *v_cache, const int32_t *seqlens,
                                  const float *cos_table, const float *sin_table, void *o, int B,
                                  int h_q, int h_kv, int S, int d, gqa_dtype dt, int num_splits,
                                  void *workspace, size_t workspace_bytes, void *hip_stream);

/* Bytes of workspace gqa_decode_append_rope needs (0 when an argument is invalid). */
size_t gqa_decode_rope_workspace_bytes(int B, int h_q, int h_kv, int d, int num_splits);

/* Bytes of decode workspace needed for these sizes and num_splits (0 =
 * default); returns 0 when an argument is invalid. */
size_t gqa_decode_workspace_bytes(int B, int h_q, int h_kv, int d, int num_splits);

/* The number of slices gqa_decode uses when passed num_splits == 0. */
int gqa_decode_default_splits(void);

/* Static, NUL-terminated description of a status code. */
const char *gqa_status_string(gqa_status s);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */
