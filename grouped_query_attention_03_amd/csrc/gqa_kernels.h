// gqa_kernels.h -- internal launch interface between the C ABI and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

// Prefill work map: a work-group covers GW query heads of one group (a
// "subgroup"; nsub = G / GW of them per key/value head) times BM positions.
// L query positions attend to Lk >= L keys per sequence; query row i sits at
// position off + i, off = Lk - L (0 for the square prefill).
struct PrefillArgs {
    const void *q, *k, *v;
    void *o;
    int B, L, Lk, off, h_q, h_kv, G;
    int GW, nsub, BM;
    int n_units;   // B * h_kv * nsub
    int n_qtiles;  // ceil(L / BM)
    float c;       // scale * log2(e)
    // c is an exact power of two: q * c is exact in bf16 and may be folded
    // into q (the plain bf16 form only); otherwise c multiplies the fp32 scores
    int fold;
    // rotary tables cos, sin [positions][d/2] fp32 (row p for position p);
    // non-null only in the rotary form, where q is rotated as it is loaded
    const float *rope_cos, *rope_sin;
    // per-sequence key lengths [B] (key j of sequence b visible iff j <
    // kv_lens[b]), or null: all Lk keys
    const int32_t *kv_lens;
    // keep-mask bytes, or null: key j is visible to query row i of sequence b
    // only if mask[b * mask_batch + i * mask_row + j] != 0 (strides in bytes;
    // mask_row a multiple of 16, L * mask_row < 2^32)
    const uint8_t *mask;
    long long mask_row, mask_batch;
    // keep-mask form, bf16: the mask's summary per (sequence, query tile,
    // 64-key tile), [B][n_qtiles][mc_stride] bytes (mc_stride = ceil(L_k / 64)
    // rounded up to a multiple of 8), and the order [B * n_qtiles] in which
    // the prefill takes the (sequence, query tile) items, both written by
    // first passes and read by the prefill
    uint8_t *mcodes;
    int32_t *morder;
    int *mwork;  // the persistent prefill's work counters (one per XCD), zeroed by the ordering pass
    int mc_stride;
};

// Rotary embedding of rows x [rows][d] into out, tables cos, sin [L][d/2].
// Without pos the rows are in [B][L][h] order and row r sits at position
// (r / h) % L; with pos ([B], one new token per sequence) the rows are in
// [B][h] order and row r sits at position pos[r / h], clamped to [0, L - 1].
struct RopeArgs {
    const void *x;
    void *out;
    const float *cos, *sin;
    long long rows;  // B * L * h, or B * h with pos
    int L, h;
    const int32_t *pos;
    // optional second segment of rows, rotated in the same launch (the new
    // token's k rows after its q rows): x2 -> out2, rows2 rows of h2 heads
    const void *x2;
    void *out2;
    long long rows2;
    int h2;
};

// Waves per work-group of the decode split pass; with one work-group per CU
// resident (its LDS ring fills the CU), 256 CUs x kDecodeWaves waves run at once.
constexpr int kDecodeWaves = 4;

// Where row j of (sequence b, key/value head g) of a decode cache sits.
enum DecodeLayout {
    kLayoutHeadMajor = 0,   // [B][h_kv][S][d]
    kLayoutTokenMajor = 1,  // [B][S][h_kv][d]
    kLayoutPaged = 2        // pool [pages][h_kv][page_size][d], block_table[b][j / page_size]
};

struct DecodeArgs {
    const void *q, *k_cache, *v_cache;
    const void *k_new, *v_new;  // [B, h_kv, d] rows appended at seqlens[b] (append form), else null
    int extra;                  // rows attended = seqlens[b] + extra (1 for the append form)
    const int32_t *seqlens;
    void *o;
    float *opart;  // [NW + segments][16][d] per-slot partial outputs (normalised)
    float *lse;    // [NW + segments][16] base-2 log-sum-exp of each partial, scaled units
    int B, h_q, h_kv, G, S;
    int NW;        // waves in the split pass (number of slices of the block list)
    int n_qsub;    // query-head subgroups of at most 16 heads per key/value head
    float c;       // log2(e) / sqrt(d)
    int layout;    // DecodeLayout of k_cache / v_cache
    const int32_t *block_table;  // paged: [B][max_blocks] page of each block of page_size rows
    int page_size, max_blocks;   // paged: page_size a multiple of 32
};

int launch_prefill_bf16(const PrefillArgs &a, int d, bool causal, hipStream_t stream);
int launch_rope_k_bf16(const RopeArgs &a, int d, hipStream_t stream);
int launch_prefill_f32(const PrefillArgs &a, int d, bool causal, hipStream_t stream);
int launch_decode_bf16(const DecodeArgs &a, int d, hipStream_t stream);

}  // namespace gqa
