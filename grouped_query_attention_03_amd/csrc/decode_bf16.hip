// decode_bf16.hip -- grouped-query attention decode over a head-major KV cache.
//
// One new query position per sequence attends to cache rows [0, seqlens[b]) of
// k_cache/v_cache [B, h_kv, S, d] ("What is Grouped-Query Attention", §2.2 step 2
// for the cache layout, §3.2 for attending over the appended cache).  In the
// append form the new token's key and value rows are written into cache row
// seqlens[b] and attended as part of the same pass (rows [0, seqlens[b] + 1)),
// the order of §3.2.  The pass is bound by reading the cache, so every valid
// cache byte is read exactly once per key/value head, never once per query
// head, and the reads are kept streaming without bubbles:
//
// decode_split: a persistent, evenly balanced stream per wave.  The valid
//   32-key blocks of all (sequence, key/value head) segments form one list of
//   T blocks; wave w of NW takes the contiguous slice [w*T/NW, (w+1)*T/NW),
//   which may span several segments.  The G query heads of the segment's group
//   are stacked as the N dimension of v_mfma_f32_16x16x32_bf16 (S^T = K Q^T,
//   keys on M), so one read of a cache row serves every query head of the
//   group.  Q, K and V rows move with direct 16-byte loads into a per-wave LDS
//   ring; K comes back as the MFMA A operand, V transposed
//   (ds_read_b64_tr_b16) as the A operand of O^T = V^T P^T.  The next block's
//   loads are always in flight, also across segment boundaries.
//   For every segment it touches, a wave writes the segment's partial output
//   (normalised) and its log-sum-exp (base 2, in units of scale*log2(e)) to
//   slot w + segment of the workspace: the (wave, segment) pairs form a
//   monotone staircase, so those slots are distinct.
// decode_merge: one wave per (sequence, query head) finds the waves whose
//   slices cover its segment and combines their partials with weights
//   2^(lse - max lse): the exact log-sum-exp merge.
// Rows at or beyond seqlens[b] (seqlens[b] + 1 when appending) are never loaded
// from the cache.
#include "gqa_device.h"
#include "gqa_kernels.h"

namespace gqa {
namespace {

constexpr int DC_WAVES = kDecodeWaves;      // waves per work-group of the split pass
constexpr int DC_THREADS = 64 * DC_WAVES;
constexpr int DC_LDS_BYTES = 160 * 1024;    // LDS of one CU
constexpr int DC_BK = 32;          // keys per block
constexpr float DC_TAU = 8.0f;     // lazy-rescale threshold, log2 units

template <int D>
struct DcLayout {
    static constexpr int KSTEPS = D / 32;              // 16x16x32 k-steps over d
    static constexpr int ROW_BYTES = 2 * D;            // one cache row
    static constexpr int CPR = D / 8;                  // 16-byte chunks per row
    static constexpr int ROWS_PER_DMA = 64 / CPR;      // rows one 64-lane 16-byte load covers
    static constexpr int KV_DMA = DC_BK / ROWS_PER_DMA;  // loads per K (and per V) block
    static constexpr int TILE = DC_BK * ROW_BYTES;     // one K or V block in LDS
    static constexpr int ROWS_PER_SWEEP = 256 / ROW_BYTES;  // rows per pass over the 64 banks
};

// Tiles sit in LDS unpadded (each direct load writes 64 consecutive 16-byte
// chunks); chunk c of row r is stored at chunk position c ^ swz(r).
//   kswz: 16 lanes reading one 16-byte chunk of 16 consecutive rows (the
//         MFMA A/B operand reads of K and Q) hit 16 distinct 4-bank groups.
//   vswz: the 8 rows x 32 bytes of one half-wave transposing read of V hit
//         64 distinct banks.
template <int D>
__device__ __forceinline__ int kswz(int r) {
    using Lay = DcLayout<D>;
    return (r / Lay::ROWS_PER_SWEEP) % Lay::CPR;
}
template <int D>
__device__ __forceinline__ int vswz(int r) {
    using Lay = DcLayout<D>;
    return 2 * ((r / Lay::ROWS_PER_SWEEP) % (Lay::CPR / 2));
}

// Direct loads of `n_dma` x 1 KiB into `dst`: load i, lane l fetches row
// i * ROWS_PER_DMA + l / CPR (clamped to last_row), logical chunk
// (l % CPR) ^ swz(row), and the hardware stores it at byte 1024 i + 16 l.
// With LAST_ELSEWHERE, row last_row (and the clamped rows past it) is taken
// from the single row at last_src instead: the appended row, which is not in
// the cache yet.
template <int D, bool VSW, bool LAST_ELSEWHERE = false>
__device__ __forceinline__ void dc_dma_rows(const __bf16 *__restrict__ src, size_t row_stride,
                                            int row0, int last_row, int n_dma, GQA_LDS char *dst,
                                            const __bf16 *last_src = nullptr) {
    using Lay = DcLayout<D>;
    const int lane = threadIdx.x & 63;
    for (int i = 0; i < n_dma; ++i) {
        const int row = i * Lay::ROWS_PER_DMA + lane / Lay::CPR;
        const int chunk = (lane % Lay::CPR) ^ (VSW ? vswz<D>(row) : kswz<D>(row));
        const int srow = min(row0 + row, last_row);
        const __bf16 *p = src + (size_t)srow * row_stride + 8 * chunk;
        if (LAST_ELSEWHERE) p = srow == last_row ? last_src + 8 * chunk : p;
        dma16_to_lds(p, dst + i * 1024);
    }
}

// 16-byte read of logical chunk c of row r from a kswz-swizzled tile.
template <int D>
__device__ __forceinline__ bf16x8 dc_read_row_chunk(const GQA_LDS char *tile, int r, int c) {
    using Lay = DcLayout<D>;
    return *reinterpret_cast<const GQA_LDS bf16x8 *>(tile + r * Lay::ROW_BYTES +
                                                     16 * (c ^ kswz<D>(r)));
}

// One 32-key block: S^T = K Q^T, online-softmax update, O^T += V^T P^T, with
// Q, K and V read from this slot's LDS tiles.
template <int D, int QROWS>
__device__ __forceinline__ void dc_block(const GQA_LDS char *qt, const GQA_LDS char *kt,
                                         const GQA_LDS char *vt, int key0, int kend, bool qvalid,
                                         float c, float &m_run, float &l_run,
                                         f32x4 (&acc)[D / 16]) {
    using Lay = DcLayout<D>;
    constexpr int DB = D / 16;
    const int lane = threadIdx.x & 63, g = lane >> 4, jl = lane & 15;
    f32x4 s[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int ks = 0; ks < Lay::KSTEPS; ++ks) {
        // A = K rows (key jl of the m-block), B = Q^T (query column jl); d-chunk 4 ks + g.
        // Columns beyond the tile's QROWS heads read its last row and are zeroed.
        bf16x8 qf = dc_read_row_chunk<D>(qt, jl < QROWS ? jl : QROWS - 1, 4 * ks + g);
        qf = qvalid ? qf : bf16x8{};
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
            s[mb] = mfma16x16x32(dc_read_row_chunk<D>(kt, 16 * mb + jl, 4 * ks + g), qf, s[mb]);
    }
    if (key0 + DC_BK > kend) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (key0 + 16 * mb + 4 * g + r >= kend) s[mb][r] = -INFINITY;
    }
    // block max over the 32 keys of this query column (4 lanes share a column)
    float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                     fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, other_half(mx));
    const float mnew = mx * c;
    if (__any(mnew > m_run + DC_TAU)) {
        const float m2 = fmaxf(m_run, mnew);
        const float alpha = (m2 == -INFINITY) ? 1.f : fast_exp2(m_run - m2);
        m_run = m2;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] *= alpha;
    }
    const float mu = (m_run == -INFINITY) ? 0.f : m_run;
    bf16x8 pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float p = fast_exp2(fmaf(s[i >> 2][i & 3], c, -mu));
        l_run += p;
        pb[i] = (__bf16)p;
    }
    // V^T operand: transposing reads of rows 4g + jl/4 (and 16 rows further down)
    const int r0 = 4 * g + (jl >> 2);
    const int sw = vswz<D>(r0);  // also the swizzle of row r0 + 16
    const GQA_LDS char *rp = vt + r0 * Lay::ROW_BYTES + 8 * (jl & 1);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        const int chunk = (2 * db + ((jl & 3) >> 1)) ^ sw;
        const GQA_LDS char *p0 = rp + 16 * chunk;
        short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GQA_LDS short4v *)p0);
        short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((GQA_LDS short4v *)(p0 + 16 * Lay::ROW_BYTES));
        acc[db] = mfma16x16x32(join_tr(lo, hi), pb, acc[db]);
    }
}

// Rows sequence b attends: its length clamped to [0, S - extra], plus extra
// (1 when the new token's row is appended and attended).  The clamp keeps a
// length outside its precondition from reading past the sequence's cache
// rows (or its block-table row); every use of a length goes through here.
__device__ __forceinline__ int dc_clamp_rows(int len, int extra, int S) {
    return min(max(len, 0), S - extra) + extra;
}
__device__ __forceinline__ int dc_rows(const int32_t *seqlens, int b, int extra, int S) {
    return dc_clamp_rows(load_const(seqlens, b), extra, S);
}

// Segment bookkeeping shared by the split and merge passes.  Segments are
// ordered (sequence b, key/value head, query-head subgroup); segment
// (b, kv, qs) has nblk(b) = ceil(rows(b) / 32) blocks.
__device__ __forceinline__ int dc_nblk(const int32_t *seqlens, int b, int extra, int S) {
    return (dc_rows(seqlens, b, extra, S) + DC_BK - 1) / DC_BK;
}

// floor(w * T / NW), the first block of wave w's slice.  A 64-bit integer
// division is a long vector-ALU sequence; the quotient is taken in double
// (off by at most one for T < 2^51) and corrected with exact products.
__device__ __forceinline__ long long dc_slice_start(int w, long long T, int NW) {
    const long long x = (long long)w * T;
    long long s = (long long)((double)x / (double)NW);
    if (s * NW > x) --s;
    else if ((s + 1) * NW <= x) ++s;
    return s;
}

// A wave-uniform 64-bit value held in vector registers, made scalar.
__device__ __forceinline__ long long dc_uniform(long long x) {
    const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)(unsigned long long)x);
    const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)((unsigned long long)x >> 32));
    return (long long)(((unsigned long long)hi << 32) | lo);
}

__device__ __forceinline__ long long dc_wave_sum(long long x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    return x;
}

// Blocks of the whole list (T) and blocks of the sequences before `upto` (P),
// one sequence per lane, 64 at a time.
__device__ __forceinline__ void dc_block_totals(const int32_t *seqlens, int extra, int S, int B,
                                                int segs_per_b, int upto, long long &T,
                                                long long &P) {
    const int lane = threadIdx.x & 63;
    long long t = 0, p = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
        const int bb = b0 + lane;
        if (bb < B) {
            const long long n =
                (long long)((dc_clamp_rows(seqlens[bb], extra, S) + DC_BK - 1) / DC_BK) *
                segs_per_b;
            t += n;
            if (bb < upto) p += n;
        }
    }
    T = dc_uniform(dc_wave_sum(t));
    P = dc_uniform(dc_wave_sum(p));
}

// The sequence whose segments hold global block `pos` (0 <= pos < T) and the
// number of blocks before its first segment: an inclusive scan over 64
// sequences at a time and a ballot.
__device__ __forceinline__ void dc_locate(const int32_t *seqlens, int extra, int S, int B,
                                          int segs_per_b, long long pos, int &b_out,
                                          long long &cum_out) {
    const int lane = threadIdx.x & 63;
    long long base = 0;
    b_out = B;
    cum_out = 0;
    for (int b0 = 0; b0 < B; b0 += 64) {
        const int bb = b0 + lane;
        const long long n =
            bb < B ? (long long)((dc_clamp_rows(seqlens[bb], extra, S) + DC_BK - 1) / DC_BK) *
                         segs_per_b
                   : 0;
        long long incl = n;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const long long up = __shfl_up(incl, off);
            if (lane >= off) incl += up;
        }
        const unsigned long long hit = __ballot(bb < B && pos < base + incl);
        if (hit) {
            const int l = __ffsll((long long)hit) - 1;
            b_out = b0 + l;
            cum_out = dc_uniform(base + __shfl(incl - n, l));
            return;
        }
        base = dc_uniform(base + __shfl(incl, 63));
    }
}

// Ring depth per wave: as many (Q, K, V) slots as the CU's LDS holds for
// DC_WAVES waves, at most 4, and few enough that the loads of the other slots
// fit the 6-bit s_waitcnt vmcnt count.
template <int D, int QD>
constexpr int dc_slots() {
    constexpr int per_slot = QD * 1024 + 2 * DcLayout<D>::TILE;
    constexpr int ops = QD + 2 * DcLayout<D>::KV_DMA;
    constexpr int by_lds = DC_LDS_BYTES / (DC_WAVES * per_slot);
    constexpr int by_count = 63 / ops + 1;
    return by_lds < by_count ? (by_lds < 4 ? by_lds : 4) : (by_count < 4 ? by_count : 4);
}

// QD = 1 KiB loads per block for the query tile (ceil(query heads x 2d / 1024)).
// LAYOUT: where row j of (sequence b, key/value head g) sits (DecodeLayout).
// APPEND (head-major only): the new token's key/value rows (k_new, v_new) are
// attended as row seqlens[b] and written into that cache row by the wave that
// owns the segment's last block (query-head subgroup 0 only); no wave reads
// that cache row, so the write races with nothing.
template <int D, int QD, int LAYOUT, bool APPEND>
__global__ __launch_bounds__(DC_THREADS, 1) void decode_split_kernel(DecodeArgs a) {
    static_assert(!APPEND || LAYOUT == kLayoutHeadMajor, "append writes a head-major cache");
    using Lay = DcLayout<D>;
    constexpr int DB = D / 16;  // 16-wide blocks of the head dimension
    constexpr int OPS = QD + 2 * Lay::KV_DMA;  // memory instructions issued per block
    constexpr int DC_SLOTS = dc_slots<D, QD>();
    static_assert(DC_SLOTS >= 2, "double buffering fits");
    // a ring of DC_SLOTS slots per wave, each with its own Q, K and V tiles
    __shared__ __attribute__((aligned(1024))) char q_s[DC_WAVES][DC_SLOTS][QD * 1024];
    __shared__ __attribute__((aligned(1024))) char k_s[DC_WAVES][DC_SLOTS][Lay::TILE];
    __shared__ __attribute__((aligned(1024))) char v_s[DC_WAVES][DC_SLOTS][Lay::TILE];

    const int lane = threadIdx.x & 63, wave = wave_id();
    const int w = blockIdx.x * DC_WAVES + wave;
    if (w >= a.NW) return;
    const int g = lane >> 4, qcol = lane & 15;
    const int segs_per_b = a.h_kv * a.n_qsub;

    // total blocks and this wave's slice
    long long T, unused;
    dc_block_totals(a.seqlens, a.extra, a.S, a.B, segs_per_b, 0, T, unused);
    const long long pos = dc_slice_start(w, T, a.NW);
    const long long end = dc_slice_start(w + 1, T, a.NW);
    if (pos >= end) return;

    struct Cur {
        int b, seg, blk;
    };
    Cur cur{0, 0, 0};
    {
        int b0;
        long long cum;
        dc_locate(a.seqlens, a.extra, a.S, a.B, segs_per_b, pos, b0, cum);
        b0 = __builtin_amdgcn_readfirstlane(b0);
        const long long nb = dc_nblk(a.seqlens, b0, a.extra, a.S);  // > 0: the block at pos lies in b0
        cur = Cur{b0, (int)((pos - cum) / nb), (int)((pos - cum) % nb)};
    }
    const float c = a.c;

    auto advance = [&](Cur &u) {
        if (++u.blk == dc_nblk(a.seqlens, u.b, a.extra, a.S)) {
            u.blk = 0;
            if (++u.seg == segs_per_b) {
                u.seg = 0;
                do {
                    ++u.b;
                } while (u.b < a.B && dc_nblk(a.seqlens, u.b, a.extra, a.S) == 0);
            }
        }
    };
    auto heads_in = [&](const Cur &u) { return min(16, a.G - 16 * (u.seg % a.n_qsub)); };
    // every issue is OPS direct loads: Q rows (query heads of the subgroup,
    // clamped to its last head), K rows, V rows (clamped to the last valid key)
    auto issue = [&](const Cur &u, GQA_LDS char *qt, GQA_LDS char *kt, GQA_LDS char *vt) {
        const int kvh = u.seg / a.n_qsub, qs = u.seg % a.n_qsub;
        const int kend = dc_rows(a.seqlens, u.b, a.extra, a.S);
        const int head0 = kvh * a.G + 16 * qs;
        const int key0 = DC_BK * u.blk;
        // rows key0 .. key0 + 31 of (b, kvh): base, row stride and the block's
        // rows as seen by dc_dma_rows (first row, last valid row)
        size_t base, stride = D;
        int row0 = key0, last = kend - 1;
        if (LAYOUT == kLayoutHeadMajor) {
            base = ((size_t)u.b * a.h_kv + kvh) * (size_t)a.S * D;
        } else if (LAYOUT == kLayoutTokenMajor) {
            base = (size_t)u.b * a.S * a.h_kv * D + (size_t)kvh * D;
            stride = (size_t)a.h_kv * D;
        } else {  // paged: the block lies inside one page (page_size is a multiple of 32)
            const int page = load_const(a.block_table, u.b * a.max_blocks + key0 / a.page_size);
            base = (((size_t)page * a.h_kv + kvh) * a.page_size + key0 % a.page_size) * D;
            row0 = 0;
            last = kend - 1 - key0;
        }
        const size_t new_row = ((size_t)u.b * a.h_kv + kvh) * D;  // in k_new / v_new
        dc_dma_rows<D, false>(static_cast<const __bf16 *>(a.q) + ((size_t)u.b * a.h_q + head0) * D, D, 0,
                              heads_in(u) - 1, QD, qt);
        dc_dma_rows<D, false, APPEND>(static_cast<const __bf16 *>(a.k_cache) + base, stride, row0,
                                      last, Lay::KV_DMA, kt,
                                      static_cast<const __bf16 *>(a.k_new) + new_row);
        dc_dma_rows<D, true, APPEND>(static_cast<const __bf16 *>(a.v_cache) + base, stride, row0,
                                     last, Lay::KV_DMA, vt,
                                     static_cast<const __bf16 *>(a.v_new) + new_row);
    };
    // APPEND: copy the new key and value rows into cache row seqlens[b], one
    // 16-byte chunk per lane, from the block's LDS tiles, which hold them
    // already (chunk c of tile row r at r * ROW_BYTES + 16 (c ^ swz(r))), so
    // no global load has to be waited for.
    // Skipped when seqlens[b] is outside [0, S - 1], a broken precondition
    // (the attention then sees the clamped length's rows and the new row).
    auto store_new_rows = [&](const Cur &u, const GQA_LDS char *kt, const GQA_LDS char *vt) {
        constexpr int CPR = Lay::CPR;
        const int kvh = u.seg / a.n_qsub;
        const int row = load_const(a.seqlens, u.b);
        if (row < 0 || row >= a.S || lane >= 2 * CPR) return;
        const bool is_v = lane >= CPR;
        const int ch = is_v ? lane - CPR : lane;
        const int r = row - DC_BK * u.blk;  // the row's place in the tile
        const int phys = ch ^ (is_v ? vswz<D>(r) : kswz<D>(r));
        const u32x4 val = *reinterpret_cast<const GQA_LDS u32x4 *>((is_v ? vt : kt) +
                                                                  r * Lay::ROW_BYTES + 16 * phys);
        const size_t off = (((size_t)u.b * a.h_kv + kvh) * a.S + row) * D + 8 * ch;
        // the pointers pass through readfirstlane so that the per-lane choice
        // is made between two values, not between two argument addresses
        // (which would read the arguments with vector loads)
        const unsigned long long base = is_v ? uniform_addr(a.v_cache) : uniform_addr(a.k_cache);
        *reinterpret_cast<GQA_GLOBAL u32x4 *>(base + 2 * off) = val;
    };

    long long left = end - pos;  // blocks left to compute
    long long issued = 0;        // blocks whose loads have been issued
    Cur nxt = cur;
    bool seg_open = false;
    f32x4 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x4{};
    float m_run = -INFINITY, l_run = 0.f;

    auto close_segment = [&](const Cur &u) {
        float l_tot = l_run + __shfl_xor(l_run, 16);
        l_tot += other_half(l_tot);
        const size_t slot = (size_t)w + (size_t)u.b * segs_per_b + u.seg;
        if (qcol < heads_in(u)) {
            const float inv = 1.f / l_tot;
            float *op = a.opart + (slot * 16 + qcol) * D + 4 * g;
#pragma unroll
            for (int db = 0; db < DB; ++db)
                *reinterpret_cast<float4 *>(op + 16 * db) =
                    make_float4(acc[db][0] * inv, acc[db][1] * inv, acc[db][2] * inv, acc[db][3] * inv);
            if (g == 0) a.lse[slot * 16 + qcol] = m_run + __log2f(l_tot);
        }
        seg_open = false;
    };
    auto step = [&](const GQA_LDS char *qt, const GQA_LDS char *kt, const GQA_LDS char *vt) {
        if (!seg_open) {
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[db] = f32x4{};
            m_run = -INFINITY;
            l_run = 0.f;
            seg_open = true;
        }
        // this slot's loads are complete once at most the loads of the other
        // DC_SLOTS - 1 slots (issued after them) are still in flight; stores
        // issued in between only make the wait stricter
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((DC_SLOTS - 1) * OPS) : "memory");
        dc_block<D, QD * Lay::ROWS_PER_DMA>(qt, kt, vt, DC_BK * cur.blk,
                    dc_rows(a.seqlens, cur.b, a.extra, a.S), qcol < heads_in(cur), c, m_run, l_run,
                    acc);
        --left;
        const bool last_block = cur.blk + 1 == dc_nblk(a.seqlens, cur.b, a.extra, a.S);
        if (APPEND && last_block && cur.seg % a.n_qsub == 0) store_new_rows(cur, kt, vt);
        if (last_block || left == 0) close_segment(cur);
        advance(cur);
    };
    // the load cursor stops at the slice's last block; later issues repeat it
    auto next_issue = [&](GQA_LDS char *qt, GQA_LDS char *kt, GQA_LDS char *vt) {
        if (issued > 0 && issued < end - pos) advance(nxt);
        ++issued;
        issue(nxt, qt, kt, vt);
    };

    // block i of the slice lives in slot i % DC_SLOTS; block i + DC_SLOTS - 1
    // is issued into the slot of block i - 1, whose reads are complete
    auto qs_ = [&](int i) { return (GQA_LDS char *)q_s[wave][i]; };
    auto ks_ = [&](int i) { return (GQA_LDS char *)k_s[wave][i]; };
    auto vs_ = [&](int i) { return (GQA_LDS char *)v_s[wave][i]; };
#pragma unroll
    for (int i = 0; i < DC_SLOTS - 1; ++i) next_issue(qs_(i), ks_(i), vs_(i));
    int si = 0;  // slot of the block computed next
    while (left > 0) {
        const int sn = si == 0 ? DC_SLOTS - 1 : si - 1;
        next_issue(qs_(sn), ks_(sn), vs_(sn));
        step(qs_(si), ks_(si), vs_(si));
        si = si + 1 == DC_SLOTS ? 0 : si + 1;
    }
}

template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63;
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wid >= a.B * a.h_q) return;
    const int b = wid / a.h_q, h = wid % a.h_q;
    const int kvh = h / a.G, hg = h % a.G, qs = hg / 16, qcol = hg % 16;
    const int segs_per_b = a.h_kv * a.n_qsub;
    __bf16 *op = static_cast<__bf16 *>(a.o) + (size_t)wid * D + PER * lane;
    const int nb = dc_nblk(a.seqlens, b, a.extra, a.S);
    if (nb == 0) {
#pragma unroll
        for (int e = 0; e < PER; ++e) op[e] = (__bf16)0.f;
        return;
    }
    long long T, P;
    dc_block_totals(a.seqlens, a.extra, a.S, a.B, segs_per_b, b, T, P);
    const int seg_in_b = kvh * a.n_qsub + qs;
    P += (long long)seg_in_b * nb;  // first block of this segment
    const long long seg_global = (long long)b * segs_per_b + seg_in_b;
    // waves whose slices intersect [P, P + nb)
    int w0 = (int)min((double)a.NW - 1, (double)P * a.NW / (double)T);
    while (w0 > 0 && dc_slice_start(w0, T, a.NW) > P) --w0;
    while (dc_slice_start(w0 + 1, T, a.NW) <= P) ++w0;
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float wsum = 0.f, Mrun = -INFINITY;
    const long long seg_end = P + nb;
    // The waves that cover the segment follow from the slice bounds alone.
    // When at most MQ of them do (the usual case), every log-sum-exp and
    // partial row is requested at once: one memory round trip, not one per
    // step.  An empty slice wrote no partial row, so its (stale) row is
    // dropped by a select, never multiplied.
    constexpr int MQ = 8;
    int n_cov = 1;
    while (n_cov <= MQ && w0 + n_cov < a.NW && dc_slice_start(w0 + n_cov, T, a.NW) < seg_end)
        ++n_cov;
    if (n_cov <= MQ) {
        const bool mine = lane < n_cov && dc_slice_start(w0 + lane + 1, T, a.NW) >
                                              dc_slice_start(w0 + lane, T, a.NW);
        const float lse_l = mine ? a.lse[((size_t)(w0 + lane) + seg_global) * 16 + qcol] : -INFINITY;
        float v[MQ][PER];
#pragma unroll
        for (int u = 0; u < MQ; ++u) {
#pragma unroll
            for (int e = 0; e < PER; ++e) v[u][e] = 0.f;
            if (u < n_cov) {
                const size_t slot = (size_t)(w0 + u) + seg_global;
                const float *pp = a.opart + (slot * 16 + qcol) * D + PER * lane;
#pragma unroll
                for (int e = 0; e < PER; ++e) v[u][e] = pp[e];
            }
        }
        float M = lse_l;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
#pragma unroll
        for (int u = 0; u < MQ; ++u) {
            const float lu = __shfl(lse_l, u);
            const bool ok = u < n_cov && lu != -INFINITY;
            const float f = ok ? fast_exp2(lu - M) : 0.f;
            wsum += f;
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] = ok ? fmaf(f, v[u][e], acc[e]) : acc[e];
        }
        const float inv = 1.f / wsum;
#pragma unroll
        for (int e = 0; e < PER; ++e) op[e] = (__bf16)(acc[e] * inv);
        return;
    }
    // More waves: rounds of 64 (one round unless more than 64 waves cover the
    // segment): lane j holds the log-sum-exp of wave wb + j, or -inf for an
    // empty slice or a wave past the segment; the partial rows of up to four
    // waves are fetched together, then combined.
    for (int wb = w0; wb < a.NW && dc_slice_start(wb, T, a.NW) < seg_end; wb += 64) {
        const int wl = wb + lane;
        float lse_l = -INFINITY;
        if (wl < a.NW && dc_slice_start(wl, T, a.NW) < seg_end &&
            dc_slice_start(wl + 1, T, a.NW) > dc_slice_start(wl, T, a.NW))
            lse_l = a.lse[((size_t)wl + seg_global) * 16 + qcol];
        float M = lse_l;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
        const float Mnew = fmaxf(Mrun, M);
        if (Mrun != -INFINITY && Mnew > Mrun) {  // earlier rounds to the new max
            const float sc = fast_exp2(Mrun - Mnew);
            wsum *= sc;
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] *= sc;
        }
        Mrun = Mnew;
        const unsigned long long live = __ballot(lse_l != -INFINITY);
        const int n_live = live ? 64 - __clzll((long long)live) : 0;  // highest live lane + 1
        for (int u0 = 0; u0 < n_live; u0 += 4) {
            float f[4], v[4][PER];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float lu = __shfl(lse_l, min(u0 + u, 63));
                const bool ok = u0 + u < n_live && lu != -INFINITY;
                f[u] = ok ? fast_exp2(lu - Mrun) : 0.f;
#pragma unroll
                for (int e = 0; e < PER; ++e) v[u][e] = 0.f;
                if (ok) {
                    const size_t slot = (size_t)(wb + u0 + u) + seg_global;
                    const float *pp = a.opart + (slot * 16 + qcol) * D + PER * lane;
#pragma unroll
                    for (int e = 0; e < PER; ++e) v[u][e] = pp[e];
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                wsum += f[u];
#pragma unroll
                for (int e = 0; e < PER; ++e) acc[e] = fmaf(f[u], v[u][e], acc[e]);
            }
        }
    }
    const float inv = 1.f / wsum;
#pragma unroll
    for (int e = 0; e < PER; ++e) op[e] = (__bf16)(acc[e] * inv);
}

}  // namespace

template <int D, int QD>
void launch_split(const DecodeArgs &a, hipStream_t stream) {
    const dim3 grid((a.NW + DC_WAVES - 1) / DC_WAVES), block(DC_THREADS);
    if (a.layout == kLayoutTokenMajor)
        hipLaunchKernelGGL((decode_split_kernel<D, QD, kLayoutTokenMajor, false>), grid, block, 0,
                           stream, a);
    else if (a.layout == kLayoutPaged)
        hipLaunchKernelGGL((decode_split_kernel<D, QD, kLayoutPaged, false>), grid, block, 0,
                           stream, a);
    else if (a.extra)
        hipLaunchKernelGGL((decode_split_kernel<D, QD, kLayoutHeadMajor, true>), grid, block, 0,
                           stream, a);
    else
        hipLaunchKernelGGL((decode_split_kernel<D, QD, kLayoutHeadMajor, false>), grid, block, 0,
                           stream, a);
}

int launch_decode_bf16(const DecodeArgs &a, int d, hipStream_t stream) {
    const int qh = a.G < 16 ? a.G : 16;  // query heads per subgroup
    const int qkib = (qh * 2 * d + 1023) / 1024;
    dim3 grid2((a.B * a.h_q + 3) / 4), block(256);  // merge: one wave per (sequence, head)
    if (d == 128) {
        if (qkib <= 1) launch_split<128, 1>(a, stream);
        else if (qkib <= 2) launch_split<128, 2>(a, stream);
        else launch_split<128, 4>(a, stream);
        hipLaunchKernelGGL(decode_merge_kernel<128>, grid2, block, 0, stream, a);
    } else {
        if (qkib <= 1) launch_split<64, 1>(a, stream);
        else launch_split<64, 2>(a, stream);
        hipLaunchKernelGGL(decode_merge_kernel<64>, grid2, block, 0, stream, a);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqa
