// prefill_bf16.hip -- grouped-query attention prefill on bf16 MFMA (gfx950).
//
// Computes o = softmax(q k^T * scale) v for every query row, where query head h
// reads key/value head floor(h / G), G = h_q / h_kv ("Modern LLM architecture
// (1): GQA and RMSNorm", §2.1 formula, §2.3 grouping; "Attention in Qwen,
// DeepSeek and LLaMA3", §2.2 head map).  The softmax is evaluated tile by tile
// with running statistics (the on-chip, no-HBM-round-trip form that "What is
// Grouped-Query Attention", §4.3 credits to FlashAttention), an exact
// rearrangement of the row softmax.
//
// Work decomposition
//   One work-group (8 waves) owns 256 query rows: GW query heads of ONE group
//   times BM = 256 / GW consecutive positions (GW = the largest power of two
//   dividing G, at most 8; larger groups are split over G / GW work-groups).
//   Each key/value tile is loaded into LDS once and used by all GW heads: the
//   group-sharing saving; the key/value head is never copied per query head.
//   Wave w owns one row block of 32 rows (one head x 32 positions).
//
// Per wave and per key tile of 64 keys (S^T formulation)
//   S^T[key][query] = K Q^T on v_mfma_f32_32x32x16_bf16: A = K rows read from
//   LDS, B = Q^T held in registers for the whole kernel.  Each lane holds 16
//   keys of ONE query column, so row max and row sum are in-lane reductions
//   plus one exchange with the other half-wave.
//   P = exp2(S * scale*log2(e) - m) with a lazily updated running max m: the
//   accumulators are rescaled only when a row max grows by more than TAU (in
//   log2 units), so every P <= 2^TAU and almost no rescale is executed.
//   The factor scale*log2(e) multiplies the fp32 scores (one fma per score,
//   fused with the subtraction of m), so q enters the product exactly as
//   given.  Only when the factor is an exact power of two is it folded into q
//   instead (q * 2^e is exact in bf16), which saves that fma.
//   O^T[d][query] += V^T P^T: P^T comes straight out of the S^T accumulators
//   (keys permuted consistently on both operands), V^T is read from the
//   row-major V tile with the transposing ds_read_b64_tr_b16.
//
// Schedule
//   Two waves of a work-group share each SIMD (and at d = 64, where two
//   work-groups fit in a CU's LDS and registers, four), so one wave's matrix
//   products run while another computes exponentials or waits for LDS.
//   K/V tiles move with direct buffer->LDS loads (waves 0-3 the K tile, waves
//   4-7 the V tile) into a 4-slot ring: tile x is issued at the start of
//   iteration x - 3 into slot x % 4, whose previous tile x - 4 was last read in
//   iteration x - 4, before the barrier that ends it.  The buffer range ends at
//   key row L - 1, so the rows of a ragged last tile past the sequence read as
//   zeros.
//   Each wave waits for its own share of the next tile (s_waitcnt vmcnt) before
//   the barrier that ends an iteration, so after that barrier the whole tile is
//   visible: one work-group barrier per tile.
//   In the folded form every QK accumulator chain starts from -mu (the MFMA C
//   operand), so S arrives in log2 units already shifted by the running max;
//   row sums are taken with v_dot2_f32_bf16 on the bf16-rounded P that the PV
//   product uses.
//   Keep-mask form: a first pass sums the mask up per query tile (the rows of
//   a work-group) and 64-key tile: none, some or all of the keys the rows may
//   see are visible.  It runs once per call, not once per key/value head.  A
//   second, one-work-group pass orders the query tiles by how many key tiles
//   they see, most first.  The prefill then runs persistent work-groups, one
//   per CU, that take their (query tile, head) items in that order from a
//   counter per XCD, so the longest lists start first and no CU waits on the
//   dispatcher.  A work-group lists the key tiles some row of the item sees,
//   from the summary, and walks only those.  The mask bytes of its rows for
//   a listed tile that is not wholly visible are moved into the tile's ring
//   slot by the same direct loads (a 3-slot ring, since a slot then also
//   holds up to 256 rows x 64 bytes of mask); a wave whose 32 rows see no key
//   of such a tile skips that tile's products.
//   Causal: tiles wholly above the diagonal are never loaded or computed; the
//   diagonal and the sequence tail are masked element-wise.
//   Work-groups map to XCDs so that a key/value head's tiles share one L2, and
//   causal or variable-length work is dealt round-robin, longest first.
//   The output rows are staged in the (then free) LDS ring and stored as whole
//   rows.
#include "gqa_device.h"
#include "gqa_kernels.h"
#include "prefill_layout.h"

namespace gqa {
namespace {

constexpr int PF_WAVES = 8;
constexpr int PF_THREADS = 64 * PF_WAVES;
constexpr int kMaskCUs = 256;  // compute units of the part
constexpr int kXcds = 8;       // XCDs of the part; work-group i runs on XCD i % 8

// The LDS ring: SLOTS slots, each the K tile, the V tile and (keep-mask form)
// the mask bytes of up to 256 rows x 64 keys; tile x is issued PF_DIST = SLOTS - 1
// iterations ahead into slot x % SLOTS.
template <int D, int FORM>
struct PfRing {
    static constexpr int MASK_BYTES = FORM == kPfMask ? 256 * 64 : 0;
    static constexpr int SLOT_BYTES = 2 * PfLay<D>::TILE_BYTES + MASK_BYTES;
    static constexpr int SLOTS = FORM == kPfMask ? 3 : 4;
    static constexpr int DIST = SLOTS - 1;
    // keep-mask form: a 16-bit list entry per key tile (the tile, and in bit
    // 15 whether all its keys are visible to the work-group's rows), up to
    // LIST tiles, and the per-wave counts of the list's prefix sum
    static constexpr int LIST = FORM == kPfMask ? 4096 : 0;
    static constexpr int LIST_BYTES = FORM == kPfMask ? LIST * 2 + 64 : 0;
};

// Mask tile rows are 64 bytes (4 chunks of 16); logical chunk c of row r sits
// at chunk position c ^ swz(r), so the rows read together spread over the banks.
__device__ __forceinline__ int pf_mswz(int r) { return (r >> 2) & 3; }

// s_waitcnt vmcnt with a wave-uniform count known only at run time (0 .. 15;
// larger counts wait for everything, which is only stricter).
__device__ __forceinline__ void wait_vmcnt_rt(int n) {
    switch (n) {
        case 1: wait_vmcnt<1>(); break;
        case 2: wait_vmcnt<2>(); break;
        case 3: wait_vmcnt<3>(); break;
        case 4: wait_vmcnt<4>(); break;
        case 5: wait_vmcnt<5>(); break;
        case 6: wait_vmcnt<6>(); break;
        case 7: wait_vmcnt<7>(); break;
        case 8: wait_vmcnt<8>(); break;
        case 9: wait_vmcnt<9>(); break;
        case 10: wait_vmcnt<10>(); break;
        case 11: wait_vmcnt<11>(); break;
        case 12: wait_vmcnt<12>(); break;
        case 13: wait_vmcnt<13>(); break;
        case 14: wait_vmcnt<14>(); break;
        case 15: wait_vmcnt<15>(); break;
        default: wait_vmcnt<0>(); break;
    }
}

// FORM (PfForm): kPfRope rotates q as it is loaded (the keys arrive rotated
// already); kPfVarlen gives sequence b a.kv_lens[b] visible keys (a padded
// batch); kPfMask hides key j from query row i unless its mask byte is nonzero.
// FOLD: scale * log2(e) is an exact power of two and is folded into q.
// One work item of the prefill: query tile qt of unit (sequence, key/value
// head, head subgroup) `unit`, from its Q load to its output rows.  smem is the
// work-group's LDS (the ring, then the keep-mask form's list).
template <int D, bool CAUSAL, int FORM, bool FOLD>
__device__ __forceinline__ void prefill_item(const PrefillArgs &a, char *smem, int unit, int qt) {
    using Lay = PfLay<D>;
    using Ring = PfRing<D, FORM>;
    constexpr bool ROPE = FORM == kPfRope, VARLEN = FORM == kPfVarlen, MASK = FORM == kPfMask;
    constexpr int KSTEPS = Lay::KSTEPS, DB = Lay::DB;
    constexpr int DPW = 2 * Lay::DMA_PER_TENSOR / PF_WAVES;  // direct loads per wave per tile
    constexpr int SLOTS = Ring::SLOTS, DIST = Ring::DIST, SLOT_BYTES = Ring::SLOT_BYTES;

    int lane_ = threadIdx.x & 63, wave_ = wave_id();
    if constexpr (MASK) {
        // in the persistent form the ids pass an empty asm per item, so the
        // values derived from them are computed per item and not hoisted out
        // of the item loop, where they would hold registers through it
        asm volatile("" : "+v"(lane_));
        wave_ = __builtin_amdgcn_readfirstlane(wave_);
    }
    const int lane = lane_, wave = wave_;
    // The integer divisions that produce unit and qt, and those below, run
    // partly on the vector ALU; their wave-uniform results are moved to
    // scalar registers, so they do not hold vector registers for the whole
    // kernel.
    unit = __builtin_amdgcn_readfirstlane(unit);
    qt = __builtin_amdgcn_readfirstlane(qt);
    const int sub = __builtin_amdgcn_readfirstlane(unit % a.nsub);
    const int bk = __builtin_amdgcn_readfirstlane(unit / a.nsub);
    const int kvh = __builtin_amdgcn_readfirstlane(bk % a.h_kv);
    const int b = __builtin_amdgcn_readfirstlane(bk / a.h_kv);
    const int L = a.L, off = a.off;  // query rows, position of row 0
    const int Lt = a.Lk;             // key rows per sequence in the tensors
    // visible keys of this sequence: all, or its length (clamped to [0, Lt])
    const int Lk = VARLEN ? min(max(load_const(a.kv_lens, b), 0), Lt) : Lt;
    const int PB = 8 / a.GW;  // 32-position blocks per work-group
    const int p0 = qt * a.BM;

    const int head = kvh * a.G + sub * a.GW + wave / PB;
    const int pos0 = p0 + 32 * (wave % PB);
    const int kv_end = CAUSAL ? min(Lk, off + p0 + a.BM) : Lk;
    const int ntiles = (kv_end + PF_BN - 1) / PF_BN;
    // The loop walks positions 0 .. npos - 1 of a list of key tiles: ring slot
    // = position % SLOTS, keys of tile tile_e(entry of the position).  Without
    // a mask the list is every tile, in order (the entry of position p is p).
    // The keep-mask form lists (below) only the tiles the mask leaves visible
    // to at least one of the work-group's rows, when it has at most Ring::LIST
    // tiles; full_e(entry) says that every key of the tile that a row of the
    // work-group may see is visible to it, so its mask bytes are neither
    // loaded nor applied.  The loop reads each entry once, a tile ahead.
    int npos = ntiles;
    bool use_list = false;
    const uint16_t *tlist = reinterpret_cast<const uint16_t *>(smem + SLOTS * SLOT_BYTES);
    auto entry_at = [&](int pos) -> int {
        if constexpr (MASK) {
            if (use_list) return pos < npos ? __builtin_amdgcn_readfirstlane((int)tlist[pos]) : 0;
        }
        return pos;
    };
    auto tile_e = [&](int e) -> int {
        if constexpr (MASK) {
            if (use_list) return e & 0x7fff;
        }
        return e;
    };
    auto full_e = [&](int e) -> bool {
        if constexpr (MASK) {
            if (use_list) return (e >> 15) != 0;
        }
        return false;
    };

    // ---- direct loads: waves 0-3 stream the K tile and waves 4-7 the V tile;
    // this wave moves 1 KiB pieces i0 .. i0 + DPW - 1 of every tile.
    constexpr int NLO = Lay::CPR / 4;  // distinct per-lane offsets (period of the K swizzle)
    static_assert(Lay::DMA_PER_TENSOR == DPW * PF_WAVES / 2, "half the waves load K, half V");
    static_assert(DPW % NLO == 0, "per-lane offsets repeat with the K swizzle");
    const bool loads_v = wave >= PF_WAVES / 2;
    const int i0 = (wave % (PF_WAVES / 2)) * DPW;
    const unsigned krb = (unsigned)(a.h_kv * D * 2);  // key row stride, bytes
    // rows 0 .. Lk-1 of this (sequence, key/value head); Lk * krb < 2^32 is checked
    // on the host.  Rows past the sequence end read as zeros; for the ragged
    // last tile of a sequence spanning nearly 2^32 bytes a row offset may wrap,
    // and then reads zeros or finite data of the same tensor, which the mask
    // discards.
    const u32x4 rsrc = make_buffer_rsrc(
        static_cast<const __bf16 *>(loads_v ? a.v : a.k) + ((size_t)b * Lt * a.h_kv + kvh) * D,
        (!VARLEN || Lk > 0) ? (unsigned)(Lk - 1) * krb + 2 * D : 0u);
    // per-lane byte offset of piece i within its rows; depends on i only via i % NLO
    unsigned loff[NLO];
#pragma unroll
    for (int u = 0; u < NLO; ++u) {
        const int row = u * Lay::ROWS_PER_DMA + lane / Lay::CPR;
        const int chunk = (lane % Lay::CPR) ^ (loads_v ? pf_vswz<D>(row) : pf_kswz<D>(row));
        loff[u] = (unsigned)(lane / Lay::CPR) * krb + 16u * chunk;
    }
    // Keep-mask form: the mask tile of tile x holds rows p0 .. p0 + BM - 1, keys
    // 64 x .. 64 x + 63 (64 bytes a row); one 1 KiB direct load moves 16 rows,
    // and wave w moves pieces w and w + 8 of the BM / 16.  Rows at or past L
    // read as zeros (out of the resource's range); bytes of keys at or past
    // L_k may hold the next row's bytes, which the key bound discards.
    const int mpieces = MASK ? a.BM / 16 : 0;
    const int mpw = MASK ? (wave < mpieces) + (wave + 8 < mpieces) : 0;  // this wave's pieces
    const int opw = DPW + mpw;  // this wave's direct loads per tile
    u32x4 mrsrc = u32x4{0u, 0u, 0u, 0u};
    unsigned moff = 0;
    if constexpr (MASK) {
        mrsrc = make_buffer_rsrc(a.mask + (size_t)b * (size_t)a.mask_batch,
                                 (unsigned)((long long)L * a.mask_row));
        const int r = 16 * wave + (lane >> 2);  // row of this lane's first piece
        moff = (unsigned)(p0 + r) * (unsigned)a.mask_row + 16u * ((lane & 3) ^ pf_mswz(r));
    }
    // this wave's share of the loads of list position x (entry e) into ring
    // slot x % SLOTS
    auto issue_tile = [&](int x, int e) {
        char *slot = smem + (x % SLOTS) * SLOT_BYTES;
        const int tx = tile_e(e);
#pragma unroll
        for (int u = 0; u < DPW; ++u) {
            const int i = i0 + u;
            const unsigned row0 = (unsigned)(tx * PF_BN + i * Lay::ROWS_PER_DMA);
            dma16_to_lds_buf(rsrc, loff[u % NLO] + row0 * krb,
                             (GQA_LDS char *)(slot + (loads_v ? Lay::TILE_BYTES : 0) + i * 1024));
        }
        if constexpr (MASK) {
            // piece i = wave + 8 u covers rows 16 i .. 16 i + 15; the swizzle of
            // row r depends on r % 16 only, so one lane offset serves both pieces
            const int n_mask = full_e(e) ? 0 : mpw;
#pragma unroll
            for (int u = 0; u < 2; ++u)
                if (u < n_mask)
                    dma16_to_lds_buf(mrsrc,
                                     moff + (unsigned)(128 * u) * (unsigned)a.mask_row +
                                         (unsigned)(tx * PF_BN),
                                     (GQA_LDS char *)(slot + 2 * Lay::TILE_BYTES +
                                                      (wave + 8 * u) * 1024));
        }
    };

    // Q^T operand: lane holds 8 head-dim values of one query row.
    bf16x8 qf[KSTEPS];
    auto load_q = [&]() {
        const int pos = pos0 + (lane & 31);
        if (pos < L) {
            const __bf16 *qrow = static_cast<const __bf16 *>(a.q) +
                                 (((size_t)b * L + pos) * a.h_q + head) * D;
            const __bf16 *qp = qrow + 8 * (lane >> 5);
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                if constexpr (!ROPE) {
                    const bf16x8 raw = __builtin_bit_cast(bf16x8, load16(qp + 16 * ks));
                    if constexpr (FOLD) {
                        // scale * log2(e) = 2^e: q * 2^e is exact in bf16, and S^T
                        // then comes out of the MFMA already in log2 units
#pragma unroll
                        for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)((float)raw[e] * a.c);
                    } else {
                        qf[ks] = raw;
                    }
                } else {
                    // rotated columns c0 .. c0 + 7: pairs i0 .. i0 + 7 of the row,
                    // first half x0 cos - x1 sin, second half x0 sin + x1 cos
                    // (position off + pos; whether c0 is in the first half is
                    // fixed per k-step since d/2 is a multiple of 16)
                    const int c0 = 16 * ks + 8 * (lane >> 5);
                    const bool first = 16 * ks < D / 2;
                    const int i0 = first ? c0 : c0 - D / 2;
                    const bf16x8 xa = __builtin_bit_cast(bf16x8, load16(qrow + 2 * i0));
                    const bf16x8 xb = __builtin_bit_cast(bf16x8, load16(qrow + 2 * i0 + 8));
                    const size_t t0 = (size_t)(off + pos) * (D / 2) + i0;
                    const float4 ca = *reinterpret_cast<const float4 *>(a.rope_cos + t0);
                    const float4 cb = *reinterpret_cast<const float4 *>(a.rope_cos + t0 + 4);
                    const float4 sa = *reinterpret_cast<const float4 *>(a.rope_sin + t0);
                    const float4 sb = *reinterpret_cast<const float4 *>(a.rope_sin + t0 + 4);
                    const float cc[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
                    const float ss[8] = {sa.x, sa.y, sa.z, sa.w, sb.x, sb.y, sb.z, sb.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float x0 = (float)(e < 4 ? xa[2 * e] : xb[2 * e - 8]);
                        const float x1 = (float)(e < 4 ? xa[2 * e + 1] : xb[2 * e - 7]);
                        const float r = first ? x0 * cc[e] - x1 * ss[e] : x0 * ss[e] + x1 * cc[e];
                        // the rotated q, rounded to bf16 once
                        qf[ks][e] = (__bf16)(FOLD ? r * a.c : r);
                    }
                }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = bf16x8{};
        }
    };
    // The keep-mask form reads its summary row first and q right after, so
    // that q's latency passes under the list's construction (which waits for
    // the summary only); the other forms read q while tile 0 streams in.
    unsigned long long c8 = 0ull;  // keep-mask form: this thread's 8 tiles' summary bytes
    if constexpr (MASK) {
        const int t0 = 8 * threadIdx.x;
        // a summary row is a multiple of 8 bytes long, so 8 tiles are one
        // aligned load
        if (ntiles <= Ring::LIST && t0 < ntiles)
            c8 = *reinterpret_cast<const unsigned long long *>(
                a.mcodes + ((size_t)b * a.n_qtiles + qt) * a.mc_stride + t0);
        load_q();
    }

    // Keep-mask form: list the key tiles with a visible key for some row of
    // the work-group, from the summary of its query tile (bit 0: some key
    // visible; bit 1: every key its rows may see visible), 8 tiles a thread,
    // then a prefix sum over the tiles kept writes the list in tile order.
    if constexpr (MASK) {
        if (ntiles <= Ring::LIST) {
            use_list = true;
            uint16_t *list = reinterpret_cast<uint16_t *>(smem + SLOTS * SLOT_BYTES);
            int *wsum = reinterpret_cast<int *>(list + Ring::LIST);
            static_assert(Ring::LIST == 8 * PF_THREADS, "a thread owns 8 tiles of the list");
            const int t0 = 8 * threadIdx.x;
            int bits = 0, fbits = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const bool in = t0 + e < ntiles;
                bits |= (in && ((c8 >> (8 * e)) & 1ull)) ? (1 << e) : 0;
                fbits |= ((c8 >> (8 * e + 1)) & 1ull) ? (1 << e) : 0;
            }
            const int cnt = __builtin_popcount(bits);
            int incl = cnt;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int up = __shfl_up(incl, o);
                if (lane >= o) incl += up;
            }
            if (lane == 63) wsum[wave] = incl;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            block_barrier();
            int base = 0, total = 0;
#pragma unroll
            for (int w = 0; w < PF_WAVES; ++w) {
                const int ws = wsum[w];
                base += w < wave ? ws : 0;
                total += ws;
            }
            int at = base + incl - cnt;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (bits & (1 << e))
                    list[at++] = (uint16_t)((t0 + e) | ((fbits >> e) & 1 ? 0x8000 : 0));
            npos = __builtin_amdgcn_readfirstlane(total);
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            block_barrier();
        }
    }

    // V rows past the sequence end meet P = 0 and must be finite: zero the V
    // halves of the ring once, in case an out-of-range load leaves its LDS
    // bytes untouched.
    for (int i = threadIdx.x; i < SLOTS * Lay::TILE_BYTES / 16; i += PF_THREADS) {
        const int sl = i / (Lay::TILE_BYTES / 16), off = i % (Lay::TILE_BYTES / 16);
        store16_lds(smem + sl * SLOT_BYTES + Lay::TILE_BYTES + 16 * off, u32x4{0u, 0u, 0u, 0u});
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    block_barrier();
    // Tile 0 streams in while q is read.  A zero-length sequence has no tile;
    // its buffer range is empty, so these loads read zeros without touching
    // memory.
    issue_tile(0, entry_at(0));

    // q has been read (in the keep-mask form, before the list was built) or is
    // read here while tile 0 streams in.
    if constexpr (!MASK) load_q();

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
    f32x16 s[2] = {f32x16{}, f32x16{}};
    // Folded form: -mu in every element, the C operand of the first QK MFMA of
    // each chain, so the accumulators hold S * scale*log2(e) - mu with no VALU
    // work.  mu is the reference the exponentials are taken against: 0 until a
    // row sees its first key, then the running max (raised lazily).
    f32x16 negm = f32x16{};
    float mu = 0.f;
    const float c = a.c;
    bf16x8 pb[2][2];  // P^T of the current tile: [key block][16-key half]
    float m_run = -INFINITY, l_run = 0.f;
    const bool has_rows = pos0 < L;
    // whether this wave's rows may see a key of tile t
    auto active = [&](int t) { return has_rows && (!CAUSAL || t * PF_BN <= off + pos0 + 31); };

    // LDS operand reads for step st of the two products (16-byte K chunk;
    // transposed V pair); st runs over (k-step, key block) for QK and over
    // (key block, 16-key half, d block) for PV.
    constexpr int NSTEP = 2 * KSTEPS;  // == 4 * DB
    static_assert(NSTEP == 4 * DB, "QK and PV have the same number of MFMA steps");
    auto kread = [&](const char *kt, int st) {
        const int ks = st >> 1, kb = st & 1;
        const int r = 32 * kb + (lane & 31);
        const int ch = (2 * ks + (lane >> 5)) ^ pf_kswz<D>(r);
        return *reinterpret_cast<const bf16x8 *>(kt + r * Lay::ROW_BYTES + 16 * ch);
    };
    auto vread = [&](const char *vt, int st) {
        const int grp = lane >> 4, jl = lane & 15;
        const int vrq = 4 * (grp >> 1) + (jl >> 2);      // V row within a 16-key step (+8 for hi)
        const int vcq = 2 * (grp & 1) + ((jl & 3) >> 1);  // 16-byte chunk within a 32-wide d block
        const int vsw = pf_vswz<D>(vrq);                  // same for vrq + 8 and every step
        const int kh = st / DB, db = st % DB;             // kh = 2 * key block + half
        const char *p0 = vt + vrq * Lay::ROW_BYTES + 8 * (jl & 1) + 16 * kh * Lay::ROW_BYTES +
                         16 * ((4 * db + vcq) ^ vsw);
        short4v lo = lds_read_tr16(reinterpret_cast<const __bf16 *>(p0));
        short4v hi = lds_read_tr16(reinterpret_cast<const __bf16 *>(p0 + 8 * Lay::ROW_BYTES));
        return join_tr(lo, hi);
    };
    auto qk = [&](int j) {  // S^T = K Q^T (folded form: minus mu) for tile j
        const char *kt = smem + (j % SLOTS) * SLOT_BYTES;
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            const int ks = st >> 1, kb = st & 1;
            if constexpr (FOLD)
                s[kb] = mfma32x32x16(kread(kt, st), qf[ks], ks == 0 ? negm : s[kb]);
            else
                s[kb] = mfma32x32x16(kread(kt, st), qf[ks], ks == 0 ? f32x16{} : s[kb]);
        }
    };
    // At d = 128 the V^T operands of the whole tile are read into registers
    // right after QK, so their LDS latency passes under the softmax; at d = 64
    // the extra registers would cost a wave per SIMD, and PV reads them as it goes
    // (as it does in the keep-mask form, whose softmax needs registers for the mask).
    constexpr bool V_EARLY = D == 128 && !MASK;
    bf16x8 vf[V_EARLY ? NSTEP : 1];
    auto vload = [&](int j) {
        const char *vt = smem + (j % SLOTS) * SLOT_BYTES + Lay::TILE_BYTES;
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) vf[V_EARLY ? st : 0] = vread(vt, st);
    };
    auto pv = [&](int j) {  // O^T += V^T P^T for tile j
        const char *vt = smem + (j % SLOTS) * SLOT_BYTES + Lay::TILE_BYTES;
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            const int kh = st / DB, db = st % DB;
            acc[db] = mfma32x32x16(V_EARLY ? vf[V_EARLY ? st : 0] : vread(vt, st),
                                   pb[kh >> 1][kh & 1], acc[db]);
        }
    };
    // Keep-mask form: this lane's mask bytes of tile j, mk[g] = the 4 bytes of
    // keys 64 j + 8 g + 4 (lane / 32) .. + 3 for its query row (the keys of
    // scores s[g / 4][4 (g % 4) .. + 3]).
    unsigned mk[8];
    auto mask_read = [&](int j) {
        const int r = 32 * (wave % PB) + (lane & 31);  // the lane's row in the mask tile
        const char *mrow = smem + (j % SLOTS) * SLOT_BYTES + 2 * Lay::TILE_BYTES + r * 64 +
                           4 * (lane >> 5);
#pragma unroll
        for (int ch = 0; ch < 4; ++ch) {
            // dwords 4 ch + h and 4 ch + h + 2 of the row: g = 2 ch and 2 ch + 1
            const char *p = mrow + 16 * (ch ^ pf_mswz(r));
            mk[2 * ch] = *reinterpret_cast<const unsigned *>(p);
            mk[2 * ch + 1] = *reinterpret_cast<const unsigned *>(p + 8);
        }
    };
    // Softmax of tile j: mask, running max, P = exp2(S c - m), row sums.
    // The max is raised (and O, l rescaled) only when a row's new max exceeds
    // mu by more than TAU, or when the row sees its first key.
    // full_tile (keep-mask form): every mask byte of the tile is nonzero.
    auto softmax = [&](int j, int tile, bool full_tile) {  // list position j, key tile
        const int j0 = tile * PF_BN;
        if ((MASK && !full_tile) || j0 + PF_BN > Lk || (CAUSAL && j0 + PF_BN - 1 > off + pos0)) {
            pf_keep_branch();  // only diagonal, tail and partly hidden tiles pay for it
            if constexpr (MASK) {
                // read again here rather than kept in registers since the
                // tile test (the empty asm keeps the two reads apart); a tile
                // whose keys are all visible to the work-group's rows has no
                // mask bytes in its slot and needs none
                asm volatile("" ::: "memory");
                if (!full_tile) {
                    mask_read(j);
                } else {
#pragma unroll
                    for (int g = 0; g < 8; ++g) mk[g] = 0xffffffffu;
                }
            }
            const int pos = pos0 + (lane & 31);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j0 + 32 * kb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    bool masked = key >= Lk || (CAUSAL && key > off + pos);
                    if constexpr (MASK)
                        masked = masked || ((mk[4 * kb + (r >> 2)] >> (8 * (r & 3))) & 0xffu) == 0u;
                    s[kb][r] = masked ? -INFINITY : s[kb][r];
                }
        }
        // a tree of three-input maxima (v_max3_f32): 32 values in 16 instructions
        float x[32];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            x[r] = s[0][r];
            x[16 + r] = s[1][r];
        }
        float t[11];
#pragma unroll
        for (int i = 0; i < 10; ++i) t[i] = fmaxf(fmaxf(x[3 * i], x[3 * i + 1]), x[3 * i + 2]);
        t[10] = fmaxf(x[30], x[31]);
        const float u0 = fmaxf(fmaxf(t[0], t[1]), t[2]), u1 = fmaxf(fmaxf(t[3], t[4]), t[5]);
        const float u2 = fmaxf(fmaxf(t[6], t[7]), t[8]), u3 = fmaxf(t[9], t[10]);
        const float m0 = fmaxf(fmaxf(u0, u1), fmaxf(u2, u3));
        const float mx = fmaxf(m0, other_half(m0));  // tile row max (folded: relative to mu)
        // a row that has seen no key and sees none in this tile (a padding row,
        // a row the mask hides) changes nothing and must not trigger the
        // wave-wide rescale, so that it leaves the other rows' schedule alone
        if constexpr (FOLD) {
            if (__any((m_run == -INFINITY && mx != -INFINITY) || mx > PF_TAU)) {
                pf_keep_branch();  // rarely taken: no rescale work on other tiles
                const float m2 = m_run == -INFINITY ? mu + mx : fmaxf(m_run, mu + mx);
                const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m2);
                const float delta = (m2 == -INFINITY) ? 0.f : m2 - mu;
                m_run = m2;
                mu += delta;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[db] *= alpha;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) s[kb] -= delta;
#pragma unroll
                for (int r = 0; r < 16; ++r) negm[r] = -mu;
            }
        } else {
            // the scores are raw q.k; c (> 0) keeps their order, so the tile
            // max in log2 units is mx * c
            const float mt = mx * c;
            if (__any((m_run == -INFINITY && mt != -INFINITY) || mt > mu + PF_TAU)) {
                pf_keep_branch();  // rarely taken: no rescale work on other tiles
                const float m2 = fmaxf(m_run, mt);  // -inf while nothing is visible
                const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2(m_run - m2);
                m_run = m2;
                mu = (m2 == -INFINITY) ? mu : m2;
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[db] *= alpha;
            }
        }
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        // folded form: s holds S c - mu; else s holds S and one fma gives S c - mu
        auto arg = [&](float v) { return FOLD ? v : fmaf(v, c, -mu); };
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    const bf16x2 p2 = {(__bf16)fast_exp2(arg(s[kb][8 * hh + i])),
                                       (__bf16)fast_exp2(arg(s[kb][8 * hh + i + 1]))};
                    pb[kb][hh][i] = p2[0];
                    pb[kb][hh][i + 1] = p2[1];
                    // row sum of the bf16-rounded P that the PV product uses
                    l_run = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, l_run, false);
                }
    };

    // q has landed: the compiler's own wait for the q loads stands here, where
    // it also covers tile 0, and not inside the loop, where it would drain the
    // prefetched tiles every iteration
    pf_settle(qf);
    if constexpr (MASK) {
        // list entries of positions j .. j + DIST, read a tile ahead, so that
        // their LDS latency passes under the ring's wait and the barrier
        int ent[DIST + 1];
#pragma unroll
        for (int i = 0; i <= DIST; ++i) ent[i] = entry_at(i);
#pragma unroll
        for (int x = 1; x < DIST; ++x)
            if (x < npos) issue_tile(x, ent[x]);
        // Tile x has landed once at most the loads issued after it are
        // pending: those of positions x + 1 .. x + pending (pending < DIST =
        // 2: at most x + 1, entry e1), opw loads, or DPW when its mask bytes
        // are not loaded.
        static_assert(DIST == 2, "one tile pending at most");
        auto wait_landed = [&](int pending, int e1) {
            if (pending < 1) wait_vmcnt<0>();
            else if (full_e(e1)) wait_vmcnt<DPW>();
            else wait_vmcnt_rt(opw);
        };
        wait_landed(min(npos, DIST) - 1, ent[1]);
        block_barrier();
        for (int j = 0; j < npos; ++j) {
            if (j + DIST < npos) issue_tile(j + DIST, ent[DIST]);
            const int t = tile_e(ent[0]);
            if (active(t)) {
                bool go = true, full = true;
                if (!full_e(ent[0])) {
                    // skip a tile whose mask hides every key from this wave's rows
                    mask_read(j);
                    unsigned any = 0, zero = 0;
#pragma unroll
                    for (int g = 0; g < 8; ++g) {
                        any |= mk[g];
                        zero |= (mk[g] - 0x01010101u) & ~mk[g] & 0x80808080u;  // a zero byte
                    }
                    go = __any(any != 0u);
                    full = !__any(zero != 0u);
                }
                if (go) {
                    qk(j);
                    softmax(j, t, full);
                    pv(j);
                }
            }
            const int nxt = entry_at(j + 1 + DIST);
            // tile j + 1 must have landed; tiles j + 2 .. j + DIST may be pending
            wait_landed(max(min(npos - 1, j + DIST) - (j + 1), 0), ent[2]);
            block_barrier();
#pragma unroll
            for (int i = 0; i < DIST; ++i) ent[i] = ent[i + 1];
            ent[DIST] = nxt;
        }
    } else {
#pragma unroll
        for (int x = 1; x < DIST; ++x)
            if (x < npos) issue_tile(x, x);
        // Tile x has landed once at most the loads issued after it are
        // pending: those of tiles x + 1 .. x + DIST - 1 that exist, DPW loads
        // each, so the counts are immediates.
        auto wait_tile = [&](int pending) {
            static_assert(DIST == 3, "the immediate waits assume a prefetch distance of 3");
            if (pending >= 2) wait_vmcnt<2 * DPW>();
            else if (pending == 1) wait_vmcnt<DPW>();
            else wait_vmcnt<0>();
        };
        wait_tile(min(npos, DIST) - 1);
        block_barrier();
        for (int j = 0; j < npos; ++j) {
            if (j + DIST < npos) issue_tile(j + DIST, j + DIST);
            if (active(j)) {
                qk(j);
                if (V_EARLY) {
                    vload(j);
                    __builtin_amdgcn_sched_barrier(0);
                }
                softmax(j, j, true);
                pv(j);
            }
            // tile j + 1 must have landed; tiles j + 2 .. j + DIST may be pending
            wait_tile(max(min(npos - 1, j + DIST) - (j + 1), 0));
            block_barrier();
        }
    }

    // ---- epilogue: O / l, round to bf16, store.  The ring is free after the
    // last barrier; each wave stages its 32 rows in its own part of it and
    // writes them back as whole rows (16-byte lanes, consecutive within a
    // row), not as the accumulators' scattered 8-byte pieces of 32 rows.
    const float lt = l_run + other_half(l_run);
    // no visible key (a zero-length sequence, a fully masked row): a zero row
    const float inv = (!(VARLEN || MASK) || lt > 0.f) ? 1.f / lt : 0.f;
    // the lane id passes an empty asm, so the addresses below are computed
    // here and not kept in registers across the tile loop
    int le = lane;
    asm volatile("" : "+v"(le));
    char *stage = smem + wave * 32 * Lay::ROW_BYTES;
    {
        // row r = lane % 32 holds columns 32 db + 8 rq + 4 h .. + 3 (h = lane / 32):
        // 8 bytes of 16-byte chunk 4 db + rq, stored at chunk position
        // (4 db + rq) ^ swz(r), the K tiles' swizzle, so that the rows written
        // together fall in different banks
        const int r = le & 31, h = le >> 5;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                bf16x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[db][4 * rq + e] * inv);
                const int ch = (4 * db + rq) ^ pf_kswz<D>(r);
                *reinterpret_cast<bf16x4 *>(stage + r * Lay::ROW_BYTES + 16 * ch + 8 * h) = w;
            }
    }
    {
        // one pass covers 64 / CPR rows, lane = (row in pass) * CPR + chunk
        constexpr int RPP = 64 / Lay::CPR;
        const int rr = le / Lay::CPR, ch = le % Lay::CPR;
#pragma unroll
        for (int p = 0; p < 32 / RPP; ++p) {
            const int r = p * RPP + rr;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(
                stage + r * Lay::ROW_BYTES + 16 * (ch ^ pf_kswz<D>(r)));
            if (pos0 + r < L)
                *reinterpret_cast<u32x4 *>(static_cast<__bf16 *>(a.o) +
                                           (((size_t)b * L + pos0 + r) * a.h_q + head) * D +
                                           8 * ch) = v;
        }
    }
}

// The prefill kernel.  Work-group -> (unit, query tile): dispatch sends
// work-group i to XCD i % 8.  Equal-cost tiles are mapped XCD-contiguously, so
// the tiles of one key/value head run on one XCD and share its L2.  Causal and
// variable-length tiles differ in cost, so they are dealt round-robin over the
// units instead, longest first: with a multiple of 8 units each unit still
// stays on one XCD, and otherwise (one head, say) every XCD still gets an
// equal mix of long and short tiles.
// The keep-mask form is persistent: one work-group per CU takes work items in
// the order the ordering pass wrote, the items of one (sequence, query tile)
// (its key/value heads and head subgroups) in a row, so a CU that finishes an
// item starts the next at once.  Work-group i runs on XCD x = i % 8 and takes
// the items r = 8 k + x, k from XCD x's own counter (the eight zeroed by the
// ordering pass): with a multiple of 8 items per query tile, each key/value
// head's items stay on one XCD, whose L2 then holds its keys and values.
template <int D, bool CAUSAL, int FORM, bool FOLD>
__global__ __launch_bounds__(PF_THREADS, D == 64 ? 4 : 2)  // waves per SIMD
void prefill_bf16_kernel(PrefillArgs a) {
    using Ring = PfRing<D, FORM>;
    constexpr bool VARLEN = FORM == kPfVarlen, MASK = FORM == kPfMask;
    __shared__ __attribute__((aligned(1024))) char smem[Ring::SLOTS * Ring::SLOT_BYTES +
                                                        Ring::LIST_BYTES];
    if constexpr (MASK) {
        __shared__ int next;
        const int hpi = a.h_kv * a.nsub;  // items per (sequence, query tile)
        const int total = a.n_units * a.n_qtiles;
        const int xcd = blockIdx.x % kXcds;
        for (;;) {
            // every wave has read the previous value (a barrier lies between)
            // and finished the previous item's epilogue (the barrier below)
            if (threadIdx.x == 0) next = atomicAdd(a.mwork + xcd, 1);
            asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
            block_barrier();
            const int r = __builtin_amdgcn_readfirstlane(next) * kXcds + xcd;
            if (r >= total) break;
            const int item = load_const(a.morder, r / hpi);
            prefill_item<D, CAUSAL, FORM, FOLD>(a, smem, (item / a.n_qtiles) * hpi + r % hpi,
                                                item % a.n_qtiles);
        }
    } else {
        int unit, qt;
        if (CAUSAL || VARLEN) {
            unit = blockIdx.x % a.n_units;
            qt = blockIdx.x / a.n_units;
        } else {
            const int lid = xcd_contiguous_id(blockIdx.x, gridDim.x);
            unit = lid / a.n_qtiles;
            qt = lid % a.n_qtiles;
        }
        if (CAUSAL) qt = a.n_qtiles - 1 - qt;  // longest rows first
        prefill_item<D, CAUSAL, FORM, FOLD>(a, smem, unit, qt);
    }
}


// Keep-mask summary: one wave per (sequence b, query tile qt of BM rows,
// 64-key tile t) writes mcodes[(b * n_qtiles + qt) * mc_stride + t]: bit 0
// set when some row of the query tile (below L) has a visible key among those
// it may see in the key tile (below L_k, and causally up to its position),
// bit 1 set when every such key is visible (also when the rows may see none
// of the tile's keys).  Lane l reads 32 bytes of row 32 p + l / 2 of the
// query tile in pass p, only where the row may see a key of them, so every
// read stays inside the row's first L_k bytes rounded up to 16.
__global__ __launch_bounds__(256) void mask_summary_kernel(PrefillArgs a, bool causal) {
    const int lane = threadIdx.x & 63;
    const long long id = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nkt = (a.Lk + PF_BN - 1) / PF_BN;
    const long long item = id / nkt;  // b * n_qtiles + qt
    if (item >= (long long)a.B * a.n_qtiles) return;
    const int t = (int)(id % nkt);
    const int qt = (int)(item % a.n_qtiles), b = (int)(item / a.n_qtiles);
    const int k0 = PF_BN * t + 32 * (lane & 1);
    const u32x4 z = u32x4{0u, 0u, 0u, 0u};
    bool any = false, hole = false;
    for (int p = 0; p < a.BM / 32; ++p) {
        const int row = qt * a.BM + 32 * p + (lane >> 1);
        const int seen = row < a.L ? min(a.Lk, causal ? a.off + row + 1 : a.Lk) : 0;
        const int lim = min(max(seen - k0, 0), 32);  // bytes of this lane that count
        const uint8_t *mp = a.mask + (size_t)b * (size_t)a.mask_batch +
                            (size_t)row * (size_t)a.mask_row + k0;
        const u32x4 m0 = lim > 0 ? load16(mp) : z;
        const u32x4 m1 = lim > 16 ? load16(mp + 16) : z;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const unsigned x = w < 4 ? m0[w] : m1[w - 4];
            const int nb = min(max(lim - 4 * w, 0), 4);
            const unsigned keep = nb == 4 ? 0xffffffffu : (1u << (8 * nb)) - 1u;
            any = any || (x & keep) != 0u;
            const unsigned y = x | ~keep;  // bytes that do not count read as 0xff
            hole = hole || ((y - 0x01010101u) & ~y & 0x80808080u) != 0u;  // a zero byte
        }
    }
    const bool any_w = __any(any), hole_w = __any(hole);
    if (lane == 0)
        a.mcodes[(size_t)item * a.mc_stride + t] = (uint8_t)((any_w ? 1 : 0) | (hole_w ? 0 : 2));
}

// Keep-mask order: one work-group ranks the (sequence, query tile) items by
// the number of key tiles their rows see, most first, ties by item index,
// and writes morder[rank] = item.  Beyond kOrderItems items it writes the
// static order instead: query tiles latest first (causally the longest rows),
// sequences in turn.
constexpr int kOrderItems = 4096;
__global__ __launch_bounds__(1024) void mask_order_kernel(PrefillArgs a, bool causal) {
    __shared__ int cnt[kOrderItems];
    const int n = a.B * a.n_qtiles, tid = threadIdx.x;
    if (tid < kXcds) a.mwork[tid] = 0;  // the prefill's work counters, one per XCD
    if (n > kOrderItems) {
        for (int r = tid; r < n; r += 1024)
            a.morder[r] = (r % a.B) * a.n_qtiles + (a.n_qtiles - 1 - r / a.B);
        return;
    }
    for (int i = tid; i < n; i += 1024) cnt[i] = 0;
    __syncthreads();
    // one thread per (item, 8 key tiles): the items' summary rows are read in
    // parallel, eight loads a thread in flight, and summed in LDS
    const int chunks = a.mc_stride / 8;  // 8-tile pieces of a summary row
    const long long work = (long long)n * chunks;
    for (long long w0 = tid; w0 < work; w0 += 8 * 1024) {
        unsigned long long x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const long long w = w0 + 1024 * u;
            x[u] = w < work ? *reinterpret_cast<const unsigned long long *>(a.mcodes + 8 * w) : 0ull;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const long long w = w0 + 1024 * u;
            if (w >= work) continue;
            const int i = (int)(w / chunks), t8 = 8 * (int)(w % chunks);
            const int qt = i % a.n_qtiles;
            const int kv_end = causal ? min(a.Lk, a.off + (qt + 1) * a.BM) : a.Lk;
            const int nt = (kv_end + PF_BN - 1) / PF_BN;  // the item's key tiles
            unsigned long long y = x[u] & 0x0101010101010101ull;  // bit 0 of each byte
            y = nt - t8 >= 8 ? y : nt - t8 <= 0 ? 0ull : y & ((1ull << (8 * (nt - t8))) - 1ull);
            const int c = __builtin_popcountll(y);
            if (c) atomicAdd(&cnt[i], c);
        }
    }
    __syncthreads();
    for (int i = tid; i < n; i += 1024) {
        const int ci = cnt[i];
        int r = 0;
        for (int j = 0; j < n; ++j) {
            const int cj = cnt[j];
            r += (cj > ci || (cj == ci && j < i)) ? 1 : 0;
        }
        a.morder[r] = i;
    }
}

template <int D, bool C>
void launch_form(const PrefillArgs &a, dim3 grid, dim3 block, hipStream_t stream) {
    if (a.rope_cos != nullptr)
        hipLaunchKernelGGL((prefill_bf16_kernel<D, C, kPfRope, false>), grid, block, 0, stream, a);
    else if (a.kv_lens != nullptr)
        hipLaunchKernelGGL((prefill_bf16_kernel<D, C, kPfVarlen, false>), grid, block, 0, stream,
                           a);
    else if (a.mask != nullptr)
        hipLaunchKernelGGL((prefill_bf16_kernel<D, C, kPfMask, false>), grid, block, 0, stream, a);
    else if (a.fold)
        hipLaunchKernelGGL((prefill_bf16_kernel<D, C, kPfPlain, true>), grid, block, 0, stream, a);
    else
        hipLaunchKernelGGL((prefill_bf16_kernel<D, C, kPfPlain, false>), grid, block, 0, stream, a);
}

}  // namespace

int launch_prefill_bf16(const PrefillArgs &a, int d, bool causal, hipStream_t stream) {
    if (a.mask != nullptr) {
        const long long waves = (long long)a.B * a.n_qtiles * ((a.Lk + PF_BN - 1) / PF_BN);
        hipLaunchKernelGGL(mask_summary_kernel, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0,
                           stream, a, causal);
        hipLaunchKernelGGL(mask_order_kernel, dim3(1), dim3(1024), 0, stream, a, causal);
    }
    // the keep-mask form is persistent: one work-group per CU (its LDS ring
    // fills the CU), at most one per work item
    const int items = a.n_units * a.n_qtiles;
    dim3 grid(a.mask != nullptr ? (items < kMaskCUs ? items : kMaskCUs) : items),
        block(PF_THREADS);
    if (d == 128) {
        if (causal) launch_form<128, true>(a, grid, block, stream);
        else launch_form<128, false>(a, grid, block, stream);
    } else {
        if (causal) launch_form<64, true>(a, grid, block, stream);
        else launch_form<64, false>(a, grid, block, stream);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqa
