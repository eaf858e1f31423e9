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
//   Scale * log2(e) is folded into Q once, and every QK accumulator chain
//   starts from -mu (the MFMA C operand), so S arrives in log2 units already
//   shifted by the running max; row sums are taken with v_dot2_f32_bf16 on the
//   bf16-rounded P that the PV product uses.
//   Causal: tiles wholly above the diagonal are never loaded or computed; the
//   diagonal and the sequence tail are masked element-wise.
//   Work-groups map to XCDs so that a key/value head's tiles share one L2, and
//   causal or variable-length work is dealt round-robin, longest first.
//   The output rows are staged in the (then free) LDS ring and stored as whole
//   rows.
#include "gqa_device.h"
#include "gqa_kernels.h"

namespace gqa {
namespace {

constexpr int PF_WAVES = 8;
constexpr int PF_THREADS = 64 * PF_WAVES;
constexpr int PF_BN = 64;       // keys per tile
constexpr int PF_SLOTS = 4;     // LDS ring depth (tiles)
constexpr float PF_TAU = 8.0f;  // lazy-rescale threshold, log2 units
constexpr int PF_DIST = 3;      // tiles issued ahead of the one being computed

template <int D>
struct PfLay {
    static constexpr int ROW_BYTES = 2 * D;
    static constexpr int CPR = D / 8;                        // 16-byte chunks per row
    static constexpr int ROWS_PER_DMA = 64 / CPR;            // rows per 64-lane 16-byte load
    static constexpr int TILE_BYTES = PF_BN * ROW_BYTES;     // one K or V tile
    static constexpr int DMA_PER_TENSOR = TILE_BYTES / 1024;
    static constexpr int DMA_PER_WAVE = 2 * DMA_PER_TENSOR / PF_WAVES;
    static constexpr int SLOT_BYTES = 2 * TILE_BYTES;        // K tile then V tile
    static constexpr int ROWS_PER_SWEEP = 256 / ROW_BYTES;   // rows per pass over the banks
    static constexpr int KSTEPS = D / 16;                    // MFMA k-steps over d
    static constexpr int DB = D / 32;                        // 32-wide blocks of d
};

// Tiles are stored unpadded (each direct load writes 64 consecutive 16-byte
// chunks); 16-byte chunk c of row r sits at chunk position c ^ swz(r).
//   K: 16 lanes reading one chunk of 16 consecutive rows hit distinct banks.
//   V: a half-wave transposing read (4 rows x 64 bytes) hits distinct banks.
template <int D>
__device__ __forceinline__ int pf_kswz(int r) {
    using Lay = PfLay<D>;
    return (r / Lay::ROWS_PER_SWEEP) % Lay::CPR;
}
template <int D>
__device__ __forceinline__ int pf_vswz(int r) {
    return D == 128 ? 4 * (r % 4) : 4 * ((r / 2) % 2);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void block_barrier() {
    asm volatile("s_barrier" ::: "memory");
}

// ROPE: q is rotated as it is loaded (the keys arrive rotated already).
// VARLEN: sequence b has a.kv_lens[b] visible keys (a padded batch).
template <int D, bool CAUSAL, bool ROPE, bool VARLEN>
__global__ __launch_bounds__(PF_THREADS, D == 64 ? 4 : 2)  // waves per SIMD
void prefill_bf16_kernel(PrefillArgs a) {
    using Lay = PfLay<D>;
    constexpr int KSTEPS = Lay::KSTEPS, DB = Lay::DB, DPW = Lay::DMA_PER_WAVE;
    __shared__ __attribute__((aligned(1024))) char smem[PF_SLOTS * Lay::SLOT_BYTES];

    const int lane = threadIdx.x & 63, wave = wave_id();
    // Work-group -> (unit, query tile).  Dispatch sends work-group i to XCD
    // i % 8.  Equal-cost tiles are mapped XCD-contiguously, so the tiles of one
    // key/value head run on one XCD and share its L2.  Causal and
    // variable-length tiles differ in cost, so they are dealt round-robin over
    // the units instead, longest first: with a multiple of 8 units each unit
    // still stays on one XCD, and otherwise (one head, say) every XCD still gets
    // an equal mix of long and short tiles.
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
    // The integer divisions above and below run partly on the vector ALU; their
    // wave-uniform results are moved to scalar registers, so they do not hold
    // vector registers for the whole kernel.
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
    // this wave's share of the loads of tile x into ring slot x % PF_SLOTS
    auto issue_tile = [&](int x) {
#pragma unroll
        for (int u = 0; u < DPW; ++u) {
            const int i = i0 + u;
            const unsigned row0 = (unsigned)(x * PF_BN + i * Lay::ROWS_PER_DMA);
            dma16_to_lds_buf(rsrc, loff[u % NLO] + row0 * krb,
                             (GQA_LDS char *)(smem + (x % PF_SLOTS) * Lay::SLOT_BYTES +
                                              (loads_v ? Lay::TILE_BYTES : 0) + i * 1024));
        }
    };

    // Q^T operand: lane holds 8 head-dim values of one query row.
    bf16x8 qf[KSTEPS];
    {
        const int pos = pos0 + (lane & 31);
        if (pos < L) {
            const __bf16 *qrow = static_cast<const __bf16 *>(a.q) +
                                 (((size_t)b * L + pos) * a.h_q + head) * D;
            const __bf16 *qp = qrow + 8 * (lane >> 5);
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
                // fold scale * log2(e) into Q once (rounded to bf16): S^T then
                // comes out of the MFMA already in log2 units
                if (!ROPE) {
                    const bf16x8 raw = __builtin_bit_cast(bf16x8, load16(qp + 16 * ks));
#pragma unroll
                    for (int e = 0; e < 8; ++e) qf[ks][e] = (__bf16)((float)raw[e] * a.c);
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
                        qf[ks][e] = (__bf16)(r * a.c);
                    }
                }
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = bf16x8{};
        }
    }

    f32x16 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
    f32x16 s[2] = {f32x16{}, f32x16{}};
    // -mu in every element: the C operand of the first QK MFMA of each chain,
    // so the accumulators hold S * scale*log2(e) - mu with no VALU work.
    // mu is the running max (0 before the first tile).
    f32x16 negm = f32x16{};
    float mu = 0.f;
    bf16x8 pb[2][2];  // P^T of the current tile: [key block][16-key half]
    float m_run = -INFINITY, l_run = 0.f;
    const bool has_rows = pos0 < L;
    auto active = [&](int j) { return has_rows && (!CAUSAL || j * PF_BN <= off + pos0 + 31); };

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
    auto qk = [&](int j) {  // S^T = K Q^T - mu for tile j
        const char *kt = smem + (j % PF_SLOTS) * Lay::SLOT_BYTES;
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            const int ks = st >> 1, kb = st & 1;
            s[kb] = mfma32x32x16(kread(kt, st), qf[ks], ks == 0 ? negm : s[kb]);
        }
    };
    // At d = 128 the V^T operands of the whole tile are read into registers
    // right after QK, so their LDS latency passes under the softmax; at d = 64
    // the extra registers would cost a wave per SIMD, and PV reads them as it goes.
    constexpr bool V_EARLY = D == 128;
    bf16x8 vf[V_EARLY ? NSTEP : 1];
    auto vload = [&](int j) {
        const char *vt = smem + (j % PF_SLOTS) * Lay::SLOT_BYTES + Lay::TILE_BYTES;
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) vf[V_EARLY ? st : 0] = vread(vt, st);
    };
    auto pv = [&](int j) {  // O^T += V^T P^T for tile j
        const char *vt = smem + (j % PF_SLOTS) * Lay::SLOT_BYTES + Lay::TILE_BYTES;
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
            const int kh = st / DB, db = st % DB;
            acc[db] = mfma32x32x16(V_EARLY ? vf[V_EARLY ? st : 0] : vread(vt, st),
                                   pb[kh >> 1][kh & 1], acc[db]);
        }
    };
    // Softmax of tile j: mask, running max, P = exp2(S c - m), row sums.
    // s holds S c - mu.  The max is raised (and O, l rescaled) only when a row's
    // new max exceeds mu by more than TAU, or on the first tile.
    auto softmax = [&](int j) {
        const int j0 = j * PF_BN;
        if (j0 + PF_BN > Lk || (CAUSAL && j0 + PF_BN - 1 > off + pos0)) {
            const int pos = pos0 + (lane & 31);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = j0 + 32 * kb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    const bool masked = key >= Lk || (CAUSAL && key > off + pos);
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
        const float mx = fmaxf(m0, other_half(m0));  // tile row max, relative to mu
        if (__any(m_run == -INFINITY || mx > PF_TAU)) {
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
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    const bf16x2 p2 = {(__bf16)fast_exp2(s[kb][8 * hh + i]),
                                       (__bf16)fast_exp2(s[kb][8 * hh + i + 1])};
                    pb[kb][hh][i] = p2[0];
                    pb[kb][hh][i + 1] = p2[1];
                    // row sum of the bf16-rounded P that the PV product uses
                    l_run = __builtin_amdgcn_fdot2_f32_bf16(p2, ones, l_run, false);
                }
    };

    // V rows past the sequence end meet P = 0 and must be finite: zero the V
    // halves of the ring once, in case an out-of-range load leaves its LDS
    // bytes untouched.
    for (int i = threadIdx.x; i < PF_SLOTS * Lay::TILE_BYTES / 16; i += PF_THREADS) {
        const int sl = i / (Lay::TILE_BYTES / 16), off = i % (Lay::TILE_BYTES / 16);
        store16_lds(smem + sl * Lay::SLOT_BYTES + Lay::TILE_BYTES + 16 * off, u32x4{0u, 0u, 0u, 0u});
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    block_barrier();
    // a zero-length sequence has no tile; its buffer range is empty, so these
    // loads read zeros without touching memory
    issue_tile(0);
#pragma unroll
    for (int x = 1; x < PF_DIST; ++x)
        if (x < ntiles) issue_tile(x);
    // tile 0 has landed once at most the loads of tiles 1 .. PF_DIST - 1 are pending
    if (ntiles >= 3) wait_vmcnt<2 * DPW>();
    else if (ntiles == 2) wait_vmcnt<DPW>();
    else wait_vmcnt<0>();
    block_barrier();
    for (int j = 0; j < ntiles; ++j) {
        if (j + PF_DIST < ntiles) issue_tile(j + PF_DIST);
        if (active(j)) {
            qk(j);
            if (V_EARLY) {
                vload(j);
                __builtin_amdgcn_sched_barrier(0);
            }
            softmax(j);
            pv(j);
        }
        // tile j + 1 must have landed; tiles j + 2 .. j + PF_DIST may be pending
        const int pending = min(ntiles - 1, j + PF_DIST) - (j + 1);
        if (pending >= 2) wait_vmcnt<2 * DPW>();
        else if (pending == 1) wait_vmcnt<DPW>();
        else wait_vmcnt<0>();
        block_barrier();
    }

    // ---- epilogue: O / l, round to bf16, store.  The ring is free after the
    // last barrier; each wave stages its 32 rows in its own part of it and
    // writes them back as whole rows (16-byte lanes, consecutive within a
    // row), not as the accumulators' scattered 8-byte pieces of 32 rows.
    const float lt = l_run + other_half(l_run);
    // no visible key (only a zero-length sequence): a zero row
    const float inv = (!VARLEN || lt > 0.f) ? 1.f / lt : 0.f;
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

}  // namespace

int launch_prefill_bf16(const PrefillArgs &a, int d, bool causal, hipStream_t stream) {
    dim3 grid(a.n_units * a.n_qtiles), block(PF_THREADS);
    // forms: plain, rotary (q rotated at load), variable length
    const int form = a.rope_cos != nullptr ? 1 : a.kv_lens != nullptr ? 2 : 0;
#define GQA_PF_LAUNCH(D_, C_)                                                                  \
    do {                                                                                       \
        if (form == 1)                                                                         \
            hipLaunchKernelGGL((prefill_bf16_kernel<D_, C_, true, false>), grid, block, 0,     \
                               stream, a);                                                     \
        else if (form == 2)                                                                    \
            hipLaunchKernelGGL((prefill_bf16_kernel<D_, C_, false, true>), grid, block, 0,     \
                               stream, a);                                                     \
        else                                                                                   \
            hipLaunchKernelGGL((prefill_bf16_kernel<D_, C_, false, false>), grid, block, 0,    \
                               stream, a);                                                     \
    } while (0)
    if (d == 128) {
        if (causal) GQA_PF_LAUNCH(128, true);
        else GQA_PF_LAUNCH(128, false);
    } else {
        if (causal) GQA_PF_LAUNCH(64, true);
        else GQA_PF_LAUNCH(64, false);
    }
#undef GQA_PF_LAUNCH
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqa
