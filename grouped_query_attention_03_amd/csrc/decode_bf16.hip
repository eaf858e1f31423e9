// decode_bf16.hip -- grouped-query attention decode over a head-major KV cache.
//
// One new query position per sequence attends to cache rows [0, seqlens[b]) of
// k_cache/v_cache [B, h_kv, S, d] ("What is Grouped-Query Attention", §2.2 step 2
// for the cache layout, §3.2 for attending over the appended cache).  The pass
// is bound by reading the cache, so the design goal is to read every valid
// cache byte exactly once per key/value head, never once per query head:
//
// decode_split: one work-group per (sequence, key/value head, chunk of CH keys).
//   The G query heads of the group are stacked as the N dimension of a
//   v_mfma_f32_16x16x32_bf16 (S^T = K Q^T, keys on M), so one read of a cache
//   row serves every query head of the group.  K rows go straight from HBM into
//   MFMA A-operand registers with 16-byte loads; V rows go through a
//   wave-private LDS buffer and come back transposed (ds_read_b64_tr_b16) as the
//   A operand of O^T = V^T P^T.  The 4 waves take interleaved 32-key blocks of
//   the chunk and prefetch the next block while computing the current one.
//   Each chunk leaves, per query head, its normalised partial output and its
//   log-sum-exp (base 2, in units of scale*log2(e)) in the workspace.
// decode_merge: one wave per (sequence, query head) combines the chunks with
//   weights 2^(lse_c - max lse), i.e. the exact log-sum-exp merge.
// Rows at or beyond seqlens[b] are never loaded.
#include "gqa_device.h"
#include "gqa_kernels.h"

namespace gqa {
namespace {

constexpr int DC_THREADS = 256;
constexpr int DC_WAVES = 4;
constexpr int DC_BK = 32;          // keys per block
constexpr float DC_TAU = 8.0f;     // lazy-rescale threshold, log2 units

template <int D>
struct DcLayout {
    static constexpr int VS = D + 16;                  // V row stride in LDS, elements
    static constexpr int V_ELEMS = DC_BK * VS;         // one wave's V block
    static constexpr int KSTEPS = D / 32;              // 16x16x32 k-steps over d
    static constexpr int KLOADS = 2 * KSTEPS;          // 16-byte K loads per lane per block
    static constexpr int VLOADS = DC_BK * D / 8 / 64;  // 16-byte V loads per lane per block
    static constexpr int OS = D + 1;                   // combine buffer row stride, floats
    static constexpr int V_BYTES = DC_WAVES * V_ELEMS * 2;
    static constexpr int C_BYTES = DC_WAVES * (16 * OS + 32) * 4;
    static constexpr int BYTES = V_BYTES > C_BYTES ? V_BYTES : C_BYTES;
};

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int D>
__device__ __forceinline__ void dc_load_block(const __bf16 *__restrict__ kb,
                                              const __bf16 *__restrict__ vb, int key0, int kend,
                                              u32x4 (&kr)[DcLayout<D>::KLOADS],
                                              u32x4 (&vr)[DcLayout<D>::VLOADS]) {
    using Lay = DcLayout<D>;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const int key = key0 + 16 * mb + (lane & 15);
        const bool ok = key < kend;
#pragma unroll
        for (int ks = 0; ks < Lay::KSTEPS; ++ks)
            kr[mb * Lay::KSTEPS + ks] =
                ok ? load16(kb + (size_t)key * D + 32 * ks + 8 * (lane >> 4)) : u32x4{0u, 0u, 0u, 0u};
    }
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < Lay::VLOADS; ++i) {
        const int cidx = lane + 64 * i;
        const int row = cidx / CPR, col = cidx % CPR;
        const int key = key0 + row;
        vr[i] = key < kend ? load16(vb + (size_t)key * D + 8 * col) : u32x4{0u, 0u, 0u, 0u};
    }
}

template <int D>
__global__ __launch_bounds__(DC_THREADS) void decode_split_kernel(DecodeArgs a) {
    using Lay = DcLayout<D>;
    constexpr int DB = D / 16;  // 16-wide blocks of the head dimension
    __shared__ __attribute__((aligned(16))) char smem[Lay::BYTES];

    const int chunk = blockIdx.x;
    const int kvh = blockIdx.y / a.n_qsub, qs = blockIdx.y % a.n_qsub;
    const int b = blockIdx.z;
    const int seqlen = a.seqlens[b];
    const int c0 = chunk * a.CH;
    if (c0 >= seqlen) return;  // whole work-group exits together
    const int kend = min(seqlen, c0 + a.CH);
    const int nblocks = (kend - c0 + DC_BK - 1) / DC_BK;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, jl = lane & 15;
    const int heads_here = min(16, a.G - 16 * qs);
    const int qcol = lane & 15;  // query head (within the subgroup) of this lane's column
    const int head_base = kvh * a.G + 16 * qs;

    // Q^T operand: lane holds 8 head-dim values of query column qcol.
    bf16x8 qf[Lay::KSTEPS];
    if (qcol < heads_here) {
        const __bf16 *qp = static_cast<const __bf16 *>(a.q) +
                           ((size_t)b * a.h_q + head_base + qcol) * D + 8 * g;
#pragma unroll
        for (int ks = 0; ks < Lay::KSTEPS; ++ks)
            qf[ks] = __builtin_bit_cast(bf16x8, load16(qp + 32 * ks));
    } else {
#pragma unroll
        for (int ks = 0; ks < Lay::KSTEPS; ++ks) qf[ks] = bf16x8{};
    }

    const size_t slab = ((size_t)b * a.h_kv + kvh) * (size_t)a.S * D;
    const __bf16 *kb = static_cast<const __bf16 *>(a.k_cache) + slab;
    const __bf16 *vb = static_cast<const __bf16 *>(a.v_cache) + slab;
    __bf16 *vw = reinterpret_cast<__bf16 *>(smem) + wave * Lay::V_ELEMS;

    f32x4 acc[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[db] = f32x4{};
    float m_run = -INFINITY, l_run = 0.f;
    const float c = a.c;

    u32x4 kr[Lay::KLOADS], vr[Lay::VLOADS];
    int blk = wave;
    if (blk < nblocks) dc_load_block<D>(kb, vb, c0 + DC_BK * blk, kend, kr, vr);

    for (; blk < nblocks; blk += DC_WAVES) {
        const int key0 = c0 + DC_BK * blk;
        // stage this block's V rows in the wave's LDS buffer
        constexpr int CPR = D / 8;
#pragma unroll
        for (int i = 0; i < Lay::VLOADS; ++i) {
            const int cidx = lane + 64 * i;
            store16_lds(vw + (cidx / CPR) * Lay::VS + 8 * (cidx % CPR), vr[i]);
        }
        u32x4 kcur[Lay::KLOADS];
#pragma unroll
        for (int i = 0; i < Lay::KLOADS; ++i) kcur[i] = kr[i];
        // prefetch the wave's next block
        if (blk + DC_WAVES < nblocks) dc_load_block<D>(kb, vb, key0 + DC_BK * DC_WAVES, kend, kr, vr);

        // S^T = K Q^T: two 16-key m-blocks
        f32x4 s[2] = {f32x4{}, f32x4{}};
#pragma unroll
        for (int ks = 0; ks < Lay::KSTEPS; ++ks)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb)
                s[mb] = mfma16x16x32(__builtin_bit_cast(bf16x8, kcur[mb * Lay::KSTEPS + ks]), qf[ks], s[mb]);
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
        wave_sync();  // the V block written above is visible to the whole wave
        const __bf16 *vp = vw + (4 * g + (jl >> 2)) * Lay::VS + 4 * (jl & 3);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            short4v lo = lds_read_tr16(vp + 16 * db);
            short4v hi = lds_read_tr16(vp + 16 * Lay::VS + 16 * db);
            acc[db] = mfma16x16x32(join_tr(lo, hi), pb, acc[db]);
        }
        wave_sync();  // reads of this block finish before the next block is staged
    }

    // ---- combine the 4 waves of the work-group
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += other_half(l_tot);
    __syncthreads();  // V buffers are reused below
    float *cO = reinterpret_cast<float *>(smem);                // [wave][16][OS]
    float *cm = cO + DC_WAVES * 16 * Lay::OS;                   // [wave][16]
    float *cl = cm + DC_WAVES * 16;                             // [wave][16]
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 4; ++r) cO[(wave * 16 + qcol) * Lay::OS + 16 * db + 4 * g + r] = acc[db][r];
    if (g == 0) {
        cm[wave * 16 + qcol] = m_run;
        cl[wave * 16 + qcol] = l_tot;
    }
    __syncthreads();
    float *opart = a.opart;
    float *lse = a.lse;
    for (int idx = tid; idx < heads_here * D; idx += DC_THREADS) {
        const int q = idx / D, dd = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < DC_WAVES; ++w) M = fmaxf(M, cm[w * 16 + q]);
        float wsum = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < DC_WAVES; ++w) {
            const float mw = cm[w * 16 + q];
            const float f = (mw == -INFINITY) ? 0.f : fast_exp2(mw - M);
            wsum += f * cl[w * 16 + q];
            o += f * cO[(w * 16 + q) * Lay::OS + dd];
        }
        const size_t row = ((size_t)b * a.h_q + head_base + q) * a.NC + chunk;
        opart[row * D + dd] = o / wsum;
        if (dd == 0) lse[row] = M + __log2f(wsum);
    }
}

template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs a) {
    constexpr int PER = D / 64;
    const int lane = threadIdx.x & 63;
    const int wid = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wid >= a.B * a.h_q) return;
    const int b = wid / a.h_q;
    const int seqlen = a.seqlens[b];
    const int n = (seqlen + a.CH - 1) / a.CH;
    __bf16 *op = static_cast<__bf16 *>(a.o) + (size_t)wid * D + PER * lane;
    if (n <= 0) {
#pragma unroll
        for (int e = 0; e < PER; ++e) op[e] = (__bf16)0.f;
        return;
    }
    const float *lp = a.lse + (size_t)wid * a.NC;
    const float *pp = a.opart + (size_t)wid * a.NC * D + PER * lane;
    float M = -INFINITY;
    for (int cidx = 0; cidx < n; ++cidx) M = fmaxf(M, lp[cidx]);
    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.f;
    float wsum = 0.f;
    for (int cidx = 0; cidx < n; ++cidx) {
        const float w = fast_exp2(lp[cidx] - M);
        wsum += w;
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] = fmaf(w, pp[(size_t)cidx * D + e], acc[e]);
    }
    const float inv = 1.f / wsum;
#pragma unroll
    for (int e = 0; e < PER; ++e) op[e] = (__bf16)(acc[e] * inv);
}

}  // namespace

int launch_decode_bf16(const DecodeArgs &a, int d, hipStream_t stream) {
    dim3 grid1(a.NC, a.h_kv * a.n_qsub, a.B), block(DC_THREADS);
    dim3 grid2((a.B * a.h_q + 3) / 4);
    if (d == 128) {
        hipLaunchKernelGGL(decode_split_kernel<128>, grid1, block, 0, stream, a);
        hipLaunchKernelGGL(decode_merge_kernel<128>, grid2, block, 0, stream, a);
    } else {
        hipLaunchKernelGGL(decode_split_kernel<64>, grid1, block, 0, stream, a);
        hipLaunchKernelGGL(decode_merge_kernel<64>, grid2, block, 0, stream, a);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqa
