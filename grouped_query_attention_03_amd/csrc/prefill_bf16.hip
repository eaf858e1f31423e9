// prefill_bf16.hip -- grouped-query attention prefill on bf16 MFMA (gfx950).
//
// Computes o = softmax(q k^T * scale) v for every query row, where query head h
// reads key/value head floor(h / G), G = h_q / h_kv ("Modern LLM architecture
// (1): GQA and RMSNorm", §2.1 formula, §2.3 grouping; "Attention in Qwen,
// DeepSeek and LLaMA3", §2.2 head map).  The softmax is evaluated tile by tile
// with running statistics (the on-chip, no-HBM-round-trip form that "What is
// Grouped-Query Attention", §4.3 credits to FlashAttention), which is an exact
// rearrangement of the row softmax.
//
// Work decomposition
//   One work-group (4 waves) owns 256 query rows: GW query heads of ONE group
//   times BM = 256 / GW consecutive positions (GW = the largest power of two
//   dividing G, at most 8; larger groups are split over G / GW work-groups).
//   Each key/value tile is loaded into LDS once and used by all GW heads: this
//   is the group-sharing saving, the key/value head is never copied per query
//   head.  Rows are cut into 8 row blocks of 32 (one head x 32 positions);
//   wave w owns row blocks 2w and 2w+1.
//
// Per wave and per key tile of 64 keys (S^T formulation)
//   S^T[key][query] = K Q^T on v_mfma_f32_32x32x16_bf16: A = K rows read from
//   LDS (16-byte reads), B = Q^T kept in registers for the whole kernel.  In
//   the accumulator layout each lane holds 16 keys of ONE query column, so the
//   row max and row sum are in-lane reductions plus one exchange with the
//   other half-wave.
//   P = exp2(S * scale*log2(e) - m) with a lazily updated running max m: the
//   accumulators are rescaled only when a row max grows by more than TAU (in
//   log2 units), which keeps every P <= 2^TAU and skips almost all rescales.
//   O^T[d][query] += V^T P^T: P^T comes straight out of the S^T accumulators
//   (keys permuted consistently on both operands), V^T is read from the
//   row-major V tile with the transposing ds_read_b64_tr_b16.
//   Causal: tiles wholly above the diagonal are never visited, the diagonal
//   and the sequence tail are masked element-wise.
#include <stdlib.h>

#include "gqa_device.h"
#include "gqa_kernels.h"

namespace gqa {
namespace {

constexpr int PF_ROWS = 256;     // query rows per work-group (8 row blocks of 32)
constexpr int PF_BN = 64;       // keys per tile
constexpr float PF_TAU = 8.0f;  // lazy-rescale threshold, log2 units

template <int D, int THREADS>
struct PfLayout {
    // K rows padded by 16 bytes: 16 lanes reading 16 rows at one column hit
    // 16 distinct 4-bank groups.  V rows padded so the 4-row x 32-byte blocks
    // of a transposing read fall in distinct banks.
    static constexpr int KS = D + 8;   // K row stride, elements
    static constexpr int VS = D + 32;  // V row stride, elements
    static constexpr int K_ELEMS = PF_BN * KS;
    static constexpr int V_ELEMS = PF_BN * VS;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
    static constexpr int CHUNKS = PF_BN * D / 8;          // 16-byte chunks per tile
    static constexpr int PER_THREAD = CHUNKS / THREADS;   // per K (and per V)
};

template <int D, int THREADS>
__device__ __forceinline__ void pf_load_tile(const __bf16 *__restrict__ src, size_t row_stride,
                                             int j0, int L,
                                             u32x4 (&r)[PfLayout<D, THREADS>::PER_THREAD]) {
    constexpr int CPR = D / 8;  // chunks per row
#pragma unroll
    for (int i = 0; i < PfLayout<D, THREADS>::PER_THREAD; ++i) {
        int c = threadIdx.x + THREADS * i;
        int row = c / CPR, col = c % CPR;
        int key = j0 + row;
        if (key < L)
            r[i] = load16(src + (size_t)key * row_stride + 8 * col);
        else
            r[i] = u32x4{0u, 0u, 0u, 0u};
    }
}

template <int D, int THREADS, int STRIDE>
__device__ __forceinline__ void pf_store_tile(__bf16 *lds,
                                              const u32x4 (&r)[PfLayout<D, THREADS>::PER_THREAD]) {
    constexpr int CPR = D / 8;
#pragma unroll
    for (int i = 0; i < PfLayout<D, THREADS>::PER_THREAD; ++i) {
        int c = threadIdx.x + THREADS * i;
        int row = c / CPR, col = c % CPR;
        store16_lds(lds + row * STRIDE + 8 * col, r[i]);
    }
}

// NW waves per work-group; each wave owns RB = 8 / NW row blocks of 32 rows.
template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(NW * 64, 1) void prefill_bf16_kernel(PrefillArgs a) {
    constexpr int THREADS = NW * 64;
    constexpr int RB = 8 / NW;
    using Lay = PfLayout<D, THREADS>;
    constexpr int KSTEPS = D / 16;  // MFMA k-steps over the head dimension
    constexpr int DB = D / 32;      // 32-wide blocks of the head dimension
    __shared__ __attribute__((aligned(16))) __bf16 smem[2 * Lay::STAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = wave_id();
    const int lid = xcd_contiguous_id(blockIdx.x, gridDim.x);
    const int unit = lid / a.n_qtiles;
    int qt = lid % a.n_qtiles;
    if (CAUSAL) qt = a.n_qtiles - 1 - qt;  // longest rows first
    const int sub = unit % a.nsub;
    const int bk = unit / a.nsub;
    const int kvh = bk % a.h_kv;
    const int b = bk / a.h_kv;
    const int L = a.L;
    const int PB = 8 / a.GW;  // 32-position blocks per work-group
    const int p0 = qt * a.BM;

    const __bf16 *kbase = static_cast<const __bf16 *>(a.k) + ((size_t)b * L * a.h_kv + kvh) * D;
    const __bf16 *vbase = static_cast<const __bf16 *>(a.v) + ((size_t)b * L * a.h_kv + kvh) * D;
    const size_t kv_row = (size_t)a.h_kv * D;

    int head[RB], pos0[RB];
#pragma unroll
    for (int t = 0; t < RB; ++t) {
        int rb = RB * wave + t;
        head[t] = kvh * a.G + sub * a.GW + rb / PB;
        pos0[t] = p0 + 32 * (rb % PB);
    }

    // Q^T operands: lane holds 8 head-dim values of one query row.
    bf16x8 qf[RB][KSTEPS];
#pragma unroll
    for (int t = 0; t < RB; ++t) {
        int pos = pos0[t] + (lane & 31);
        if (pos < L) {
            const __bf16 *qp = static_cast<const __bf16 *>(a.q) +
                               (((size_t)b * L + pos) * a.h_q + head[t]) * D + 8 * (lane >> 5);
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks)
                qf[t][ks] = __builtin_bit_cast(bf16x8, load16(qp + 16 * ks));
        } else {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) qf[t][ks] = bf16x8{};
        }
    }

    f32x16 acc[RB][DB];
#pragma unroll
    for (int t = 0; t < RB; ++t)
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[t][db] = f32x16{};
    float m_run[RB], l_run[RB];
#pragma unroll
    for (int t = 0; t < RB; ++t) {
        m_run[t] = -INFINITY;
        l_run[t] = 0.f;
    }

    const int kv_end = CAUSAL ? min(L, p0 + a.BM) : L;
    const int ntiles = (kv_end + PF_BN - 1) / PF_BN;
    int wave_last_pos = pos0[0] + 31, wave_first_pos = pos0[0];
#pragma unroll
    for (int t = 1; t < RB; ++t) {
        wave_last_pos = max(wave_last_pos, pos0[t] + 31);
        wave_first_pos = min(wave_first_pos, pos0[t]);
    }
    const bool wave_has_rows = wave_first_pos < L;
    const float c = a.c;

    u32x4 kr[Lay::PER_THREAD], vr[Lay::PER_THREAD];
    pf_load_tile<D, THREADS>(kbase, kv_row, 0, L, kr);
    pf_load_tile<D, THREADS>(vbase, kv_row, 0, L, vr);
    pf_store_tile<D, THREADS, Lay::KS>(smem, kr);
    pf_store_tile<D, THREADS, Lay::VS>(smem + Lay::K_ELEMS, vr);
    __syncthreads();

    for (int j = 0; j < ntiles; ++j) {
        const int j0 = j * PF_BN;
        const bool more = j + 1 < ntiles;
        if (more) {
            pf_load_tile<D, THREADS>(kbase, kv_row, j0 + PF_BN, L, kr);
            pf_load_tile<D, THREADS>(vbase, kv_row, j0 + PF_BN, L, vr);
        }
        const __bf16 *ks_lds = smem + (j & 1) * Lay::STAGE;
        const __bf16 *vs_lds = ks_lds + Lay::K_ELEMS;

        if (wave_has_rows && (!CAUSAL || j0 <= wave_last_pos)) {
            // ---- S^T = K Q^T for 2 key blocks x RB row blocks
            f32x16 s[RB][2];
#pragma unroll
            for (int t = 0; t < RB; ++t) s[t][0] = s[t][1] = f32x16{};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    bf16x8 ka = *reinterpret_cast<const bf16x8 *>(
                        ks_lds + (32 * kb + (lane & 31)) * Lay::KS + 16 * ks + 8 * (lane >> 5));
#pragma unroll
                    for (int t = 0; t < RB; ++t) s[t][kb] = mfma32x32x16(ka, qf[t][ks], s[t][kb]);
                }
            }
            // ---- mask the diagonal tile and the tail of the sequence
            const bool need_mask = (j0 + PF_BN > L) || (CAUSAL && j0 + PF_BN - 1 > wave_first_pos);
            if (need_mask) {
#pragma unroll
                for (int t = 0; t < RB; ++t) {
                    const int pos = pos0[t] + (lane & 31);
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            int key = j0 + 32 * kb + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                            bool masked = key >= L || (CAUSAL && key > pos);
                            s[t][kb][r] = masked ? -INFINITY : s[t][kb][r];
                        }
                }
            }
            // ---- running max with lazy rescale
            float mnew[RB];
            bool grow = false;
#pragma unroll
            for (int t = 0; t < RB; ++t) {
                float mx = s[t][0][0];
#pragma unroll
                for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[t][0][r]);
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][1][r]);
                mx = fmaxf(mx, other_half(mx));
                mnew[t] = mx * c;
                grow = grow || (mnew[t] > m_run[t] + PF_TAU);
            }
            if (__any(grow)) {
#pragma unroll
                for (int t = 0; t < RB; ++t) {
                    float m2 = fmaxf(m_run[t], mnew[t]);
                    float alpha = (m2 == -INFINITY) ? 1.f : fast_exp2(m_run[t] - m2);
                    m_run[t] = m2;
                    l_run[t] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db) acc[t][db] *= alpha;
                }
            }
            // ---- P = exp2(S*c - m), row sums, pack to bf16 as the B operand of PV
            bf16x8 pb[RB][2][2];  // [row block][key block][16-key half]
#pragma unroll
            for (int t = 0; t < RB; ++t) {
                const float mu = (m_run[t] == -INFINITY) ? 0.f : m_run[t];
                float lsum = 0.f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                        for (int i = 0; i < 8; ++i) {
                            float p = fast_exp2(fmaf(s[t][kb][8 * hh + i], c, -mu));
                            lsum += p;
                            pb[t][kb][hh][i] = (__bf16)p;
                        }
                l_run[t] += lsum;
            }
            // ---- O^T += V^T P^T
            const int grp = lane >> 4, jl = lane & 15;
            const int vrow = 4 * (grp >> 1) + (jl >> 2);
            const int vcol = 16 * (grp & 1) + 4 * (jl & 3);
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const __bf16 *vp = vs_lds + (32 * kb + 16 * hh + vrow) * Lay::VS + vcol;
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        short4v lo = lds_read_tr16(vp + 32 * db);
                        short4v hi = lds_read_tr16(vp + 8 * Lay::VS + 32 * db);
                        bf16x8 va = join_tr(lo, hi);
#pragma unroll
                        for (int t = 0; t < RB; ++t)
                            acc[t][db] = mfma32x32x16(va, pb[t][kb][hh], acc[t][db]);
                    }
                }
        }
        if (more) {
            __bf16 *nxt = smem + ((j + 1) & 1) * Lay::STAGE;
            pf_store_tile<D, THREADS, Lay::KS>(nxt, kr);
            pf_store_tile<D, THREADS, Lay::VS>(nxt + Lay::K_ELEMS, vr);
        }
        __syncthreads();
    }

    // ---- epilogue: O / l, round to bf16, store
#pragma unroll
    for (int t = 0; t < RB; ++t) {
        float lt = l_run[t] + other_half(l_run[t]);
        float inv = 1.f / lt;
        int pos = pos0[t] + (lane & 31);
        if (pos < L) {
            __bf16 *op = static_cast<__bf16 *>(a.o) +
                         (((size_t)b * L + pos) * a.h_q + head[t]) * D + 4 * (lane >> 5);
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int rq = 0; rq < 4; ++rq) {
                    bf16x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[t][db][4 * rq + e] * inv);
                    *reinterpret_cast<bf16x4 *>(op + 32 * db + 8 * rq) = w;
                }
        }
    }
}

template <int D, bool CAUSAL>
void launch_variant(const PrefillArgs &a, hipStream_t stream) {
    dim3 grid(a.n_units * a.n_qtiles);
    // GQA_PREFILL_WAVES selects 4 or 8 waves per work-group (default 8)
    static const int nw = [] {
        const char *e = getenv("GQA_PREFILL_WAVES");
        return (e && atoi(e) == 4) ? 4 : 8;
    }();
    if (nw == 4)
        hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, 4>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((prefill_bf16_kernel<D, CAUSAL, 8>), grid, dim3(512), 0, stream, a);
}

}  // namespace

int launch_prefill_bf16(const PrefillArgs &a, int d, bool causal, hipStream_t stream) {
    if (d == 128) {
        if (causal) launch_variant<128, true>(a, stream);
        else launch_variant<128, false>(a, stream);
    } else {
        if (causal) launch_variant<64, true>(a, stream);
        else launch_variant<64, false>(a, stream);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqa
