// prefill_f32.hip -- grouped-query attention prefill in fp32 (vector ALU).
//
// The fp32 path keeps every product and sum in fp32 (no bf16 rounding of the
// probabilities), for inputs that must match an fp64 result to 1e-4.  It uses
// the same work map as the bf16 kernel: a work-group owns GW query heads of one
// group times BM positions (256 rows, one per thread), and each key/value tile
// is staged once in LDS and read by all of them (query head h reads key/value
// head floor(h / G): "Modern LLM architecture (1): GQA and RMSNorm", §2.3).
// The softmax is the exact running-max form: per 32-key tile, new max, rescale
// of the running sum and output, then accumulation of exp2(s - m) v.
// Key j is hidden from a row past the sequence's length (kv_lens), above the
// causal diagonal, or where the keep-mask byte of (row, j) is zero.
#include "gqa_device.h"
#include "gqa_kernels.h"

namespace gqa {
namespace {

constexpr int PF32_THREADS = 256;
constexpr int PF32_BN = 32;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(PF32_THREADS) void prefill_f32_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) float ksm[PF32_BN * D];
    __shared__ __attribute__((aligned(16))) float vsm[PF32_BN * D];

    const int tid = threadIdx.x;
    const int lid = xcd_contiguous_id(blockIdx.x, gridDim.x);
    const int unit = lid / a.n_qtiles;
    int qt = lid % a.n_qtiles;
    if (CAUSAL) qt = a.n_qtiles - 1 - qt;
    const int sub = unit % a.nsub;
    const int bk = unit / a.nsub;
    const int kvh = bk % a.h_kv;
    const int b = bk / a.h_kv;
    const int L = a.L, off = a.off;  // query rows, position of row 0
    const int Lt = a.Lk;             // key rows per sequence in the tensors
    // visible keys of this sequence: all, or its length (clamped to [0, Lt])
    const int Lk = a.kv_lens ? min(max(load_const(a.kv_lens, b), 0), Lt) : Lt;
    const int p0 = qt * a.BM;
    const int hl = tid / a.BM, pp = tid % a.BM;
    const int pos = p0 + pp;
    const int head = kvh * a.G + sub * a.GW + hl;

    const float *qg = static_cast<const float *>(a.q);
    const float *kg = static_cast<const float *>(a.k) + ((size_t)b * Lt * a.h_kv + kvh) * D;
    const float *vg = static_cast<const float *>(a.v) + ((size_t)b * Lt * a.h_kv + kvh) * D;
    const size_t kv_row = (size_t)a.h_kv * D;
    // this row's keep-mask bytes (keep-mask form), keys 0 .. Lk - 1
    const uint8_t *mrow = a.mask && pos < L
                              ? a.mask + (size_t)b * (size_t)a.mask_batch +
                                    (size_t)pos * (size_t)a.mask_row
                              : nullptr;

    float qv[D], ov[D];
    if (pos < L) {
        const float *qp = qg + (((size_t)b * L + pos) * a.h_q + head) * D;
#pragma unroll
        for (int cc = 0; cc < D; ++cc) qv[cc] = qp[cc] * a.c;
    } else {
#pragma unroll
        for (int cc = 0; cc < D; ++cc) qv[cc] = 0.f;
    }
#pragma unroll
    for (int cc = 0; cc < D; ++cc) ov[cc] = 0.f;
    float m = -INFINITY, l = 0.f;

    const int kv_end = CAUSAL ? min(Lk, off + p0 + a.BM) : Lk;
    for (int j0 = 0; j0 < kv_end; j0 += PF32_BN) {
        __syncthreads();
        constexpr int F4_PER_ROW = D / 4;
        for (int idx = tid; idx < PF32_BN * F4_PER_ROW; idx += PF32_THREADS) {
            int row = idx / F4_PER_ROW, col = idx % F4_PER_ROW;
            int key = j0 + row;
            float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
            if (key < Lk) {
                kx = *reinterpret_cast<const float4 *>(kg + (size_t)key * kv_row + 4 * col);
                vx = *reinterpret_cast<const float4 *>(vg + (size_t)key * kv_row + 4 * col);
            }
            *reinterpret_cast<float4 *>(ksm + row * D + 4 * col) = kx;
            *reinterpret_cast<float4 *>(vsm + row * D + 4 * col) = vx;
        }
        __syncthreads();

        float s[PF32_BN];
        float mx = -INFINITY;
#pragma unroll
        for (int kk = 0; kk < PF32_BN; ++kk) {
            float dot = 0.f;
#pragma unroll
            for (int cc = 0; cc < D; ++cc) dot = fmaf(qv[cc], ksm[kk * D + cc], dot);
            int key = j0 + kk;
            bool masked = key >= Lk || (CAUSAL && key > off + pos);
            if (a.mask) masked = masked || mrow == nullptr || mrow[key] == 0;
            s[kk] = masked ? -INFINITY : dot;
            mx = fmaxf(mx, s[kk]);
        }
        float m2 = fmaxf(m, mx);
        if (m2 == -INFINITY) continue;  // nothing visible to this row yet
        float alpha = fast_exp2(m - m2);
        m = m2;
        l *= alpha;
#pragma unroll
        for (int cc = 0; cc < D; ++cc) ov[cc] *= alpha;
#pragma unroll
        for (int kk = 0; kk < PF32_BN; ++kk) {
            float p = fast_exp2(s[kk] - m);
            l += p;
#pragma unroll
            for (int cc = 0; cc < D; ++cc) ov[cc] = fmaf(p, vsm[kk * D + cc], ov[cc]);
        }
    }

    if (pos < L) {
        float inv = l > 0.f ? 1.f / l : 0.f;  // no visible key: a zero row
        float *op = static_cast<float *>(a.o) + (((size_t)b * L + pos) * a.h_q + head) * D;
#pragma unroll
        for (int cc = 0; cc < D; cc += 4)
            *reinterpret_cast<float4 *>(op + cc) =
                make_float4(ov[cc] * inv, ov[cc + 1] * inv, ov[cc + 2] * inv, ov[cc + 3] * inv);
    }
}

}  // namespace

int launch_prefill_f32(const PrefillArgs &a, int d, bool causal, hipStream_t stream) {
    dim3 grid(a.n_units * a.n_qtiles), block(PF32_THREADS);
    if (d == 128) {
        if (causal) hipLaunchKernelGGL((prefill_f32_kernel<128, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((prefill_f32_kernel<128, false>), grid, block, 0, stream, a);
    } else {
        if (causal) hipLaunchKernelGGL((prefill_f32_kernel<64, true>), grid, block, 0, stream, a);
        else hipLaunchKernelGGL((prefill_f32_kernel<64, false>), grid, block, 0, stream, a);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqa
