// rope_bf16.hip -- rotary position embedding of the keys (gfx950).
//
// For a key row x of even length d at position p, with tables cos, sin
// [L][d/2] indexed by position ("Attention in Qwen, DeepSeek and LLaMA3", §1,
// apply_rotary_pos_emb):
//   out[i]       = x[2i] cos[p][i] - x[2i+1] sin[p][i]
//   out[d/2 + i] = x[2i] sin[p][i] + x[2i+1] cos[p][i]        (0 <= i < d/2)
// the even/odd pairs rotated and the two results concatenated along the row.
// The rotation runs in fp32 and each output is rounded to bf16 once.  The keys
// are rotated once here, not once per query tile, and the rotated rows are
// what a cache stores; the prefill kernel then reads them like plain keys.
//
// In a decode step the rows are the new token's q or k rows, one position per
// sequence (its length before the append).
//
// One thread per (row, 4 pairs): one 16-byte load of the row, 16-byte loads
// of the 4 cosines and 4 sines, two 8-byte stores (one into each half).
#include "gqa_device.h"
#include "gqa_kernels.h"

namespace gqa {
namespace {

template <int D>
__global__ __launch_bounds__(256) void rope_k_kernel(RopeArgs a) {
    constexpr int QUADS = D / 8;  // 4-pair pieces per row
    const long long n1 = (long long)a.rows * QUADS;
    const long long n = n1 + (long long)a.rows2 * QUADS;
    for (long long t = (long long)blockIdx.x * blockDim.x + threadIdx.x; t < n;
         t += (long long)gridDim.x * blockDim.x) {
        const bool second = t >= n1;
        const long long row = (second ? t - n1 : t) / QUADS;  // [B][L][h] or [B][h] order
        const int quad = (int)(t % QUADS);
        const int h = second ? a.h2 : a.h;
        const int p = a.pos ? min(max(a.pos[row / h], 0), a.L - 1) : (int)((row / h) % a.L);
        const __bf16 *xr = static_cast<const __bf16 *>(second ? a.x2 : a.x) + row * D;
        __bf16 *orow = static_cast<__bf16 *>(second ? a.out2 : a.out) + row * D;
        const int i0 = 4 * quad;  // first pair
        const bf16x8 x = __builtin_bit_cast(bf16x8, load16(xr + 2 * i0));
        const float4 c = *reinterpret_cast<const float4 *>(a.cos + (size_t)p * (D / 2) + i0);
        const float4 s = *reinterpret_cast<const float4 *>(a.sin + (size_t)p * (D / 2) + i0);
        const float cc[4] = {c.x, c.y, c.z, c.w}, ss[4] = {s.x, s.y, s.z, s.w};
        bf16x4 lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x0 = (float)x[2 * e], x1 = (float)x[2 * e + 1];
            lo[e] = (__bf16)(x0 * cc[e] - x1 * ss[e]);
            hi[e] = (__bf16)(x0 * ss[e] + x1 * cc[e]);
        }
        *reinterpret_cast<bf16x4 *>(orow + i0) = lo;
        *reinterpret_cast<bf16x4 *>(orow + D / 2 + i0) = hi;
    }
}

}  // namespace

int launch_rope_k_bf16(const RopeArgs &a, int d, hipStream_t stream) {
    const long long n = ((long long)a.rows + a.rows2) * (d / 8);
    const int blocks = (int)(n / 256 + 1 < 256 * 16 ? n / 256 + 1 : 256 * 16);
    if (d == 128) hipLaunchKernelGGL(rope_k_kernel<128>, dim3(blocks), dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(rope_k_kernel<64>, dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace gqa
