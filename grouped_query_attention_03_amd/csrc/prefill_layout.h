// prefill_layout.h -- tile geometry and helpers shared by the bf16 prefill
// kernels: 64-key tiles of K and V moved into LDS by direct loads, their
// bank swizzles, and the wait and barrier primitives of the tile loop.
#pragma once

#include "gqa_device.h"

namespace gqa {
namespace {

constexpr int PF_BN = 64;       // keys per tile
constexpr float PF_TAU = 8.0f;  // lazy-rescale threshold, log2 units

// Forms of the kernel: q rotated at load (ROPE), per-sequence key lengths
// (VARLEN), a keep-mask of bytes (MASK).
enum PfForm { kPfPlain = 0, kPfRope = 1, kPfVarlen = 2, kPfMask = 3 };

template <int D>
struct PfLay {
    static constexpr int ROW_BYTES = 2 * D;
    static constexpr int CPR = D / 8;                        // 16-byte chunks per row
    static constexpr int ROWS_PER_DMA = 64 / CPR;            // rows per 64-lane 16-byte load
    static constexpr int TILE_BYTES = PF_BN * ROW_BYTES;     // one K or V tile
    static constexpr int DMA_PER_TENSOR = TILE_BYTES / 1024;  // 1 KiB direct loads per tile
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

// Make the compiler wait for the loads behind x here.  It does not see the
// direct-to-LDS loads (inline asm), so its own count of pending vector loads
// holds only the q loads; consumed here, they need no wait inside the loop.
template <int N>
__device__ __forceinline__ void pf_settle(const bf16x8 (&x)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" ::"v"(x[i]));
}

// An empty statement with side effects.  Placed in a rarely taken,
// wave-uniform branch it keeps the compiler from speculating the branch into
// straight-line selects and multiplies that would then run on every tile.
__device__ __forceinline__ void pf_keep_branch() { asm volatile(""); }

__device__ __forceinline__ void block_barrier() {
    asm volatile("s_barrier" ::: "memory");
}

}  // namespace
}  // namespace gqa
