// gqa_device.h -- gfx950 device helpers shared by the GQA kernels.
//
// Lane layouts of the two bf16 MFMA shapes used here (wave64):
//
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds A[m = l%32][k = 8*(l/32) + i], i = 0..7
//     B: lane l holds B[k = 8*(l/32) + i][n = l%32]
//     D: lane l, element r holds D[m = 8*(r/4) + 4*(l/32) + r%4][n = l%32]
//
//   v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] * B[32x16]
//     A: lane l holds A[m = l%16][k = 8*(l/16) + i]
//     B: lane l holds B[k = 8*(l/16) + i][n = l%16]
//     D: lane l, element r holds D[m = 4*(l/16) + r][n = l%16]
//
//   ds_read_b64_tr_b16: in each group of 16 lanes, lanes 4e..4e+3 each point at
//   4 consecutive b16 values; together they form row e (16 values) of a 4x16
//   block, and lane j of the group receives column j of that block.
//
// These were checked on the hardware with exact small-integer products.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

#define GQA_LDS __attribute__((address_space(3)))

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Transposing 64-bit LDS read (4 b16 values), see the layout note above.
__device__ __forceinline__ short4v lds_read_tr16(const __bf16 *lds_ptr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((GQA_LDS short4v *)(lds_ptr));
}

__device__ __forceinline__ bf16x8 join_tr(short4v lo, short4v hi) {
    typedef short short8v __attribute__((ext_vector_type(8)));
    short8v s = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, s);
}

// Value held by lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float other_half(float x) {
    auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(threadIdx.x % 64 < 32 ? p[1] : p[0]);
}

// Read a kernel-lifetime read-only int32 array through the constant address
// space, so that a wave-uniform index becomes a scalar (s_load) read.
__device__ __forceinline__ int load_const(const int32_t *p, int i) {
    return reinterpret_cast<const __attribute__((address_space(4))) int32_t *>(
        reinterpret_cast<uintptr_t>(p))[i];
}

#define GQA_GLOBAL __attribute__((address_space(1)))

// A wave-uniform global address as a scalar value.  readfirstlane returns a
// signed 32-bit int: each half goes through unsigned before it is widened, or
// a low word with bit 31 set would be sign-extended into the high word.
__device__ __forceinline__ unsigned long long uniform_addr(const void *p) {
    const unsigned long long a = (unsigned long long)(uintptr_t)p;
    const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)a);
    const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(a >> 32));
    return ((unsigned long long)hi << 32) | (unsigned long long)lo;
}

// Index of this wave in its work-group, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Work-group ids are handed to the 8 XCDs round-robin (id % 8).  Renumber them
// so that XCD x receives one contiguous range of logical ids: consecutive
// logical ids (tiles that share a key/value head) then run on one XCD and
// share its L2.
__device__ __forceinline__ int xcd_contiguous_id(int id, int total) {
    const int nx = 8;
    int per = total / nx, rem = total % nx;
    int x = id % nx, slot = id / nx;
    return x * per + (x < rem ? x : rem) + slot;
}

// 16-byte direct load from global memory into LDS (global_load_lds_dwordx4):
// lane l's 16 bytes land at LDS byte address lds_base + 16 * l.  lds_base must
// be wave-uniform.  Issued from inline assembly so that the compiler neither
// reorders it across other memory operations ("memory" clobber) nor inserts
// its own conservative waits for it; the caller waits with s_waitcnt vmcnt
// before reading the destination.  It has no register result.
__device__ __forceinline__ void dma16_to_lds(const void *gptr, const GQA_LDS void *lds_base) {
    const unsigned m0v = (unsigned)(uintptr_t)lds_base;
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %0, off"
        :
        : "v"(gptr), "s"(m0v)
        : "memory", "m0");
}

// Raw buffer resource for a byte range [base, base + bytes): reads at offsets
// at or beyond `bytes` are out of range and return zeros.  All fields must be
// wave-uniform so that the descriptor lives in scalar registers.
__device__ __forceinline__ u32x4 make_buffer_rsrc(const void *base, unsigned bytes) {
    const unsigned long long a = (unsigned long long)(uintptr_t)base;
    // readfirstlane: the compiler may have computed a uniform value in vector
    // registers, and the descriptor operand must be scalar
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((unsigned)a);
    r[1] = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32) & 0xffffu);  // stride 0: raw bytes
    r[2] = __builtin_amdgcn_readfirstlane(bytes);                        // num_records, in bytes
    r[3] = 0x00020000u;                                                  // 32-bit data format
    return r;
}

// 16-byte direct load through a buffer resource into LDS
// (buffer_load_dwordx4 ... lds): lane l reads bytes [voffset, voffset + 16)
// of the resource's range (zeros when out of range) and its 16 bytes land at
// lds_base + 16 * l.  Same ordering and waiting rules as dma16_to_lds.
__device__ __forceinline__ void dma16_to_lds_buf(u32x4 rsrc, unsigned voffset,
                                                 const GQA_LDS void *lds_base) {
    const unsigned m0v = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_base);
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(voffset), "s"(rsrc), "s"(m0v)
        : "memory", "m0");
}

__device__ __forceinline__ u32x4 load16(const void *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ void store16_lds(void *p, u32x4 v) {
    *reinterpret_cast<u32x4 *>(p) = v;
}

}  // namespace gqa
