// Device-side vocabulary shared by the gfx950 kernels: vector types, the
// MFMA fragment maps, the LDS tile swizzle and the XCD-aware work mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rettn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4* lds_i16x4_ptr;

// ---------------------------------------------------------------------------
// Work mapping.  Work-groups are dispatched round-robin over the 8 XCDs
// (work-group i runs on XCD i % 8).  Remap so that each XCD receives a
// contiguous range of work items: consecutive query blocks of the same
// (batch, head) then share that XCD's L2, which holds the head's K/V blocks.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xcd_remap(int wg, int total) {
    const int q = total >> 3, r = total & 7;
    const int x = wg & 7, j = wg >> 3;
    return x * q + (x < r ? x : r) + j;
}

// ---------------------------------------------------------------------------
// LDS tile of K or V: one row per key, RS 16-bit elements per row, stored as
// 16-byte chunks.  Chunk c of key row `key` sits at physical chunk
// c ^ swz(key).  swz gives
//   * 8 distinct chunks for 8 consecutive keys: the ds_read_b128 of a K
//     operand fragment (8 lanes, 8 keys, one logical chunk) is conflict-free;
//   * 4 distinct 32-byte windows for 4 consecutive keys: the transposed
//     ds_read_b64_tr_b16 of a V operand fragment (16 lanes, 4 keys x 32 bytes)
//     is conflict-free.
// ---------------------------------------------------------------------------
__host__ __device__ __forceinline__ int swz(int key) { return ((key & 3) << 1) | ((key >> 2) & 1); }

__device__ __forceinline__ float xhalf_max(float x) {
    // lanes l and l^32 hold the two halves of one query row's keys
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float xhalf_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Wave-wide max / min without LDS: DPP swaps partners at distance 1 and 2
// (quad permutes), then mirrors inside 8 and 16 lanes (each half already
// reduced, so the mirror meets the other half), then the gfx950 permlane
// swaps join lanes 16 and 32 apart.  Every lane ends with the result.
#define RETTN_DPP(X, CTRL) ((uint32_t)__builtin_amdgcn_update_dpp(0, (int)(X), (CTRL), 0xf, 0xf, false))
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, __uint_as_float(RETTN_DPP(__float_as_uint(x), 0xB1)));    // quad_perm [1,0,3,2]
    x = fmaxf(x, __uint_as_float(RETTN_DPP(__float_as_uint(x), 0x4E)));    // quad_perm [2,3,0,1]
    x = fmaxf(x, __uint_as_float(RETTN_DPP(__float_as_uint(x), 0x141)));   // row_half_mirror
    x = fmaxf(x, __uint_as_float(RETTN_DPP(__float_as_uint(x), 0x140)));   // row_mirror
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
    r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ int wave_min(int x) {
    x = min(x, (int)RETTN_DPP(x, 0xB1));
    x = min(x, (int)RETTN_DPP(x, 0x4E));
    x = min(x, (int)RETTN_DPP(x, 0x141));
    x = min(x, (int)RETTN_DPP(x, 0x140));
    auto r = __builtin_amdgcn_permlane16_swap((uint32_t)x, (uint32_t)x, false, false);
    x = min((int)r[0], (int)r[1]);
    r = __builtin_amdgcn_permlane32_swap((uint32_t)x, (uint32_t)x, false, false);
    return min((int)r[0], (int)r[1]);
}
#undef RETTN_DPP

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-uniform reads of read-only tables (CSR row pointers and column ids,
// mask bytes) through the constant address space: they become scalar loads,
// which are counted by lgkmcnt, so waiting for them never drains the vector
// loads (K/V prefetches) that are in flight.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;
__device__ __forceinline__ int32_t scalar_load(const int32_t* p, int64_t i) { return ((const_i32_ptr)p)[i]; }

// One mask byte, wave-uniform.  gfx950 has no scalar byte load: a byte read
// through the constant address space becomes a vector load, and its wait
// (vmcnt) would drain every prefetch issued before it.  So the aligned dword
// holding the byte is read with a scalar load and the byte shifted out.  That
// dword never crosses a page, so its other bytes (possibly just outside the
// mask) are always mapped; they are discarded.
__device__ __forceinline__ uint32_t mask_byte(const uint8_t* p, int64_t i) {
    const uintptr_t addr = (uintptr_t)(p + i);
    const uint32_t w = *(const_u32_ptr)(addr & ~(uintptr_t)3);
    return (w >> (8u * (uint32_t)(addr & 3u))) & 0xffu;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bfloat16 (nearest even) and pack them, low half first.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Round two floats to float16 (nearest even) and pack them, low half first.
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 v = {(_Float16)lo, (_Float16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Eight bfloat16 values (one 16-byte chunk) re-encoded as float16.
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 w) {
    u32x4 o;
    o[0] = pack_f16(bf16_lo(w[0]), bf16_hi(w[0]));
    o[1] = pack_f16(bf16_lo(w[1]), bf16_hi(w[1]));
    o[2] = pack_f16(bf16_lo(w[2]), bf16_hi(w[2]));
    o[3] = pack_f16(bf16_lo(w[3]), bf16_hi(w[3]));
    return o;
}

}  // namespace rettn
