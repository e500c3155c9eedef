// Device-side helpers shared by the libkdv kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kdv.h"

namespace kdv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short i16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// One 32x32x16 bf16 MFMA: D[32][32] += A[32][16] * B[16][32], fp32 accumulate.
// Lane l holds A[l%32][(l/32)*8 + 0..7], B[(l/32)*8 + 0..7][l%32] and
// D[(r/4)*8 + (l/32)*4 + r%4][l%32] in register r (checked on gfx950).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16: within each 16-lane group, lane q supplies the address of four consecutive
// 16-bit elements at row (q/4), columns 4*(q%4)..+3 of a 4x16 block; lane i then receives column i of
// that block (rows 0..3).  Used to read an MFMA operand whose contraction index runs down LDS rows.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

__device__ __forceinline__ bf16x8 concat_tr(i16x4 lo, i16x4 hi) {
  i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Vector global stores with the SC1 bit (agent scope, the form an agent-scope atomic store takes): the data is
// written through to memory as it is stored rather than left dirty in this XCD's L2 for the end-of-kernel
// writeback, which the next kernel's workgroups (on any XCD) would otherwise wait for.  For results a kernel
// writes in bulk at its end and the next kernel reads.
// The compiler treats an asm block's inputs as read once the block is issued and may overwrite them with the
// next instruction, but a vector store reads more than 8 bytes of data over several cycles: on gfx940 and later
// a VALU write to such a store's data registers must wait 2 states.  The compiler inserts that wait after its
// own stores only, so these blocks end with it (s_nop 1 = 2 wait states).
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;
__device__ __forceinline__ void store_agent16(void* p, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1\n\ts_nop 1" ::"v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_agent8(void* p, u32x2 v) {
  asm volatile("global_store_dwordx2 %0, %1, off sc1\n\ts_nop 1" ::"v"(p), "v"(v) : "memory");
}

// Combine a value across the lane pair (l, l ^ 32) with one VALU swap (v_permlane32_swap) instead of an LDS
// permute.  Swapping a register with itself leaves lane l holding v[l & 31] in the first result and
// v[(l & 31) + 32] in the second; both lanes of a pair combine the two in the same order, so they get the same bits.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

}  // namespace kdv
