// Tile helpers shared by the prefill and backward kernels for gfx950: vector
// types, the LDS layouts of 32-row tiles that feed v_mfma_f32_32x32x16_*, and
// bounded buffer resources over the rows of one (b, h).
#pragma once

#include "kernels.h"

namespace diffattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Position (in units of 4 keys) of key group kg inside a transposed row.  Key
// k = 16s + 8m + 4h + r of a 32-key tile must sit at 16s + 8h + 4m + r, so that
// lane half h reads the 8 keys {16s + 8m + 4h + r} of product step s as one
// contiguous 16-byte word: the same keys, in the same slot order, that half h
// holds in a 32x32 accumulator (register i is row 8(i/4) + 4h + i%4).  That is
// a swap of bits 0 and 1 of kg.
__device__ __forceinline__ int kVPos(int kg) { return (kg & 4) | ((kg & 1) << 1) | ((kg >> 1) & 1); }

// 16-byte chunk swizzle of 128-byte rows: row r's chunk c sits at
// c ^ kSwz(r).  Any 8 consecutive rows, and the 8 even or the 8 odd rows of
// any 16, read the same logical chunk from 8 distinct chunk slots, so a
// 16-byte read by 8 or 16 lanes (one row each) is free of bank conflicts on 32
// or 64 banks.
__device__ __forceinline__ int kSwz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Buffer resource over rows k0 .. kend-1 of one (b, h) (row stride `stride`
// elements, rows of `row` 16-bit elements): loads past the last valid row
// return zero in hardware, so tile loads need no per-row branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint16_t* base, int64_t stride, int k0, int kend,
                                                             int row) {
  const uint16_t* p = base + (int64_t)k0 * stride;
  const int nrec = kend > k0 ? (int)(((int64_t)(kend - k0 - 1) * stride + row) * 2) : 0;
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, nrec, 0x00020000);
}

// Waits for this wave's outstanding memory loads, the LDS-destination ones
// included (vmcnt 0; export and LDS counters left alone).
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

}  // namespace diffattn
