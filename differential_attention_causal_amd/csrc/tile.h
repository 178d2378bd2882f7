// Tile helpers shared by the prefill and backward kernels for gfx950: vector
// types, the LDS layouts of 32-row tiles that feed v_mfma_f32_32x32x16_*, and
// bounded buffer resources over the rows of one (b, h).
#pragma once

#include "extent.h"
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
  const int nrec = (int)rows_extent_bytes(stride, k0, kend, row);
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0, nrec, 0x00020000);
}

// Buffer resource over the fp16 V^T tiles (vtiles.hip) of the bh-th (b, h)
// of a T-key tensor: tiles past the last read as zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t vt_tiles_rsrc(const uint16_t* vt, int64_t bh, int T) {
  const int nt = (T + 31) / 32;
  const uint16_t* p = vt + bh * nt * (kVtTileBytes / 2);
  return __builtin_amdgcn_make_buffer_rsrc((void*)p, (short)0,
                                           (int)rows_extent_bytes(kVtTileBytes / 2, 0, nt, kVtTileBytes / 2),
                                           0x00020000);
}

// Memory -> LDS of one 8 KiB V^T tile by the four waves that stage it: wave
// `part` moves bytes 2048 part .. +2047 (two loads of 64 lanes x 16 bytes).
// The instruction's immediate offset would move the LDS destination as well,
// so the second half's 1 KiB step goes into the per-lane offset.
__device__ __forceinline__ void dma_vt(__amdgpu_buffer_rsrc_t r, char* vt_lds, int tile, int part, int lane) {
  char* dst = vt_lds + part * 2048;
  const uint32_t off = (uint32_t)tile * kVtTileBytes + part * 2048 + lane * 16;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, off, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(dst + 1024), 16, off + 1024, 0, 0, 0);
}

// The V^T operand of one P V product from a DMA'd tile: channel row
// 32 cb + lq, keys 16 s .. 16 s + 15, lane half hf's eight (one swizzled chunk).
__device__ __forceinline__ f16x8 vt_operand(const char* vt, int lq, int hf, int cb, int s) {
  return *reinterpret_cast<const f16x8*>(vt + (32 * cb + lq) * 64 + (((2 * s + hf) ^ ((lq >> 2) & 3)) << 4));
}

// Waits for this wave's outstanding memory loads, the LDS-destination ones
// included (vmcnt 0; export and LDS counters left alone).
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Waits: vmcnt(n) alone, lgkmcnt(0) alone (gfx9 s_waitcnt encoding).
template <int n>
__device__ __forceinline__ void wait_vm() { __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | 0x0F70); }
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier with no memory wait of its own; the asm memory clobber
// keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Lazy rebase bound of the online softmax (base-2 units): a map's reference
// max is raised only when a score exceeds it by more than this, so the
// probabilities 2^(c s - m) stay <= 2^kSlack, far inside fp16 range.
constexpr float kSlack = 8.0f;

// Probabilities 2^(c s - m) of a tile as the two f16 operands of the P^T V^T
// product, and the running sum l += their sum, taken over the rounded f16
// values the product uses, two per instruction (dot product with (1, 1), fp32
// accumulation).  The sixteen values go into two interleaved chains of four
// dependent instructions, not one of eight: the wave issues in order, and the
// end of the softmax phase otherwise waits on that chain's latency.
__device__ __forceinline__ void softmax_probs(const f32x16& s, float c, float m, float& l, f16x8& p0, f16x8& p1) {
  float p[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -m));
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p0[j] = (_Float16)p[j];
    p1[j] = (_Float16)p[8 + j];
  }
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  float d0 = l, d1 = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; j += 2) {
    d0 = __builtin_amdgcn_fdot2(f16x2{p0[2 * j], p0[2 * j + 1]}, one, d0, false);
    d1 = __builtin_amdgcn_fdot2(f16x2{p0[2 * j + 2], p0[2 * j + 3]}, one, d1, false);
  }
#pragma unroll
  for (int j = 0; j < 4; j += 2) {
    d0 = __builtin_amdgcn_fdot2(f16x2{p1[2 * j], p1[2 * j + 1]}, one, d0, false);
    d1 = __builtin_amdgcn_fdot2(f16x2{p1[2 * j + 2], p1[2 * j + 3]}, one, d1, false);
  }
  l = d0 + d1;
}

__device__ __forceinline__ float tile_max(const f32x16& s) {
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
  return mx;
}

// One map's online-softmax step on a 32x32 score tile held as S^T (lane: one
// query, 16 keys).  Keeps the running reference max m (base-2 units) unless
// a score lies more than kSlack above it: only when some lane of the wave sees
// one are the two lanes of each query pair reconciled, and the queries over
// the bound raise m to their tile max and rescale that map's O^T and partial
// sum l.  Returns the tile's probabilities
// 2^(c s - m) <= 2^kSlack as the two f16 operands of the P^T V^T product.
__device__ __forceinline__ void softmax_rebase(const f32x16& s, float c, float& m, float& l, f32x16 (&O)[4]) {
  float mx = tile_max(s);
  if (__any(mx * c > m + kSlack)) {
    // Each query decides from its own scores only (its two lanes agree after
    // the exchange), so a row's result never depends on other rows' data.
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mc = mx * c;
    const float mn = mc > m + kSlack ? mc : m;
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    l *= alpha;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) O[cb] *= alpha;
    m = mn;
  }
}

__device__ __forceinline__ void softmax_step(f32x16& s, float c, float& m, float& l, f32x16 (&O)[4],
                                             f16x8& p0, f16x8& p1) {
  softmax_rebase(s, c, m, l, O);
  softmax_probs(s, c, m, l, p0, p1);
}

// End-of-loop merge buffer of a split-key workgroup (two groups of four
// waves on the same queries; it reuses the stage memory): one map's O^T of
// the four group-1 waves stored [wave][register][lane], then their
// (max, sum) pairs.
constexpr int kMergeO = 4 * 64 * 64 * 4;
constexpr int kMergeML = 4 * 64 * 2 * 4;
constexpr int kMergeBytes = kMergeO + kMergeML;

// Merge one map's (m, l, O^T) of a group-1 wave into the matching group-0 wave
// through LDS.  Every thread of the workgroup calls it (it holds two barriers).
__device__ __forceinline__ void merge_map(char* smem, int grp, int wq, int lane, bool live, float& m, float& l,
                                          f32x16 (&O)[4]) {
  float* mo = reinterpret_cast<float*>(smem);
  float* ml = reinterpret_cast<float*>(smem + kMergeO);
  if (grp == 1 && live) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mo[((wq * 64) + cb * 16 + i) * 64 + lane] = O[cb][i];
    ml[(wq * 64 + lane) * 2 + 0] = m;
    ml[(wq * 64 + lane) * 2 + 1] = l;
  }
  __syncthreads();
  if (grp == 0 && live) {
    const float mb = ml[(wq * 64 + lane) * 2 + 0];
    const float lb = ml[(wq * 64 + lane) * 2 + 1];
    const float mn = fmaxf(m, mb);  // every query sees at least itself
    const float aa = __builtin_amdgcn_exp2f(m - mn);
    const float ab = __builtin_amdgcn_exp2f(mb - mn);
    l = l * aa + lb * ab;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) O[cb][i] = O[cb][i] * aa + mo[((wq * 64) + cb * 16 + i) * 64 + lane] * ab;
    m = mn;
  }
  __syncthreads();
}

}  // namespace diffattn
