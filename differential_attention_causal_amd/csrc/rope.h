// Device helpers for the rotary position embedding of 64-wide vectors,
// shared by the prefill (queries and staged key tiles), the decode (the query)
// and the standalone rotation kernel.
//
// Rotary embedding (Motif 2.6B explainer, section "The block": RoPE with base
// 500,000): pair c of a 64-wide vector turns by the angle pos * theta^(-c/32).
// Mode 1 pairs dims (c, c + 32), mode 2 pairs dims (2c, 2c + 1).
//
// Angles.  The host gives, per pair, F_c = theta^(-c/32) / (2 pi) in 0.64
// fixed point (revolutions per position).  (pos * F_c) mod 2^64 is then the
// angle in revolutions, exact apart from F_c's own rounding (< 2^-64 per
// position), so no precision is lost at large positions; its top 32 bits, as a
// signed fraction in [-1/2, 1/2), feed v_sin_f32 / v_cos_f32, which take
// revolutions.  The rotation itself is fp32.
#pragma once

#include "kernels.h"

namespace diffattn {

typedef uint32_t rope_u32x4 __attribute__((ext_vector_type(4)));

// phase[c] of the rotary arguments for a lane-dependent c (0 .. 31) without
// indexing the kernel argument dynamically: a chain of selects over the 32
// values, which arrive by scalar loads issued together (a branch per value
// would wait for each load in turn).
__device__ __forceinline__ uint64_t rope_phase_at(const RopeArgs& r, int c) {
  uint64_t v = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) v = i == c ? r.phase[i] : v;
  return v;
}

__device__ __forceinline__ void rope_cos_sin(uint32_t pos, uint64_t phase, float& c, float& s) {
  const uint32_t lo = (uint32_t)phase, hi = (uint32_t)(phase >> 32);
  const uint32_t top = __umulhi(pos, lo) + pos * hi;  // bits 32..63 of pos * phase
  const float rev = (float)(int32_t)top * 0x1p-32f;   // [-0.5, 0.5) revolutions
  s = __builtin_amdgcn_sinf(rev);
  c = __builtin_amdgcn_cosf(rev);
}

__device__ __forceinline__ void rope_unpack(rope_u32x4 w, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Packs 8 floats as bf16 or, with kF16, fp16 (both round to nearest even).
template <bool kF16>
__device__ __forceinline__ rope_u32x4 rope_pack(const float (&x)[8]) {
  rope_u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (kF16) {
      typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
      const f16x2_t v = {(_Float16)x[2 * i], (_Float16)x[2 * i + 1]};
      w[i] = __builtin_bit_cast(uint32_t, v);
    } else {
      typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
      const bf16x2_t v = {(__bf16)x[2 * i], (__bf16)x[2 * i + 1]};
      w[i] = __builtin_bit_cast(uint32_t, v);
    }
  }
  return w;
}

// Rotates chunk ch (dims 8ch .. 8ch+7) of kVecs vectors at position pos, in
// fp32, in place.  In mode 1, p holds the partner chunk ch ^ 4.
template <int kVecs>
__device__ __forceinline__ void rope_rotate(float (&x)[kVecs][8], const float (&p)[kVecs][8], int ch, uint32_t pos,
                                            int mode, const uint64_t* tab) {
  if (mode == 1) {
    // (x_c, x_{c+32}) -> (x_c cos - x_{c+32} sin, x_c sin + x_{c+32} cos)
    const float sg = ch < 4 ? -1.f : 1.f;
    const uint64_t* f = tab + 8 * (ch & 3);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float c, s;
      rope_cos_sin(pos, f[e], c, s);
#pragma unroll
      for (int k = 0; k < kVecs; ++k) x[k][e] = x[k][e] * c + sg * (p[k][e] * s);
    }
  } else {
    const uint64_t* f = tab + 4 * ch;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float c, s;
      rope_cos_sin(pos, f[e], c, s);
#pragma unroll
      for (int k = 0; k < kVecs; ++k) {
        const float a = x[k][2 * e], b = x[k][2 * e + 1];
        x[k][2 * e] = a * c - b * s;
        x[k][2 * e + 1] = a * s + b * c;
      }
    }
  }
}

// Rotates the bf16 chunks ch of kVecs vectors that sit at the same position
// pos, in place; the results are packed as bf16 or, with kOutF16, fp16.
// Eight consecutive lanes hold the eight chunks of one vector (chunk = lane %
// 8); in mode 1 the pair partner of chunk ch is chunk ch ^ 4, read from lane ^
// 4, so every lane of the wave must call this together.  tab: the 32 phases
// (any memory the lanes can read).
template <int kVecs, bool kOutF16>
__device__ __forceinline__ void rope_chunks(rope_u32x4 (&v)[kVecs], int ch, uint32_t pos, int mode,
                                            const uint64_t* tab) {
  float x[kVecs][8], p[kVecs][8];
#pragma unroll
  for (int k = 0; k < kVecs; ++k) {
    rope_unpack(v[k], x[k]);
    if (mode == 1) {
      rope_u32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = (uint32_t)__shfl_xor((int)v[k][i], 4);
      rope_unpack(w, p[k]);
    }
  }
  rope_rotate<kVecs>(x, p, ch, pos, mode, tab);
#pragma unroll
  for (int k = 0; k < kVecs; ++k) v[k] = rope_pack<kOutF16>(x[k]);
}

// One workgroup (256 threads) of the prefill's key pre-pass: key vectors
// 32 blk .. 32 blk + 31 of the flattened [B, T, H] index, K1 and K2 of one
// token in the same lanes (they share the angles), rounded to fp16 as the
// prefill's score products take them and stored C-contiguous.  tab: the 32
// phases, already in memory the whole workgroup reads.
__device__ __forceinline__ void rope_keys_block(const RopeKeysArgs& a, int64_t blk, int tid, const uint64_t* tab) {
  const int64_t vec = blk * 32 + (tid >> 3);
  const int ch = tid & 7;
  const int64_t nvec = (int64_t)a.B * a.T * a.H;
  const bool live = vec < nvec;
  const int h = live ? (int)(vec % a.H) : 0;
  const int64_t t = live ? (vec / a.H) % a.T : 0;
  const int b = live ? (int)(vec / ((int64_t)a.H * a.T)) : 0;
  rope_u32x4 v[2] = {rope_u32x4{0, 0, 0, 0}, rope_u32x4{0, 0, 0, 0}};
  if (live) {
    v[0] = *reinterpret_cast<const rope_u32x4*>(a.k1 + b * a.s1.b + t * a.s1.t + h * a.s1.h + 8 * ch);
    v[1] = *reinterpret_cast<const rope_u32x4*>(a.k2 + b * a.s2.b + t * a.s2.t + h * a.s2.h + 8 * ch);
  }
  rope_chunks<2, true>(v, ch, a.rope.pos0 + (uint32_t)t, a.rope.mode, tab);
  if (live) {
    *reinterpret_cast<rope_u32x4*>(a.out1 + vec * 64 + 8 * ch) = v[0];
    *reinterpret_cast<rope_u32x4*>(a.out2 + vec * 64 + 8 * ch) = v[1];
  }
}

// The same on fp32 chunks (no rounding of the result).
template <int kVecs>
__device__ __forceinline__ void rope_floats(float (&x)[kVecs][8], int ch, uint32_t pos, int mode,
                                            const uint64_t* tab) {
  float p[kVecs][8];
  if (mode == 1) {
#pragma unroll
    for (int k = 0; k < kVecs; ++k)
#pragma unroll
      for (int e = 0; e < 8; ++e) p[k][e] = __shfl_xor(x[k][e], 4);
  }
  rope_rotate<kVecs>(x, p, ch, pos, mode, tab);
}

}  // namespace diffattn
