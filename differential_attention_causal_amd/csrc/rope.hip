// Standalone rotary embedding of a [B, T, H, 64] bf16 tensor (results rounded
// to bf16), the prefill's key pre-pass (both key tensors rotated once into
// fp16 copies), and the host computation of the per-pair phases that every
// RoPE kernel here uses.  The angle convention is the one in rope.h.
#include <cmath>

#include "rope.h"

namespace diffattn {

void rope_phases(float theta, RopeArgs& r) {
  // Long double keeps F_c = theta^(-c/32) / (2 pi) * 2^64 within one unit.
  const long double two_pi = 6.283185307179586476925286766559005768L;
  for (int c = 0; c < 32; ++c) {
    const long double w = std::pow((long double)theta, -(long double)c / 32.0L);
    r.phase[c] = (uint64_t)std::llround(std::ldexp(w / two_pi, 64));
  }
}

namespace {

constexpr int kThreads = 256;  // 32 vectors of 8 chunks per workgroup

// One thread per 8-dim chunk; the eight chunks of a vector are eight
// consecutive lanes.  Lanes past the last vector still take part in the
// partner exchange, with zeros, and store nothing.
__global__ void __launch_bounds__(kThreads) rope_apply_kernel(RopeApplyArgs a) {
  __shared__ uint64_t tab[32];
  if (threadIdx.x < 32) tab[threadIdx.x] = rope_phase_at(a.rope, (int)threadIdx.x);
  __syncthreads();
  const int64_t vec = (int64_t)blockIdx.x * (kThreads / 8) + (threadIdx.x >> 3);
  const int ch = threadIdx.x & 7;
  const int64_t nvec = (int64_t)a.B * a.T * a.H;
  const bool live = vec < nvec;
  const int h = live ? (int)(vec % a.H) : 0;
  const int64_t t = live ? (vec / a.H) % a.T : 0;
  const int b = live ? (int)(vec / ((int64_t)a.H * a.T)) : 0;
  rope_u32x4 v[1] = {rope_u32x4{0, 0, 0, 0}};
  if (live)
    v[0] = *reinterpret_cast<const rope_u32x4*>(a.x + b * a.sx.b + t * a.sx.t + h * a.sx.h + 8 * ch);
  const uint32_t pos = a.rope.pos0 + (uint32_t)(a.pos_start ? a.pos_start[b] : 0) + (uint32_t)t;
  rope_chunks<1, false>(v, ch, pos, a.rope.mode, tab);
  if (live) *reinterpret_cast<rope_u32x4*>(a.out + b * a.so.b + t * a.so.t + h * a.so.h + 8 * ch) = v[0];
}

// The prefill's keys, rotated once per token instead of once per query block
// that reads them: K1 and K2 of one token in the same lanes (they share the
// angles), results rounded to fp16 as the prefill's score products take them.
__global__ void __launch_bounds__(kThreads) rope_keys_kernel(RopeKeysArgs a) {
  __shared__ uint64_t tab[32];
  if (threadIdx.x < 32) tab[threadIdx.x] = rope_phase_at(a.rope, (int)threadIdx.x);
  __syncthreads();
  rope_keys_block(a, (int64_t)blockIdx.x, (int)threadIdx.x, tab);
}

}  // namespace

hipError_t launch_rope_keys(const RopeKeysArgs& a, hipStream_t stream) {
  const int64_t nvec = (int64_t)a.B * a.T * a.H;
  const int64_t blocks = (nvec + kThreads / 8 - 1) / (kThreads / 8);
  return launch_kernel(rope_keys_kernel, dim3((unsigned)blocks), dim3(kThreads), stream, a);
}

hipError_t launch_rope_apply(const RopeApplyArgs& a, hipStream_t stream) {
  const int64_t nvec = (int64_t)a.B * a.T * a.H;
  const int64_t blocks = (nvec + kThreads / 8 - 1) / (kThreads / 8);
  return launch_kernel(rope_apply_kernel, dim3((unsigned)blocks), dim3(kThreads), stream, a);
}

}  // namespace diffattn
