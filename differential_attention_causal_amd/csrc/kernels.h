// Internal interface between the C-ABI front end (api.cpp) and the gfx950
// kernels.  Not installed; the public interface is include/diffattn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace diffattn {

constexpr int kDqk = 64;   // query/key head size of each map
constexpr int kDv = 128;   // value head size

struct Strides {
  int64_t b, t, h;  // element strides; the innermost dimension is contiguous
};

struct PrefillArgs {
  const uint16_t* q1;
  const uint16_t* q2;
  const uint16_t* k1;
  const uint16_t* k2;
  const uint16_t* v;
  Strides sq1, sq2, sk1, sk2, sv;
  int B, T, H;
  int window;             // > 0: query i sees keys i-window+1 .. i; 0: every key <= i
  float c;                // scale * log2(e): scores are kept in base-2 units
  float lambda;           // used when lambda_h is null
  const float* lambda_h;  // [H] or null
  const float* gain;      // [H, kDv]
  float eps;
  void* out;              // [B, T, H, kDv] bf16 or fp32
  int out_f32;
  float* o_pre;           // [B, T, H, kDv] fp32 or null
};

struct DecodeArgs {
  const uint16_t* q1;  // [B, H, kDqk]
  const uint16_t* q2;
  const uint16_t* k1;  // [B, L, H, kDqk] with strides
  const uint16_t* k2;
  const uint16_t* v;   // [B, L, H, kDv] with strides
  Strides sk1, sk2, sv;
  const int32_t* seqlens;  // [B] or null
  int B, L, H, splits;
  int window;              // > 0: attend only the last `window` positions
  int ring;                // cache of L slots is a ring: position p in slot p % L
  float c;
  float lambda;
  const float* lambda_h;
  const float* gain;
  float eps;
  float* partial;      // [B, H, splits, 2, kDv + 2] fp32 workspace
  void* out;           // [B, H, kDv]
  int out_f32;
  float* o_pre;
};

// Initial reference max of a softmax state: finite, so a query whose first
// tile holds none of its keys (sliding window) gets P = 2^(-inf) = 0, not NaN.
constexpr float kNoMax = -1.0e30f;

// Floats per (b, h, split, map) record in the decode workspace: max, sum, O[kDv].
constexpr int kPartialStride = kDv + 2;

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

}  // namespace diffattn
