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

// Rotary position embedding of the 64-wide Q1, Q2, K1, K2 vectors: pair c
// turns by pos * theta^(-c/32) radians.
struct RopeArgs {
  int mode;            // 0 none, 1 split-half pairs (c, c + 32), 2 interleaved pairs (2c, 2c + 1)
  uint32_t pos0;       // position of token 0
  uint64_t phase[32];  // pair c: theta^(-c/32) / (2 pi) revolutions per position, 0.64 fixed point
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
  RopeArgs rope;          // token t at position rope.pos0 + t
  int keys_rotated;       // rope on: k1, k2 hold the keys already rotated, as fp16
  float c;                // scale * log2(e): scores are kept in base-2 units
  float lambda;           // used when lambda_h is null
  const float* lambda_h;  // [H] or null
  const float* gain;      // [H, kDv]
  float eps;
  void* out;              // [B, T, H, kDv] bf16 or fp32
  int out_f32;
  float* o_pre;           // [B, T, H, kDv] fp32 or null
  // Training outputs (all or none): each map's normalised output O_m / l_m,
  // fp32 [B, T, H, kDv], and its base-2 log-sum-exp m_m + log2 l_m of the
  // scores in base-2 units, fp32 [B, T, H, 2].
  float* o1n;
  float* o2n;
  float* lse;
  // The values as fp16 V^T tiles (vtiles.hip), or null: the kernels then
  // convert and transpose V while staging it.
  const uint16_t* vt;
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
  RopeArgs rope;           // the query of a sequence of n tokens sits at rope.pos0 + n - 1
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

// Standalone rotation of a [B, T, H, 64] bf16 tensor (for writing rotated
// keys into a decode cache): token t of batch row b at position
// rope.pos0 + pos_start[b] + t.
struct RopeApplyArgs {
  const uint16_t* x;
  uint16_t* out;
  Strides sx, so;
  const int32_t* pos_start;  // [B] or null
  int B, T, H;
  RopeArgs rope;
};

// Both key tensors of a prefill rotated once (rope.h) into fp16 copies,
// C-contiguous [B, T, H, 64].
struct RopeKeysArgs {
  const uint16_t* k1;
  const uint16_t* k2;
  Strides s1, s2;
  uint16_t* out1;
  uint16_t* out2;
  int B, T, H;
  RopeArgs rope;
};

// Backward pass of the causal prefill (no window, no rotary embedding).
struct BackwardArgs {
  const uint16_t* q1;
  const uint16_t* q2;
  const uint16_t* k1;
  const uint16_t* k2;
  const uint16_t* v;
  Strides sq1, sq2, sk1, sk2, sv;
  int B, T, H;
  float c;                // scale * log2(e)
  float scale;            // score factor
  float lambda;
  const float* lambda_h;  // [H] or null
  const float* gain;      // [H, kDv]
  float eps;
  const float* o1n;       // forward training outputs (see PrefillArgs)
  const float* o2n;
  const float* lse;
  const void* dy;         // [B, T, H, kDv] bf16 or fp32
  int dy_f32;
  float* dq1;             // [B, T, H, kDqk] fp32, contiguous
  float* dq2;
  float* dk1;
  float* dk2;
  float* dv;              // [B, T, H, kDv] fp32
  float* dlam;            // [H]
  float* dgain;           // [H, kDv]
  // workspace
  uint16_t* q1h;          // fp16 copies of the inputs, contiguous [B, T, H, d] (the
  uint16_t* q2h;          // product kernels take every tile by DMA and every
  uint16_t* k1h;          // transposed operand by transposed LDS reads)
  uint16_t* k2h;
  uint16_t* vh;
  uint16_t* dO;           // [B, T, H, kDv] fp16: gradient of the pre-norm output
  float* dstat;           // [B, T, H, 2]: D_m = rowsum(dO_m * O_m) per map
  float* partial;         // [H, nchunks, kDv + 1]: gain and lambda gradient partials
  int nchunks;
  int window;             // > 0: sliding window of that many keys (as the forward's)
  RopeArgs rope;          // rotary embedding of Q1, Q2, K1, K2 (mode 0: none)
};

// Grouped differential attention with token-wise lambda and output gate:
// n_H = nS + nN heads, signal heads 0 .. nS-1, noise heads nS .. n_H-1,
// signal head s paired with noise head nS + s / g.
struct GroupedArgs {
  const uint16_t* q;  // [B, T, n_H, kDqk] with strides
  const uint16_t* k;
  const uint16_t* v;  // [B, T, n_H, kDv] with strides
  Strides sq, sk, sv;
  int B, T, nH, g, nN, nS;
  float c;               // scale * log2(e)
  const float* lam;      // [B, T, nS] fp32
  const uint16_t* gate;  // [B, T, nS, kDv] bf16 logits, or null
  void* out;             // [B, T, nS, kDv] bf16 or fp32
  int out_f32;
  float* hw;             // workspace [B, T, nH, kDv] fp32: every head's normalised output
  const uint16_t* vt;    // workspace for fp16 V^T tiles (vtiles.hip) of every (b, head), or null
};

hipError_t launch_grouped(const GroupedArgs& a, hipStream_t stream);

// Single-query decode of the grouped form: head h's query q[b, h] against its
// own cache rows (n_H heads, each plain softmax attention), then signal head
// s combined with noise head nS + s / g as the prefill does.
struct GroupedDecodeArgs {
  const uint16_t* q;       // [B, nH, kDqk]
  const uint16_t* k;       // [B, L, nH, kDqk] with strides
  const uint16_t* v;       // [B, L, nH, kDv] with strides
  Strides sk, sv;
  const int32_t* seqlens;  // [B] or null (L each)
  int B, L, nH, g, nN, nS, splits;
  int window;              // > 0: the last `window` positions
  int ring;                // cache of L slots is a ring: position p in slot p % L
  float c;                 // scale * log2(e)
  const float* lam;        // [B, nS] fp32
  const uint16_t* gate;    // [B, nS, kDv] bf16 logits, or null
  float* partial;          // [B, nH, splits, kDv + 2] fp32 workspace
  void* out;               // [B, nS, kDv] bf16 or fp32
  int out_f32;
};

hipError_t launch_grouped_decode(const GroupedDecodeArgs& a, hipStream_t stream);

// Rows (b, t) of one head per workgroup of the backward's first kernel.
constexpr int kBwdRowsPerChunk = 64;

// Fills rope.phase for base theta (host).
void rope_phases(float theta, RopeArgs& r);

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);
// Whether the kernel launch_prefill picks for `a` reads V^T tiles (a.vt).
bool prefill_takes_vt(const PrefillArgs& a);

// V of a prefill as fp16 V^T tiles, each the exact LDS image the prefill
// kernels read: per (b, h) and 32-key tile, 128 channel rows of 64 bytes,
// keys in the score accumulator's order, 16-byte chunks swizzled by row.
constexpr int kVtTileBytes = 128 * 32 * 2;
struct VTilesArgs {
  const uint16_t* v;  // [B, T, H, kDv] bf16 with strides
  Strides sv;
  int B, T, H;
  int ntiles;         // ceil(T / 32)
  uint16_t* out;      // [B * H][ntiles][kVtTileBytes / 2]
};
// The pre-pass arguments for V ([B, T, H, kDv] bf16 with strides sv) into out.
inline VTilesArgs make_vtiles_args(const uint16_t* v, const Strides& sv, int B, int T, int H, uint16_t* out) {
  VTilesArgs t{};
  t.v = v;
  t.sv = sv;
  t.B = B;
  t.T = T;
  t.H = H;
  t.ntiles = (T + 31) / 32;
  t.out = out;
  return t;
}
hipError_t launch_vtiles(const VTilesArgs& a, hipStream_t stream);
// The key rotation and the V^T tiles of one rotary prefill in one launch
// (both results exactly as launch_rope_keys and launch_vtiles give them).
hipError_t launch_prepass(const RopeKeysArgs& r, const VTilesArgs& t, hipStream_t stream);

// Compute units of the current device, queried once per device and cached.
int device_cu_count();

template <class T>
struct NoDeduce {
  using type = T;
};

// Enqueues kernel f on `stream` with one argument struct and returns the
// status of this launch alone (hipLaunchKernel reports its own result, so a
// sticky error left by an earlier, unrelated call is not taken for this one).
template <class A>
inline hipError_t launch_kernel(void (*f)(A), dim3 grid, dim3 block, hipStream_t stream,
                                typename NoDeduce<A>::type arg) {
  void* args[] = {&arg};
  return hipLaunchKernel(reinterpret_cast<const void*>(f), grid, block, args, 0, stream);
}
// The sliding-window streaming kernel (window.hip): whether it takes a's
// configuration (window of at most 129 keys, no rotary embedding, no training
// outputs), and its launch.
bool prefill_window_kernel_fits(const PrefillArgs& a);
hipError_t launch_prefill_window(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Split partials of the no-allocation decode: a file-scope device array of
// this many bytes (decode.hip), one per device, shared by every such call.
constexpr size_t kDecodeScratchBytes = size_t(16) << 20;
// Device address of the current device's array, looked up with
// hipGetSymbolAddress on the first call on that device and kept per device.
hipError_t decode_scratch(float** ptr);
hipError_t launch_rope_apply(const RopeApplyArgs& a, hipStream_t stream);
hipError_t launch_rope_keys(const RopeKeysArgs& a, hipStream_t stream);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream);

}  // namespace diffattn
