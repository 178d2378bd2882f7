// C-ABI front end of libdiffattn.so: argument validation (before any HIP
// call), stride defaults and kernel launch.  The operation and every argument
// are documented in include/diffattn.h.
#include "diffattn.h"

#include <atomic>
#include <cmath>
#include <cstdint>

#include "kernels.h"

namespace {

using diffattn::kDqk;
using diffattn::kDv;
using diffattn::Strides;

constexpr int kDefaultSplits = 8;
constexpr int kMaxSplits = 64;
constexpr int64_t kMaxWorkgroups = int64_t(1) << 23;
constexpr float kLog2e = 1.4426950408889634f;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Strides: non-negative multiples of 8 elements (16-byte rows), and a token
// stride below kMaxTokenStride elements, so that the per-lane byte offsets of a
// 32-row tile fit the 32-bit offsets of buffer loads.
constexpr int64_t kMaxTokenStride = int64_t(1) << 25;

bool strides_ok(const diffattn_strides& s) {
  return s.b >= 0 && s.t >= 0 && s.h >= 0 && s.b % 8 == 0 && s.t % 8 == 0 && s.h % 8 == 0 &&
         s.t < kMaxTokenStride;
}

Strides to_internal(const diffattn_strides& s) { return Strides{s.b, s.t, s.h}; }

diffattn_strides contiguous(int T, int H, int D) {
  return diffattn_strides{(int64_t)T * H * D, (int64_t)H * D, (int64_t)D};
}

int check_common(int B, int H, int d_qk, int d_v, float lambda, float eps, float scale, int out_dtype) {
  if (B <= 0 || H <= 0) return DIFFATTN_ERR_SHAPE;
  if ((int64_t)B * H > (int64_t(1) << 24)) return DIFFATTN_ERR_SHAPE;
  if (d_qk != kDqk || d_v != kDv) return DIFFATTN_ERR_UNSUPPORTED;
  if (!std::isfinite(lambda) || !std::isfinite(eps) || eps < 0.f || std::isnan(scale) || std::isinf(scale))
    return DIFFATTN_ERR_VALUE;
  if (out_dtype != DIFFATTN_OUT_BF16 && out_dtype != DIFFATTN_OUT_F32) return DIFFATTN_ERR_VALUE;
  return DIFFATTN_OK;
}

// Options shared by prefill and decode; the kv_ring field is checked by the
// caller (it is meaningful for decode only).
int check_options(const diffattn_options* opt) {
  if (!opt) return DIFFATTN_OK;
  if (opt->window < 0) return DIFFATTN_ERR_VALUE;
  if (opt->ws_prepared != 0 && opt->ws_prepared != 1) return DIFFATTN_ERR_VALUE;
  for (int r : opt->reserved)
    if (r != 0) return DIFFATTN_ERR_VALUE;
  if (opt->rope < DIFFATTN_ROPE_NONE || opt->rope > DIFFATTN_ROPE_INTERLEAVED) return DIFFATTN_ERR_VALUE;
  if (opt->rope != DIFFATTN_ROPE_NONE && (!std::isfinite(opt->rope_theta) || !(opt->rope_theta > 0.f) ||
                                          opt->rope_pos0 < 0))
    return DIFFATTN_ERR_VALUE;
  return DIFFATTN_OK;
}

diffattn::RopeArgs rope_args(const diffattn_options* opt) {
  diffattn::RopeArgs r{};
  if (opt && opt->rope != DIFFATTN_ROPE_NONE) {
    r.mode = opt->rope;
    r.pos0 = (uint32_t)opt->rope_pos0;
    diffattn::rope_phases(opt->rope_theta, r);
  }
  return r;
}

float score_factor(float scale) {
  const float s = scale > 0.f ? scale : 1.0f / std::sqrt((float)kDqk);
  return s * kLog2e;
}

}  // namespace

namespace diffattn {

int device_cu_count() {
  // One slot per device ordinal; a racing first query stores the same value.
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) return 256;
  if (dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace diffattn

extern "C" {

int diffattn_abi_version(void) { return 112; }

const char* diffattn_status_string(int status) {
  switch (status) {
    case DIFFATTN_OK: return "ok";
    case DIFFATTN_ERR_NULL: return "diffattn: a required pointer is NULL";
    case DIFFATTN_ERR_SHAPE: return "diffattn: a size is non-positive or beyond the supported range";
    case DIFFATTN_ERR_UNSUPPORTED: return "diffattn: unsupported head size (needs d_qk=64, d_v=128)";
    case DIFFATTN_ERR_LAYOUT: return "diffattn: pointer not 16-byte aligned or stride not a multiple of 8 elements";
    case DIFFATTN_ERR_WORKSPACE: return "diffattn: workspace missing, misaligned or too small";
    case DIFFATTN_ERR_HIP: return "diffattn: the HIP runtime refused the kernel launch";
    case DIFFATTN_ERR_VALUE:
      return "diffattn: invalid scalar argument (lambda, eps, scale, dtype, split count or option)";
    default: return "diffattn: unknown status";
  }
}

namespace {

// Bytes of one fp16 copy of a [B, T, H, 64] key tensor in the prefill
// workspace (256-byte aligned slices).
size_t rope_keys_bytes(int B, int T, int H) {
  return ((size_t)B * T * H * diffattn::kDqk * 2 + 255) & ~size_t(255);
}

// Bytes of the fp16 V^T tiles in the prefill workspace (vtiles.hip).
size_t vtiles_bytes(int B, int T, int H) {
  return (size_t)B * H * ((T + 31) / 32) * diffattn::kVtTileBytes;
}

// The prefill workspace, [rotated K1, K2 (with rope)] [V^T tiles]: its size and
// alignment checked, its pre-pass kernels launched when `launch` (else the
// caller vouches that diffattn_prefill_prepare wrote it for these arguments),
// and the prefill's arguments pointed at it.  The V^T tiles exist when the
// launch plan of `a` takes them, a function of the sizes, the key and value
// strides and the options only.
int ws_pre_pass(diffattn::PrefillArgs& a, void* ws, size_t ws_bytes, hipStream_t hs, bool launch) {
  const int B = a.B, T = a.T, H = a.H;
  const size_t rope_part = a.rope.mode != 0 ? 2 * rope_keys_bytes(B, T, H) : 0;
  if (ws_bytes < rope_part + vtiles_bytes(B, T, H) || reinterpret_cast<uintptr_t>(ws) % 256 != 0)
    return DIFFATTN_ERR_WORKSPACE;
  const bool rope = a.rope.mode != 0;
  diffattn::RopeKeysArgs r{};
  if (rope) {
    // Rotate both key tensors once into the workspace (fp16, C-contiguous);
    // the prefill then stages them like plain keys.
    const size_t one = rope_keys_bytes(B, T, H);
    r.k1 = a.k1;
    r.k2 = a.k2;
    r.s1 = a.sk1;
    r.s2 = a.sk2;
    r.out1 = static_cast<uint16_t*>(ws);
    r.out2 = reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + one);
    r.B = B;
    r.T = T;
    r.H = H;
    r.rope = a.rope;
    const diffattn::Strides kc = to_internal(contiguous(T, H, kDqk));
    a.k1 = r.out1;
    a.k2 = r.out2;
    a.sk1 = kc;
    a.sk2 = kc;
    a.keys_rotated = 1;
  }
  // V converted and transposed once into fp16 V^T tiles that the prefill
  // kernels move into LDS by DMA (the kernel choice depends on the rotated
  // keys, so this is asked after the fields above are set).
  const bool vt = diffattn::prefill_takes_vt(a);
  const diffattn::VTilesArgs t = diffattn::make_vtiles_args(
      a.v, a.sv, B, T, H, reinterpret_cast<uint16_t*>(static_cast<char*>(ws) + rope_part));
  // one launch of 256-thread workgroups covers every key vector (32 per
  // workgroup) and every V^T tile: its work-items must fit 32 bits
  const int64_t blocks = (rope ? ((int64_t)B * T * H + 31) / 32 : 0) + (vt ? (int64_t)B * H * t.ntiles : 0);
  if (blocks * 256 > (int64_t)UINT32_MAX) return DIFFATTN_ERR_SHAPE;
  if (launch) {
    // with both pre-passes, one launch does the two
    hipError_t e = hipSuccess;
    if (rope && vt)
      e = diffattn::launch_prepass(r, t, hs);
    else if (rope)
      e = diffattn::launch_rope_keys(r, hs);
    else if (vt)
      e = diffattn::launch_vtiles(t, hs);
    if (e != hipSuccess) return DIFFATTN_ERR_HIP;
  }
  if (vt) a.vt = t.out;
  return DIFFATTN_OK;
}

// Shared by diffattn_fwd_prefill_ex, _ws and _train; `train` holds the three
// training outputs or nulls; `ws`: the prefill workspace (rotated keys) or
// null for the rotation inside the kernels.
int prefill_impl(const diffattn_options* opt, const void* q1, const void* q2, const void* k1, const void* k2,
                 const void* v, const diffattn_strides* strides, int B, int T, int H, int d_qk, int d_v,
                 float lambda, const float* lambda_per_head, const float* gain, float gn_eps, float scale, void* out,
                 int out_dtype, float* o_pre, float* const train[3], void* stream, void* ws = nullptr,
                 size_t ws_bytes = 0) {
  if (!q1 || !q2 || !k1 || !k2 || !v || !gain || !out) return DIFFATTN_ERR_NULL;
  int rc = check_common(B, H, d_qk, d_v, lambda, gn_eps, scale, out_dtype);
  if (rc != DIFFATTN_OK) return rc;
  rc = check_options(opt);
  if (rc != DIFFATTN_OK) return rc;
  if (opt && opt->kv_ring != 0) return DIFFATTN_ERR_VALUE;
  if (T <= 0 || T > (1 << 22)) return DIFFATTN_ERR_SHAPE;
  // One 256-thread workgroup per 128 queries of each (b, h); the launch must
  // stay below 2^32 threads.
  if ((int64_t)((T + 127) / 128) * B * H > kMaxWorkgroups) return DIFFATTN_ERR_SHAPE;
  const void* ptrs[5] = {q1, q2, k1, k2, v};
  for (const void* p : ptrs)
    if (!aligned16(p)) return DIFFATTN_ERR_LAYOUT;
  if (!aligned16(out) || !aligned16(gain) || (o_pre && !aligned16(o_pre))) return DIFFATTN_ERR_LAYOUT;
  diffattn_strides st[5];
  for (int i = 0; i < 5; ++i) {
    st[i] = strides ? strides[i] : contiguous(T, H, i == 4 ? d_v : d_qk);
    if (!strides_ok(st[i])) return DIFFATTN_ERR_LAYOUT;
  }

  diffattn::PrefillArgs a{};
  a.q1 = static_cast<const uint16_t*>(q1);
  a.q2 = static_cast<const uint16_t*>(q2);
  a.k1 = static_cast<const uint16_t*>(k1);
  a.k2 = static_cast<const uint16_t*>(k2);
  a.v = static_cast<const uint16_t*>(v);
  a.sq1 = to_internal(st[0]);
  a.sq2 = to_internal(st[1]);
  a.sk1 = to_internal(st[2]);
  a.sk2 = to_internal(st[3]);
  a.sv = to_internal(st[4]);
  a.B = B;
  a.T = T;
  a.H = H;
  a.window = opt ? opt->window : 0;
  a.rope = rope_args(opt);
  a.c = score_factor(scale);
  a.lambda = lambda;
  a.lambda_h = lambda_per_head;
  a.gain = gain;
  a.eps = gn_eps;
  a.out = out;
  a.out_f32 = out_dtype == DIFFATTN_OUT_F32;
  a.o_pre = o_pre;
  if (train) {
    a.o1n = train[0];
    a.o2n = train[1];
    a.lse = train[2];
  }
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (opt && opt->ws_prepared && ws == nullptr) return DIFFATTN_ERR_WORKSPACE;
  if (ws != nullptr) {
    rc = ws_pre_pass(a, ws, ws_bytes, hs, !(opt && opt->ws_prepared));
    if (rc != DIFFATTN_OK) return rc;
  }
  if (diffattn::launch_prefill(a, hs) != hipSuccess) return DIFFATTN_ERR_HIP;
  return DIFFATTN_OK;
}

}  // namespace

int diffattn_fwd_prefill_ex(const diffattn_options* opt, const void* q1, const void* q2, const void* k1,
                            const void* k2, const void* v, const diffattn_strides* strides, int B, int T, int H,
                            int d_qk, int d_v, float lambda, const float* lambda_per_head, const float* gain,
                            float gn_eps, float scale, void* out, int out_dtype, float* o_pre, void* stream) {
  if (opt && opt->ws_prepared != 0) return DIFFATTN_ERR_VALUE;  // a workspace entry point's option
  return prefill_impl(opt, q1, q2, k1, k2, v, strides, B, T, H, d_qk, d_v, lambda, lambda_per_head, gain, gn_eps,
                      scale, out, out_dtype, o_pre, nullptr, stream);
}

size_t diffattn_prefill_workspace_bytes(const diffattn_options* opt, int B, int T, int H) {
  if (B <= 0 || T <= 0 || H <= 0 || (int64_t)B * H > (1 << 24) || T > (1 << 22)) return 0;
  if ((int64_t)((T + 127) / 128) * B * H > kMaxWorkgroups) return 0;
  const size_t rope_part = opt && opt->rope != DIFFATTN_ROPE_NONE ? 2 * rope_keys_bytes(B, T, H) : 0;
  return rope_part + vtiles_bytes(B, T, H);
}

int diffattn_fwd_prefill_ws(const diffattn_options* opt, const void* q1, const void* q2, const void* k1,
                            const void* k2, const void* v, const diffattn_strides* strides, int B, int T, int H,
                            int d_qk, int d_v, float lambda, const float* lambda_per_head, const float* gain,
                            float gn_eps, float scale, void* out, int out_dtype, float* o_pre, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (opt && opt->rope != DIFFATTN_ROPE_NONE && workspace == nullptr) return DIFFATTN_ERR_WORKSPACE;
  return prefill_impl(opt, q1, q2, k1, k2, v, strides, B, T, H, d_qk, d_v, lambda, lambda_per_head, gain, gn_eps,
                      scale, out, out_dtype, o_pre, nullptr, stream, workspace, workspace_bytes);
}

int diffattn_prefill_prepare(const diffattn_options* opt, const void* k1, const void* k2, const void* v,
                             const diffattn_strides* strides, int B, int T, int H, int d_qk, int d_v, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!k1 || !k2 || !v) return DIFFATTN_ERR_NULL;
  if (workspace == nullptr) return DIFFATTN_ERR_WORKSPACE;
  int rc = check_common(B, H, d_qk, d_v, 0.0f, 0.0f, 0.0f, DIFFATTN_OUT_BF16);
  if (rc != DIFFATTN_OK) return rc;
  rc = check_options(opt);
  if (rc != DIFFATTN_OK) return rc;
  if (opt && (opt->kv_ring != 0 || opt->ws_prepared != 0)) return DIFFATTN_ERR_VALUE;
  if (T <= 0 || T > (1 << 22)) return DIFFATTN_ERR_SHAPE;
  if ((int64_t)((T + 127) / 128) * B * H > kMaxWorkgroups) return DIFFATTN_ERR_SHAPE;
  if (!aligned16(k1) || !aligned16(k2) || !aligned16(v)) return DIFFATTN_ERR_LAYOUT;
  diffattn_strides st[5];
  for (int i = 2; i < 5; ++i) {
    st[i] = strides ? strides[i] : contiguous(T, H, i == 4 ? d_v : d_qk);
    if (!strides_ok(st[i])) return DIFFATTN_ERR_LAYOUT;
  }
  // The arguments the workspace depends on, as prefill_impl fills them.
  diffattn::PrefillArgs a{};
  a.k1 = static_cast<const uint16_t*>(k1);
  a.k2 = static_cast<const uint16_t*>(k2);
  a.v = static_cast<const uint16_t*>(v);
  a.sk1 = to_internal(st[2]);
  a.sk2 = to_internal(st[3]);
  a.sv = to_internal(st[4]);
  a.B = B;
  a.T = T;
  a.H = H;
  a.window = opt ? opt->window : 0;
  a.rope = rope_args(opt);
  return ws_pre_pass(a, workspace, workspace_bytes, static_cast<hipStream_t>(stream), true);
}

int diffattn_fwd_prefill_train(const void* q1, const void* q2, const void* k1, const void* k2, const void* v,
                               const diffattn_strides* strides, int B, int T, int H, int d_qk, int d_v,
                               float lambda, const float* lambda_per_head, const float* gain, float gn_eps,
                               float scale, void* out, int out_dtype, float* o_pre, float* o1, float* o2,
                               float* lse, void* stream) {
  return diffattn_fwd_prefill_train_ex(nullptr, q1, q2, k1, k2, v, strides, B, T, H, d_qk, d_v, lambda,
                                       lambda_per_head, gain, gn_eps, scale, out, out_dtype, o_pre, o1, o2, lse,
                                       stream);
}

int diffattn_fwd_prefill_train_ex(const diffattn_options* opt, const void* q1, const void* q2, const void* k1,
                                  const void* k2, const void* v, const diffattn_strides* strides, int B, int T,
                                  int H, int d_qk, int d_v, float lambda, const float* lambda_per_head,
                                  const float* gain, float gn_eps, float scale, void* out, int out_dtype,
                                  float* o_pre, float* o1, float* o2, float* lse, void* stream) {
  if (!o1 || !o2 || !lse) return DIFFATTN_ERR_NULL;
  if (!aligned16(o1) || !aligned16(o2) || !aligned16(lse)) return DIFFATTN_ERR_LAYOUT;
  if (opt && opt->ws_prepared != 0) return DIFFATTN_ERR_VALUE;  // a workspace entry point's option
  float* const train[3] = {o1, o2, lse};
  return prefill_impl(opt, q1, q2, k1, k2, v, strides, B, T, H, d_qk, d_v, lambda, lambda_per_head, gain, gn_eps,
                      scale, out, out_dtype, o_pre, train, stream);
}

namespace {

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

struct BwdLayout {
  size_t q1h, q2h, k1h, k2h, vh, dO, dstat, partial, total;
  int nchunks;
};

// Workspace of the backward pass: fp16 copies of Q_1, Q_2, K_1, K_2
// [B,T,H,d_qk] and V [B,T,H,d_v], dO fp16 [B,T,H,d_v], D fp32 [B,T,H,2],
// gain/lambda partials fp32 [H, nchunks, d_v + 1].
BwdLayout bwd_layout(int B, int T, int H) {
  BwdLayout l;
  const size_t rows = (size_t)B * T * H;
  l.nchunks = (int)(((int64_t)B * T + diffattn::kBwdRowsPerChunk - 1) / diffattn::kBwdRowsPerChunk);
  l.q1h = 0;
  l.q2h = l.q1h + align256(rows * kDqk * 2);
  l.k1h = l.q2h + align256(rows * kDqk * 2);
  l.k2h = l.k1h + align256(rows * kDqk * 2);
  l.vh = l.k2h + align256(rows * kDqk * 2);
  l.dO = l.vh + align256(rows * kDv * 2);
  l.dstat = l.dO + align256(rows * kDv * 2);
  l.partial = l.dstat + align256(rows * 2 * sizeof(float));
  l.total = l.partial + align256((size_t)H * l.nchunks * (kDv + 1) * sizeof(float));
  return l;
}

}  // namespace

size_t diffattn_bwd_workspace_bytes(int B, int T, int H, int d_v) {
  if (B <= 0 || T <= 0 || H <= 0 || d_v != kDv || T > (1 << 22)) return 0;
  if ((int64_t)B * H > (int64_t(1) << 24) || (int64_t)((T + 127) / 128) * B * H > kMaxWorkgroups) return 0;
  return bwd_layout(B, T, H).total;
}

int diffattn_bwd_prefill(const void* q1, const void* q2, const void* k1, const void* k2, const void* v,
                         const diffattn_strides* strides, int B, int T, int H, int d_qk, int d_v, float lambda,
                         const float* lambda_per_head, const float* gain, float gn_eps, float scale, const float* o1,
                         const float* o2, const float* lse, const void* dy, int dy_dtype, float* dq1, float* dq2,
                         float* dk1, float* dk2, float* dv, float* dlambda, float* dgain, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return diffattn_bwd_prefill_ex(nullptr, q1, q2, k1, k2, v, strides, B, T, H, d_qk, d_v, lambda, lambda_per_head,
                                 gain, gn_eps, scale, o1, o2, lse, dy, dy_dtype, dq1, dq2, dk1, dk2, dv, dlambda,
                                 dgain, workspace, workspace_bytes, stream);
}

int diffattn_bwd_prefill_ex(const diffattn_options* opt, const void* q1, const void* q2, const void* k1,
                            const void* k2, const void* v, const diffattn_strides* strides, int B, int T, int H,
                            int d_qk, int d_v, float lambda, const float* lambda_per_head, const float* gain,
                            float gn_eps, float scale, const float* o1, const float* o2, const float* lse,
                            const void* dy, int dy_dtype, float* dq1, float* dq2, float* dk1, float* dk2, float* dv,
                            float* dlambda, float* dgain, void* workspace, size_t workspace_bytes, void* stream) {
  if (!q1 || !q2 || !k1 || !k2 || !v || !gain || !o1 || !o2 || !lse || !dy || !dq1 || !dq2 || !dk1 || !dk2 ||
      !dv || !dlambda || !dgain)
    return DIFFATTN_ERR_NULL;
  int rc = check_common(B, H, d_qk, d_v, lambda, gn_eps, scale, dy_dtype);
  if (rc != DIFFATTN_OK) return rc;
  rc = check_options(opt);
  if (rc != DIFFATTN_OK) return rc;
  if (opt && (opt->kv_ring != 0 || opt->ws_prepared != 0)) return DIFFATTN_ERR_VALUE;
  if (T <= 0 || T > (1 << 22)) return DIFFATTN_ERR_SHAPE;
  if ((int64_t)((T + 127) / 128) * B * H > kMaxWorkgroups) return DIFFATTN_ERR_SHAPE;
  const void* ptrs[] = {q1, q2, k1, k2, v, gain, o1, o2, lse, dy, dq1, dq2, dk1, dk2, dv, dgain};
  for (const void* p : ptrs)
    if (!aligned16(p)) return DIFFATTN_ERR_LAYOUT;
  diffattn_strides st[5];
  for (int i = 0; i < 5; ++i) {
    st[i] = strides ? strides[i] : contiguous(T, H, i == 4 ? d_v : d_qk);
    if (!strides_ok(st[i])) return DIFFATTN_ERR_LAYOUT;
  }
  const BwdLayout lay = bwd_layout(B, T, H);
  if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return DIFFATTN_ERR_WORKSPACE;
  if (workspace_bytes < lay.total) return DIFFATTN_ERR_WORKSPACE;

  diffattn::BackwardArgs a{};
  a.q1 = static_cast<const uint16_t*>(q1);
  a.q2 = static_cast<const uint16_t*>(q2);
  a.k1 = static_cast<const uint16_t*>(k1);
  a.k2 = static_cast<const uint16_t*>(k2);
  a.v = static_cast<const uint16_t*>(v);
  a.sq1 = to_internal(st[0]);
  a.sq2 = to_internal(st[1]);
  a.sk1 = to_internal(st[2]);
  a.sk2 = to_internal(st[3]);
  a.sv = to_internal(st[4]);
  a.B = B;
  a.T = T;
  a.H = H;
  a.c = score_factor(scale);
  a.scale = scale > 0.f ? scale : 1.0f / std::sqrt((float)kDqk);
  a.lambda = lambda;
  a.lambda_h = lambda_per_head;
  a.gain = gain;
  a.eps = gn_eps;
  a.o1n = o1;
  a.o2n = o2;
  a.lse = lse;
  a.dy = dy;
  a.dy_f32 = dy_dtype == DIFFATTN_OUT_F32;
  a.dq1 = dq1;
  a.dq2 = dq2;
  a.dk1 = dk1;
  a.dk2 = dk2;
  a.dv = dv;
  a.dlam = dlambda;
  a.dgain = dgain;
  char* ws = static_cast<char*>(workspace);
  a.q1h = reinterpret_cast<uint16_t*>(ws + lay.q1h);
  a.q2h = reinterpret_cast<uint16_t*>(ws + lay.q2h);
  a.k1h = reinterpret_cast<uint16_t*>(ws + lay.k1h);
  a.k2h = reinterpret_cast<uint16_t*>(ws + lay.k2h);
  a.vh = reinterpret_cast<uint16_t*>(ws + lay.vh);
  a.dO = reinterpret_cast<uint16_t*>(ws + lay.dO);
  a.dstat = reinterpret_cast<float*>(ws + lay.dstat);
  a.partial = reinterpret_cast<float*>(ws + lay.partial);
  a.nchunks = lay.nchunks;
  a.window = opt ? opt->window : 0;
  a.rope = rope_args(opt);
  if (diffattn::launch_backward(a, static_cast<hipStream_t>(stream)) != hipSuccess) return DIFFATTN_ERR_HIP;
  return DIFFATTN_OK;
}

int diffattn_fwd_prefill(const void* q1, const void* q2, const void* k1, const void* k2, const void* v,
                         const diffattn_strides* strides, int B, int T, int H, int d_qk, int d_v,
                         float lambda, const float* lambda_per_head, const float* gain, float gn_eps,
                         float scale, void* out, int out_dtype, float* o_pre, void* stream) {
  return diffattn_fwd_prefill_ex(nullptr, q1, q2, k1, k2, v, strides, B, T, H, d_qk, d_v, lambda,
                                 lambda_per_head, gain, gn_eps, scale, out, out_dtype, o_pre, stream);
}

size_t diffattn_decode_workspace_bytes(int B, int H, int d_v, int num_splits) {
  if (num_splits <= 0) num_splits = kDefaultSplits;
  if (B <= 0 || H <= 0 || d_v != kDv || num_splits > kMaxSplits) return 0;
  if ((int64_t)B * H > (int64_t(1) << 24)) return 0;
  return (size_t)B * H * num_splits * 2 * diffattn::kPartialStride * sizeof(float);
}

}  // extern "C"

namespace {

// Shared by diffattn_fwd_decode_ex (the caller's workspace) and
// diffattn_fwd_decode_noalloc (scratch: the library's per-device array, whose
// address is looked up only once every argument has passed validation).
int decode_impl(const diffattn_options* opt, const void* q1, const void* q2, const void* k1, const void* k2,
                const void* v, const diffattn_strides* cache_strides, const int32_t* seqlens, int B, int L, int H,
                int d_qk, int d_v, float lambda, const float* lambda_per_head, const float* gain, float gn_eps,
                float scale, int num_splits, void* workspace, size_t workspace_bytes, bool scratch, void* out,
                int out_dtype, float* o_pre, void* stream) {
  if (!q1 || !q2 || !k1 || !k2 || !v || !gain || !out) return DIFFATTN_ERR_NULL;
  int rc = check_common(B, H, d_qk, d_v, lambda, gn_eps, scale, out_dtype);
  if (rc != DIFFATTN_OK) return rc;
  rc = check_options(opt);
  if (rc != DIFFATTN_OK) return rc;
  if (opt && opt->ws_prepared != 0) return DIFFATTN_ERR_VALUE;  // a prefill workspace option
  if (L <= 0 || L > (1 << 26)) return DIFFATTN_ERR_SHAPE;
  const bool ring = opt && opt->kv_ring != 0;
  if (ring && opt->window > L) return DIFFATTN_ERR_VALUE;
  if (num_splits <= 0) num_splits = kDefaultSplits;
  if (num_splits > kMaxSplits) return DIFFATTN_ERR_VALUE;
  if ((int64_t)B * H * num_splits > kMaxWorkgroups) return DIFFATTN_ERR_SHAPE;
  const void* ptrs[5] = {q1, q2, k1, k2, v};
  for (const void* p : ptrs)
    if (!aligned16(p)) return DIFFATTN_ERR_LAYOUT;
  if (!aligned16(out) || !aligned16(gain) || (o_pre && !aligned16(o_pre))) return DIFFATTN_ERR_LAYOUT;
  if (scratch) {
    if (diffattn_decode_workspace_bytes(B, H, d_v, num_splits) > diffattn::kDecodeScratchBytes)
      return DIFFATTN_ERR_WORKSPACE;
  } else {
    if (!workspace || !aligned16(workspace)) return DIFFATTN_ERR_WORKSPACE;
    if (workspace_bytes < diffattn_decode_workspace_bytes(B, H, d_v, num_splits)) return DIFFATTN_ERR_WORKSPACE;
  }
  diffattn_strides st[3];
  for (int i = 0; i < 3; ++i) {
    st[i] = cache_strides ? cache_strides[i] : contiguous(L, H, i == 2 ? d_v : d_qk);
    if (!strides_ok(st[i])) return DIFFATTN_ERR_LAYOUT;
  }
  if (scratch) {
    float* p = nullptr;
    if (diffattn::decode_scratch(&p) != hipSuccess) return DIFFATTN_ERR_HIP;
    workspace = p;
  }

  diffattn::DecodeArgs a{};
  a.q1 = static_cast<const uint16_t*>(q1);
  a.q2 = static_cast<const uint16_t*>(q2);
  a.k1 = static_cast<const uint16_t*>(k1);
  a.k2 = static_cast<const uint16_t*>(k2);
  a.v = static_cast<const uint16_t*>(v);
  a.sk1 = to_internal(st[0]);
  a.sk2 = to_internal(st[1]);
  a.sv = to_internal(st[2]);
  a.seqlens = seqlens;
  a.B = B;
  a.L = L;
  a.H = H;
  a.splits = num_splits;
  a.window = opt ? opt->window : 0;
  a.ring = ring;
  if (ring && a.window == 0) a.window = L;
  a.rope = rope_args(opt);
  a.c = score_factor(scale);
  a.lambda = lambda;
  a.lambda_h = lambda_per_head;
  a.gain = gain;
  a.eps = gn_eps;
  a.partial = static_cast<float*>(workspace);
  a.out = out;
  a.out_f32 = out_dtype == DIFFATTN_OUT_F32;
  a.o_pre = o_pre;
  if (diffattn::launch_decode(a, static_cast<hipStream_t>(stream)) != hipSuccess) return DIFFATTN_ERR_HIP;
  return DIFFATTN_OK;
}

}  // namespace

extern "C" {

int diffattn_fwd_decode_ex(const diffattn_options* opt, const void* q1, const void* q2, const void* k1,
                           const void* k2, const void* v, const diffattn_strides* cache_strides,
                           const int32_t* seqlens, int B, int L, int H, int d_qk, int d_v, float lambda,
                           const float* lambda_per_head, const float* gain, float gn_eps, float scale,
                           int num_splits, void* workspace, size_t workspace_bytes, void* out, int out_dtype,
                           float* o_pre, void* stream) {
  return decode_impl(opt, q1, q2, k1, k2, v, cache_strides, seqlens, B, L, H, d_qk, d_v, lambda, lambda_per_head,
                     gain, gn_eps, scale, num_splits, workspace, workspace_bytes, false, out, out_dtype, o_pre,
                     stream);
}

int diffattn_fwd_decode_noalloc(const diffattn_options* opt, const void* q1, const void* q2, const void* k1,
                                const void* k2, const void* v, const diffattn_strides* cache_strides,
                                const int32_t* seqlens, int B, int L, int H, int d_qk, int d_v, float lambda,
                                const float* lambda_per_head, const float* gain, float gn_eps, float scale,
                                int num_splits, void* out, int out_dtype, float* o_pre, void* stream) {
  return decode_impl(opt, q1, q2, k1, k2, v, cache_strides, seqlens, B, L, H, d_qk, d_v, lambda, lambda_per_head,
                     gain, gn_eps, scale, num_splits, nullptr, 0, true, out, out_dtype, o_pre, stream);
}

int diffattn_fwd_decode(const void* q1, const void* q2, const void* k1, const void* k2, const void* v,
                        const diffattn_strides* cache_strides, const int32_t* seqlens, int B, int L, int H,
                        int d_qk, int d_v, float lambda, const float* lambda_per_head, const float* gain,
                        float gn_eps, float scale, int num_splits, void* workspace, size_t workspace_bytes,
                        void* out, int out_dtype, float* o_pre, void* stream) {
  return diffattn_fwd_decode_ex(nullptr, q1, q2, k1, k2, v, cache_strides, seqlens, B, L, H, d_qk, d_v, lambda,
                                lambda_per_head, gain, gn_eps, scale, num_splits, workspace, workspace_bytes, out,
                                out_dtype, o_pre, stream);
}

int diffattn_rope_apply(const void* x, const diffattn_strides* x_strides, void* out,
                        const diffattn_strides* out_strides, int B, int T, int H, int d, int mode, float theta,
                        int pos0, const int32_t* pos_start, void* stream) {
  if (!x || !out) return DIFFATTN_ERR_NULL;
  if (B <= 0 || T <= 0 || H <= 0 || (int64_t)B * T * H > (int64_t(1) << 34)) return DIFFATTN_ERR_SHAPE;
  if (d != kDqk) return DIFFATTN_ERR_UNSUPPORTED;
  if ((mode != DIFFATTN_ROPE_HALF && mode != DIFFATTN_ROPE_INTERLEAVED) || !std::isfinite(theta) ||
      !(theta > 0.f) || pos0 < 0)
    return DIFFATTN_ERR_VALUE;
  if (!aligned16(x) || !aligned16(out)) return DIFFATTN_ERR_LAYOUT;
  const diffattn_strides sx = x_strides ? *x_strides : contiguous(T, H, d);
  const diffattn_strides so = out_strides ? *out_strides : contiguous(T, H, d);
  if (!strides_ok(sx) || !strides_ok(so)) return DIFFATTN_ERR_LAYOUT;
  diffattn::RopeApplyArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.out = static_cast<uint16_t*>(out);
  a.sx = to_internal(sx);
  a.so = to_internal(so);
  a.pos_start = pos_start;
  a.B = B;
  a.T = T;
  a.H = H;
  a.rope.mode = mode;
  a.rope.pos0 = (uint32_t)pos0;
  diffattn::rope_phases(theta, a.rope);
  if (diffattn::launch_rope_apply(a, static_cast<hipStream_t>(stream)) != hipSuccess) return DIFFATTN_ERR_HIP;
  return DIFFATTN_OK;
}

size_t diffattn_grouped_workspace_bytes(int B, int T, int n_heads, int group, int d_v) {
  if (B <= 0 || T <= 0 || n_heads <= 0 || group <= 0 || n_heads % (group + 1) != 0 || d_v != kDv) return 0;
  return (size_t)B * T * n_heads * kDv * sizeof(float) + vtiles_bytes(B, T, n_heads);
}

int diffattn_fwd_grouped(const void* q, const void* k, const void* v, const diffattn_strides* strides, int B, int T,
                         int n_heads, int group, int d_qk, int d_v, const float* lambda_t, const void* gate,
                         float scale, void* out, int out_dtype, void* workspace, size_t workspace_bytes,
                         void* stream) {
  if (!q || !k || !v || !lambda_t || !out) return DIFFATTN_ERR_NULL;
  if (B <= 0 || T <= 0 || T > (1 << 22) || n_heads <= 0 || group <= 0) return DIFFATTN_ERR_SHAPE;
  if (n_heads % (group + 1) != 0) return DIFFATTN_ERR_SHAPE;
  if ((int64_t)B * n_heads > (int64_t(1) << 24)) return DIFFATTN_ERR_SHAPE;
  if ((int64_t)((T + 127) / 128) * B * n_heads > kMaxWorkgroups) return DIFFATTN_ERR_SHAPE;
  if (d_qk != kDqk || d_v != kDv) return DIFFATTN_ERR_UNSUPPORTED;
  if (std::isnan(scale) || std::isinf(scale)) return DIFFATTN_ERR_VALUE;
  if (out_dtype != DIFFATTN_OUT_BF16 && out_dtype != DIFFATTN_OUT_F32) return DIFFATTN_ERR_VALUE;
  const void* ptrs[] = {q, k, v, lambda_t, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return DIFFATTN_ERR_LAYOUT;
  if (gate && (reinterpret_cast<uintptr_t>(gate) & 7u) != 0) return DIFFATTN_ERR_LAYOUT;
  diffattn_strides st[3];
  for (int i = 0; i < 3; ++i) {
    st[i] = strides ? strides[i] : contiguous(T, n_heads, i == 2 ? d_v : d_qk);
    if (!strides_ok(st[i])) return DIFFATTN_ERR_LAYOUT;
  }
  if (!workspace || !aligned16(workspace)) return DIFFATTN_ERR_WORKSPACE;
  if (workspace_bytes < diffattn_grouped_workspace_bytes(B, T, n_heads, group, d_v)) return DIFFATTN_ERR_WORKSPACE;
  diffattn::GroupedArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.sq = to_internal(st[0]);
  a.sk = to_internal(st[1]);
  a.sv = to_internal(st[2]);
  a.B = B;
  a.T = T;
  a.nH = n_heads;
  a.g = group;
  a.nN = n_heads / (group + 1);
  a.nS = group * a.nN;
  a.c = score_factor(scale);
  a.lam = lambda_t;
  a.gate = static_cast<const uint16_t*>(gate);
  a.out = out;
  a.out_f32 = out_dtype == DIFFATTN_OUT_F32;
  a.hw = static_cast<float*>(workspace);
  // fp16 V^T tiles after the head outputs, for the ping-pong kernel, which
  // addresses a head's key rows with 32-bit offsets (up to about T + 320
  // rows) and whose pre-pass covers every tile with one 256-thread workgroup
  const int64_t tiles = (int64_t)B * n_heads * ((T + 31) / 32);
  if ((int64_t)(T + 320) * a.sk.t * 2 < (int64_t(1) << 31) && tiles * 256 <= (int64_t)UINT32_MAX)
    a.vt = reinterpret_cast<const uint16_t*>(static_cast<char*>(workspace) + (size_t)B * T * n_heads * kDv * 4);
  if (diffattn::launch_grouped(a, static_cast<hipStream_t>(stream)) != hipSuccess) return DIFFATTN_ERR_HIP;
  return DIFFATTN_OK;
}

size_t diffattn_grouped_decode_workspace_bytes(int B, int n_heads, int d_v, int num_splits) {
  if (num_splits <= 0) num_splits = kDefaultSplits;
  if (B <= 0 || n_heads <= 0 || d_v != kDv || num_splits > kMaxSplits) return 0;
  if ((int64_t)B * n_heads > (int64_t(1) << 24)) return 0;
  return (size_t)B * n_heads * num_splits * (kDv + 2) * sizeof(float);
}

int diffattn_fwd_grouped_decode(const diffattn_options* opt, const void* q, const void* k, const void* v,
                                const diffattn_strides* strides, const int32_t* seqlens, int B, int L, int n_heads,
                                int group, int d_qk, int d_v, const float* lambda_t, const void* gate, float scale,
                                int num_splits, void* workspace, size_t workspace_bytes, void* out, int out_dtype,
                                void* stream) {
  if (!q || !k || !v || !lambda_t || !out) return DIFFATTN_ERR_NULL;
  int rc = check_options(opt);
  if (rc != DIFFATTN_OK) return rc;
  if (opt && (opt->rope != DIFFATTN_ROPE_NONE || opt->ws_prepared != 0)) return DIFFATTN_ERR_VALUE;
  if (B <= 0 || L <= 0 || L > (1 << 26) || n_heads <= 0 || group <= 0) return DIFFATTN_ERR_SHAPE;
  if (n_heads % (group + 1) != 0) return DIFFATTN_ERR_SHAPE;
  if ((int64_t)B * n_heads > (int64_t(1) << 24)) return DIFFATTN_ERR_SHAPE;
  if (d_qk != kDqk || d_v != kDv) return DIFFATTN_ERR_UNSUPPORTED;
  if (std::isnan(scale) || std::isinf(scale)) return DIFFATTN_ERR_VALUE;
  if (out_dtype != DIFFATTN_OUT_BF16 && out_dtype != DIFFATTN_OUT_F32) return DIFFATTN_ERR_VALUE;
  const bool ring = opt && opt->kv_ring != 0;
  if (ring && opt->window > L) return DIFFATTN_ERR_VALUE;
  if (num_splits <= 0) num_splits = kDefaultSplits;
  if (num_splits > kMaxSplits) return DIFFATTN_ERR_VALUE;
  if ((int64_t)B * n_heads * num_splits > kMaxWorkgroups) return DIFFATTN_ERR_SHAPE;
  const void* ptrs[] = {q, k, v, lambda_t, out};
  for (const void* p : ptrs)
    if (!aligned16(p)) return DIFFATTN_ERR_LAYOUT;
  if (gate && (reinterpret_cast<uintptr_t>(gate) & 7u) != 0) return DIFFATTN_ERR_LAYOUT;
  if (seqlens && (reinterpret_cast<uintptr_t>(seqlens) & 3u) != 0) return DIFFATTN_ERR_LAYOUT;
  diffattn_strides st[2];
  for (int i = 0; i < 2; ++i) {
    st[i] = strides ? strides[i] : contiguous(L, n_heads, i == 1 ? d_v : d_qk);
    if (!strides_ok(st[i])) return DIFFATTN_ERR_LAYOUT;
  }
  if (!workspace || !aligned16(workspace)) return DIFFATTN_ERR_WORKSPACE;
  if (workspace_bytes < diffattn_grouped_decode_workspace_bytes(B, n_heads, d_v, num_splits))
    return DIFFATTN_ERR_WORKSPACE;
  diffattn::GroupedDecodeArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.sk = to_internal(st[0]);
  a.sv = to_internal(st[1]);
  a.seqlens = seqlens;
  a.B = B;
  a.L = L;
  a.nH = n_heads;
  a.g = group;
  a.nN = n_heads / (group + 1);
  a.nS = group * a.nN;
  a.splits = num_splits;
  a.window = opt ? opt->window : 0;
  a.ring = ring ? 1 : 0;
  if (ring && a.window == 0) a.window = L;  // a ring holds the last L positions
  a.c = score_factor(scale);
  a.lam = lambda_t;
  a.gate = static_cast<const uint16_t*>(gate);
  a.partial = static_cast<float*>(workspace);
  a.out = out;
  a.out_f32 = out_dtype == DIFFATTN_OUT_F32;
  if (diffattn::launch_grouped_decode(a, static_cast<hipStream_t>(stream)) != hipSuccess) return DIFFATTN_ERR_HIP;
  return DIFFATTN_OK;
}

}  // extern "C"
