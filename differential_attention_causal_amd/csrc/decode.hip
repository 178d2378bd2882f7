// Split-KV single-query decode for causal differential attention on gfx950.
//
// One query per (b, h) attends every cached position of its sequence (the
// cache includes the current token).  The cache is HBM-bound work: each byte
// of K1, K2 and V is read once.  The positions are cut into `splits` equal
// ranges; a workgroup per (b, h, split) keeps BOTH maps' softmax states (running
// max, sum, unnormalised 128-channel output) and writes them to the workspace.
// A merge kernel per (b, h) rescales the splits to a common max per map, keeps
// the maps apart until o = O1/L1 - lambda O2/L2, then applies the per-head
// GroupNorm (Motif 2.6B explainer, "Differential attention", figure 1 caption).
// With one split the split kernel does that epilogue itself.
//
// Inside a split, keys go in blocks of kKB: scores (8 lanes per key, exact
// bf16 products, fp32 accumulation) -> LDS; block max and exp2 in fp32 (P stays
// fp32 here; there is no matrix product to feed); then the P V pass with 16
// lanes per 256-byte V row.  Scores are kept in base-2 units (c = scale log2 e).
// Every cache byte is read exactly once, so the cache loads are non-temporal:
// they stream past the caches instead of evicting other data.
#include <algorithm>
#include <mutex>

#include "kernels.h"
#include "rope.h"

namespace diffattn {

// The split partials of diffattn_fwd_decode_noalloc.  In host code `scratch`
// names a host-side stand-in, not the device array: kernels and copies get
// the address decode_scratch() looked up.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

hipError_t decode_scratch(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static float* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = static_cast<float*>(p);
  }
  *ptr = addr[dev];
  return hipSuccess;
}

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kKB = 512;                   // keys per block inside a split
constexpr int kPerThread = kKB / kThreads; // scores each thread reduces

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Dot product of 8 bf16 pairs: products are exact in fp32, sums in fp32.
// q (8 floats, dims in order) . b (8 packed bf16), fp32 FMAs in dim order.
__device__ __forceinline__ float dot8(const float (&q)[8], const u32x4& b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc = __builtin_fmaf(q[2 * i], bf16_lo(b[i]), acc);
    acc = __builtin_fmaf(q[2 * i + 1], bf16_hi(b[i]), acc);
  }
  return acc;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Positions 0 .. n-1 of sequence b have been cached.  A linear cache holds at
// most L of them; a ring cache keeps the last L, so n may exceed L there.
__device__ __forceinline__ int seq_len(const DecodeArgs& a, int b) {
  int n = a.seqlens ? a.seqlens[b] : a.L;
  return (!a.ring && n > a.L) ? a.L : n;
}

// What a workgroup of (b, h, split) reads: its range of visible positions,
// the slot of the first, its query (rotated when the cache holds rotated
// keys) and the row bases of its keys and values.
struct SplitView {
  int bh, head, n;
  int r0, r1;     // visible positions lo + r for r in [r0, r1)
  int slot0;      // slot of position lo
  float* rec;     // the split's two records
  float q[2][8];  // lane e of a key group holds dims 8e .. 8e+7 of q1 and q2 (query_unpack)
  const uint16_t *k1b, *k2b, *vb;
};

__device__ __forceinline__ void split_view(const DecodeArgs& a, SplitView& v) {
  const int tid = threadIdx.x;
  const int split = (int)(blockIdx.x % a.splits);
  v.bh = (int)(blockIdx.x / a.splits);
  v.head = v.bh % a.H;
  const int b = v.bh / a.H;
  v.n = seq_len(a, b);
  const int lo = (a.window > 0 && v.n > a.window) ? v.n - a.window : 0;  // oldest visible position
  const int nvis = v.n - lo;  // visible positions lo .. n-1 (at most L)
  const int chunk = nvis > 0 ? (nvis + a.splits - 1) / a.splits : 0;
  v.r0 = split * chunk;
  v.r1 = min(nvis, v.r0 + chunk);
  // Slot of position lo + r: slot0 + r, less L if that reaches L (the visible
  // positions span at most L slots, so they wrap at most once).  A linear
  // cache has n <= L and slot = position.
  v.slot0 = a.ring ? lo % a.L : lo;
  v.rec = a.partial + ((int64_t)v.bh * a.splits + split) * 2 * kPartialStride;
  const int e = tid & 7, cg = tid & 15;
  v.k1b = a.k1 + (int64_t)b * a.sk1.b + (int64_t)v.head * a.sk1.h + 8 * e;
  v.k2b = a.k2 + (int64_t)b * a.sk2.b + (int64_t)v.head * a.sk2.h + 8 * e;
  v.vb = a.v + (int64_t)b * a.sv.b + (int64_t)v.head * a.sv.h + 8 * cg;
}

// The query's raw bf16 chunks (lane e of a key group: dims 8e .. 8e+7), and
// their unpacking into the view (rotated when the cache holds rotated keys).
__device__ __forceinline__ void query_load(const DecodeArgs& a, const SplitView& v, u32x4 (&raw)[2]) {
  const int e = threadIdx.x & 7;
  raw[0] = *reinterpret_cast<const u32x4*>(a.q1 + (int64_t)v.bh * kDqk + 8 * e);
  raw[1] = *reinterpret_cast<const u32x4*>(a.q2 + (int64_t)v.bh * kDqk + 8 * e);
}

__device__ __forceinline__ void query_unpack(const DecodeArgs& a, SplitView& v, const u32x4 (&raw)[2]) {
  const int tid = threadIdx.x, e = tid & 7;
  rope_unpack(raw[0], v.q[0]);
  rope_unpack(raw[1], v.q[1]);
  if (a.rope.mode != 0) {
    // The query is the sequence's last token, rotated in fp32 (no rounding);
    // cached keys are already rotated.
    __shared__ uint64_t rope_tab[32];
    if (tid < 32) rope_tab[tid] = rope_phase_at(a.rope, tid);
    __syncthreads();
    rope_floats<2>(v.q, e, a.rope.pos0 + (uint32_t)(v.n - 1), a.rope.mode, rope_tab);
  }
}

// The end of a split: the 16 key groups' partial outputs summed (4 per wave by
// shuffles, then the 4 waves in LDS), then either the split's record
// (max, sum, O) of each map, or with one split the merge kernel's epilogue.
__device__ __forceinline__ void finish_split(const DecodeArgs& a, float (&o1)[8], float (&o2)[8], float m1, float m2,
                                             float l1, float l2, float* rec, int bh, int head,
                                             float (*acc)[2][kDv], float (*red)[kWaves][2]) {
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int cg = tid & 15;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    o1[k] += __shfl_xor(o1[k], 16);
    o2[k] += __shfl_xor(o2[k], 16);
    o1[k] += __shfl_xor(o1[k], 32);
    o2[k] += __shfl_xor(o2[k], 32);
  }
  if (lane < 16) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      acc[wave][0][8 * cg + k] = o1[k];
      acc[wave][1][8 * cg + k] = o2[k];
    }
  }
  __syncthreads();
  const int map = tid >> 7, ch = tid & 127;
  float sum = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) sum += acc[w][map][ch];
  if (a.splits > 1) {
    float* r = rec + map * kPartialStride;
    r[2 + ch] = sum;
    if (ch == 0) {
      r[0] = map ? m2 : m1;
      r[1] = map ? l2 : l1;
    }
    return;
  }
  // One split: the merge of a single record is the record itself (weight
  // 2^0 = 1), so the epilogue runs here with the merge kernel's arithmetic,
  // threads 0 .. 127 one channel each (the other two waves only pass the
  // barriers).
  __syncthreads();  // every wave has read acc
  acc[0][map][ch] = sum;
  __syncthreads();
  const bool chan = tid < kDv;
  const bool empty = m1 == -__builtin_inff();  // no cached position (uniform)
  float o = 0.f, y = 0.f;
  if (!empty) {
    const float lam = a.lambda_h ? a.lambda_h[head] : a.lambda;
    if (chan) {
#pragma clang fp contract(off)
      o = acc[0][0][ch] / l1 - lam * (acc[0][1][ch] / l2);
    }
    const float s = wave_sum(o);
    if (lane == 0 && chan) red[0][wave][0] = s;
    __syncthreads();
    const float mu = (red[0][0][0] + red[0][1][0]) * (1.0f / kDv);
    const float d = chan ? o - mu : 0.f;
    const float v = wave_sum(d * d);
    if (lane == 0 && chan) red[1][wave][0] = v;
    __syncthreads();
    const float var = (red[1][0][0] + red[1][1][0]) * (1.0f / kDv);
    if (chan) y = d * (1.0f / __builtin_sqrtf(var + a.eps)) * a.gain[(int64_t)head * kDv + ch];
  }
  if (!chan) return;
  const int64_t row = (int64_t)bh * kDv + ch;
  if (a.o_pre) a.o_pre[row] = o;
  if (a.out_f32)
    static_cast<float*>(a.out)[row] = y;
  else
    static_cast<__bf16*>(a.out)[row] = (__bf16)y;
}

__global__ void __launch_bounds__(kThreads) decode_split_kernel(DecodeArgs a) {
  __shared__ float sc[2][kKB];          // scores, then probabilities
  __shared__ float red[2][kWaves][2];   // per-wave max / sum of each map
  __shared__ float acc[kWaves][2][kDv]; // per-wave partial outputs

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  SplitView sv;
  split_view(a, sv);
  {
    u32x4 raw[2];
    query_load(a, sv, raw);
    query_unpack(a, sv, raw);
  }
  const int bh = sv.bh, head = sv.head, r0 = sv.r0, r1 = sv.r1, slot0 = sv.slot0;
  float* const rec = sv.rec;
  const float(&q)[2][8] = sv.q;
  const uint16_t *k1b = sv.k1b, *k2b = sv.k2b, *vb = sv.vb;
  const int e = tid & 7, ks = tid >> 3;
  const int kq = tid >> 4;

  float m1 = -__builtin_inff(), m2 = -__builtin_inff(), l1 = 0.f, l2 = 0.f;
  float o1[8], o2[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o1[k] = o2[k] = 0.f;

  for (int kb = r0; kb < r1; kb += kKB) {
    const int cnt = min(kKB, r1 - kb);
    // Scores of both maps for this block (32 keys per pass, 8 lanes per key).
#pragma unroll 4
    for (int p = 0; p < kKB / 32; ++p) {
      const int kk = p * 32 + ks;
      float d1 = 0.f, d2 = 0.f;
      if (kk < cnt) {
        int slot = slot0 + kb + kk;
        slot -= slot >= a.L ? a.L : 0;
        const int64_t pos = slot;
        const u32x4 x1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k1b + pos * a.sk1.t));
        const u32x4 x2 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k2b + pos * a.sk2.t));
        d1 = dot8(q[0], x1, 0.f);
        d2 = dot8(q[1], x2, 0.f);
      }
      d1 += __shfl_xor(d1, 1);
      d2 += __shfl_xor(d2, 1);
      d1 += __shfl_xor(d1, 2);
      d2 += __shfl_xor(d2, 2);
      d1 += __shfl_xor(d1, 4);
      d2 += __shfl_xor(d2, 4);
      if (e == 0) {
        sc[0][kk] = kk < cnt ? d1 * a.c : -__builtin_inff();
        sc[1][kk] = kk < cnt ? d2 * a.c : -__builtin_inff();
      }
    }
    __syncthreads();
    // Block max per map, raise the running max, rescale.
    float t1[kPerThread], t2[kPerThread];
    float bm1 = -__builtin_inff(), bm2 = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      t1[i] = sc[0][tid + i * kThreads];
      t2[i] = sc[1][tid + i * kThreads];
      bm1 = fmaxf(bm1, t1[i]);
      bm2 = fmaxf(bm2, t2[i]);
    }
    bm1 = wave_max(bm1);
    bm2 = wave_max(bm2);
    if (lane == 0) {
      red[0][wave][0] = bm1;
      red[1][wave][0] = bm2;
    }
    __syncthreads();
    bm1 = red[0][0][0];
    bm2 = red[1][0][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      bm1 = fmaxf(bm1, red[0][w][0]);
      bm2 = fmaxf(bm2, red[1][w][0]);
    }
    const float nm1 = fmaxf(m1, bm1), nm2 = fmaxf(m2, bm2);
    const float al1 = __builtin_amdgcn_exp2f(m1 - nm1), al2 = __builtin_amdgcn_exp2f(m2 - nm2);
    m1 = nm1;
    m2 = nm2;
    float ps1 = 0.f, ps2 = 0.f;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const float p1 = __builtin_amdgcn_exp2f(t1[i] - m1), p2 = __builtin_amdgcn_exp2f(t2[i] - m2);
      sc[0][tid + i * kThreads] = p1;
      sc[1][tid + i * kThreads] = p2;
      ps1 += p1;
      ps2 += p2;
    }
    ps1 = wave_sum(ps1);
    ps2 = wave_sum(ps2);
    if (lane == 0) {
      red[0][wave][1] = ps1;
      red[1][wave][1] = ps2;
    }
    __syncthreads();
    float bs1 = 0.f, bs2 = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      bs1 += red[0][w][1];
      bs2 += red[1][w][1];
    }
    l1 = l1 * al1 + bs1;
    l2 = l2 * al2 + bs2;
    // P V for both maps (16 keys per pass, 16 lanes per V row).
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      o1[k] *= al1;
      o2[k] *= al2;
    }
#pragma unroll 8
    for (int p = 0; p < kKB / 16; ++p) {
      const int kk = p * 16 + kq;
      if (kk < cnt) {
        int slot = slot0 + kb + kk;
        slot -= slot >= a.L ? a.L : 0;
        const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + (int64_t)slot * a.sv.t));
        const float p1 = sc[0][kk], p2 = sc[1][kk];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float lo = bf16_lo(x[w]), hi = bf16_hi(x[w]);
          o1[2 * w] = __builtin_fmaf(p1, lo, o1[2 * w]);
          o1[2 * w + 1] = __builtin_fmaf(p1, hi, o1[2 * w + 1]);
          o2[2 * w] = __builtin_fmaf(p2, lo, o2[2 * w]);
          o2[2 * w + 1] = __builtin_fmaf(p2, hi, o2[2 * w + 1]);
        }
      }
    }
    __syncthreads();  // sc is rewritten by the next block
  }

  finish_split(a, o1, o2, m1, m2, l1, l2, rec, bh, head, acc, red);
}

// A split of at most kSmallKB positions (a short cache, or a sliding window
// of Motif 3's 128 tokens): one block, and every load of it, keys and values,
// issued before any arithmetic, so the workgroup waits for memory once.  The
// scores and the P V pass are the split kernel's; the softmax takes one value
// per thread (map tid / 128, position tid % 128).
constexpr int kSmallKB = 128;

__global__ void __launch_bounds__(kThreads) decode_small_kernel(DecodeArgs a) {
  __shared__ float sc[2][kSmallKB];     // scores, then probabilities
  __shared__ float red[2][kWaves][2];   // per-wave max / sum of each map
  __shared__ float acc[kWaves][2][kDv]; // per-wave partial outputs

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  SplitView sv;
  split_view(a, sv);
  const int e = tid & 7, ks = tid >> 3, kq = tid >> 4;
  const int cnt = max(0, sv.r1 - sv.r0);  // at most kSmallKB (the host checks)
  // Loads go out unconditionally, all at once: a position past the split's
  // last reads that last one (or slot 0 when the split is empty) and is
  // masked afterwards, so no load sits behind a branch.
  const int last = max(cnt - 1, 0);
  auto slot_of = [&](int kk) {
    int slot = sv.slot0 + sv.r0 + min(kk, last);
    return slot - (slot >= a.L ? a.L : 0);
  };
  u32x4 qraw[2];
  query_load(a, sv, qraw);
  u32x4 x1[kSmallKB / 32], x2[kSmallKB / 32], xv[kSmallKB / 16];
#pragma unroll
  for (int p = 0; p < kSmallKB / 32; ++p) {
    const int64_t pos = slot_of(p * 32 + ks);
    x1[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sv.k1b + pos * a.sk1.t));
    x2[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sv.k2b + pos * a.sk2.t));
  }
#pragma unroll
  for (int p = 0; p < kSmallKB / 16; ++p)
    xv[p] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sv.vb + (int64_t)slot_of(p * 16 + kq) * a.sv.t));
  query_unpack(a, sv, qraw);
  // Scores of both maps (32 keys per pass, 8 lanes per key).
#pragma unroll
  for (int p = 0; p < kSmallKB / 32; ++p) {
    const int kk = p * 32 + ks;
    float d1 = dot8(sv.q[0], x1[p], 0.f), d2 = dot8(sv.q[1], x2[p], 0.f);
    d1 += __shfl_xor(d1, 1);
    d2 += __shfl_xor(d2, 1);
    d1 += __shfl_xor(d1, 2);
    d2 += __shfl_xor(d2, 2);
    d1 += __shfl_xor(d1, 4);
    d2 += __shfl_xor(d2, 4);
    if (e == 0 && kk < cnt) {
      sc[0][kk] = d1 * a.c;
      sc[1][kk] = d2 * a.c;
    }
  }
  __syncthreads();
  // Max, exponentials and sum: waves 0-1 take map 1, waves 2-3 map 2.
  const int mp = tid >> 7, k = tid & (kSmallKB - 1);
  const float t = k < cnt ? sc[mp][k] : -__builtin_inff();
  float bm = wave_max(t);
  if (lane == 0) red[mp][wave & 1][0] = bm;
  __syncthreads();
  const float m1 = fmaxf(red[0][0][0], red[0][1][0]), m2 = fmaxf(red[1][0][0], red[1][1][0]);
  const float pr = k < cnt ? __builtin_amdgcn_exp2f(t - (mp ? m2 : m1)) : 0.f;
  sc[mp][k] = pr;
  const float ps = wave_sum(pr);
  if (lane == 0) red[mp][wave & 1][1] = ps;
  __syncthreads();
  const float l1 = red[0][0][1] + red[0][1][1], l2 = red[1][0][1] + red[1][1][1];
  // P V for both maps (16 keys per pass, 16 lanes per V row); positions past
  // the last get probability 0 and an in-range value row.
  float o1[8], o2[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o1[i] = o2[i] = 0.f;
  if (cnt > 0) {
#pragma unroll
    for (int p = 0; p < kSmallKB / 16; ++p) {
      const int kk = p * 16 + kq;
      const float p1 = kk < cnt ? sc[0][kk] : 0.f, p2 = kk < cnt ? sc[1][kk] : 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float lo = bf16_lo(xv[p][w]), hi = bf16_hi(xv[p][w]);
        o1[2 * w] = __builtin_fmaf(p1, lo, o1[2 * w]);
        o1[2 * w + 1] = __builtin_fmaf(p1, hi, o1[2 * w + 1]);
        o2[2 * w] = __builtin_fmaf(p2, lo, o2[2 * w]);
        o2[2 * w + 1] = __builtin_fmaf(p2, hi, o2[2 * w + 1]);
      }
    }
  }
  finish_split(a, o1, o2, m1, m2, l1, l2, sv.rec, sv.bh, sv.head, acc, red);
}

// Merge the splits of one (b, h): one thread per channel.  Every split
// record's (max, sum, O[channel]) is loaded up front, kMergeChunk splits at a
// time with independent loads, so the kernel waits for memory once per chunk.
constexpr int kMergeChunk = 8;

__global__ void __launch_bounds__(kDv) decode_merge_kernel(DecodeArgs a) {
  __shared__ float red[2][2];
  const int ch = threadIdx.x;
  const int wave = ch >> 6;
  const int bh = blockIdx.x;
  const int head = bh % a.H;
  const float* rec = a.partial + (int64_t)bh * a.splits * 2 * kPartialStride;

  float M[2] = {-__builtin_inff(), -__builtin_inff()};
  float L[2] = {0.f, 0.f}, O[2] = {0.f, 0.f};
  for (int s0 = 0; s0 < a.splits; s0 += kMergeChunk) {
    float m[kMergeChunk][2], l[kMergeChunk][2], o[kMergeChunk][2];
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
#pragma unroll
      for (int map = 0; map < 2; ++map) {
        const bool ok = s0 + u < a.splits;
        const float* r = rec + ((s0 + u) * 2 + map) * kPartialStride;
        m[u][map] = ok ? r[0] : -__builtin_inff();
        l[u][map] = ok ? r[1] : 0.f;
        o[u][map] = ok ? r[2 + ch] : 0.f;
      }
    }
#pragma unroll
    for (int map = 0; map < 2; ++map) {
      float mn = M[map];
#pragma unroll
      for (int u = 0; u < kMergeChunk; ++u) mn = fmaxf(mn, m[u][map]);
      if (mn == -__builtin_inff()) continue;  // nothing seen yet (uniform)
      const float sc = __builtin_amdgcn_exp2f(M[map] - mn);
      float Ls = L[map] * sc, Os = O[map] * sc;
#pragma unroll
      for (int u = 0; u < kMergeChunk; ++u) {
        const float w = __builtin_amdgcn_exp2f(m[u][map] - mn);
        Ls += w * l[u][map];
        Os += w * o[u][map];
      }
      M[map] = mn;
      L[map] = Ls;
      O[map] = Os;
    }
  }
  const bool empty = M[0] == -__builtin_inff();  // no cached position (uniform)
  const int64_t row = (int64_t)bh * kDv + ch;
  float o = 0.f, y = 0.f;
  if (!empty) {
    const float lam = a.lambda_h ? a.lambda_h[head] : a.lambda;
    {
#pragma clang fp contract(off)
      o = O[0] / L[0] - lam * (O[1] / L[1]);
    }
    float s = wave_sum(o);
    if ((ch & 63) == 0) red[0][wave] = s;
    __syncthreads();
    const float mu = (red[0][0] + red[0][1]) * (1.0f / kDv);
    const float d = o - mu;
    float v = wave_sum(d * d);
    if ((ch & 63) == 0) red[1][wave] = v;
    __syncthreads();
    const float var = (red[1][0] + red[1][1]) * (1.0f / kDv);
    y = d * (1.0f / __builtin_sqrtf(var + a.eps)) * a.gain[(int64_t)head * kDv + ch];
  }
  if (a.o_pre) a.o_pre[row] = o;
  if (a.out_f32)
    static_cast<float*>(a.out)[row] = y;
  else
    static_cast<__bf16*>(a.out)[row] = (__bf16)y;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  const int64_t bh = (int64_t)a.B * a.H;
  // Visible positions per sequence: at most the window, and at most L.
  const int vis = a.window > 0 ? std::min(a.window, a.L) : a.L;
  const bool small = (vis + a.splits - 1) / a.splits <= kSmallKB;
  const hipError_t e = launch_kernel(small ? decode_small_kernel : decode_split_kernel, dim3((unsigned)(bh * a.splits)),
                                     dim3(kThreads), stream, a);
  if (e != hipSuccess || a.splits == 1) return e;  // one split finishes in the split kernel
  return launch_kernel(decode_merge_kernel, dim3((unsigned)bh), dim3(kDv), stream, a);
}

}  // namespace diffattn
