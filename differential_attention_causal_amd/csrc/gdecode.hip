// Split-KV single-query decode of grouped differential attention with a
// token-wise lambda and an output gate (picx.dev summary of the Motif 3
// report, section 2.2, "Grouped Differential Attention" and "Output Gating")
// on gfx950.
//
// n_H = nS + nN heads; every head is plain causal softmax attention with its
// own keys and values, H_h = softmax(scale q_h K_h^T) V_h over the cached
// positions, and signal head s gives
//   out_s = sigmoid(G_s) * (H_s - lambda_s H_(nS + s / g))
// (no GroupNorm).  The cache is HBM-bound work: each byte of K and V is read
// once.  gdecode_split_kernel: one workgroup per (b, head, split) keeps one
// softmax state (running max, sum, unnormalised 128-channel output) of its
// range of positions and writes it to the workspace, so every head, noise
// heads included, is computed once.  gdecode_merge_kernel: one workgroup per
// (b, signal head) merges the splits of its signal head and of its noise head
// to a common max each, then forms out_s.
//
// Inside a split, keys go in blocks of kKB: scores (8 lanes per key, exact
// bf16 products, fp32 accumulation) -> LDS; block max and exp2 in fp32; then
// the P V pass with 16 lanes per 256-byte V row.  Scores are in base-2 units
// (c = scale log2 e).  Cache loads are non-temporal (read once).
#include "kernels.h"

namespace diffattn {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kKB = 512;                    // keys per block inside a split
constexpr int kPerThread = kKB / kThreads;  // scores each thread reduces
constexpr int kRec = kDv + 2;               // floats per (b, head, split) record: max, sum, O[kDv]

__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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
__device__ __forceinline__ int gseq_len(const GroupedDecodeArgs& a, int b) {
  const int n = a.seqlens ? a.seqlens[b] : a.L;
  return (!a.ring && n > a.L) ? a.L : n;
}

__global__ void __launch_bounds__(kThreads) gdecode_split_kernel(GroupedDecodeArgs a) {
  __shared__ float sc[kKB];           // scores, then probabilities
  __shared__ float red[kWaves][2];    // per-wave max / sum
  __shared__ float acc[kWaves][kDv];  // per-wave partial outputs

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int split = (int)(blockIdx.x % a.splits);
  const int bh = (int)(blockIdx.x / a.splits);
  const int head = bh % a.nH, b = bh / a.nH;

  const int n = gseq_len(a, b);
  const int lo = (a.window > 0 && n > a.window) ? n - a.window : 0;  // oldest visible position
  const int nvis = n - lo;
  const int chunk = nvis > 0 ? (nvis + a.splits - 1) / a.splits : 0;
  const int r0 = split * chunk;
  const int r1 = min(nvis, r0 + chunk);
  // slot of visible position lo + r: slot0 + r, less L once it reaches L
  const int slot0 = a.ring ? lo % a.L : lo;

  // Query chunk: lane e of a key group holds dims 8e .. 8e+7.
  const int e = tid & 7, ks = tid >> 3;
  float q[8];
  {
    const u32x4 w = *reinterpret_cast<const u32x4*>(a.q + (int64_t)bh * kDqk + 8 * e);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      q[2 * i] = lo16(w[i]);
      q[2 * i + 1] = hi16(w[i]);
    }
  }
  const uint16_t* kb0 = a.k + (int64_t)b * a.sk.b + (int64_t)head * a.sk.h + 8 * e;
  const int cg = tid & 15, kq = tid >> 4;
  const uint16_t* vb0 = a.v + (int64_t)b * a.sv.b + (int64_t)head * a.sv.h + 8 * cg;

  float m = -__builtin_inff(), l = 0.f;
  float o[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] = 0.f;

  for (int kb = r0; kb < r1; kb += kKB) {
    const int cnt = min(kKB, r1 - kb);
    // Scores of this block: 32 keys per pass, 8 lanes per key.
#pragma unroll 4
    for (int p = 0; p < kKB / 32; ++p) {
      const int kk = p * 32 + ks;
      float d = 0.f;
      if (kk < cnt) {
        int slot = slot0 + kb + kk;
        slot -= slot >= a.L ? a.L : 0;
        const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb0 + (int64_t)slot * a.sk.t));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          d = __builtin_fmaf(q[2 * i], lo16(x[i]), d);
          d = __builtin_fmaf(q[2 * i + 1], hi16(x[i]), d);
        }
      }
      d += __shfl_xor(d, 1);
      d += __shfl_xor(d, 2);
      d += __shfl_xor(d, 4);
      if (e == 0) sc[kk] = kk < cnt ? d * a.c : -__builtin_inff();
    }
    __syncthreads();
    // Block max, raise the running max, rescale.
    float t[kPerThread];
    float bm = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      t[i] = sc[tid + i * kThreads];
      bm = fmaxf(bm, t[i]);
    }
    bm = wave_max(bm);
    if (lane == 0) red[wave][0] = bm;
    __syncthreads();
    bm = red[0][0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) bm = fmaxf(bm, red[w][0]);
    const float nm = fmaxf(m, bm);
    const float al = __builtin_amdgcn_exp2f(m - nm);
    m = nm;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const float p = __builtin_amdgcn_exp2f(t[i] - m);
      sc[tid + i * kThreads] = p;
      ps += p;
    }
    ps = wave_sum(ps);
    if (lane == 0) red[wave][1] = ps;
    __syncthreads();
    float bs = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) bs += red[w][1];
    l = l * al + bs;
    // P V: 16 keys per pass, 16 lanes per V row.
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] *= al;
#pragma unroll 8
    for (int p = 0; p < kKB / 16; ++p) {
      const int kk = p * 16 + kq;
      if (kk < cnt) {
        int slot = slot0 + kb + kk;
        slot -= slot >= a.L ? a.L : 0;
        const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb0 + (int64_t)slot * a.sv.t));
        const float pk = sc[kk];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          o[2 * w] = __builtin_fmaf(pk, lo16(x[w]), o[2 * w]);
          o[2 * w + 1] = __builtin_fmaf(pk, hi16(x[w]), o[2 * w + 1]);
        }
      }
    }
    __syncthreads();  // sc is rewritten by the next block
  }

  // Sum the 16 key groups: 4 per wave by shuffles, then the 4 waves in LDS.
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    o[k] += __shfl_xor(o[k], 16);
    o[k] += __shfl_xor(o[k], 32);
  }
  if (lane < 16) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[wave][8 * cg + k] = o[k];
  }
  __syncthreads();
  if (tid >= kDv) return;
  float sum = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) sum += acc[w][tid];
  float* r = a.partial + ((int64_t)bh * a.splits + split) * kRec;
  r[2 + tid] = sum;
  if (tid == 0) {
    r[0] = m;
    r[1] = l;
  }
}

// One head's splits merged to a common max: (M, L, O[ch]) for this thread's
// channel.  Every record of a chunk is loaded up front (independent loads).
constexpr int kMergeChunk = 8;

__device__ __forceinline__ void merge_head(const GroupedDecodeArgs& a, const float* rec, int ch, float& M, float& L,
                                           float& O) {
  M = -__builtin_inff();
  L = 0.f;
  O = 0.f;
  for (int s0 = 0; s0 < a.splits; s0 += kMergeChunk) {
    float m[kMergeChunk], l[kMergeChunk], o[kMergeChunk];
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      const bool ok = s0 + u < a.splits;
      const float* r = rec + (s0 + u) * kRec;
      m[u] = ok ? r[0] : -__builtin_inff();
      l[u] = ok ? r[1] : 0.f;
      o[u] = ok ? r[2 + ch] : 0.f;
    }
    float mn = M;
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) mn = fmaxf(mn, m[u]);
    if (mn == -__builtin_inff()) continue;  // nothing seen yet (uniform)
    const float sc = __builtin_amdgcn_exp2f(M - mn);
    float Ls = L * sc, Os = O * sc;
#pragma unroll
    for (int u = 0; u < kMergeChunk; ++u) {
      const float w = __builtin_amdgcn_exp2f(m[u] - mn);
      Ls += w * l[u];
      Os += w * o[u];
    }
    M = mn;
    L = Ls;
    O = Os;
  }
}

// out[b, s, ch] = sigmoid(G) * (H_s - lambda H_noise): one thread per channel.
__global__ void __launch_bounds__(kDv) gdecode_merge_kernel(GroupedDecodeArgs a) {
  const int ch = threadIdx.x;
  const int bs = blockIdx.x;
  const int s = bs % a.nS, b = bs / a.nS;
  const int hn = a.nS + s / a.g;  // the paired noise head
  const float* rs = a.partial + ((int64_t)b * a.nH + s) * a.splits * kRec;
  const float* rn = a.partial + ((int64_t)b * a.nH + hn) * a.splits * kRec;
  float Ms, Ls, Os, Mn, Ln, On;
  merge_head(a, rs, ch, Ms, Ls, Os);
  merge_head(a, rn, ch, Mn, Ln, On);
  float y = 0.f;
  if (Ms != -__builtin_inff()) {  // a sequence with no cached position gives 0 (uniform)
    const float lam = a.lam[(int64_t)b * a.nS + s];
    {
      // both quotients rounded before the subtraction (no FMA contraction)
#pragma clang fp contract(off)
      y = Os / Ls - lam * (On / Ln);
    }
    if (a.gate) {
      const uint16_t gb = a.gate[((int64_t)b * a.nS + s) * kDv + ch];
      const float gl = __uint_as_float((uint32_t)gb << 16);
      y *= 1.0f / (1.0f + __builtin_amdgcn_exp2f(-gl * 1.4426950408889634f));  // sigmoid, as the prefill's
    }
  }
  const int64_t row = (int64_t)bs * kDv + ch;
  if (a.out_f32)
    static_cast<float*>(a.out)[row] = y;
  else
    static_cast<__bf16*>(a.out)[row] = (__bf16)y;
}

}  // namespace

hipError_t launch_grouped_decode(const GroupedDecodeArgs& a, hipStream_t stream) {
  const int64_t bh = (int64_t)a.B * a.nH;
  const hipError_t e = launch_kernel(gdecode_split_kernel, dim3((unsigned)(bh * a.splits)), dim3(kThreads), stream, a);
  if (e != hipSuccess) return e;
  return launch_kernel(gdecode_merge_kernel, dim3((unsigned)((int64_t)a.B * a.nS)), dim3(kDv), stream, a);
}

}  // namespace diffattn
