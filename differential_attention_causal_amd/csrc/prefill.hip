// Fused causal differential-attention prefill for gfx950 (MI355X).
//
// Computes, per (b, h) and query i (Motif 2.6B explainer, "Differential
// attention" and the figure 1 caption):
//   o_i = sum_{j<=i} [P1_ij - lambda P2_ij] v_j,   Pm = softmax_j(Qm Km^T * scale)
//   y_i = GroupNorm(o_i)  (one group = the head's 128 channels, with gain)
// in one pass over the keys, with two independent online-softmax states.
//
// Work split.  A workgroup owns 128 consecutive queries of one (b, h): four
// wave64s with 32 queries each.  Keys stream through LDS in tiles of 32; tiles
// past the causal diagonal are never loaded, and a wave skips tiles past its
// own diagonal.
//
// Transposed products.  Each wave computes S^T = K Q^T (32 keys x 32 queries)
// on v_mfma_f32_32x32x16_bf16 with K from LDS and Q^T held in registers for the
// whole kernel, and O^T = V^T P^T (128 channels x 32 queries) on
// v_mfma_f32_32x32x16_f16.  In this orientation lane l holds query l % 32 in
// both the score accumulator and the output accumulator, so the softmax state,
// the rescale of O and the GroupNorm are lane-local, with one exchange between
// the two lanes (l, l ^ 32) that share a query.  P^T feeds the second product
// straight from registers: the score accumulator already holds, per lane, the
// key indices the f16 operand needs, provided V^T's keys are stored in LDS in
// the matching order (see kVPos below).
//
// Precision.  Scores: bf16 inputs, fp32 accumulation.  Softmax in fp32 base-2
// units (c = scale * log2 e).  P is rounded to fp16 and V is converted
// bf16 -> fp16 (exact for |v| in [2^-14, 65504)) for the f16 product, fp32
// accumulation.  The running max is only raised when a tile's max exceeds it
// by more than kSlack (base 2), so P <= 2^kSlack stays far inside fp16 range and
// the O rescale is rare after the first tiles.
#include "kernels.h"

namespace diffattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;            // queries per workgroup
constexpr int kBN = 32;                     // keys per LDS tile
constexpr int kKRow = kDqk * 2;             // 128 bytes per key row
constexpr int kKBytes = kBN * kKRow;        // 4 KiB per K tile
constexpr int kVRow = (kBN + 8) * 2;        // 80 bytes per V^T channel row (16-byte pad)
constexpr int kVBytes = kDv * kVRow;        // 10 KiB per V^T tile
constexpr int kStage = 2 * kKBytes + kVBytes;
constexpr float kSlack = 8.0f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Position (in units of 4 keys) of key group kg inside a V^T row.  Key
// k = 16s + 8m + 4h + r of a tile must sit at 16s + 8h + 4m + r, so that lane
// half h reads the 8 keys {16s + 8m + 4h + r} of product step s as one
// contiguous 16-byte word: the same keys, in the same slot order, that half h
// holds in its score accumulator.  That is a swap of bits 0 and 1 of kg.
__device__ __forceinline__ int kVPos(int kg) { return (kg & 4) | ((kg & 1) << 1) | ((kg >> 1) & 1); }

__device__ __forceinline__ u32x4 load16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 load8(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }

struct Staged {
  u32x4 k1, k2;
  u32x2 v[4];
};

// Global -> registers for key tile starting at k0.  Thread t loads 16 bytes of
// K1 and K2 (key t/8, chunk t%8) and a 4-key x 4-channel block of V.
__device__ __forceinline__ void stage_load(Staged& st, const PrefillArgs& a, int b, int head, int k0,
                                           int tid) {
  const int kr = tid >> 3, ch = tid & 7;
  const int key = k0 + kr;
  if (key < a.T) {
    st.k1 = load16(a.k1 + (int64_t)b * a.sk1.b + (int64_t)key * a.sk1.t + (int64_t)head * a.sk1.h + 8 * ch);
    st.k2 = load16(a.k2 + (int64_t)b * a.sk2.b + (int64_t)key * a.sk2.t + (int64_t)head * a.sk2.h + 8 * ch);
  } else {
    st.k1 = u32x4{0, 0, 0, 0};
    st.k2 = u32x4{0, 0, 0, 0};
  }
  const int kg = tid & 7, cg = tid >> 3;
  const uint16_t* vb = a.v + (int64_t)b * a.sv.b + (int64_t)head * a.sv.h + 4 * cg;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int kv = k0 + 4 * kg + r;
    st.v[r] = (kv < a.T) ? load8(vb + (int64_t)kv * a.sv.t) : u32x2{0, 0};
  }
}

// Registers -> LDS: K rows with the 16-byte chunk index XOR-swizzled by the
// row, V transposed to [channel][key] in fp16 with the kVPos key order.
__device__ __forceinline__ void stage_store(const Staged& st, char* stage, int tid) {
  const int kr = tid >> 3, ch = tid & 7;
  const int koff = kr * kKRow + ((ch ^ (kr & 7)) << 4);
  *reinterpret_cast<u32x4*>(stage + koff) = st.k1;
  *reinterpret_cast<u32x4*>(stage + kKBytes + koff) = st.k2;
  const int kg = tid & 7, cg = tid >> 3;
  float e[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    e[r][0] = bf16_lo(st.v[r].x);
    e[r][1] = bf16_hi(st.v[r].x);
    e[r][2] = bf16_lo(st.v[r].y);
    e[r][3] = bf16_hi(st.v[r].y);
  }
  char* vt = stage + 2 * kKBytes + kVPos(kg) * 8;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    f16x4 h = {(_Float16)e[0][c], (_Float16)e[1][c], (_Float16)e[2][c], (_Float16)e[3][c]};
    *reinterpret_cast<f16x4*>(vt + (4 * cg + c) * kVRow) = h;
  }
}

// One map's online-softmax step on a 32x32 score tile held as S^T (lane: one
// query, 16 keys).  Updates the running max m (base-2 units) and the lane's
// partial sum l, rescales that map's O^T when the max is raised, and returns
// the tile's probabilities as the two f16 operands of the P^T V^T product.
__device__ __forceinline__ void softmax_step(f32x16& s, float c, float& m, float& l, f32x16 (&O)[4],
                                             f16x8& p0, f16x8& p1) {
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mc = mx * c;
  const bool need = mc > m + kSlack;
  if (__any(need)) {
    const float mn = need ? mc : m;
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    l *= alpha;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) O[cb] *= alpha;
    m = mn;
  }
  float p[16];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c, -m));
    sum += p[i];
  }
  l += sum;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p0[j] = (_Float16)p[j];
    p1[j] = (_Float16)p[8 + j];
  }
}

__global__ void __launch_bounds__(kThreads) prefill_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hf = lane >> 5;  // lane half
  const int lq = lane & 31;  // query within the wave

  // Longest rows first; consecutive workgroups take different (b, h), so all
  // query blocks of one (b, h) are dispatched to the same XCD when B*H is a
  // multiple of 8 and share its L2.
  const int nqb = (a.T + kBM - 1) / kBM;
  const int BH = a.B * a.H;
  const int qb = nqb - 1 - (int)(blockIdx.x / BH);
  const int bh = (int)(blockIdx.x % BH);
  const int head = bh % a.H;
  const int b = bh / a.H;

  const int q_first = qb * kBM + 32 * wave;  // first query of this wave
  const int q = q_first + lq;                // this lane's query
  const bool wave_live = q_first < a.T;
  const int last_tile = min(qb * (kBM / kBN) + (kBM / kBN) - 1, (a.T - 1) / kBN);
  const int wave_last_tile = q_first / kBN;  // the wave's diagonal tile

  // Q1^T, Q2^T operands: lane holds query lq, dims 16s + 8hf .. +7.
  bf16x8 qa[4], qb2[4];
  {
    const bool ok = q < a.T;
    const uint16_t* p1 = a.q1 + (int64_t)b * a.sq1.b + (int64_t)q * a.sq1.t + (int64_t)head * a.sq1.h + 8 * hf;
    const uint16_t* p2 = a.q2 + (int64_t)b * a.sq2.b + (int64_t)q * a.sq2.t + (int64_t)head * a.sq2.h + 8 * hf;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 x1 = ok ? load16(p1 + 16 * s) : u32x4{0, 0, 0, 0};
      u32x4 x2 = ok ? load16(p2 + 16 * s) : u32x4{0, 0, 0, 0};
      qa[s] = __builtin_bit_cast(bf16x8, x1);
      qb2[s] = __builtin_bit_cast(bf16x8, x2);
    }
  }

  f32x16 O1[4], O2[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    O1[cb] = f32x16{};
    O2[cb] = f32x16{};
  }
  float m1 = -__builtin_inff(), m2 = -__builtin_inff(), l1 = 0.f, l2 = 0.f;
  const float c = a.c;

  Staged st;
  stage_load(st, a, b, head, 0, tid);
  stage_store(st, smem, tid);
  __syncthreads();

  for (int j = 0; j <= last_tile; ++j) {
    char* cur = smem + (j & 1) * kStage;
    char* nxt = smem + ((j + 1) & 1) * kStage;
    const bool more = j < last_tile;
    if (more) stage_load(st, a, b, head, (j + 1) * kBN, tid);

    if (wave_live && j <= wave_last_tile) {
      f32x16 s1 = f32x16{}, s2 = f32x16{};
      const int krow = lq * kKRow;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int off = krow + (((2 * s + hf) ^ (lq & 7)) << 4);
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(cur + off);
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(cur + kKBytes + off);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qa[s], s1, 0, 0, 0);
        s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, qb2[s], s2, 0, 0, 0);
      }
      if (j == wave_last_tile) {
        // Diagonal tile (its first key is the wave's first query): key row
        // 8(i/4) + 4hf + i%4 is visible to query lq iff it is <= lq.
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kr = 8 * (i >> 2) + 4 * hf + (i & 3);
          if (kr > lq) {
            s1[i] = -__builtin_inff();
            s2[i] = -__builtin_inff();
          }
        }
      }
      f16x8 p1a, p1b, p2a, p2b;
      softmax_step(s1, c, m1, l1, O1, p1a, p1b);
      softmax_step(s2, c, m2, l2, O2, p2a, p2b);
      const char* vt = cur + 2 * kKBytes + lq * kVRow + hf * 16;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const f16x8 va0 = *reinterpret_cast<const f16x8*>(vt + cb * 32 * kVRow);
        const f16x8 va1 = *reinterpret_cast<const f16x8*>(vt + cb * 32 * kVRow + 32);
        O1[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va0, p1a, O1[cb], 0, 0, 0);
        O2[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va0, p2a, O2[cb], 0, 0, 0);
        O1[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va1, p1b, O1[cb], 0, 0, 0);
        O2[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va1, p2b, O2[cb], 0, 0, 0);
      }
    }

    if (more) stage_store(st, nxt, tid);
    __syncthreads();
  }

  if (!wave_live) return;

  // Combine the two maps, then GroupNorm over the 128 channels of the query.
  // Lane (hf, lq) holds channels 32cb + 8(i/4) + 4hf + i%4; its partner lane
  // (lane ^ 32) holds the other 64.
  l1 += __shfl_xor(l1, 32);
  l2 += __shfl_xor(l2, 32);
  const float lam = a.lambda_h ? a.lambda_h[head] : a.lambda;
  const float r1 = 1.0f / l1;
  const float r2 = lam / l2;
  float sum = 0.f;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // Both products rounded before the subtraction (no FMA contraction), so
      // two identical maps at lambda = 1 cancel to exactly zero.
#pragma clang fp contract(off)
      const float o = O1[cb][i] * r1 - O2[cb][i] * r2;
      O1[cb][i] = o;
      sum += o;
    }
  }
  sum += __shfl_xor(sum, 32);
  const float mu = sum * (1.0f / kDv);
  float ss = 0.f;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float d = O1[cb][i] - mu;
      ss += d * d;
    }
  }
  ss += __shfl_xor(ss, 32);
  const float inv = 1.0f / __builtin_sqrtf(ss * (1.0f / kDv) + a.eps);

  if (q >= a.T) return;
  const int64_t row = (((int64_t)b * a.T + q) * a.H + head) * kDv;
  const float* g = a.gain + (int64_t)head * kDv;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int ch = 32 * cb + 8 * r4 + 4 * hf;
      const f32x4 gv = *reinterpret_cast<const f32x4*>(g + ch);
      f32x4 o, y;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        o[r] = O1[cb][4 * r4 + r];
        y[r] = (o[r] - mu) * inv * gv[r];
      }
      if (a.o_pre) *reinterpret_cast<f32x4*>(a.o_pre + row + ch) = o;
      if (a.out_f32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row + ch) = y;
      } else {
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 yb = {(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
        *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(a.out) + row + ch) = yb;
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int nqb = (a.T + kBM - 1) / kBM;
  const int64_t grid = (int64_t)nqb * a.B * a.H;
  hipLaunchKernelGGL(prefill_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace diffattn
