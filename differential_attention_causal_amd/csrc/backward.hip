// Backward pass of causal differential attention for gfx950 (MI355X).
//
// Forward (Motif 2.6B explainer, "Differential attention" and the figure 1
// caption): P_m = softmax(scale * Q_m K_m^T) causally, O_m = P_m V,
// o = O_1 - lambda O_2, y = GroupNorm(o) * gain.  Given dy, the calculus of
// that definition is, per (b, h):
//   GroupNorm:  x = (o - mu) / sigma, dgain += dy x,
//               do = (g - mean(g) - x mean(g x)) / sigma  with g = dy gain
//   combine:    dO_1 = do, dO_2 = -lambda do, dlambda += -sum(do O_2)
//   each map:   dP_m = dO_m V^T, dS_m = P_m (dP_m - D_m), D_m = rowsum(dO_m O_m)
//               dQ_m = scale dS_m K_m, dK_m = scale dS_m^T Q_m
//   values:     dV = P_1^T dO_1 + P_2^T dO_2 = (P_1 - lambda P_2)^T do
// Since both maps share V and dO_2 = -lambda dO_1, dP_2 = -lambda dP_1: one
// product serves both maps.
//
// Kernels (all deterministic, no atomics):
//   bwd_pre_kernel     per row: do (fp16), D_1, D_2; gain/lambda partials
//   bwd_reduce_kernel  per head: sum of the partials
//   bwd_dq_kernel      queries own lanes (the forward's orientation): recompute
//                      S^T, P^T from the saved log-sum-exp, dP^T = V dO^T,
//                      dQ^T += K^T dS^T
//   bwd_dkv_kernel     keys own lanes, two kinds of waves on the same keys and
//                      query tiles: S = Q K^T, dP = dO V^T, dK^T += Q^T dS;
//                      and S = Q K^T, dV^T += dO^T (P_1 - lambda P_2)
// The last two use v_mfma_f32_32x32x16 like the prefill: a 32x32 accumulator
// held by a wave is used directly as the next product's operand, with the
// transposed LDS tiles stored in the matching (kVPos) order.  Scores are bf16
// products of the exact inputs; dO, P, dS, V^T, K^T and Q^T enter the other
// products as fp16 (inputs converted exactly, |x| in [2^-14, 65504)).
#include "kernels.h"
#include "tile.h"

namespace diffattn {
namespace {

constexpr int kWaves = 4;
constexpr int kRows = 32 * kWaves;      // queries (dQ) or keys (dK, dV) per workgroup
constexpr int kKRow = kDqk * 2;         // 128-byte bf16 rows of Q or K
constexpr int kQKTile = 32 * kKRow;     // 4 KiB: one map's 32-row bf16 tile
constexpr int kD16Row = kDv * 2;        // 256-byte fp16 rows of dO or V
constexpr int kD16Tile = 32 * kD16Row;  // 8 KiB
constexpr int kTRow = (32 + 8) * 2;     // 80-byte transposed fp16 rows (16-byte pad)
constexpr int kQKT = kDqk * kTRow;      // 5 KiB: one map's transposed 64 x 32 tile

// 16-byte chunk swizzle of 256-byte rows (16 chunks): rows r and r ^ 16 share
// it, so a 16-byte read by 32 lanes of consecutive rows is at most 2-way
// conflicted.
__device__ __forceinline__ int swz16(int r) { return r & 15; }

// ---------------------------------------------------------------------------
// Per row: the GroupNorm backward, do, D_1 = rowsum(do O_1),
// D_2 = rowsum(-lambda do O_2), and partial sums of dgain and dlambda over a
// chunk of kBwdRowsPerChunk rows of one head.  Sixteen lanes per row (eight
// channels each), four rows per wave at a time; row sums are reduced within
// the 16-lane DPP row in four steps.

// Sum over the 16 lanes of a DPP row, the same value in every lane: xor 1 and
// xor 2 within quads, then the mirrored halves of 8, then of 16.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

__device__ __forceinline__ float sum16(float x) {
  x += dpp_f32<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_f32<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_f32<0x141>(x);  // row_half_mirror
  x += dpp_f32<0x140>(x);  // row_mirror
  return x;
}

__global__ void __launch_bounds__(256) bwd_pre_kernel(BackwardArgs a) {
  constexpr int kRowsPerPass = 4 * kWaves;  // 16: four per wave
  __shared__ float red[kRowsPerPass][kDv + 1];
  const int chunk = blockIdx.x, h = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int grp = lane >> 4, li = lane & 15;  // row within the wave's four, lane within the row
  const int BT = a.B * a.T;
  const float lam = a.lambda_h ? a.lambda_h[h] : a.lambda;
  const float* gp = a.gain + (int64_t)h * kDv + 8 * li;
  float g[8];
  {
    const f32x4 g0 = *reinterpret_cast<const f32x4*>(gp), g1 = *reinterpret_cast<const f32x4*>(gp + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      g[e] = g0[e];
      g[4 + e] = g1[e];
    }
  }
  float dg[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float dl = 0.f;
#pragma unroll 1
  for (int pass = 0; pass < kBwdRowsPerChunk / kRowsPerPass; ++pass) {
    const int rbt = chunk * kBwdRowsPerChunk + pass * kRowsPerPass + wave * 4 + grp;
    if (rbt >= BT) continue;  // per-lane; the DPP rows of a wave are independent
    const int64_t off = ((int64_t)rbt * a.H + h) * kDv + 8 * li;
    float o1[8], o2[8], dy[8], x[8];
    {
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(a.o1n + off), a1 = *reinterpret_cast<const f32x4*>(a.o1n + off + 4);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(a.o2n + off), b1 = *reinterpret_cast<const f32x4*>(a.o2n + off + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o1[e] = a0[e];
        o1[4 + e] = a1[e];
        o2[e] = b0[e];
        o2[4 + e] = b1[e];
      }
      if (a.dy_f32) {
        const float* d = static_cast<const float*>(a.dy) + off;
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(d), d1 = *reinterpret_cast<const f32x4*>(d + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dy[e] = d0[e];
          dy[4 + e] = d1[e];
        }
      } else {
        const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.dy) + off);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dy[2 * e] = bf16_lo(w[e]);
          dy[2 * e + 1] = bf16_hi(w[e]);
        }
      }
    }
    float sx = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = o1[e] - lam * o2[e];
      sx += x[e];
    }
    const float mu = sum16(sx) * (1.0f / kDv);
    float sd = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] -= mu;
      sd += x[e] * x[e];
    }
    const float rs = 1.0f / __builtin_sqrtf(sum16(sd) * (1.0f / kDv) + a.eps);
    float sg = 0.f, sgx = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] *= rs;  // x-hat
      dg[e] += dy[e] * x[e];
      dy[e] *= g[e];  // g = dy * gain
      sg += dy[e];
      sgx += dy[e] * x[e];
    }
    const float mg = sum16(sg) * (1.0f / kDv), mgx = sum16(sgx) * (1.0f / kDv);
    float sdl = 0.f, sd1 = 0.f, sd2 = 0.f;
    f16x8 hv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = rs * (dy[e] - mg - x[e] * mgx);
      sdl += d * o2[e];
      // D_m from the fp16 dO the products use, so that sum_j P_ij dP_ij = D_i
      // holds up to fp32 rounding (at T = 1, dS is then 0 as it must be).
      hv[e] = (_Float16)d;
      sd1 += (float)hv[e] * o1[e];
      sd2 += (float)hv[e] * o2[e];
    }
    dl -= sum16(sdl);
    const float dd1 = sum16(sd1), s2 = sum16(sd2);
    *reinterpret_cast<f16x8*>(a.dO + off) = hv;
    if (li == 0) *reinterpret_cast<f32x2*>(a.dstat + (off / kDv) * 2) = f32x2{dd1, -lam * s2};
  }
  const int rr = wave * 4 + grp;
#pragma unroll
  for (int e = 0; e < 8; ++e) red[rr][8 * li + e] = dg[e];
  if (li == 0) red[rr][kDv] = dl;
  __syncthreads();
  const int t = threadIdx.x;
  if (t <= kDv) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < kRowsPerPass; ++r) s += red[r][t];
    a.partial[((int64_t)h * a.nchunks + chunk) * (kDv + 1) + t] = s;
  }
}

// dgain[h, c] and dlambda[h]: the partials summed in chunk order.
__global__ void __launch_bounds__(192) bwd_reduce_kernel(BackwardArgs a) {
  const int h = blockIdx.x, t = threadIdx.x;
  if (t > kDv) return;
  const float* p = a.partial + (int64_t)h * a.nchunks * (kDv + 1) + t;
  // Eight running sums in a fixed order: eight independent loads in flight.
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int c = 0;
  for (; c + 8 <= a.nchunks; c += 8)
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] += p[(int64_t)(c + u) * (kDv + 1)];
  for (; c < a.nchunks; ++c) acc[0] += p[(int64_t)c * (kDv + 1)];
  const float s = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  if (t < kDv)
    a.dgain[(int64_t)h * kDv + t] = s;
  else
    a.dlam[h] = s;
}

// ---------------------------------------------------------------------------
// Tile staging shared by the three product kernels.  A tile is 32 rows
// (keys or queries) of one (b, h), rows r0 .. r0+31, rows at or past `end`
// reading as zero.  Threads 0..255 of the workgroup take part.

// Row-major bf16 tiles of both maps (Q or K) by DMA into [map][32][128 B]
// with the kSwz chunk swizzle: thread t fetches row t/8, logical chunk
// (t % 8) ^ kSwz(t / 8), landing at chunk position t.
__device__ __forceinline__ void dma_qk(const uint16_t* b1, const uint16_t* b2, int64_t st1, int64_t st2, int r0,
                                       int end, char* dst, int tid) {
  const int r = tid >> 3, c = (tid & 7) ^ kSwz(r);
  char* d = dst + (tid >> 6) * 1024;  // each wave fills 1 KiB of each map's tile
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc(b1, st1, r0, end, kDqk), (lds_ptr_t)d, 16,
                                           (uint32_t)((r * st1 + 8 * c) * 2), 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc(b2, st2, r0, end, kDqk), (lds_ptr_t)(d + kQKTile), 16,
                                           (uint32_t)((r * st2 + 8 * c) * 2), 0, 0, 0);
}

// Row-major fp16 dO tile by DMA into [32][256 B] with the swz16 swizzle: the
// tile's 512 chunks, two per thread (chunk positions t and t + 256).
__device__ __forceinline__ void dma_do(const uint16_t* base, int64_t stride, int r0, int end, char* dst, int tid) {
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc(base, stride, r0, end, kDv);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int p = tid + 256 * k;
    const int r = p >> 4, c = (p & 15) ^ swz16(r);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + 1024 * (p >> 6)), 16,
                                             (uint32_t)((r * stride + 8 * c) * 2), 0, 0, 0);
  }
}

// Transposed fp16 tiles of both maps (Q^T or K^T): [map][64 dims][80 B], row
// d holding rows r0..r0+31 of dim d in kVPos order.  Thread t loads rows
// 4(t%8) .. +3, dims 2(t/8), 2(t/8)+1 of each map (4-byte loads) ...
struct StagedT {
  uint32_t w[2][4];
};

__device__ __forceinline__ void load_qkT(StagedT& s, const uint16_t* b1, const uint16_t* b2, int64_t st1,
                                         int64_t st2, int r0, int end, int tid) {
  const int kg = tid & 7, dg = tid >> 3;
  const __amdgpu_buffer_rsrc_t x1 = rows_rsrc(b1, st1, r0, end, kDqk);
  const __amdgpu_buffer_rsrc_t x2 = rows_rsrc(b2, st2, r0, end, kDqk);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    s.w[0][r] = __builtin_amdgcn_raw_buffer_load_b32(x1, (uint32_t)(((4 * kg + r) * st1 + 2 * dg) * 2), 0, 0);
    s.w[1][r] = __builtin_amdgcn_raw_buffer_load_b32(x2, (uint32_t)(((4 * kg + r) * st2 + 2 * dg) * 2), 0, 0);
  }
}

// ... and writes them converted to fp16.
__device__ __forceinline__ void store_qkT(const StagedT& s, char* dst, int tid) {
  const int kg = tid & 7, dg = tid >> 3;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const f16x4 lo = {(_Float16)bf16_lo(s.w[m][0]), (_Float16)bf16_lo(s.w[m][1]), (_Float16)bf16_lo(s.w[m][2]),
                      (_Float16)bf16_lo(s.w[m][3])};
    const f16x4 hi = {(_Float16)bf16_hi(s.w[m][0]), (_Float16)bf16_hi(s.w[m][1]), (_Float16)bf16_hi(s.w[m][2]),
                      (_Float16)bf16_hi(s.w[m][3])};
    char* d = dst + m * kQKT + kVPos(kg) * 8;
    *reinterpret_cast<f16x4*>(d + (2 * dg) * kTRow) = lo;
    *reinterpret_cast<f16x4*>(d + (2 * dg + 1) * kTRow) = hi;
  }
}

// Row-major fp16 V tile (keys x 128 channels) through registers: thread t
// takes row t/8, channels 16(t%8) .. +15 (two 16-byte loads), stores them
// converted at logical chunks 2(t%8), 2(t%8)+1 with the swz16 swizzle.
struct StagedV {
  u32x4 w[2];
};

__device__ __forceinline__ void load_v(StagedV& s, const uint16_t* base, int64_t stride, int r0, int end, int tid) {
  const int r = tid >> 3, p = tid & 7;
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc(base, stride, r0, end, kDv);
  s.w[0] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)((r * stride + 16 * p) * 2), 0, 0);
  s.w[1] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)((r * stride + 16 * p + 8) * 2), 0, 0);
}

__device__ __forceinline__ void store_v(const StagedV& s, char* dst, int tid) {
  const int r = tid >> 3, p = tid & 7;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    f16x8 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[2 * i] = (_Float16)bf16_lo(s.w[k][i]);
      h[2 * i + 1] = (_Float16)bf16_hi(s.w[k][i]);
    }
    *reinterpret_cast<f16x8*>(dst + r * kD16Row + (((2 * p + k) ^ swz16(r)) << 4)) = h;
  }
}

// Packs a 32x32 accumulator (16 values per lane) as the two fp16 operands of
// the next product's k-steps: registers 0..7, then 8..15.
__device__ __forceinline__ void pack16(const f32x16& v, f16x8& p0, f16x8& p1) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p0[j] = (_Float16)v[j];
    p1[j] = (_Float16)v[8 + j];
  }
}

// acc (32 rows x 32 lanes' columns) += T^T(rows 32blk.., kVPos-ordered 32)
// * B for one 32-row block of a transposed fp16 tile.
__device__ __forceinline__ f32x16 mfma_T(const char* tT, int blk, int lq, int hf, const f16x8& b0, const f16x8& b1,
                                         f32x16 acc) {
  const char* t = tT + (32 * blk + lq) * kTRow + hf * 16;
  const f16x8 a0 = *reinterpret_cast<const f16x8*>(t);
  const f16x8 a1 = *reinterpret_cast<const f16x8*>(t + 32);
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, b0, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, b1, acc, 0, 0, 0);
}

// Stores a lane's column of a 32-row accumulator block (rows 32blk + 8(i/4) +
// 4hf + i%4), times f, into dst[rows] (fp32, 16-byte stores).
__device__ __forceinline__ void store_col(float* dst, const f32x16& acc, int blk, int hf, float f) {
#pragma unroll
  for (int r4 = 0; r4 < 4; ++r4) {
    f32x4 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = acc[4 * r4 + r] * f;
    *reinterpret_cast<f32x4*>(dst + 32 * blk + 8 * r4 + 4 * hf) = v;
  }
}

// The transposed operand of a row-major fp16 tile (32 rows x 128 columns,
// swz16-swizzled 256-byte rows) by ds_read_b64_tr_b16, which hands lane i of
// each 16-lane group element i % 4 of the 8-byte reads of lanes 4k + i / 4,
// k = 0..3.  For column block blk and k-half kh, lane (hf, g, L) (g: 16-lane
// group within the half, L: lane within it) reads 4 columns 32blk + 16g +
// 4(L % 4) .. +3 of row 16kh + 8h + 4hf + L / 4 for h = 0, 1, so it receives
// column 32blk + 16g + L of rows 16kh + 8(j / 4) + 4hf + j % 4, j = 0..7:
// the A operand of a product whose B operand is a 32x32 accumulator packed by
// pack16 (rows in the accumulator's order).
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ f16x8 tr_operand(const char* tile, int blk, int kh, int lane) {
  const int hf = lane >> 5, g = (lane >> 4) & 1, L = lane & 15;
  const int col = 32 * blk + 16 * g + 4 * (L & 3);
  auto rd = [&](int h) {
    const int row = 16 * kh + 8 * h + 4 * hf + (L >> 2);
    const char* p = tile + row * kD16Row + (((col >> 3) ^ swz16(row)) << 4) + (col & 7) * 2;
    return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
  };
  const f16x4 lo = rd(0), hi = rd(1);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// ---------------------------------------------------------------------------
// dQ_1, dQ_2: a workgroup owns 128 queries of one (b, h); wave w queries
// 32w .. 32w+31, lane (hf, lq) query lq.  Key tiles stream through LDS:
// K_1, K_2 row-major bf16 (score operands), V row-major fp16 (dP^T operand),
// K_1^T, K_2^T fp16 (dQ^T operands).
constexpr int kDqStage = 2 * kQKTile + kD16Tile + 2 * kQKT;

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) bwd_dq_kernel(BackwardArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kDqStage];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, lq = lane & 31;
  const int nqb = (a.T + kRows - 1) / kRows, BH = a.B * a.H;
  const int qb = nqb - 1 - (int)(blockIdx.x / BH);  // longest rows first
  const int bh = (int)(blockIdx.x % BH), head = bh % a.H, b = bh / a.H;
  const int q_first = qb * kRows + 32 * wave, q = q_first + lq;
  const bool wave_live = q_first < a.T, ok = q < a.T;
  const int ntiles = min(qb * (kRows / 32) + kRows / 32, (a.T + 31) / 32);
  const int kend = min(a.T, ntiles * 32);
  const int last_tile = q_first / 32;

  // Operands held for the whole kernel: Q_m^T (score B operands, bf16) and
  // dO^T (dP^T B operand, fp16), both for this lane's query.
  bf16x8 qa[4], qb2[4];
  f16x8 dot[8];
  const int64_t rq = ((int64_t)b * a.T + q) * a.H + head;
  {
    const uint16_t* p1 = a.q1 + (int64_t)b * a.sq1.b + (int64_t)q * a.sq1.t + (int64_t)head * a.sq1.h + 8 * hf;
    const uint16_t* p2 = a.q2 + (int64_t)b * a.sq2.b + (int64_t)q * a.sq2.t + (int64_t)head * a.sq2.h + 8 * hf;
    const uint16_t* pd = a.dO + rq * kDv + 8 * hf;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qa[s] = ok ? *reinterpret_cast<const bf16x8*>(p1 + 16 * s) : bf16x8{};
      qb2[s] = ok ? *reinterpret_cast<const bf16x8*>(p2 + 16 * s) : bf16x8{};
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) dot[s] = ok ? *reinterpret_cast<const f16x8*>(pd + 16 * s) : f16x8{};
  }
  const float lse1 = ok ? a.lse[rq * 2] : 0.f, lse2 = ok ? a.lse[rq * 2 + 1] : 0.f;
  const float D1 = ok ? a.dstat[rq * 2] : 0.f, D2 = ok ? a.dstat[rq * 2 + 1] : 0.f;
  const float lam = a.lambda_h ? a.lambda_h[head] : a.lambda;
  const float c = a.c;

  const uint16_t* kb1 = a.k1 + (int64_t)b * a.sk1.b + (int64_t)head * a.sk1.h;
  const uint16_t* kb2 = a.k2 + (int64_t)b * a.sk2.b + (int64_t)head * a.sk2.h;
  const uint16_t* vb = a.v + (int64_t)b * a.sv.b + (int64_t)head * a.sv.h;

  f32x16 dq1[2] = {f32x16{}, f32x16{}}, dq2[2] = {f32x16{}, f32x16{}};
  const int ksw = kSwz(lq);

  StagedV sv;
  StagedT sk;
  auto stage_issue = [&](int j, char* st) {
    dma_qk(kb1, kb2, a.sk1.t, a.sk2.t, 32 * j, kend, st, tid);
    load_v(sv, vb, a.sv.t, 32 * j, kend, tid);
    load_qkT(sk, kb1, kb2, a.sk1.t, a.sk2.t, 32 * j, kend, tid);
  };
  auto stage_store = [&](char* st) {
    store_v(sv, st + 2 * kQKTile, tid);
    store_qkT(sk, st + 2 * kQKTile + kD16Tile, tid);
  };
  stage_issue(0, smem);
  stage_store(smem);
  wait_dma();
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    char* cur = smem + (j & 1) * kDqStage;
    char* nxt = smem + ((j + 1) & 1) * kDqStage;
    const bool more = j + 1 < ntiles;
    if (more) stage_issue(j + 1, nxt);
    if (wave_live && j <= last_tile) {
      // S_m^T = K_m Q_m^T (32 keys x 32 queries)
      f32x16 s1 = f32x16{}, s2 = f32x16{};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int off = lq * kKRow + (((2 * s + hf) ^ ksw) << 4);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(cur + off), qa[s], s1, 0, 0, 0);
        s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(cur + kQKTile + off), qb2[s],
                                                     s2, 0, 0, 0);
      }
      // dP^T = V dO^T
      f32x16 dp = f32x16{};
      const char* vt = cur + 2 * kQKTile + lq * kD16Row;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            *reinterpret_cast<const f16x8*>(vt + (((2 * s + hf) ^ swz16(lq)) << 4)), dot[s], dp, 0, 0, 0);
      // P_m^T from the saved log-sum-exp, then dS_m^T; the diagonal tile
      // keeps keys <= query only (register i is key 8(i/4) + 4hf + i%4).
      if (j == last_tile) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i >> 2) + 4 * hf + (i & 3) > lq) s1[i] = s2[i] = -__builtin_inff();  // P = 0, dS = 0
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, -lse1));
        const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[i], c, -lse2));
        s1[i] = p1 * (dp[i] - D1);
        s2[i] = p2 * (-lam * dp[i] - D2);
      }
      f16x8 a0, a1, b0, b1;
      pack16(s1, a0, a1);
      pack16(s2, b0, b1);
      // dQ_m^T += K_m^T dS_m^T
      const char* kt = cur + 2 * kQKTile + kD16Tile;
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        dq1[blk] = mfma_T(kt, blk, lq, hf, a0, a1, dq1[blk]);
        dq2[blk] = mfma_T(kt + kQKT, blk, lq, hf, b0, b1, dq2[blk]);
      }
    }
    if (more) stage_store(nxt);
    wait_dma();
    __syncthreads();
  }
  if (!ok) return;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    store_col(a.dq1 + rq * kDqk, dq1[blk], blk, hf, a.scale);
    store_col(a.dq2 + rq * kDqk, dq2[blk], blk, hf, a.scale);
  }
}

// ---------------------------------------------------------------------------
// dK and dV: a workgroup owns 128 keys of one (b, h); wave w keys 32w ..
// 32w+31, lane (hf, lk) key lk.  Query tiles from the workgroup's diagonal on
// stream through LDS.  Scores are S = Q K^T (32 queries x 32 keys), so the
// accumulator's columns are this lane's key and its rows queries.

// Per-query statistics of a query tile in LDS: [lse_1, lse_2, D_1, D_2][32].
// Rows past T get lse = +inf, so their probabilities are 0.
__device__ __forceinline__ void stage_stats(const BackwardArgs& a, int b, int head, int q0, float* st, int tid) {
  if (tid < 32) {
    const int q = q0 + tid;
    f32x2 l = {__builtin_inff(), __builtin_inff()}, d = {0.f, 0.f};
    if (q < a.T) {
      const int64_t r = ((int64_t)b * a.T + q) * a.H + head;
      l = *reinterpret_cast<const f32x2*>(a.lse + r * 2);
      d = *reinterpret_cast<const f32x2*>(a.dstat + r * 2);
    }
    st[tid] = l.x;
    st[32 + tid] = l.y;
    st[64 + tid] = d.x;
    st[96 + tid] = d.y;
  }
}

// S_m = Q_m K_m^T for one map from a row-major bf16 Q tile.
__device__ __forceinline__ f32x16 scores_qk(const char* qt, const bf16x8 (&kt)[4], int lq, int hf) {
  f32x16 acc = f32x16{};
  const int sw = kSwz(lq);
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        *reinterpret_cast<const bf16x8*>(qt + lq * kKRow + (((2 * s + hf) ^ sw) << 4)), kt[s], acc, 0, 0, 0);
  return acc;
}

// Loads this lane's key row as the score B operand (K_m^T: dims 16s + 8hf ..).
__device__ __forceinline__ void load_krow(bf16x8 (&kt)[4], const uint16_t* base, int64_t stride, int key, bool ok,
                                          int hf) {
  const uint16_t* p = base + (int64_t)key * stride + 8 * hf;
#pragma unroll
  for (int s = 0; s < 4; ++s) kt[s] = ok ? *reinterpret_cast<const bf16x8*>(p + 16 * s) : bf16x8{};
}

// dK and dV in one launch: a workgroup of 8 waves owns 128 keys of one (b, h).
// Waves 0-3 compute dK_1, dK_2 and waves 4-7 dV for the same keys, so each SIMD holds one wave of each kind and every
// query tile is staged once for both: Q_1, Q_2 row-major bf16 and dO
// row-major fp16 by DMA plus Q^T by registers (staged by the dK waves), and
// the per-query statistics (staged by the dV waves, which read dO^T from the
// row-major dO tile by transposed reads).  Each role runs its own copy of the
// loop (same trip count, one barrier per query tile), so its registers are
// allocated for that role alone.
constexpr int kDkvStage = 2 * kQKTile + kD16Tile + 2 * kQKT + 4 * 32 * 4;
constexpr int kOffDo = 2 * kQKTile, kOffQT = kOffDo + kD16Tile, kOffSt = kOffQT + 2 * kQKT;

template <bool kDV>
__device__ __forceinline__ void dkv_role(const BackwardArgs& a, char* smem, int tid) {
  const int rt = tid & 255;                                   // thread within its role
  const int rw = __builtin_amdgcn_readfirstlane(rt >> 6);     // wave within its role
  const int lane = tid & 63, hf = lane >> 5, lk = lane & 31;
  const int BH = a.B * a.H;
  const int kb = (int)(blockIdx.x / BH);  // longest column blocks first
  const int bh = (int)(blockIdx.x % BH), head = bh % a.H, b = bh / a.H;
  const int k_first = kb * kRows + 32 * rw, key = k_first + lk;
  const bool wave_live = k_first < a.T, ok = key < a.T;
  const int nqt = (a.T + 31) / 32, qt0 = kb * (kRows / 32);
  const int diag = k_first / 32;  // this wave's first (diagonal) query tile

  bf16x8 k1t[4], k2t[4];
  load_krow(k1t, a.k1 + (int64_t)b * a.sk1.b + (int64_t)head * a.sk1.h, a.sk1.t, key, ok, hf);
  load_krow(k2t, a.k2 + (int64_t)b * a.sk2.b + (int64_t)head * a.sk2.h, a.sk2.t, key, ok, hf);
  f16x8 vt[kDV ? 1 : 8];
  if constexpr (!kDV) {
    const uint16_t* p = a.v + (int64_t)b * a.sv.b + (int64_t)key * a.sv.t + (int64_t)head * a.sv.h + 8 * hf;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const u32x4 w = ok ? *reinterpret_cast<const u32x4*>(p + 16 * s) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        vt[s][2 * i] = (_Float16)bf16_lo(w[i]);
        vt[s][2 * i + 1] = (_Float16)bf16_hi(w[i]);
      }
    }
  }
  const float lam = a.lambda_h ? a.lambda_h[head] : a.lambda;
  const float c = a.c;
  const uint16_t* qb1 = a.q1 + (int64_t)b * a.sq1.b + (int64_t)head * a.sq1.h;
  const uint16_t* qb2 = a.q2 + (int64_t)b * a.sq2.b + (int64_t)head * a.sq2.h;
  const uint16_t* dob = a.dO + (int64_t)b * a.T * a.H * kDv + (int64_t)head * kDv;
  const int64_t sdo = (int64_t)a.H * kDv;

  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};  // dK_1 (0, 1), dK_2 (2, 3) or dV^T (0 .. 3)
  StagedT sq;
  auto stage_issue = [&](int qt, char* st) {
    if constexpr (!kDV) {
      dma_qk(qb1, qb2, a.sq1.t, a.sq2.t, 32 * qt, a.T, st, rt);
      dma_do(dob, sdo, 32 * qt, a.T, st + kOffDo, rt);
      load_qkT(sq, qb1, qb2, a.sq1.t, a.sq2.t, 32 * qt, a.T, rt);
    }
  };
  auto stage_store = [&](int qt, char* st) {
    if constexpr (!kDV)
      store_qkT(sq, st + kOffQT, rt);
    else
      stage_stats(a, b, head, 32 * qt, reinterpret_cast<float*>(st + kOffSt), rt);
  };
  if (qt0 < nqt) {
    stage_issue(qt0, smem);
    stage_store(qt0, smem);
  }
  wait_dma();
  __syncthreads();

  for (int qt = qt0; qt < nqt; ++qt) {
    const int it = qt - qt0;
    char* cur = smem + (it & 1) * kDkvStage;
    char* nxt = smem + ((it + 1) & 1) * kDkvStage;
    const bool more = qt + 1 < nqt;
    if (more) stage_issue(qt + 1, nxt);
    if (wave_live && qt >= diag) {
      f32x16 s1 = scores_qk(cur, k1t, lk, hf);
      f32x16 s2 = scores_qk(cur + kQKTile, k2t, lk, hf);
      const float* stats = reinterpret_cast<const float*>(cur + kOffSt);
      if (qt == diag) {  // rows are queries 8(i/4) + 4hf + i%4 of the tile, the column key lk
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (lk > 8 * (i >> 2) + 4 * hf + (i & 3)) s1[i] = s2[i] = -__builtin_inff();  // P = 0
      }
      if constexpr (!kDV) {
        // dP = dO V^T (32 queries x 32 keys)
        f32x16 dp = f32x16{};
        const char* dt = cur + kOffDo + lk * kD16Row;
#pragma unroll
        for (int s = 0; s < 8; ++s)
          dp = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              *reinterpret_cast<const f16x8*>(dt + (((2 * s + hf) ^ swz16(lk)) << 4)), vt[s], dp, 0, 0, 0);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r0 = 8 * g + 4 * hf;
          const f32x4 l1 = *reinterpret_cast<const f32x4*>(stats + r0);
          const f32x4 l2 = *reinterpret_cast<const f32x4*>(stats + 32 + r0);
          const f32x4 d1 = *reinterpret_cast<const f32x4*>(stats + 64 + r0);
          const f32x4 d2 = *reinterpret_cast<const f32x4*>(stats + 96 + r0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * g + r;
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, -l1[r]));
            const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[i], c, -l2[r]));
            s1[i] = p1 * (dp[i] - d1[r]);
            s2[i] = p2 * (-lam * dp[i] - d2[r]);
          }
        }
        f16x8 a0, a1, b0, b1;
        pack16(s1, a0, a1);
        pack16(s2, b0, b1);
        // dK_m^T += Q_m^T dS_m
        const char* qtT = cur + kOffQT;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
          acc[blk] = mfma_T(qtT, blk, lk, hf, a0, a1, acc[blk]);
          acc[2 + blk] = mfma_T(qtT + kQKT, blk, lk, hf, b0, b1, acc[2 + blk]);
        }
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r0 = 8 * g + 4 * hf;
          const f32x4 l1 = *reinterpret_cast<const f32x4*>(stats + r0);
          const f32x4 l2 = *reinterpret_cast<const f32x4*>(stats + 32 + r0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * g + r;
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, -l1[r]));
            const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[i], c, -l2[r]));
            s1[i] = p1 - lam * p2;
          }
        }
        f16x8 p0, p1;
        pack16(s1, p0, p1);
        // dV^T += dO^T (P_1 - lambda P_2), dO^T read transposed from the dO tile
        const char* dt = cur + kOffDo;
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) {
          acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(tr_operand(dt, blk, 0, lane), p0, acc[blk], 0, 0, 0);
          acc[blk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(tr_operand(dt, blk, 1, lane), p1, acc[blk], 0, 0, 0);
        }
      }
    }
    if (more) stage_store(qt + 1, nxt);
    wait_dma();
    __syncthreads();
  }
  if (!ok) return;
  const int64_t rk = ((int64_t)b * a.T + key) * a.H + head;
  if constexpr (!kDV) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      store_col(a.dk1 + rk * kDqk, acc[blk], blk, hf, a.scale);
      store_col(a.dk2 + rk * kDqk, acc[2 + blk], blk, hf, a.scale);
    }
  } else {
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) store_col(a.dv + rk * kDv, acc[blk], blk, hf, 1.0f);
  }
}

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) bwd_dkv_kernel(BackwardArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kDkvStage];
  const int tid = threadIdx.x;
  if (__builtin_amdgcn_readfirstlane(tid >> 6) >= kWaves)
    dkv_role<true>(a, smem, tid);
  else
    dkv_role<false>(a, smem, tid);
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(bwd_pre_kernel, dim3((unsigned)a.nchunks, (unsigned)a.H), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)a.H), dim3(192), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t blocks = (int64_t)((a.T + kRows - 1) / kRows) * a.B * a.H;
  hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dkv_kernel, dim3((unsigned)blocks), dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace diffattn
