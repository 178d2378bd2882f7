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
//   bwd_pre_kernel     per row: do (fp16), D_1, D_2; gain/lambda partials; the
//                      fp16 copies of Q_1, Q_2, K_1, K_2, V in the workspace
//   bwd_reduce_kernel  per head: sum of the partials
//   bwd_dq_kernel      queries own lanes (the forward's orientation): recompute
//                      S^T, P^T from the saved log-sum-exp, dP^T = V dO^T,
//                      dQ^T += K^T dS^T
//   bwd_dkv_kernel     keys own lanes, two kinds of waves on the same keys and
//                      query tiles: S = Q K^T, dP = dO V^T, dK^T += Q^T dS;
//                      and S = Q K^T, dV^T += dO^T (P_1 - lambda P_2)
// The last two use v_mfma_f32_32x32x16_f16 like the prefill: a 32x32
// accumulator held by a wave is used directly as the next product's operand.
// Every tile is a row-major fp16 tile moved by DMA; the transposed operands
// (K^T, Q^T, dO^T) come from the same tiles by ds_read_b64_tr_b16, with
// addresses chosen so that their k order matches the accumulator's rows.  All
// inputs enter the products as fp16 (bf16 converted exactly for |x| in
// [2^-14, 65504)), so the scores are the same products of the inputs as the
// forward's bf16 ones; P, dS and dO are rounded to fp16; fp32 accumulation.
#include "kernels.h"
#include "rope.h"
#include "tile.h"

namespace diffattn {
namespace {

constexpr int kWaves = 4;
constexpr int kRows = 32 * kWaves;      // queries (dQ) or keys (dK, dV) per workgroup
constexpr int kKRow = kDqk * 2;         // 128-byte fp16 rows of Q or K
constexpr int kQKTile = 32 * kKRow;     // 4 KiB: one map's 32-row fp16 tile
constexpr int kD16Row = kDv * 2;        // 256-byte fp16 rows of dO or V
constexpr int kD16Tile = 32 * kD16Row;  // 8 KiB

// 16-byte chunk swizzles of the tiles' rows, logical chunk c of row r stored
// at chunk c ^ swz(r).  Two kinds of reads must be conflict-free on 64 banks:
// a 16-byte read by lanes of consecutive rows at one logical chunk (row-major
// operands), and a transposed 8-byte read (ds_read_b64_tr_b16) whose 32
// lanes of a pass cover four consecutive rows 4m .. 4m+3 and four chunks of
// one aligned group.  256-byte rows (16 chunks; every row spans all banks):
// swz16 is a bijection on r % 16 for the first, and gives rows 4m .. 4m+3
// different chunk groups for the second.  128-byte rows (8 chunks; rows r and
// r + 1 share the banks' halves): swz8 takes 8 distinct values over the even
// rows and over the odd rows of 16 consecutive ones, and rows 4m and 4m + 2
// differ in its group bit.
__device__ __forceinline__ int swz16(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
__device__ __forceinline__ int swz8(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// ---------------------------------------------------------------------------
// Per row: the GroupNorm backward, do, D_1 = rowsum(do O_1),
// D_2 = rowsum(-lambda do O_2), partial sums of dgain and dlambda over a
// chunk of kBwdRowsPerChunk rows of one head, and the row's fp16 input copies.  Sixteen lanes per row (eight
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
  __shared__ uint64_t rope_tab[32];
  if (a.rope.mode != 0) {
    if (threadIdx.x < 32) rope_tab[threadIdx.x] = rope_phase_at(a.rope, (int)threadIdx.x);
    __syncthreads();
  }
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
    // fp16 copies of this row's inputs for the product kernels (exact for |x|
    // in [2^-14, 65504), like every fp16 operand of the products): V's eight
    // channels 8li.., and two 8-dim chunks of Q_1, Q_2, K_1 or K_2 (tensor
    // li / 4, chunks li % 4 and li % 4 + 4).
    {
      const int bb = rbt / a.T, tt = rbt - bb * a.T;
      const int64_t row = (int64_t)rbt * a.H + h;
      const int m = li >> 2, c0 = li & 3;
      const uint16_t* base = m == 0 ? a.q1 : m == 1 ? a.q2 : m == 2 ? a.k1 : a.k2;
      const Strides& st = m == 0 ? a.sq1 : m == 1 ? a.sq2 : m == 2 ? a.sk1 : a.sk2;
      uint16_t* dst = m == 0 ? a.q1h : m == 1 ? a.q2h : m == 2 ? a.k1h : a.k2h;
      const uint16_t* src = base + (int64_t)bb * st.b + (int64_t)tt * st.t + (int64_t)h * st.h;
      const uint16_t* vsrc = a.v + (int64_t)bb * a.sv.b + (int64_t)tt * a.sv.t + (int64_t)h * a.sv.h + 8 * li;
      const u32x4 w0 = *reinterpret_cast<const u32x4*>(src + 8 * c0);
      const u32x4 w1 = *reinterpret_cast<const u32x4*>(src + 8 * (c0 + 4));
      const u32x4 wv = *reinterpret_cast<const u32x4*>(vsrc);
      float x0[8], x1[8];
      rope_unpack(w0, x0);
      rope_unpack(w1, x1);
      if (a.rope.mode != 0) {
        // The rotary embedding at position pos0 + t, in fp32 with the
        // forward's arithmetic (each pair (u, w) -> (u cos - w sin,
        // u sin + w cos)), then rounded to fp16 like the forward's rotated
        // score operands: chunk c0 pairs with chunk c0 + 4 in split-half
        // mode, each chunk with itself in interleaved mode.
        const uint32_t pos = a.rope.pos0 + (uint32_t)tt;
        auto turn = [&](float& u, float& w, int pair) __attribute__((always_inline)) {
          float cs, sn;
          rope_cos_sin(pos, rope_tab[pair], cs, sn);
          const float uu = u, ww = w;
          u = uu * cs - ww * sn;
          w = uu * sn + ww * cs;
        };
        if (a.rope.mode == 1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) turn(x0[e], x1[e], 8 * c0 + e);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            turn(x0[2 * i], x0[2 * i + 1], 4 * c0 + i);
            turn(x1[2 * i], x1[2 * i + 1], 4 * (c0 + 4) + i);
          }
        }
      }
      f16x8 h0, h1, hv8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        h0[i] = (_Float16)x0[i];
        h1[i] = (_Float16)x1[i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hv8[2 * i] = (_Float16)bf16_lo(wv[i]);
        hv8[2 * i + 1] = (_Float16)bf16_hi(wv[i]);
      }
      *reinterpret_cast<f16x8*>(dst + row * kDqk + 8 * c0) = h0;
      *reinterpret_cast<f16x8*>(dst + row * kDqk + 8 * (c0 + 4)) = h1;
      *reinterpret_cast<f16x8*>(a.vh + row * kDv + 8 * li) = hv8;
    }
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

// Row-major fp16 tiles of both maps (Q or K) by DMA into [map][32][128 B]
// with the swz8 chunk swizzle: thread t fetches row t/8, logical chunk
// (t % 8) ^ swz8(t / 8), landing at chunk position t.
__device__ __forceinline__ void dma_qk(const uint16_t* b1, const uint16_t* b2, int64_t st1, int64_t st2, int r0,
                                       int end, char* dst, int tid) {
  const int r = tid >> 3, c = (tid & 7) ^ swz8(r);
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

// Packs a 32x32 accumulator (16 values per lane) as the two fp16 operands of
// the next product's k-steps: registers 0..7, then 8..15.
__device__ __forceinline__ void pack16(const f32x16& v, f16x8& p0, f16x8& p1) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p0[j] = (_Float16)v[j];
    p1[j] = (_Float16)v[8 + j];
  }
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

// The transposed operand of a row-major fp16 tile of 32 rows (kRowBytes-byte
// rows: 256 with the swz16 chunk swizzle, 128 with swz8) by
// ds_read_b64_tr_b16, which hands lane i of each 16-lane group element i % 4
// of the 8-byte reads of lanes 4k + i / 4, k = 0..3.  For column block blk
// and k-half kh, lane (hf, g, L) (g: 16-lane group within the half, L: lane
// within it) reads 4 columns 32blk + 16g + 4(L % 4) .. +3 of row 16kh + 8h +
// 4hf + L / 4 for h = 0, 1, so it receives column 32blk + 16g + L of rows
// 16kh + 8(j / 4) + 4hf + j % 4, j = 0..7: the A operand of a product whose B
// operand is a 32x32 accumulator packed by pack16 (rows in the accumulator's
// order).
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int kRowBytes>
__device__ __forceinline__ f16x8 tr_operand(const char* tile, int blk, int kh, int lane) {
  const int hf = lane >> 5, g = (lane >> 4) & 1, L = lane & 15;
  const int col = 32 * blk + 16 * g + 4 * (L & 3);
  auto rd = [&](int h) {
    const int row = 16 * kh + 8 * h + 4 * hf + (L >> 2);
    const int sw = kRowBytes == 256 ? swz16(row) : swz8(row);
    const char* p = tile + row * kRowBytes + (((col >> 3) ^ sw) << 4) + (col & 7) * 2;
    return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p));
  };
  const f16x4 lo = rd(0), hi = rd(1);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// acc += T^T P for column block blk of a row-major tile T (32 rows): the two
// k-halves of the product, P packed by pack16.
template <int kRowBytes>
__device__ __forceinline__ f32x16 mfma_tr(const char* tile, int blk, int lane, const f16x8& p0, const f16x8& p1,
                                          f32x16 acc) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(tr_operand<kRowBytes>(tile, blk, 0, lane), p0, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(tr_operand<kRowBytes>(tile, blk, 1, lane), p1, acc, 0, 0, 0);
}

// The gradient of an unrotated query or key from that of its rotated copy
// (the rotary embedding R at the row's position pos is orthogonal, so the
// gradient is R^T times it): each pair (g_u, g_w) -> (g_u cos + g_w sin,
// -g_u sin + g_w cos), in fp32.  g0, g1 hold dims 8 (i / 4) + 4 hf + i % 4
// and 32 more in register i, so both members of every pair are in the lane.
__device__ __forceinline__ void unrotate_grad(f32x16& g0, f32x16& g1, int hf, uint32_t pos, const RopeArgs& r) {
  // pair (u, w) = (x[iu], y[iw])
  auto turn_back = [&](f32x16& x, int iu, f32x16& y, int iw, uint64_t phase) __attribute__((always_inline)) {
    float cs, sn;
    rope_cos_sin(pos, phase, cs, sn);
    const float u = x[iu], w = y[iw];
    x[iu] = u * cs + w * sn;
    y[iw] = w * cs - u * sn;
  };
  if (r.mode == 1) {
    // pair c = dims c, c + 32 (c = 8 r4 + 4 hf + e)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        turn_back(g0, 4 * r4 + e, g1, 4 * r4 + e, hf ? r.phase[8 * r4 + 4 + e] : r.phase[8 * r4 + e]);
  } else {
    // pair c = dims 2c, 2c + 1 (2c = 32 blk + 8 r4 + 4 hf + 2 e)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int c0 = 4 * r4 + e;
        turn_back(g0, 4 * r4 + 2 * e, g0, 4 * r4 + 2 * e + 1, hf ? r.phase[c0 + 2] : r.phase[c0]);
        turn_back(g1, 4 * r4 + 2 * e, g1, 4 * r4 + 2 * e + 1, hf ? r.phase[16 + c0 + 2] : r.phase[16 + c0]);
      }
  }
}

// ---------------------------------------------------------------------------
// dQ_1, dQ_2: 128 queries of one (b, h) per work item; wave w of a group
// queries 32w .. 32w+31, lane (hf, lq) query lq.  Two groups of four waves
// take alternate key tiles of the same queries and add their dQ at the end.
// Key tiles of the fp16 copies stream through LDS by DMA alone: K_1, K_2
// (score operands, and K^T by transposed reads for dQ^T) and V (dP^T
// operand), all row-major.  Workgroup r * B*H + bh runs the items of rows r
// and nqb - 1 - r (longest-first order) of (b, h) = bh back to back, so every
// workgroup carries the same number of key tiles.
constexpr int kDqTile = 2 * kQKTile + kD16Tile;  // one group's key tile
constexpr int kDqStage = 2 * kDqTile;             // one step: a tile for each group
static_assert(4 * 64 * 64 * 4 <= 2 * kDqStage, "the dQ merge must fit in the stages");

__device__ __forceinline__ void dq_item(const BackwardArgs& a, char* smem, int item) {
  const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, lq = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2, wq = wave & 3, rt = tid & 255;
  const int nqb = (a.T + kRows - 1) / kRows, BH = a.B * a.H;
  const int qb = nqb - 1 - item / BH;
  const int bh = item % BH, head = bh % a.H, b = bh / a.H;
  const int q_first = qb * kRows + 32 * wq, q = q_first + lq;
  const bool wave_live = q_first < a.T, ok = q < a.T;
  const int ntiles = min(qb * (kRows / 32) + kRows / 32, (a.T + 31) / 32);
  const int kend = min(a.T, ntiles * 32);
  const int last_tile = q_first / 32;
  // With a sliding window, the key tiles below every query's window are
  // skipped (the forward's tile range).
  const int W = a.window;
  const int tile0 = W > 0 ? max(0, qb * kRows - W + 1) / 32 : 0;
  const int first_tile = W > 0 ? max(0, q_first - W + 1) / 32 : 0;
  const int nsteps = (ntiles - tile0 + 1) / 2;

  // Operands held for the whole item: Q_m^T (score B operands) and dO^T
  // (dP^T B operand), fp16, both for this lane's query.
  f16x8 qa[4], qb2[4];
  f16x8 dot[8];
  const int64_t rq = ((int64_t)b * a.T + q) * a.H + head;
  {
    const uint16_t* p1 = a.q1h + rq * kDqk + 8 * hf;
    const uint16_t* p2 = a.q2h + rq * kDqk + 8 * hf;
    const uint16_t* pd = a.dO + rq * kDv + 8 * hf;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qa[s] = ok ? *reinterpret_cast<const f16x8*>(p1 + 16 * s) : f16x8{};
      qb2[s] = ok ? *reinterpret_cast<const f16x8*>(p2 + 16 * s) : f16x8{};
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) dot[s] = ok ? *reinterpret_cast<const f16x8*>(pd + 16 * s) : f16x8{};
  }
  const float lse1 = ok ? a.lse[rq * 2] : 0.f, lse2 = ok ? a.lse[rq * 2 + 1] : 0.f;
  const float D1 = ok ? a.dstat[rq * 2] : 0.f, D2 = ok ? a.dstat[rq * 2 + 1] : 0.f;
  const float lam = a.lambda_h ? a.lambda_h[head] : a.lambda;
  const float c = a.c;

  const int64_t row0 = (int64_t)b * a.T * a.H + head;  // (b, t = 0, head)
  const uint16_t* kb1 = a.k1h + row0 * kDqk;
  const uint16_t* kb2 = a.k2h + row0 * kDqk;
  const uint16_t* vb = a.vh + row0 * kDv;
  const int64_t sk = (int64_t)a.H * kDqk, sv = (int64_t)a.H * kDv;

  f32x16 dq1[2] = {f32x16{}, f32x16{}}, dq2[2] = {f32x16{}, f32x16{}};
  const int ksw = swz8(lq);

  // Each group stages its own tile of the step (tile 2 it + grp; past the
  // last tile the rows read as zero).
  auto stage_issue = [&](int it, char* st) {
    const int j = tile0 + 2 * it + grp;
    char* t = st + grp * kDqTile;
    dma_qk(kb1, kb2, sk, sk, 32 * j, kend, t, rt);
    dma_do(vb, sv, 32 * j, kend, t + 2 * kQKTile, rt);
  };
  stage_issue(0, smem);
  wait_dma();
  __syncthreads();

  for (int it = 0; it < nsteps; ++it) {
    char* cur = smem + (it & 1) * kDqStage + grp * kDqTile;
    const int j = tile0 + 2 * it + grp;
    const bool act = wave_live && j >= first_tile && j <= last_tile;
    // K_m^T operands of the dQ products, read transposed before the next
    // tile's DMA goes out: the compiler orders transposed LDS reads behind
    // every LDS DMA in flight, which would make these products wait for the
    // prefetch.
    f16x8 kt1[2][2], kt2[2][2];
    if (act) {
#pragma unroll
      for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          kt1[blk][kh] = tr_operand<kKRow>(cur, blk, kh, lane);
          kt2[blk][kh] = tr_operand<kKRow>(cur + kQKTile, blk, kh, lane);
        }
    }
    if (it + 1 < nsteps) stage_issue(it + 1, smem + ((it + 1) & 1) * kDqStage);
    if (act) {
      // S_m^T = K_m Q_m^T (32 keys x 32 queries)
      f32x16 s1 = f32x16{}, s2 = f32x16{};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int off = lq * kKRow + (((2 * s + hf) ^ ksw) << 4);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*reinterpret_cast<const f16x8*>(cur + off), qa[s], s1, 0, 0, 0);
        s2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(*reinterpret_cast<const f16x8*>(cur + kQKTile + off), qb2[s], s2,
                                                    0, 0, 0);
      }
      // dP^T = V dO^T
      f32x16 dp = f32x16{};
      const char* vt = cur + 2 * kQKTile + lq * kD16Row;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        dp = __builtin_amdgcn_mfma_f32_32x32x16_f16(
            *reinterpret_cast<const f16x8*>(vt + (((2 * s + hf) ^ swz16(lq)) << 4)), dot[s], dp, 0, 0, 0);
      // P_m^T from the saved log-sum-exp, then dS_m^T; on the diagonal tile the
      // keys past the query (register i is key 8(i/4) + 4hf + i%4) get P = 0.
      if (j == last_tile) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i >> 2) + 4 * hf + (i & 3) > lq) s1[i] = s2[i] = -__builtin_inff();  // P = 0, dS = 0
      }
      if (W > 0 && 32 * j < q_first + 32 - W) {
        // lower window edge: key 32 j + kr is visible to query q iff it is > q - W
        const int lim = q - W - 32 * j;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i >> 2) + 4 * hf + (i & 3) <= lim) s1[i] = s2[i] = -__builtin_inff();
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
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        dq1[blk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kt1[blk][0], a0, dq1[blk], 0, 0, 0);
        dq1[blk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kt1[blk][1], a1, dq1[blk], 0, 0, 0);
        dq2[blk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kt2[blk][0], b0, dq2[blk], 0, 0, 0);
        dq2[blk] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kt2[blk][1], b1, dq2[blk], 0, 0, 0);
      }
    }
    wait_dma();
    __syncthreads();
  }
  // Group 1's sums through LDS (the stages are free after the last barrier),
  // added to group 0's in a fixed order: group 0's partial + group 1's.
  float* mo = reinterpret_cast<float*>(smem);
  auto slot = [&](int k, int i) { return ((wq * 64) + k * 16 + i) * 64 + lane; };
  if (grp == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      mo[slot(0, i)] = dq1[0][i];
      mo[slot(1, i)] = dq1[1][i];
      mo[slot(2, i)] = dq2[0][i];
      mo[slot(3, i)] = dq2[1][i];
    }
  }
  __syncthreads();
  if (grp == 0 && ok) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dq1[0][i] += mo[slot(0, i)];
      dq1[1][i] += mo[slot(1, i)];
      dq2[0][i] += mo[slot(2, i)];
      dq2[1][i] += mo[slot(3, i)];
    }
    if (a.rope.mode != 0) {
      const uint32_t pos = a.rope.pos0 + (uint32_t)q;
      unrotate_grad(dq1[0], dq1[1], hf, pos, a.rope);
      unrotate_grad(dq2[0], dq2[1], hf, pos, a.rope);
    }
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      store_col(a.dq1 + rq * kDqk, dq1[blk], blk, hf, a.scale);
      store_col(a.dq2 + rq * kDqk, dq2[blk], blk, hf, a.scale);
    }
  }
}

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) bwd_dq_kernel(BackwardArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[2 * kDqStage];
  const int BH = a.B * a.H;
  const int nqb = (a.T + kRows - 1) / kRows;
  const int r = (int)blockIdx.x / BH, bh = (int)blockIdx.x % BH;
  dq_item(a, smem, (int)blockIdx.x);
  if (nqb - 1 - r > r) {
    __syncthreads();  // the first item's merge is done with LDS
    dq_item(a, smem, (nqb - 1 - r) * BH + bh);
  }
}

// ---------------------------------------------------------------------------
// dK and dV: a workgroup owns 128 keys of one (b, h); wave w keys 32w ..
// 32w+31, lane (hf, lk) key lk.  Query tiles from the workgroup's diagonal on
// stream through LDS.  Scores are S = Q K^T (32 queries x 32 keys), so the
// accumulator's columns are this lane's key and its rows queries.

// Per-query statistics of a query tile in LDS: [lse_1, lse_2, D_1, D_2][32],
// in two parts: threads 0..31 load their query's values into registers (at
// the start of a step, so the loads run under its products), then store them
// (at its end).  Rows past T get lse = +inf, so their probabilities are 0.
struct QueryStats {
  f32x2 l, d;
};
__device__ __forceinline__ QueryStats load_stats(const BackwardArgs& a, int b, int head, int q0, int tid) {
  QueryStats r{{__builtin_inff(), __builtin_inff()}, {0.f, 0.f}};
  const int q = q0 + tid;
  if (tid < 32 && q < a.T) {
    const int64_t row = ((int64_t)b * a.T + q) * a.H + head;
    r.l = *reinterpret_cast<const f32x2*>(a.lse + row * 2);
    r.d = *reinterpret_cast<const f32x2*>(a.dstat + row * 2);
  }
  return r;
}
__device__ __forceinline__ void store_stats(const QueryStats& v, float* st, int tid) {
  if (tid < 32) {
    st[tid] = v.l.x;
    st[32 + tid] = v.l.y;
    st[64 + tid] = v.d.x;
    st[96 + tid] = v.d.y;
  }
}

// S_m = Q_m K_m^T for one map from a row-major fp16 Q tile.
__device__ __forceinline__ f32x16 scores_qk(const char* qt, const f16x8 (&kt)[4], int lq, int hf) {
  f32x16 acc = f32x16{};
  const int sw = swz8(lq);
#pragma unroll
  for (int s = 0; s < 4; ++s)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(
        *reinterpret_cast<const f16x8*>(qt + lq * kKRow + (((2 * s + hf) ^ sw) << 4)), kt[s], acc, 0, 0, 0);
  return acc;
}

// Loads 16-dim chunks 16s + 8hf .. of a row of an fp16 copy (row `row` of
// the [B, T, H, d] layout) as operands.
template <int kN>
__device__ __forceinline__ void load_row16(f16x8 (&r)[kN], const uint16_t* base, int64_t row, bool ok, int hf) {
  const uint16_t* p = base + row * (16 * kN) + 8 * hf;
#pragma unroll
  for (int s = 0; s < kN; ++s) r[s] = ok ? *reinterpret_cast<const f16x8*>(p + 16 * s) : f16x8{};
}

// dK and dV in one launch: a workgroup of 8 waves owns 128 keys of one (b, h).
// Waves 0-3 compute dK_1, dK_2 and waves 4-7 dV for the same keys, so each
// SIMD holds one wave of each kind and every query tile is staged once for
// both: Q_1, Q_2 and dO row-major fp16 by DMA (issued by the dK waves; Q^T and
// dO^T come from the same tiles by transposed reads) and the per-query
// statistics (stored by the dV waves).  The dV wave of a tile computes the
// scores and both maps' probabilities, takes P_1 - lambda P_2 for dV and
// leaves P_1 and P_2 (fp32) in the tile's stage; the dK wave of the same keys
// takes them one step later, with dP = dO V^T, for dS and dK.  Each kind then
// carries 16 products per tile.  Three stages keep a tile staged for the step
// after its own.  Each role runs its own copy of the loop (same trip count, one barrier
// per query tile), so its registers are allocated for that role alone.
// A stage: Q_1, Q_2, dO, the statistics, then the tile's P_1, P_2 as the dV
// waves leave them ([dK wave][f32x4 index 0..7][lane]).
constexpr int kDkvP = 4 * 8 * 64 * 16;
constexpr int kDkvStage = 2 * kQKTile + kD16Tile + 4 * 32 * 4 + kDkvP;
constexpr int kOffDo = 2 * kQKTile, kOffSt = kOffDo + kD16Tile, kOffP = kOffSt + 4 * 32 * 4;

template <bool kDV>
__device__ __forceinline__ void dkv_role(const BackwardArgs& a, char* stage0, char* stage1, char* stage2, int tid) {
  const int rt = tid & 255;                                   // thread within its role
  const int rw = __builtin_amdgcn_readfirstlane(rt >> 6);     // wave within its role
  const int lane = tid & 63, hf = lane >> 5, lk = lane & 31;
  const int BH = a.B * a.H;
  const int kb = (int)(blockIdx.x / BH);  // longest column blocks first
  const int bh = (int)(blockIdx.x % BH), head = bh % a.H, b = bh / a.H;
  const int k_first = kb * kRows + 32 * rw, key = k_first + lk;
  const bool wave_live = k_first < a.T, ok = key < a.T;
  const int qt0 = kb * (kRows / 32);
  const int diag = k_first / 32;  // this wave's first (diagonal) query tile
  // With a sliding window of W keys, query q sees key k iff q < k + W: the
  // query tiles past the last that sees one of the workgroup's keys are
  // skipped, and a wave stops at the last tile that sees one of its own.
  const int W = a.window;
  const int nqt = W > 0 ? min((a.T + 31) / 32, (kb * kRows + kRows - 1 + W - 1) / 32 + 1) : (a.T + 31) / 32;
  const int wave_last = W > 0 ? (k_first + 31 + W - 1) / 32 : nqt - 1;
  auto live = [&](int qt) { return wave_live && qt >= diag && qt <= wave_last; };

  const int64_t rk = ((int64_t)b * a.T + key) * a.H + head;
  f16x8 k1t[kDV ? 4 : 1], k2t[kDV ? 4 : 1], vt[kDV ? 1 : 8];
  if constexpr (kDV) {
    load_row16(k1t, a.k1h, rk, ok, hf);
    load_row16(k2t, a.k2h, rk, ok, hf);
  } else {
    load_row16(vt, a.vh, rk, ok, hf);
  }
  const float lam = a.lambda_h ? a.lambda_h[head] : a.lambda;
  const float c = a.c;
  const int64_t row0 = (int64_t)b * a.T * a.H + head;  // (b, t = 0, head)
  const uint16_t* qb1 = a.q1h + row0 * kDqk;
  const uint16_t* qb2 = a.q2h + row0 * kDqk;
  const uint16_t* dob = a.dO + row0 * kDv;
  const int64_t sq = (int64_t)a.H * kDqk, sdo = (int64_t)a.H * kDv;
  auto pslot = [&](char* st, int j) { return reinterpret_cast<f32x4*>(st + kOffP) + (rw * 8 + j) * 64 + lane; };

  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};  // dK_1 (0, 1), dK_2 (2, 3) or dV^T (0 .. 3)
  auto stage_issue = [&](int qt, char* st) {
    if constexpr (!kDV) {
      dma_qk(qb1, qb2, sq, sq, 32 * qt, a.T, st, rt);
      dma_do(dob, sdo, 32 * qt, a.T, st + kOffDo, rt);
    }
  };
  QueryStats nst;  // the next tile's statistics (dV role), loaded at the start of a step
  auto stats_load = [&](int qt) {
    if constexpr (kDV) nst = load_stats(a, b, head, 32 * qt, rt);
  };
  auto stats_store = [&](char* st) {
    if constexpr (kDV) store_stats(nst, reinterpret_cast<float*>(st + kOffSt), rt);
  };
  // dK wave, in this order within a step, so that its vector work comes while
  // the dV wave of its SIMD runs the score products and its products while
  // that wave computes the exponentials: dS of the previous tile (from the P
  // the dV wave left in its stage and the dP computed a step ago), then
  // dK += Q^T dS of the previous tile and dP = dO V^T of the current one.
  f32x16 dp;               // dP of the last tile this wave computed it for
  f16x8 a0, a1, b0, b1;    // dS_1, dS_2 of the previous tile, as fp16 operands
  auto dk_ds = [&](const char* st) __attribute__((always_inline)) {
    const float* stats = reinterpret_cast<const float*>(st + kOffSt);
    f32x16 p1, p2;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 x = *pslot(const_cast<char*>(st), g), y = *pslot(const_cast<char*>(st), 4 + g);
      const int r0 = 8 * g + 4 * hf;
      const f32x4 d1 = *reinterpret_cast<const f32x4*>(stats + 64 + r0);
      const f32x4 d2 = *reinterpret_cast<const f32x4*>(stats + 96 + r0);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * g + r;
        p1[i] = x[r] * (dp[i] - d1[r]);
        p2[i] = y[r] * (-lam * dp[i] - d2[r]);
      }
    }
    pack16(p1, a0, a1);
    pack16(p2, b0, b1);
  };
  auto dk_products = [&](const char* st) __attribute__((always_inline)) {
    // dK_m^T += Q_m^T dS_m, Q_m^T read transposed from the query tiles
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      acc[blk] = mfma_tr<kKRow>(st, blk, lane, a0, a1, acc[blk]);
      acc[2 + blk] = mfma_tr<kKRow>(st + kQKTile, blk, lane, b0, b1, acc[2 + blk]);
    }
  };
  auto dk_dp = [&](const char* st) __attribute__((always_inline)) {
    // dP = dO V^T (32 queries x 32 keys)
    dp = f32x16{};
    const char* dt = st + kOffDo + lk * kD16Row;
#pragma unroll
    for (int s = 0; s < 8; ++s)
      dp = __builtin_amdgcn_mfma_f32_32x32x16_f16(*reinterpret_cast<const f16x8*>(dt + (((2 * s + hf) ^ swz16(lk)) << 4)),
                                                  vt[s], dp, 0, 0, 0);
  };
  if (qt0 < nqt) {
    stage_issue(qt0, stage0);
    stats_load(qt0);
    stats_store(stage0);
  }
  wait_dma();
  __syncthreads();

  // The three stages are separate LDS objects and the loop is unrolled by
  // three, so every step names the stage it reads, the one the next tile's
  // DMA fills and the previous tile's (the compiler then adds no wait for a
  // DMA into another object before the transposed reads).
  auto step = [&](int qt, char* cur, char* nxt, char* prev) __attribute__((always_inline)) {
    const bool more = qt + 1 < nqt;
    if (more) {
      stage_issue(qt + 1, nxt);
      stats_load(qt + 1);
    }
    if constexpr (kDV) {
      if (qt < nqt && live(qt)) {
        f32x16 s1 = scores_qk(cur, k1t, lk, hf);
        f32x16 s2 = scores_qk(cur + kQKTile, k2t, lk, hf);
        const float* stats = reinterpret_cast<const float*>(cur + kOffSt);
        if (qt == diag) {  // rows are queries 8(i/4) + 4hf + i%4 of the tile, the column key lk
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (lk > 8 * (i >> 2) + 4 * hf + (i & 3)) s1[i] = s2[i] = -__builtin_inff();  // P = 0
        }
        if (W > 0 && 32 * qt + 31 >= k_first + W) {  // queries past the window of this lane's key
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (32 * qt + 8 * (i >> 2) + 4 * hf + (i & 3) >= key + W) s1[i] = s2[i] = -__builtin_inff();
        }
        f32x16 pv;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r0 = 8 * g + 4 * hf;
          const f32x4 l1 = *reinterpret_cast<const f32x4*>(stats + r0);
          const f32x4 l2 = *reinterpret_cast<const f32x4*>(stats + 32 + r0);
          f32x4 x, y;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = 4 * g + r;
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[i], c, -l1[r]));
            const float p2 = __builtin_amdgcn_exp2f(__builtin_fmaf(s2[i], c, -l2[r]));
            x[r] = p1;
            y[r] = p2;
            pv[i] = p1 - lam * p2;
          }
          *pslot(cur, g) = x;
          *pslot(cur, 4 + g) = y;
        }
        f16x8 p0, p1;
        pack16(pv, p0, p1);
        // dV^T += dO^T (P_1 - lambda P_2), dO^T read transposed from the dO tile
#pragma unroll
        for (int blk = 0; blk < 4; ++blk) acc[blk] = mfma_tr<kD16Row>(cur + kOffDo, blk, lane, p0, p1, acc[blk]);
      }
    } else {
      // the previous tile, whose P the dV wave of these keys left a step ago,
      // then the current tile's dP
      const bool lp = qt > qt0 && live(qt - 1);
      if (lp) dk_ds(prev);
      if (lp) dk_products(prev);
      if (qt < nqt && live(qt)) dk_dp(cur);
    }
    if (more) stats_store(nxt);
    wait_dma();
    __syncthreads();
  };
  // steps qt0 .. nqt: the last one finishes tile nqt - 1's dK
  int qt = qt0;
  for (; qt + 2 <= nqt; qt += 3) {
    step(qt, stage0, stage1, stage2);
    step(qt + 1, stage1, stage2, stage0);
    step(qt + 2, stage2, stage0, stage1);
  }
  if (qt <= nqt) step(qt, stage0, stage1, stage2);
  if (qt + 1 <= nqt) step(qt + 1, stage1, stage2, stage0);
  if (!ok) return;
  if constexpr (!kDV) {
    if (a.rope.mode != 0) {
      const uint32_t pos = a.rope.pos0 + (uint32_t)key;
      unrotate_grad(acc[0], acc[1], hf, pos, a.rope);
      unrotate_grad(acc[2], acc[3], hf, pos, a.rope);
    }
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
  __shared__ __attribute__((aligned(16))) char stage0[kDkvStage];
  __shared__ __attribute__((aligned(16))) char stage1[kDkvStage];
  __shared__ __attribute__((aligned(16))) char stage2[kDkvStage];
  const int tid = threadIdx.x;
  if (__builtin_amdgcn_readfirstlane(tid >> 6) >= kWaves)
    dkv_role<true>(a, stage0, stage1, stage2, tid);
  else
    dkv_role<false>(a, stage0, stage1, stage2, tid);
}

}  // namespace

hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream) {
  hipError_t e = launch_kernel(bwd_pre_kernel, dim3((unsigned)a.nchunks, (unsigned)a.H), dim3(256), stream, a);
  if (e != hipSuccess) return e;
  if ((e = launch_kernel(bwd_reduce_kernel, dim3((unsigned)a.H), dim3(192), stream, a)) != hipSuccess) return e;
  const int64_t nqb = (a.T + kRows - 1) / kRows;
  const int64_t blocks = nqb * a.B * a.H;
  e = launch_kernel(bwd_dq_kernel, dim3((unsigned)((nqb + 1) / 2 * a.B * a.H)), dim3(512), stream, a);
  if (e != hipSuccess) return e;
  return launch_kernel(bwd_dkv_kernel, dim3((unsigned)blocks), dim3(512), stream, a);
}

}  // namespace diffattn
