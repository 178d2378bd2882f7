// Shared pieces of the prefill kernels (prefill.hip) and the sliding-window
// streaming kernel (window.hip): tile geometry, key/value staging, the
// rotary prologue of the queries, the score and PV products of one tile, the
// causal/window mask, and the epilogue (combine of the two maps, GroupNorm,
// stores).  Everything is force-inlined into the kernels of each file; the
// kernels live in separate translation units so that adding one does not
// change how the compiler allocates registers in another.
#pragma once

#include <algorithm>

#include "kernels.h"
#include "rope.h"
#include "tile.h"

namespace diffattn {
namespace {


constexpr int kGroupWaves = 4;              // waves per group, 32 queries each
constexpr int kBM = 32 * kGroupWaves;       // queries per workgroup
constexpr int kBN = 32;                     // keys per tile (one tile per group per step)
constexpr int kKRow = kDqk * 2;             // 128 bytes per key row
constexpr int kKBytes = kBN * kKRow;        // 4 KiB per K tile
constexpr int kVRow = (kBN + 8) * 2;        // 80 bytes per V^T channel row (16-byte pad)
constexpr int kVBytes = kDv * kVRow;        // 10 KiB per V^T tile
constexpr int kTile = 2 * kKBytes + kVBytes;
constexpr int kTileVT = 2 * kKBytes + kVtTileBytes;  // with V^T tiles moved by DMA (vtiles.hip)
constexpr int kTileThreads = 256;           // threads that stage one tile
// merge_out's buffer: one map's O^T of four waves, then (m1, l1, m2, l2) of
// both groups' eight waves
constexpr int kMergeOutBytes = kMergeO + 8 * 64 * 16;
static_assert(kMergeBytes <= 2 * 2 * kTile, "merge buffer must fit in the stage memory");


__device__ __forceinline__ u32x4 load16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

struct Staged {
  u32x4 k1, k2;
  u32x2 v[4];
  uint32_t kpos;  // position of this thread's key row (rotary embedding)
};

// Per-thread byte offsets of the staging loads inside a tile (see stage_load).
struct StageOffsets {
  uint32_t k1, k2, v;
};

// K columns a thread stages: 16 bytes (dims 8ch .. 8ch+7), or with the
// split-half rotary embedding 8 + 8 bytes (dims 4ch .. 4ch+3 and their pair
// partners 32 + 4ch ..), so that every rotation pair stays in one thread.
// Without the rotary embedding, key tiles go from memory straight to LDS
// (buffer loads with an LDS destination: lane i of a wave writes the 16 bytes
// at its wave's base + 16 i), so thread t fetches the chunk that belongs at
// chunk position t of the swizzled tile: key t/8, logical chunk
// (t % 8) ^ kSwz(t / 8).
template <int kRope>
__device__ __forceinline__ StageOffsets stage_offsets(const PrefillArgs& a, int tid) {
  const int t = tid % kTileThreads;
  const int kr = t >> 3, ch = t & 7, kg = t & 7, cg = t >> 3;
  const int col = kRope == 1 ? 4 * ch : kRope == 2 ? 8 * ch : 8 * (ch ^ kSwz(kr));
  StageOffsets o;
  o.k1 = (uint32_t)((kr * a.sk1.t + col) * 2);
  o.k2 = (uint32_t)((kr * a.sk2.t + col) * 2);
  o.v = (uint32_t)((4 * kg * a.sv.t + 4 * cg) * 2);
  return o;
}

// Memory -> LDS for the key tiles of one step (no registers involved): each
// wave moves 64 chunks of K1 and of K2 into its quarter of its group's tile.
// Completion is counted by vmcnt; the step's barrier follows a wait for it.
// kTileBytes: the stage's bytes per tile (kTile, or kTileVT with V^T tiles).
template <int kTileBytes = kTile>
__device__ __forceinline__ void stage_dma_k(const PrefillArgs& a, const uint16_t* kb1, const uint16_t* kb2,
                                            const StageOffsets& off, char* stage, int k0, int kend, int tid) {
  const int tile = __builtin_amdgcn_readfirstlane(tid / kTileThreads);
  const int part = __builtin_amdgcn_readfirstlane((tid % kTileThreads) >> 6);  // wave within the tile's group
  const int kbase = k0 + tile * kBN;
  char* dst = stage + tile * kTileBytes + part * 1024;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc(kb1, a.sk1.t, kbase, kend, kDqk), (lds_ptr_t)dst, 16, off.k1,
                                           0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc(kb2, a.sk2.t, kbase, kend, kDqk), (lds_ptr_t)(dst + kKBytes),
                                           16, off.k2, 0, 0, 0);
}

// Buffer resource over one (b, h)'s fp16 V^T tiles (vtiles.hip).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t vt_rsrc(const PrefillArgs& a, int b, int head) {
  return vt_tiles_rsrc(a.vt, (int64_t)b * a.H + head, a.T);
}

__device__ __forceinline__ u32x4 load_krow(__amdgpu_buffer_rsrc_t r, uint32_t off, bool split) {
  if (!split) return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  const u32x2 lo = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  const u32x2 hi = __builtin_amdgcn_raw_buffer_load_b64(r, off + 64, 0, 0);  // 32 dims further
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// Global -> registers for one step: one 32-key tile per group, keys from k0 on
// (keys at or past kend read as zero).  Threads 256g .. 256g+255 stage group
// g's tile.  Within a tile, thread t loads 16 bytes of K1 and K2 (key t/8,
// chunk t%8) and a 4-key x 4-channel block of V (keys 4(t%8).., channels
// 4(t/8)..).  kb1, kb2, vb point at key 0 of this (b, h).
template <int kRope>
__device__ __forceinline__ void stage_load(Staged& st, const PrefillArgs& a, const uint16_t* kb1,
                                           const uint16_t* kb2, const uint16_t* vb, const StageOffsets& off,
                                           int k0, int kend, int tid) {
  const int tile = __builtin_amdgcn_readfirstlane(tid / kTileThreads);
  const int kbase = k0 + tile * kBN;
  if constexpr (kRope == 1 || kRope == 2) {
    st.kpos = a.rope.pos0 + (uint32_t)(kbase + ((tid % kTileThreads) >> 3));
    st.k1 = load_krow(rows_rsrc(kb1, a.sk1.t, kbase, kend, kDqk), off.k1, kRope == 1);
    st.k2 = load_krow(rows_rsrc(kb2, a.sk2.t, kbase, kend, kDqk), off.k2, kRope == 1);
  }
  const __amdgpu_buffer_rsrc_t rv = rows_rsrc(vb, a.sv.t, kbase, kend, kDv);
  const int vrow = (int)(a.sv.t * 2);
#pragma unroll
  for (int r = 0; r < 4; ++r) st.v[r] = __builtin_amdgcn_raw_buffer_load_b64(rv, off.v, r * vrow, 0);
}

// Split-half rotation of a staged key row piece: words 0-1 hold dims
// 4j .. 4j+3 of K1 (K2), words 2-3 the pair partners 32 + 4j .., so pairs
// c = 4j .. 4j+3 are complete in the thread.  Packs the result as fp16.
__device__ __forceinline__ void rope_split_half(u32x4& k1, u32x4& k2, int j, uint32_t pos, const uint64_t* tab) {
  float a[2][8];
  rope_unpack(k1, a[0]);
  rope_unpack(k2, a[1]);
  const uint64_t* f = tab + 4 * j;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float c, sn;
    rope_cos_sin(pos, f[e], c, sn);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float lo = a[k][e], hi = a[k][4 + e];
      a[k][e] = lo * c - hi * sn;
      a[k][4 + e] = lo * sn + hi * c;
    }
  }
  k1 = rope_pack<true>(a[0]);
  k2 = rope_pack<true>(a[1]);
}

// Registers -> LDS: K rows with swizzled 16-byte chunks (rotated first when
// the rotary embedding is on), V transposed to [channel][key] in fp16 with the
// kVPos key order.
template <int kRope>
__device__ __forceinline__ void stage_store(const Staged& st, char* stage, int tid, const uint64_t* rope_tab) {
  const int tile = tid / kTileThreads, t = tid % kTileThreads;
  char* base = stage + tile * kTile;
  const int kr = t >> 3, ch = t & 7;
  if constexpr (kRope == 1) {
    // dims 4ch .. 4ch+3 (words 0, 1) and their partners 32 + 4ch .. (words 2, 3)
    u32x4 k1 = st.k1, k2 = st.k2;
    rope_split_half(k1, k2, ch, st.kpos, rope_tab);
    const int c0 = ch >> 1, half = (ch & 1) * 8, sw = kSwz(kr);
    const int off_lo = kr * kKRow + ((c0 ^ sw) << 4) + half;
    const int off_hi = kr * kKRow + (((c0 + 4) ^ sw) << 4) + half;
    *reinterpret_cast<u32x2*>(base + off_lo) = u32x2{k1.x, k1.y};
    *reinterpret_cast<u32x2*>(base + off_hi) = u32x2{k1.z, k1.w};
    *reinterpret_cast<u32x2*>(base + kKBytes + off_lo) = u32x2{k2.x, k2.y};
    *reinterpret_cast<u32x2*>(base + kKBytes + off_hi) = u32x2{k2.z, k2.w};
  } else if constexpr (kRope == 2) {
    const int koff = kr * kKRow + ((ch ^ kSwz(kr)) << 4);
    rope_u32x4 kk[2] = {st.k1, st.k2};
    rope_chunks<2, true>(kk, ch, st.kpos, kRope, rope_tab);
    *reinterpret_cast<u32x4*>(base + koff) = kk[0];
    *reinterpret_cast<u32x4*>(base + kKBytes + koff) = kk[1];
  }  // without the rotary embedding the key tile came by DMA
  const int kg = t & 7, cg = t >> 3;
  float e[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    e[r][0] = bf16_lo(st.v[r].x);
    e[r][1] = bf16_hi(st.v[r].x);
    e[r][2] = bf16_lo(st.v[r].y);
    e[r][3] = bf16_hi(st.v[r].y);
  }
  char* vt = base + 2 * kKBytes + kVPos(kg) * 8;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    f16x4 h = {(_Float16)e[0][c], (_Float16)e[1][c], (_Float16)e[2][c], (_Float16)e[3][c]};
    *reinterpret_cast<f16x4*>(vt + (4 * cg + c) * kVRow) = h;
  }
}

// Rotary embedding of the lane's query vectors, held as the score product's
// operand: chunk s holds dims 16s + 8hf .. +7.  Split-half pairs (c, c + 32)
// join chunks s and s + 2 of the same lane; interleaved pairs stay inside a
// chunk.  Both maps' queries share the angles.  The rotated values are stored
// as fp16 bits (the key tiles are rotated to fp16 as well, and the score
// product then runs on fp16 operands: eight times finer than bf16, which keeps
// the rounding of rotated operands well inside the error budget).
// rope_query with a small working set: one pair of chunks (split-half) or
// one chunk (interleaved) of both queries at a time, for kernels that call it
// with most of their registers live.  The same rotation, element by element.
__device__ __forceinline__ void rope_query_lean(bf16x8 (&q1)[4], bf16x8 (&q2)[4], int hf, uint32_t pos, int mode,
                                                const RopeArgs& r) {
  if (mode == 1) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      float a1[8], b1[8], a2[8], b2[8];
      rope_unpack(__builtin_bit_cast(rope_u32x4, q1[s]), a1);
      rope_unpack(__builtin_bit_cast(rope_u32x4, q1[s + 2]), b1);
      rope_unpack(__builtin_bit_cast(rope_u32x4, q2[s]), a2);
      rope_unpack(__builtin_bit_cast(rope_u32x4, q2[s + 2]), b2);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c0 = 16 * s + e;  // pair index in lane half 0; half 1 adds 8
        float c, sn;
        rope_cos_sin(pos, hf ? r.phase[c0 + 8] : r.phase[c0], c, sn);
        float a = a1[e], b = b1[e];
        a1[e] = a * c - b * sn;
        b1[e] = a * sn + b * c;
        a = a2[e];
        b = b2[e];
        a2[e] = a * c - b * sn;
        b2[e] = a * sn + b * c;
      }
      q1[s] = __builtin_bit_cast(bf16x8, rope_pack<true>(a1));
      q1[s + 2] = __builtin_bit_cast(bf16x8, rope_pack<true>(b1));
      q2[s] = __builtin_bit_cast(bf16x8, rope_pack<true>(a2));
      q2[s + 2] = __builtin_bit_cast(bf16x8, rope_pack<true>(b2));
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float x1[8], x2[8];
      rope_unpack(__builtin_bit_cast(rope_u32x4, q1[s]), x1);
      rope_unpack(__builtin_bit_cast(rope_u32x4, q2[s]), x2);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c0 = 8 * s + e;  // pair index in lane half 0; half 1 adds 4
        float c, sn;
        rope_cos_sin(pos, hf ? r.phase[c0 + 4] : r.phase[c0], c, sn);
        float a = x1[2 * e], b = x1[2 * e + 1];
        x1[2 * e] = a * c - b * sn;
        x1[2 * e + 1] = a * sn + b * c;
        a = x2[2 * e];
        b = x2[2 * e + 1];
        x2[2 * e] = a * c - b * sn;
        x2[2 * e + 1] = a * sn + b * c;
      }
      q1[s] = __builtin_bit_cast(bf16x8, rope_pack<true>(x1));
      q2[s] = __builtin_bit_cast(bf16x8, rope_pack<true>(x2));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

__device__ __forceinline__ void rope_query(bf16x8 (&q1)[4], bf16x8 (&q2)[4], int hf, uint32_t pos, int mode,
                                           const RopeArgs& r) {
  float x1[4][8], x2[4][8];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    rope_unpack(__builtin_bit_cast(rope_u32x4, q1[s]), x1[s]);
    rope_unpack(__builtin_bit_cast(rope_u32x4, q2[s]), x2[s]);
  }
  if (mode == 1) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c0 = 16 * s + e;  // pair index in lane half 0; half 1 adds 8
        const uint64_t f = hf ? r.phase[c0 + 8] : r.phase[c0];
        float c, sn;
        rope_cos_sin(pos, f, c, sn);
        float a = x1[s][e], b = x1[s + 2][e];
        x1[s][e] = a * c - b * sn;
        x1[s + 2][e] = a * sn + b * c;
        a = x2[s][e];
        b = x2[s + 2][e];
        x2[s][e] = a * c - b * sn;
        x2[s + 2][e] = a * sn + b * c;
      }
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c0 = 8 * s + e;  // pair index in lane half 0; half 1 adds 4
        const uint64_t f = hf ? r.phase[c0 + 4] : r.phase[c0];
        float c, sn;
        rope_cos_sin(pos, f, c, sn);
        float a = x1[s][2 * e], b = x1[s][2 * e + 1];
        x1[s][2 * e] = a * c - b * sn;
        x1[s][2 * e + 1] = a * sn + b * c;
        a = x2[s][2 * e];
        b = x2[s][2 * e + 1];
        x2[s][2 * e] = a * c - b * sn;
        x2[s][2 * e + 1] = a * sn + b * c;
      }
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    q1[s] = __builtin_bit_cast(bf16x8, rope_pack<true>(x1[s]));
    q2[s] = __builtin_bit_cast(bf16x8, rope_pack<true>(x2[s]));
  }
}

// GroupNorm statistics of a query's 128 channels, taken as two halves of 64:
// channel blocks 2h and 2h + 1 (cb) of the lane pair holding the query.
// half_stats: the half's mean and sum of squared deviations from it
// (two-pass), added over the lane pair.  combine_halves: the mean and the
// variance of all 128 by the pairwise update for two equal halves, var * 128
// = M2_0 + M2_1 + 32 (mu_0 - mu_1)^2, whose operations are symmetric in the
// halves.  Every kernel normalises with these two, so outputs that agree
// before the norm agree after it bit for bit, whichever kernel (or wave group,
// when two groups finish one half each) took the statistics.
template <int h>
__device__ __forceinline__ f32x2 half_stats(const f32x16 (&O)[4]) {
  float sum = 0.f;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += O[2 * h + blk][i];
  sum += __shfl_xor(sum, 32);
  const float mu = sum * (1.0f / 64);
  float m2 = 0.f;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float d = O[2 * h + blk][i] - mu;
      m2 += d * d;
    }
  m2 += __shfl_xor(m2, 32);
  return f32x2{mu, m2};
}

// (mean, 1 / sqrt(var + eps)) from the two halves' statistics (either order).
__device__ __forceinline__ f32x2 combine_halves(f32x2 x, f32x2 y, float eps) {
  const float dmu = x[0] - y[0];
  const float mean = (x[0] + y[0]) * 0.5f;
  const float var = (x[1] + y[1] + 32.0f * (dmu * dmu)) * (1.0f / kDv);
  return f32x2{mean, 1.0f / __builtin_sqrtf(var + eps)};
}

// GroupNorm over the 128 channels of the query (o in O, lane (hf, lq)
// holding channels 32cb + 8(i/4) + 4hf + i%4, its partner lane the other 64),
// then the stores.  gain(cb, r4): the head's gain of channels 32cb + 8r4 + 4hf
// .. +3.
template <class GainFn>
__device__ __forceinline__ void norm_store_g(const PrefillArgs& a, int b, int head, int q, int hf, f32x16 (&O)[4],
                                             GainFn gain) {
  const f32x2 mi = combine_halves(half_stats<0>(O), half_stats<1>(O), a.eps);
  const float mu = mi[0], inv = mi[1];

  if (q >= a.T) return;
  const int64_t row = (((int64_t)b * a.T + q) * a.H + head) * kDv;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int ch = 32 * cb + 8 * r4 + 4 * hf;
      const f32x4 gv = gain(cb, r4);
      f32x4 o, y;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        o[r] = O[cb][4 * r4 + r];
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

// norm_store_g with the gain read from g (shared memory) at each store.
__device__ __forceinline__ void norm_store(const PrefillArgs& a, int b, int head, int q, int hf, f32x16 (&O)[4],
                                           const float* g) {
  norm_store_g(a, b, head, q, hf, O,
               [&](int cb, int r4) { return *reinterpret_cast<const f32x4*>(g + 32 * cb + 8 * r4 + 4 * hf); });
}

// A lane's 64 gains of the head (the channels norm_store_g stores) from global
// memory.  Loaded before any store of the epilogue: the memory counter also
// counts stores, so a load issued after a store waits for that store too.
__device__ __forceinline__ void load_gain(const PrefillArgs& a, int head, int hf, f32x4 (&gv)[4][4]) {
  const float* g = a.gain + (int64_t)head * kDv + 4 * hf;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) gv[cb][r4] = *reinterpret_cast<const f32x4*>(g + 32 * cb + 8 * r4);
}

// The same gains spread over the wave: lane L holds the head's gains 2L and
// 2L + 1 (one coalesced 8-byte load, two registers), and each store's four
// gains are broadcast from their lanes by v_readlane (the lane index is a
// constant once unrolled).  Used where 64 registers of gains do not fit.
struct LaneGain {
  float g0, g1;
  int hf;
  __device__ __forceinline__ f32x4 operator()(int cb, int r4) const {
    f32x4 v;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c0 = 32 * cb + 8 * r4 + r, c1 = c0 + 4;  // the channel of a lane with hf = 0, hf = 1
      const float a = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, (c0 & 1) ? g1 : g0), c0 >> 1));
      const float b = __builtin_bit_cast(
          float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, (c1 & 1) ? g1 : g0), c1 >> 1));
      v[r] = hf ? b : a;
    }
    return v;
  }
};

// The lane's two gains (lane = 0 .. 63).
__device__ __forceinline__ f32x2 load_lane_gain(const PrefillArgs& a, int head, int lane) {
  return *reinterpret_cast<const f32x2*>(a.gain + (int64_t)head * kDv + 2 * lane);
}

__device__ __forceinline__ float head_lambda(const PrefillArgs& a, int head) {
  return a.lambda_h ? a.lambda_h[head] : a.lambda;
}

// Fold the two wave groups' softmax states of each query and form the
// differential output o = O1 / l1 - lambda O2 / l2 in group 0's O1: both
// groups exchange (m, l) per map, weight their own accumulators, and group
// 1's part of o crosses LDS once.  Both groups compute the merged sums with
// the same operations (sums of two terms, commutative), so their weights
// agree bit for bit.  kTrain adds the training outputs (each map's O_m / l_m
// and log-sum-exp) through two more exchanges; o is computed the same way
// either way, so the training forward's y equals the plain forward's.  Every
// thread calls it (the barriers are unconditional).
template <bool kTrain>
__device__ __forceinline__ void merge_out(const PrefillArgs& a, char* smem, int grp, int wq, int lane, bool live,
                                          float lam, int b, int head, int q, int hf, float m1, float l1, float m2,
                                          float l2, f32x16 (&O1)[4], f32x16 (&O2)[4]) {
  float* mo = reinterpret_cast<float*>(smem);
  f32x4* ml = reinterpret_cast<f32x4*>(smem + kMergeO);  // [group][wave][lane]: m1, l1, m2, l2
  auto slot = [&](int cb, int i) { return ((wq * 64) + cb * 16 + i) * 64 + lane; };
  if (live) ml[(grp * 4 + wq) * 64 + lane] = f32x4{m1, l1, m2, l2};
  __syncthreads();
  float M1 = 0.f, M2 = 0.f, a1 = 0.f, a2 = 0.f, L1 = 1.f, L2 = 1.f;
  if (live) {
    const f32x4 ot = ml[((grp ^ 1) * 4 + wq) * 64 + lane];
    M1 = fmaxf(m1, ot[0]);
    M2 = fmaxf(m2, ot[2]);
    a1 = __builtin_amdgcn_exp2f(m1 - M1);
    a2 = __builtin_amdgcn_exp2f(m2 - M2);
    L1 = l1 * a1 + ot[1] * __builtin_amdgcn_exp2f(ot[0] - M1);
    L2 = l2 * a2 + ot[3] * __builtin_amdgcn_exp2f(ot[2] - M2);
  }
  L1 += __shfl_xor(L1, 32);
  L2 += __shfl_xor(L2, 32);
  if constexpr (kTrain) {
    // O_m / l_m of each map, summed over the two groups.
    const int64_t rq = ((int64_t)b * a.T + q) * a.H + head;
#pragma unroll
    for (int map = 0; map < 2; ++map) {
      f32x16 (&O)[4] = map == 0 ? O1 : O2;
      float* dst = map == 0 ? a.o1n : a.o2n;
      const float w = map == 0 ? a1 / L1 : a2 / L2;
      if (grp == 1 && live) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mo[slot(cb, i)] = O[cb][i] * w;
      }
      __syncthreads();
      if (grp == 0 && live && q < a.T) {
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = O[cb][4 * r4 + r] * w + mo[slot(cb, 4 * r4 + r)];
            *reinterpret_cast<f32x4*>(dst + rq * kDv + 32 * cb + 8 * r4 + 4 * hf) = v;
          }
      }
      __syncthreads();
    }
    if (grp == 0 && live && q < a.T && hf == 0) {
      a.lse[rq * 2] = M1 + __builtin_log2f(L1);
      a.lse[rq * 2 + 1] = M2 + __builtin_log2f(L2);
    }
  }
  if (live) {
    const float w1 = a1 / L1, w2 = lam * a2 / L2;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // both products rounded before the subtraction (no FMA contraction):
        // two identical maps at lambda = 1 cancel to exactly zero
#pragma clang fp contract(off)
        O1[cb][i] = O1[cb][i] * w1 - O2[cb][i] * w2;
      }
    if (grp == 1) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mo[slot(cb, i)] = O1[cb][i];
    }
  }
  __syncthreads();
  if (grp == 0 && live) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) O1[cb][i] += mo[slot(cb, i)];
  }
}

// merge_out and the GroupNorm epilogue (inference outputs) with the work split
// between the two wave groups by channel: group g finishes channel blocks
// cb = 2g, 2g + 1 of its queries.  After the (m, l) exchange each group forms
// its own weighted part of o for all four blocks, as merge_out does; the two
// blocks it does not finish cross LDS to the other group as 16-byte vectors,
// and each group adds the other's part into its two blocks (the same sums as
// merge_out's, in commutative order).  GroupNorm then needs the statistics of
// all 128 channels: each group takes its half's (half_stats), the groups
// exchange them once, and both combine them (combine_halves, symmetric in the
// halves), so both get the statistics norm_store_g would, bit for bit.  Each
// group then normalises and stores its 64 channels.  Every thread calls it
// (the barriers are unconditional).
__device__ __forceinline__ void merge_norm_split(const PrefillArgs& a, char* smem, int grp, int wq, int lane,
                                                 bool live, float lam, int b, int head, int q, int hf, float m1,
                                                 float l1, float m2, float l2, f32x16 (&O1)[4],
                                                 const f32x16 (&O2)[4], const float* gain_s) {
  f32x4* xo = reinterpret_cast<f32x4*>(smem);            // [sender][wave][block][r4][lane]
  f32x4* ml = reinterpret_cast<f32x4*>(smem + kMergeO);  // [group][wave][lane]: m1, l1, m2, l2
  f32x2* st = reinterpret_cast<f32x2*>(smem + kMergeO);  // reused: [group][wave][lane]: mean, M2
  static_assert(2 * 4 * 2 * 4 * 64 * 16 <= kMergeO, "exchange buffer");
  auto xslot = [&](int sender, int blk, int r4) { return (((sender * 4 + wq) * 2 + blk) * 4 + r4) * 64 + lane; };
  // The register blocks are indexed with compile-time constants only (a
  // runtime index would move the accumulators to scratch memory): each part
  // that depends on the group runs as one of two instantiations.
  typedef std::integral_constant<int, 0> G0;
  typedef std::integral_constant<int, 1> G1;
  auto send = [&](auto G) __attribute__((always_inline)) {
    constexpr int g = decltype(G)::value;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x16& o = O1[2 * (1 - g) + blk];
        xo[xslot(g, blk, r4)] = f32x4{o[4 * r4], o[4 * r4 + 1], o[4 * r4 + 2], o[4 * r4 + 3]};
      }
  };
  // adds the other group's part and returns the 64-channel (mean, M2)
  auto gather = [&](auto G) __attribute__((always_inline)) {
    constexpr int g = decltype(G)::value;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 o = xo[xslot(1 - g, blk, r4)];
#pragma unroll
        for (int r = 0; r < 4; ++r) O1[2 * g + blk][4 * r4 + r] += o[r];
      }
    return half_stats<g>(O1);
  };
  auto store = [&](auto G, float mean, float inv) __attribute__((always_inline)) {
    constexpr int g = decltype(G)::value;
    const int64_t row = (((int64_t)b * a.T + q) * a.H + head) * kDv;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const int cb = 2 * g + blk;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int ch = 32 * cb + 8 * r4 + 4 * hf;
        const f32x4 gv = *reinterpret_cast<const f32x4*>(gain_s + ch);
        f32x4 o, y;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          o[r] = O1[cb][4 * r4 + r];
          y[r] = (o[r] - mean) * inv * gv[r];
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
  };

  if (live) ml[(grp * 4 + wq) * 64 + lane] = f32x4{m1, l1, m2, l2};
  __syncthreads();
  if (live) {
    const f32x4 ot = ml[((grp ^ 1) * 4 + wq) * 64 + lane];
    const float M1 = fmaxf(m1, ot[0]);
    const float M2 = fmaxf(m2, ot[2]);
    const float a1 = __builtin_amdgcn_exp2f(m1 - M1);
    const float a2 = __builtin_amdgcn_exp2f(m2 - M2);
    float L1 = l1 * a1 + ot[1] * __builtin_amdgcn_exp2f(ot[0] - M1);
    float L2 = l2 * a2 + ot[3] * __builtin_amdgcn_exp2f(ot[2] - M2);
    L1 += __shfl_xor(L1, 32);
    L2 += __shfl_xor(L2, 32);
    const float w1 = a1 / L1, w2 = lam * a2 / L2;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        // both products rounded before the subtraction (no FMA contraction):
        // two identical maps at lambda = 1 cancel to exactly zero
#pragma clang fp contract(off)
        O1[cb][i] = O1[cb][i] * w1 - O2[cb][i] * w2;
      }
    if (grp == 0)
      send(G0{});
    else
      send(G1{});
  }
  __syncthreads();  // every wave has read ml and written its blocks
  f32x2 mine = f32x2{0.f, 0.f};
  if (live) {
    mine = grp == 0 ? gather(G0{}) : gather(G1{});
    st[(grp * 4 + wq) * 64 + lane] = mine;
  }
  __syncthreads();
  if (!live) return;
  const f32x2 mi = combine_halves(mine, st[((grp ^ 1) * 4 + wq) * 64 + lane], a.eps);
  const float mean = mi[0], inv = mi[1];
  if (q >= a.T) return;
  if (grp == 0)
    store(G0{}, mean, inv);
  else
    store(G1{}, mean, inv);
}

// o = O1 / l1 - lam O2 / l2 into O1 (l1, l2: the row's full sums).
__device__ __forceinline__ void combine_maps(float lam, float l1, float l2, f32x16 (&O1)[4], const f32x16 (&O2)[4]) {
  const float r1 = 1.0f / l1;
  const float r2 = lam / l2;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      // Both products rounded before the subtraction (no FMA contraction), so
      // two identical maps at lambda = 1 cancel to exactly zero.
#pragma clang fp contract(off)
      O1[cb][i] = O1[cb][i] * r1 - O2[cb][i] * r2;
    }
  }
}

// Combine the two maps of one query row (lane pair) from their final softmax
// states, write the training outputs if asked, then GroupNorm and store; lam
// is the head's lambda and gv its gains (load_gain), both read before any
// store.
__device__ __forceinline__ void finish_rows(const PrefillArgs& a, int b, int head, int q, int hf, float m1, float m2,
                                            float l1, float l2, f32x16 (&O1)[4], f32x16 (&O2)[4], float lam,
                                            const f32x4 (&gv)[4][4]) {
  l1 += __shfl_xor(l1, 32);
  l2 += __shfl_xor(l2, 32);
  if (a.o1n != nullptr && q < a.T) {
    // Training outputs for the backward pass.
    const int64_t rq = ((int64_t)b * a.T + q) * a.H + head;
    const float i1 = 1.0f / l1, i2 = 1.0f / l2;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int ch = 32 * cb + 8 * r4 + 4 * hf;
        f32x4 v1, v2;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          v1[r] = O1[cb][4 * r4 + r] * i1;
          v2[r] = O2[cb][4 * r4 + r] * i2;
        }
        *reinterpret_cast<f32x4*>(a.o1n + rq * kDv + ch) = v1;
        *reinterpret_cast<f32x4*>(a.o2n + rq * kDv + ch) = v2;
      }
    if (hf == 0) {
      a.lse[rq * 2] = m1 + __builtin_log2f(l1);
      a.lse[rq * 2 + 1] = m2 + __builtin_log2f(l2);
    }
  }
  combine_maps(lam, l1, l2, O1, O2);
  // The gains have landed before the first store (left to itself the
  // compiler waits for each gain after the stores issued before its use).
  wait_vm<0>();
  norm_store_g(a, b, head, q, hf, O1, [&](int cb, int r4) { return gv[cb][r4]; });
}

// finish_rows with lambda and the gains loaded first.
__device__ __forceinline__ void finish_rows(const PrefillArgs& a, int b, int head, int q, int hf, float m1, float m2,
                                            float l1, float l2, f32x16 (&O1)[4], f32x16 (&O2)[4]) {
  const float lam = head_lambda(a, head);
  f32x4 gv[4][4];
  load_gain(a, head, hf, gv);
  finish_rows(a, b, head, q, hf, m1, m2, l1, l2, O1, O2, lam, gv);
}

// S^T = K Q^T of one tile for both maps, K from LDS: bf16 operands, or fp16
// (kF16: rotated keys and queries, see rope_query).
template <bool kF16>
__device__ __forceinline__ void scores_tile(const char* kt, int lq, int hf, int ksw, const bf16x8 (&qa)[4],
                                            const bf16x8 (&qb2)[4], f32x16& s1, f32x16& s2) {
  s1 = f32x16{};
  s2 = f32x16{};
  const int krow = lq * kKRow;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const int off = krow + (((2 * s + hf) ^ ksw) << 4);
    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kt + off);
    const bf16x8 kb = *reinterpret_cast<const bf16x8*>(kt + kKBytes + off);
    if constexpr (kF16) {
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, ka), __builtin_bit_cast(f16x8, qa[s]), s1,
                                                  0, 0, 0);
      s2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kb), __builtin_bit_cast(f16x8, qb2[s]),
                                                  s2, 0, 0, 0);
    } else {
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qa[s], s1, 0, 0, 0);
      s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, qb2[s], s2, 0, 0, 0);
    }
  }
}

__device__ __forceinline__ void mask_tile(const PrefillArgs& a, f32x16& s1, f32x16& s2, int j, int wave_last_tile,
                                          int q_first, int q, int hf) {
  // Key row kr = 8(i/4) + 4hf + i%4 of tile j is key 32j + kr: visible to
  // query q iff it is <= q (and > q - window).  The bounds depend on j, so the
  // compiler keeps the compares inside the loop instead of holding sixteen
  // lane masks.
  if (j == wave_last_tile) {
    const int hi = q - j * kBN - 4 * hf;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (8 * (i >> 2) + (i & 3) > hi) {
        s1[i] = -__builtin_inff();
        s2[i] = -__builtin_inff();
      }
    }
  }
  if (a.window > 0 && j * kBN < q_first + 32 - a.window) {
    const int lo = q - a.window - j * kBN - 4 * hf;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (8 * (i >> 2) + (i & 3) <= lo) {
        s1[i] = -__builtin_inff();
        s2[i] = -__builtin_inff();
      }
    }
  }
}

// Two 32-channel blocks of O += V P for both maps, ordered so that
// consecutive products never share an accumulator.  kVT: the tile's V^T came
// by DMA in the vtiles.hip layout; otherwise it was staged in kVRow rows.
template <bool kVT = false>
__device__ __forceinline__ void pv_pair(const char* kt, int lq, int hf, int cb, const f16x8& p1a, const f16x8& p1b,
                                        const f16x8& p2a, const f16x8& p2b, f32x16 (&O1)[4], f32x16 (&O2)[4]) {
  if constexpr (kVT) {
    const char* vt = kt + 2 * kKBytes;
    const f16x8 a0 = vt_operand(vt, lq, hf, cb, 0);
    const f16x8 b0 = vt_operand(vt, lq, hf, cb + 1, 0);
    O1[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, p1a, O1[cb], 0, 0, 0);
    O2[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, p2a, O2[cb], 0, 0, 0);
    O1[cb + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0, p1a, O1[cb + 1], 0, 0, 0);
    O2[cb + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0, p2a, O2[cb + 1], 0, 0, 0);
    const f16x8 a1 = vt_operand(vt, lq, hf, cb, 1);
    const f16x8 b1 = vt_operand(vt, lq, hf, cb + 1, 1);
    O1[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, p1b, O1[cb], 0, 0, 0);
    O2[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, p2b, O2[cb], 0, 0, 0);
    O1[cb + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b1, p1b, O1[cb + 1], 0, 0, 0);
    O2[cb + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b1, p2b, O2[cb + 1], 0, 0, 0);
    return;
  }
  const char* vt = kt + 2 * kKBytes + lq * kVRow + hf * 16 + cb * 32 * kVRow;
  const f16x8 a0 = *reinterpret_cast<const f16x8*>(vt);
  const f16x8 b0 = *reinterpret_cast<const f16x8*>(vt + 32 * kVRow);
  O1[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, p1a, O1[cb], 0, 0, 0);
  O2[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, p2a, O2[cb], 0, 0, 0);
  O1[cb + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0, p1a, O1[cb + 1], 0, 0, 0);
  O2[cb + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0, p2a, O2[cb + 1], 0, 0, 0);
  const f16x8 a1 = *reinterpret_cast<const f16x8*>(vt + 32);
  const f16x8 b1 = *reinterpret_cast<const f16x8*>(vt + 32 * kVRow + 32);
  O1[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, p1b, O1[cb], 0, 0, 0);
  O2[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, p2b, O2[cb], 0, 0, 0);
  O1[cb + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b1, p1b, O1[cb + 1], 0, 0, 0);
  O2[cb + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b1, p2b, O2[cb + 1], 0, 0, 0);
}

}  // namespace
}  // namespace diffattn
