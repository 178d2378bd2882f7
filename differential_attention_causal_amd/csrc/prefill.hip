// Fused causal differential-attention prefill for gfx950 (MI355X).
//
// Computes, per (b, h) and query i (Motif 2.6B explainer, "Differential
// attention" and the figure 1 caption):
//   o_i = sum_{j<=i} [P1_ij - lambda P2_ij] v_j,   Pm = softmax_j(Qm Km^T * scale)
//   y_i = GroupNorm(o_i)  (one group = the head's 128 channels, with gain)
// in one pass over the keys, with two independent online-softmax states.
//
// Work split.  A workgroup owns 128 consecutive queries of one (b, h); within
// a group of four wave64s, wave w takes queries 32w .. 32w+31.  Keys stream
// through LDS in 32-key tiles; tiles past the causal diagonal are never
// loaded, and a wave skips tiles past its own diagonal.  Launch shapes:
//   - ping-pong (prefill_pp_kernel, 8 waves): two groups take alternate tiles
//     of the causal range (group 0 the even ones, group 1 the odd ones), each
//     with its own softmax states and accumulators, merged through LDS at the
//     end; group 1 runs half a step behind group 0, so that on every SIMD one
//     wave's matrix products run while the other wave does its softmax.  Used
//     for grids that fit on the chip in one round, without the rotary
//     embedding; each workgroup runs two query blocks of one (b, h) back to
//     back (the longest with the shortest), so one workgroup per CU carries
//     the same work everywhere;
//   - one group (4 waves, prefill_kernel<1, .>): two workgroups share a CU,
//     and a grid larger than the chip balances itself in longest-first order;
//   - two groups in lock step (prefill_kernel<2, .>): the split of the
//     ping-pong kernel without its phase offset, for small grids with the
//     rotary embedding (keys rotated while staged) or key spans past 2^31
//     bytes.
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
// the matching order (see kVPos in tile.h).
//
// Precision.  Scores: bf16 inputs, fp32 accumulation.  Softmax in fp32 base-2
// units (c = scale * log2 e).  P is rounded to fp16 and V is converted
// bf16 -> fp16 (exact for |v| in [2^-14, 65504)) for the f16 product, fp32
// accumulation.  The running max is only raised when a tile's max exceeds it
// by more than kSlack (base 2), so P <= 2^kSlack stays far inside fp16 range and
// the O rescale is rare after the first tiles.
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
constexpr int kTileThreads = 256;           // threads that stage one tile
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
__device__ __forceinline__ void stage_dma_k(const PrefillArgs& a, const uint16_t* kb1, const uint16_t* kb2,
                                            const StageOffsets& off, char* stage, int k0, int kend, int tid) {
  const int tile = __builtin_amdgcn_readfirstlane(tid / kTileThreads);
  const int part = __builtin_amdgcn_readfirstlane((tid % kTileThreads) >> 6);  // wave within the tile's group
  const int kbase = k0 + tile * kBN;
  char* dst = stage + tile * kTile + part * 1024;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc(kb1, a.sk1.t, kbase, kend, kDqk), (lds_ptr_t)dst, 16, off.k1,
                                           0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc(kb2, a.sk2.t, kbase, kend, kDqk), (lds_ptr_t)(dst + kKBytes),
                                           16, off.k2, 0, 0, 0);
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

// GroupNorm over the 128 channels of the query (o in O, lane (hf, lq)
// holding channels 32cb + 8(i/4) + 4hf + i%4, its partner lane the other 64),
// then the stores.  g: the head's gain (global or shared memory).
__device__ __forceinline__ void norm_store(const PrefillArgs& a, int b, int head, int q, int hf, f32x16 (&O)[4],
                                           const float* g) {
  float sum = 0.f;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += O[cb][i];
  sum += __shfl_xor(sum, 32);
  const float mu = sum * (1.0f / kDv);
  float ss = 0.f;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float d = O[cb][i] - mu;
      ss += d * d;
    }
  }
  ss += __shfl_xor(ss, 32);
  const float inv = 1.0f / __builtin_sqrtf(ss * (1.0f / kDv) + a.eps);

  if (q >= a.T) return;
  const int64_t row = (((int64_t)b * a.T + q) * a.H + head) * kDv;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int ch = 32 * cb + 8 * r4 + 4 * hf;
      const f32x4 gv = *reinterpret_cast<const f32x4*>(g + ch);
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

// Combine the two maps of one query row (lane pair) from their final softmax
// states, write the training outputs if asked, then GroupNorm and store.
__device__ __forceinline__ void finish_rows(const PrefillArgs& a, int b, int head, int q, int hf, float m1, float m2,
                                            float l1, float l2, f32x16 (&O1)[4], f32x16 (&O2)[4]) {
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
  const float lam = a.lambda_h ? a.lambda_h[head] : a.lambda;
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
  norm_store(a, b, head, q, hf, O1, a.gain + (int64_t)head * kDv);
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
// consecutive products never share an accumulator.
__device__ __forceinline__ void pv_pair(const char* kt, int lq, int hf, int cb, const f16x8& p1a, const f16x8& p1b,
                                        const f16x8& p2a, const f16x8& p2b, f32x16 (&O1)[4], f32x16 (&O2)[4]) {
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

// Buffer resources over one (b, h)'s key rows 0 .. kend-1, fixed for the whole
// kernel (rows past kend read as zero); a tile is addressed by adding its first
// key's byte offset to the per-lane offset, so the host keeps a (b, h)'s key
// span under 2^31 bytes for this kernel.
struct KeyRes {
  __amdgpu_buffer_rsrc_t k1, k2, v;
  uint32_t ks1, ks2, vs;  // bytes per key row
};

// DMA of one group's key tile (first key kbase) into the group's slot.
__device__ __forceinline__ void pp_dma_k(const KeyRes& r, const StageOffsets& off, char* slot, int kbase, int part) {
  char* dst = slot + part * 1024;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.k1, (lds_ptr_t)dst, 16, off.k1 + (uint32_t)kbase * r.ks1, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r.k2, (lds_ptr_t)(dst + kKBytes), 16, off.k2 + (uint32_t)kbase * r.ks2, 0,
                                           0, 0);
}

// Global -> registers: the thread's 4-key x 4-channel block of one group's
// value tile (first key kbase).
__device__ __forceinline__ void pp_load_v(Staged& st, const KeyRes& r, const StageOffsets& off, int kbase) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    st.v[i] = __builtin_amdgcn_raw_buffer_load_b64(r.v, off.v + (uint32_t)(kbase + i) * r.vs, 0, 0);
}

// Ping-pong split-key kernel (two groups of four waves, one wave of each group
// per SIMD).  Each group runs a two-phase step: a matrix phase (O += V P for
// its current tile, then S = K Q^T for its next tile) and a vector phase
// (softmax of that S into P, V staging).  Group 1 runs one phase behind group
// 0, so on every SIMD one wave's matrix products overlap the other's vector
// work; every phase ends in a workgroup barrier that keeps the two in step.
// Each group stages its own tiles in two slots: tile x's keys and values sit
// in slot x % 2.  In the matrix phase of step x the group reads V(x) and
// K(x + 1) while the DMA of K(x + 2) fills slot x % 2; V(x + 1) is stored in
// the vector phase of step x from registers loaded a step earlier.
constexpr int kPPStage = 2 * kTile;
constexpr int kPPSmem = 2 * kPPStage + kDv * 4 + 16;

template <bool kTrain, bool kRopeQ>
__device__ __forceinline__ void pp_item(const PrefillArgs& a, char* smem, int item) {
  constexpr int kStage = kPPStage;
  f32x4* const gain_s = reinterpret_cast<f32x4*>(smem + 2 * kStage);
  float* const lam_s = reinterpret_cast<float*>(smem + 2 * kStage + kDv * 4);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / kGroupWaves;
  const int wq = wave % kGroupWaves;
  const int lane = tid & 63;
  const int hf = lane >> 5;
  const int lq = lane & 31;

  const int nqb = (a.T + kBM - 1) / kBM;
  const int BH = a.B * a.H;
  const int qb = nqb - 1 - item / BH;
  const int bh = item % BH;
  const int head = bh % a.H;
  const int b = bh / a.H;

  const int q_first = qb * kBM + 32 * wq;
  const int q = q_first + lq;
  const bool wave_live = q_first < a.T;
  const int ntiles = min(qb * (kBM / kBN) + (kBM / kBN), (a.T + kBN - 1) / kBN);
  const int kend = min(a.T, ntiles * kBN);
  const int tile0 = a.window > 0 ? max(0, qb * kBM - a.window + 1) / kBN : 0;
  const int nsteps = (ntiles - tile0 + 1) / 2;
  const int wave_last_tile = q_first / kBN;
  const int wave_first_tile = a.window > 0 ? max(0, q_first - a.window + 1) / kBN : 0;

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
  // With pre-rotated keys, the query is rotated here (fp16 operands).
  if constexpr (kRopeQ) rope_query(qa, qb2, hf, a.rope.pos0 + (uint32_t)q, a.rope.mode, a.rope);

  f32x16 O1[4], O2[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    O1[cb] = f32x16{};
    O2[cb] = f32x16{};
  }
  float m1 = kNoMax, m2 = kNoMax, l1 = 0.f, l2 = 0.f;
  const float c = a.c;
  const int ksw = kSwz(lq);

  const uint16_t* kb1 = a.k1 + (int64_t)b * a.sk1.b + (int64_t)head * a.sk1.h;
  const uint16_t* kb2 = a.k2 + (int64_t)b * a.sk2.b + (int64_t)head * a.sk2.h;
  const uint16_t* vbase = a.v + (int64_t)b * a.sv.b + (int64_t)head * a.sv.h;
  const StageOffsets soff = stage_offsets<0>(a, tid);
  KeyRes res;
  res.k1 = rows_rsrc(kb1, a.sk1.t, 0, kend, kDqk);
  res.k2 = rows_rsrc(kb2, a.sk2.t, 0, kend, kDqk);
  res.v = rows_rsrc(vbase, a.sv.t, 0, kend, kDv);
  res.ks1 = (uint32_t)(a.sk1.t * 2);
  res.ks2 = (uint32_t)(a.sk2.t * 2);
  res.vs = (uint32_t)(a.sv.t * 2);
  auto key0 = [&](int x) { return (tile0 + 2 * x + grp) * kBN; };  // first key of the group's tile of step x
  char* const slot0 = smem + grp * kTile;                          // the group's tile in stage 0
  auto live = [&](int j) { return wave_live && j >= wave_first_tile && j <= wave_last_tile; };

  // The epilogue's gain and lambda, fetched while the first tiles load.
  f32x4 gpre = f32x4{};
  float lpre = 0.f;
  if (tid < kDv / 4) gpre = *reinterpret_cast<const f32x4*>(a.gain + (int64_t)head * kDv + 4 * tid);
  if (tid == kDv / 4) lpre = a.lambda_h ? a.lambda_h[head] : a.lambda;

  // Prologue: tile 0 complete in slot 0, K(1) in slot 1, V(1) in registers
  // (wait: everything but the four V(1) loads).
  Staged st;
  pp_dma_k(res, soff, slot0, key0(0), wq);
  pp_load_v(st, res, soff, key0(0));
  pp_dma_k(res, soff, slot0 + kStage, key0(1), wq);
  stage_store<0>(st, smem, tid, nullptr);
  pp_load_v(st, res, soff, key0(1));
  if (tid < kDv / 4) gain_s[tid] = gpre;
  if (tid == kDv / 4) *lam_s = lpre;
  wait_vm<4>();
  wait_lds();
  phase_barrier();

  f16x8 p1a, p1b, p2a, p2b;
  {
    const int j = tile0 + grp;
    if (live(j)) {
      f32x16 s1, s2;
      scores_tile<kRopeQ>(smem + grp * kTile, lq, hf, ksw, qa, qb2, s1, s2);
      mask_tile(a, s1, s2, j, wave_last_tile, q_first, q, hf);
      softmax_step(s1, c, m1, l1, O1, p1a, p1b);
      softmax_step(s2, c, m2, l2, O2, p2a, p2b);
    }
  }
  // Every wave is done reading slot 0's keys before step 0 refills them.
  phase_barrier();
  if (grp == 1) phase_barrier();  // group 1 starts one phase late

  for (int it = 0; it < nsteps; ++it) {
    char* cur = smem + (it & 1) * kStage + grp * kTile;
    char* nxt = smem + ((it + 1) & 1) * kStage + grp * kTile;
    const int j = tile0 + 2 * it + grp;
    const bool next = it + 1 < nsteps && live(j + 2);
    // Matrix phase (raised issue priority: its products go first whenever
    // both waves of a SIMD are ready).
    __builtin_amdgcn_s_setprio(1);
    f32x16 s1, s2;
    const bool lj = live(j);
    if (lj) pv_pair(cur, lq, hf, 0, p1a, p1b, p2a, p2b, O1, O2);
    // K(it + 2) into slot it % 2, issued once the first products are queued.
    // Unconditional: past the last tile the loads read zeros (rows past kend)
    // into a slot nobody reads again, and the wait counts stay the same on
    // every iteration.
    __builtin_amdgcn_sched_barrier(0);
    pp_dma_k(res, soff, slot0 + (it & 1) * kStage, key0(it + 2), wq);
    __builtin_amdgcn_sched_barrier(0);
    if (lj) pv_pair(cur, lq, hf, 2, p1a, p1b, p2a, p2b, O1, O2);
    if (next) scores_tile<kRopeQ>(nxt, lq, hf, ksw, qa, qb2, s1, s2);
    __builtin_amdgcn_s_setprio(0);
    phase_barrier();
    // Vector phase.
    if (it + 1 < nsteps) stage_store<0>(st, smem + ((it + 1) & 1) * kStage, tid, nullptr);
    pp_load_v(st, res, soff, key0(it + 2));
    if (next) {
      mask_tile(a, s1, s2, j + 2, wave_last_tile, q_first, q, hf);
      softmax_step(s1, c, m1, l1, O1, p1a, p1b);
      softmax_step(s2, c, m2, l2, O2, p2a, p2b);
    }
    wait_vm<4>();  // K(it + 2) has landed; only the four V(it + 2) loads may be in flight
    wait_lds();    // V(it + 1) stored
    phase_barrier();
  }
  if (grp == 0) phase_barrier();
  wait_vm<0>();  // the zero-filling DMAs past the last tile, before the merge reuses the stages
  __syncthreads();

  merge_out<kTrain>(a, smem, grp, wq, lane, wave_live, *lam_s, b, head, q, hf, m1, l1, m2, l2, O1, O2);
  if (grp != 0 || !wave_live) return;
  norm_store(a, b, head, q, hf, O1, reinterpret_cast<const float*>(gain_s));
}

// Persistent form: workgroup w = r * B*H + bh runs the query blocks of row r
// and of row nqb - 1 - r of the longest-first order, both of (b, h) = bh,
// back to back: the longest block with the shortest, so one workgroup per CU
// carries the same work everywhere, and a head's blocks stay on the XCD that
// holds its keys in L2 (B*H a multiple of 8).  An odd middle row runs alone.
template <bool kTrain, bool kRopeQ>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_pp_kernel(PrefillArgs a) {
  // One LDS object (the stages, then the epilogue's gain and lambda): the
  // compiler then has no per-object alias scopes to go on and adds no waits
  // of its own for the key DMA before LDS reads; the explicit waits order them.
  __shared__ __attribute__((aligned(16))) char smem[kPPSmem];
  const int BH = a.B * a.H;
  const int nqb = (a.T + kBM - 1) / kBM;
  const int r = (int)blockIdx.x / BH, bh = (int)blockIdx.x % BH;
  pp_item<kTrain, kRopeQ>(a, smem, (int)blockIdx.x);
  if (nqb - 1 - r > r) {
    __syncthreads();  // the first block's epilogue is done with LDS
    pp_item<kTrain, kRopeQ>(a, smem, (nqb - 1 - r) * BH + bh);
  }
}

// kGroups wave groups of four waves share a workgroup's 128 queries and split
// its key tiles.  Two waves per SIMD (<= 256 VGPRs each): one wave's softmax
// VALU work overlaps the other's matrix products.
// kRope: the rotary embedding, fixed at compile time so the plain kernel
// carries none of its registers: 0 none; 1 split-half and 2 interleaved, with
// the key tiles rotated while staged; 3 keys rotated beforehand (fp16 copies
// moved by DMA like plain keys), the query rotated here in mode a.rope.mode.
template <int kGroups, int kRope>
__global__ void __launch_bounds__(64 * kGroupWaves * kGroups) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_kernel(PrefillArgs a) {
  constexpr int kStage = kGroups * kTile;  // one step: a tile for each group
  __shared__ __attribute__((aligned(16))) char smem[2 * kStage];
  __shared__ uint64_t rope_tab[32];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int grp = wave / kGroupWaves;  // which half of the key tiles
  const int wq = wave % kGroupWaves;   // which 32 queries
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

  const int q_first = qb * kBM + 32 * wq;  // first query of this wave
  const int q = q_first + lq;              // this lane's query
  const bool wave_live = q_first < a.T;
  const int ntiles = min(qb * (kBM / kBN) + (kBM / kBN), (a.T + kBN - 1) / kBN);
  const int kend = min(a.T, ntiles * kBN);
  // With a sliding window, tiles below every query's window are skipped.
  const int tile0 = a.window > 0 ? max(0, qb * kBM - a.window + 1) / kBN : 0;
  const int nsteps = (ntiles - tile0 + kGroups - 1) / kGroups;
  const int wave_last_tile = q_first / kBN;  // the wave's diagonal tile
  const int wave_first_tile = a.window > 0 ? max(0, q_first - a.window + 1) / kBN : 0;

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
  if constexpr (kRope == 3) {
    rope_query(qa, qb2, hf, a.rope.pos0 + (uint32_t)q, a.rope.mode, a.rope);
  } else if constexpr (kRope != 0) {
    // Phase table for the key tiles, then the lane's own query in registers.
    if (tid < 32) {
#pragma unroll
      for (int c = 0; c < 32; ++c)
        if (c == tid) rope_tab[c] = a.rope.phase[c];
    }
    rope_query(qa, qb2, hf, a.rope.pos0 + (uint32_t)q, kRope, a.rope);
    __syncthreads();
  }

  f32x16 O1[4], O2[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    O1[cb] = f32x16{};
    O2[cb] = f32x16{};
  }
  float m1 = kNoMax, m2 = kNoMax, l1 = 0.f, l2 = 0.f;
  const float c = a.c;
  const int ksw = kSwz(lq);

  const uint16_t* kb1 = a.k1 + (int64_t)b * a.sk1.b + (int64_t)head * a.sk1.h;
  const uint16_t* kb2 = a.k2 + (int64_t)b * a.sk2.b + (int64_t)head * a.sk2.h;
  const uint16_t* vbase = a.v + (int64_t)b * a.sv.b + (int64_t)head * a.sv.h;
  const StageOffsets soff = stage_offsets<kRope>(a, tid);

  Staged st;
  if constexpr (kRope == 0 || kRope == 3) stage_dma_k(a, kb1, kb2, soff, smem, tile0 * kBN, kend, tid);
  stage_load<kRope>(st, a, kb1, kb2, vbase, soff, tile0 * kBN, kend, tid);
  stage_store<kRope>(st, smem, tid, rope_tab);
  if constexpr (kRope == 0 || kRope == 3) wait_dma();
  __syncthreads();

  for (int it = 0; it < nsteps; ++it) {
    char* cur = smem + (it & 1) * kStage;
    char* nxt = smem + ((it + 1) & 1) * kStage;
    const bool more = it + 1 < nsteps;
    if (more) {
      if constexpr (kRope == 0 || kRope == 3)
        stage_dma_k(a, kb1, kb2, soff, nxt, (tile0 + (it + 1) * kGroups) * kBN, kend, tid);
      stage_load<kRope>(st, a, kb1, kb2, vbase, soff, (tile0 + (it + 1) * kGroups) * kBN, kend, tid);
    }

    const int j = tile0 + it * kGroups + grp;  // this group's tile
    if (wave_live && j >= wave_first_tile && j <= wave_last_tile) {
      const char* kt = cur + grp * kTile;
      f32x16 s1 = f32x16{}, s2 = f32x16{};
      const int krow = lq * kKRow;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int off = krow + (((2 * s + hf) ^ ksw) << 4);
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kt + off);
        const bf16x8 kb = *reinterpret_cast<const bf16x8*>(kt + kKBytes + off);
        if constexpr (kRope != 0) {
          // rotated operands are fp16 (see rope_query)
          s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, ka),
                                                      __builtin_bit_cast(f16x8, qa[s]), s1, 0, 0, 0);
          s2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, kb),
                                                      __builtin_bit_cast(f16x8, qb2[s]), s2, 0, 0, 0);
        } else {
          s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qa[s], s1, 0, 0, 0);
          s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, qb2[s], s2, 0, 0, 0);
        }
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
      if (a.window > 0 && j * kBN < q_first + 32 - a.window) {
        // Lower window edge: key k is visible to query q iff k > q - window.
        const int lim = q - a.window - j * kBN;  // key rows <= lim are too old
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int kr = 8 * (i >> 2) + 4 * hf + (i & 3);
          if (kr <= lim) {
            s1[i] = -__builtin_inff();
            s2[i] = -__builtin_inff();
          }
        }
      }
      f16x8 p1a, p1b, p2a, p2b;
      softmax_step(s1, c, m1, l1, O1, p1a, p1b);
      softmax_step(s2, c, m2, l2, O2, p2a, p2b);
      const char* vt = kt + 2 * kKBytes + lq * kVRow + hf * 16;
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

    if (more) stage_store<kRope>(st, nxt, tid, rope_tab);
    if constexpr (kRope == 0 || kRope == 3) wait_dma();
    __syncthreads();
  }

  // Fold group 1's states into group 0 (the stage memory is free: the last
  // loop iteration ended with a barrier after every read of it).
  if constexpr (kGroups == 2) {
    merge_map(smem, grp, wq, lane, wave_live, m1, l1, O1);
    merge_map(smem, grp, wq, lane, wave_live, m2, l2, O2);
  }
  if (grp != 0 || !wave_live) return;

  finish_rows(a, b, head, q, hf, m1, m2, l1, l2, O1, O2);
}

// Sliding-window streaming kernel.  With a window w, a wave's 32 queries see
// d + 1 key tiles, d = ceil((w - 1) / 32) before the diagonal one.  A workgroup
// of four waves takes kSwBlocks consecutive query blocks of one (b, h) and
// runs each block in d + 1 steps; at step s of block qb wave w computes key
// tile 4 qb - d + s + w, so every wave works every step (the lock-step
// one-tile-per-step loop leaves each wave idle on the block's other tiles).
// The four tiles of a step are consecutive, and the next step needs one more,
// so the tiles stream through a ring of five 16 KiB slots, one prefetched per
// step; with d = 4 (windows 98 .. 129) block qb + 1 starts on block qb's last
// four tiles and the stream never stalls.  V^T rows are 64 bytes with the
// chunk swizzle sw_vsw instead of padding, so two workgroups fit on a CU.
constexpr int kSwVRow = kBN * 2;                       // 64-byte V^T rows
constexpr int kSwTile = 2 * kKBytes + kDv * kSwVRow;  // 16 KiB
constexpr int kSwSlots = 5;
constexpr int kSwBlocks = 4;  // query blocks per workgroup

// Chunk swizzle of V^T row (channel) ch: 16-byte reads by 16 lanes of
// consecutive channels at one logical chunk hit 16 distinct bank groups.
__device__ __forceinline__ int sw_vsw(int ch) { return (ch >> 2) & 3; }

// V of one key tile, staged in registers by stage_load, to fp16 V^T rows:
// thread t holds keys 4(t % 8) .. +3 and channels 4(t / 8) .. +3; keys sit in
// kVPos order, 8 bytes per 4-key group.
__device__ __forceinline__ void sw_store_v(const Staged& st, char* tile, int t) {
  const int kg = t & 7, cg = t >> 3, pos = kVPos(kg);
  float e[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    e[r][0] = bf16_lo(st.v[r].x);
    e[r][1] = bf16_hi(st.v[r].x);
    e[r][2] = bf16_lo(st.v[r].y);
    e[r][3] = bf16_hi(st.v[r].y);
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int ch = 4 * cg + c;
    const f16x4 h = {(_Float16)e[0][c], (_Float16)e[1][c], (_Float16)e[2][c], (_Float16)e[3][c]};
    *reinterpret_cast<f16x4*>(tile + 2 * kKBytes + ch * kSwVRow + (((pos >> 1) ^ sw_vsw(ch)) << 4) + (pos & 1) * 8) =
        h;
  }
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
prefill_swa_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[kSwSlots * kSwTile];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, hf = lane >> 5, lq = lane & 31;
  const int nqb = (a.T + kBM - 1) / kBM;
  const int BH = a.B * a.H;
  const int bh = (int)blockIdx.x % BH, head = bh % a.H, b = bh / a.H;
  const int qb0 = ((int)blockIdx.x / BH) * kSwBlocks;
  const int qb1 = min(nqb, qb0 + kSwBlocks);
  const int d = (a.window - 1 + kBN - 1) / kBN;  // key tiles before a wave's diagonal one
  const float c = a.c;
  const int ksw = kSwz(lq);

  const uint16_t* kb1 = a.k1 + (int64_t)b * a.sk1.b + (int64_t)head * a.sk1.h;
  const uint16_t* kb2 = a.k2 + (int64_t)b * a.sk2.b + (int64_t)head * a.sk2.h;
  const uint16_t* vbase = a.v + (int64_t)b * a.sv.b + (int64_t)head * a.sv.h;
  const StageOffsets soff = stage_offsets<0>(a, tid);
  auto slot = [&](int k) { return smem + (k % kSwSlots) * kSwTile; };  // k >= 0
  Staged st;
  // Key tile k (k >= 0; rows at or past T read as zero): K_1, K_2 by DMA, V
  // through registers (stored by store_v once the loads are back).
  auto load_kv = [&](int k) {
    stage_dma_k(a, kb1, kb2, soff, slot(k), k * kBN, a.T, tid);
    stage_load<0>(st, a, kb1, kb2, vbase, soff, k * kBN, a.T, tid);
  };
  auto store_v = [&](int k) { sw_store_v(st, slot(k), tid); };

  bf16x8 qa[4], qb2[4];
  auto load_q = [&](int qb) {
    const int q = qb * kBM + 32 * wave + lq;
    const bool ok = q < a.T;
    const uint16_t* p1 = a.q1 + (int64_t)b * a.sq1.b + (int64_t)q * a.sq1.t + (int64_t)head * a.sq1.h + 8 * hf;
    const uint16_t* p2 = a.q2 + (int64_t)b * a.sq2.b + (int64_t)q * a.sq2.t + (int64_t)head * a.sq2.h + 8 * hf;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      qa[s] = __builtin_bit_cast(bf16x8, ok ? load16(p1 + 16 * s) : u32x4{0, 0, 0, 0});
      qb2[s] = __builtin_bit_cast(bf16x8, ok ? load16(p2 + 16 * s) : u32x4{0, 0, 0, 0});
    }
  };

  // Prologue: the first block's queries and the four tiles of its first step.
  load_q(qb0);
  for (int k = 4 * qb0 - d; k < 4 * qb0 - d + 4; ++k) {
    if (k < 0) continue;
    load_kv(k);
    store_v(k);
  }
  wait_dma();
  __syncthreads();

  f32x16 O1[4], O2[4];
  for (int qb = qb0; qb < qb1; ++qb) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      O1[cb] = f32x16{};
      O2[cb] = f32x16{};
    }
    float m1 = kNoMax, m2 = kNoMax, l1 = 0.f, l2 = 0.f;
    const int q_first = qb * kBM + 32 * wave, q = q_first + lq;
    const bool wave_live = q_first < a.T;
    const int wave_last_tile = q_first / kBN;
    for (int s = 0; s <= d; ++s) {
      const int t0 = 4 * qb - d + s;  // this step's first tile (wave w takes t0 + w)
      const bool last = s == d;
      // The next step's newest tile, when it is new and has a free slot (the
      // one of tile t0 - 1): always within a block, and at a block change
      // unless the window is exactly four tiles deep (nothing new then).
      const bool next_block = last && qb + 1 < qb1;
      const int pf = (!last || (next_block && d < 4)) ? t0 + 4 : -1;
      if (pf >= 0) load_kv(pf);

      const int j = t0 + wave;
      if (wave_live && j >= 0) {
        const char* kt = slot(j);
        f32x16 s1 = f32x16{}, s2 = f32x16{};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int off = lq * kKRow + (((2 * k + hf) ^ ksw) << 4);
          s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kt + off), qa[k], s1, 0, 0, 0);
          s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(kt + kKBytes + off), qb2[k],
                                                       s2, 0, 0, 0);
        }
        mask_tile(a, s1, s2, j, wave_last_tile, q_first, q, hf);
        f16x8 p1a, p1b, p2a, p2b;
        softmax_step(s1, c, m1, l1, O1, p1a, p1b);
        softmax_step(s2, c, m2, l2, O2, p2a, p2b);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int ch = 32 * cb + lq;
          const char* vr = kt + 2 * kKBytes + ch * kSwVRow;
          const f16x8 va0 = *reinterpret_cast<const f16x8*>(vr + ((hf ^ sw_vsw(ch)) << 4));
          const f16x8 va1 = *reinterpret_cast<const f16x8*>(vr + (((2 + hf) ^ sw_vsw(ch)) << 4));
          O1[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va0, p1a, O1[cb], 0, 0, 0);
          O2[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va0, p2a, O2[cb], 0, 0, 0);
          O1[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va1, p1b, O1[cb], 0, 0, 0);
          O2[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va1, p2b, O2[cb], 0, 0, 0);
        }
      }
      if (pf >= 0) store_v(pf);
      wait_dma();
      __syncthreads();
    }
    if (wave_live) finish_rows(a, b, head, q, hf, m1, m2, l1, l2, O1, O2);
    if (qb + 1 < qb1) {
      load_q(qb + 1);
      if (d < 3) {
        // A window under three tiles deep moves the next block's first step
        // past the prefetched tile: load the rest (their slots held tiles
        // before that step).
        for (int k = 4 * qb + 5; k < 4 * (qb + 1) - d + 4; ++k) {
          load_kv(k);
          store_v(k);
        }
        wait_dma();
        __syncthreads();
      }
    }
  }
}

}  // namespace

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  const int nqb = (a.T + kBM - 1) / kBM;
  const int64_t grid = (int64_t)nqb * a.B * a.H;
  // A grid that fits on the chip in one round (two 4-wave workgroups per CU)
  // leaves the CUs holding the longest query blocks working alone at the end;
  // splitting each workgroup's key range over two wave groups halves that
  // tail.  Larger grids balance by themselves in longest-first order and run
  // better as independent 4-wave workgroups.
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  const bool split = grid <= 2 * (int64_t)cus;
  const int64_t row_max = std::max(std::max(a.sk1.t, a.sk2.t), a.sv.t);
  // Keys already rotated (fp16 copies): they are staged like plain keys, and
  // only the queries turn inside the kernels.
  const bool prerot = a.rope.mode != 0 && a.keys_rotated;
  // The ping-pong kernel addresses a (b, h)'s key rows from one buffer base
  // with 32-bit offsets (up to about T + 192 rows).
  const bool pingpong = split && (a.rope.mode == 0 || prerot) && !(prerot && a.o1n != nullptr) &&
                        (int64_t)(a.T + 256) * row_max * 2 < (int64_t(1) << 31);
  // Windowed prefill without the rotary embedding or training outputs, at
  // most four tiles before the diagonal: the streaming kernel.
  if (a.window > 0 && a.rope.mode == 0 && a.o1n == nullptr && (a.window - 1 + kBN - 1) / kBN <= 4) {
    const int64_t chunks = (nqb + kSwBlocks - 1) / kSwBlocks;
    hipLaunchKernelGGL(prefill_swa_kernel, dim3((unsigned)(chunks * a.B * a.H)), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (pingpong) {
    const dim3 gp((unsigned)((int64_t)((nqb + 1) / 2) * a.B * a.H));
    if (prerot)
      hipLaunchKernelGGL((prefill_pp_kernel<false, true>), gp, dim3(512), 0, stream, a);
    else if (a.o1n != nullptr)
      hipLaunchKernelGGL((prefill_pp_kernel<true, false>), gp, dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_pp_kernel<false, false>), gp, dim3(512), 0, stream, a);
    return hipGetLastError();
  }
  const dim3 g((unsigned)grid), b1(64 * kGroupWaves), b2(64 * kGroupWaves * 2);
  if (prerot) {
    if (split)
      hipLaunchKernelGGL((prefill_kernel<2, 3>), g, b2, 0, stream, a);
    else
      hipLaunchKernelGGL((prefill_kernel<1, 3>), g, b1, 0, stream, a);
    return hipGetLastError();
  }
  switch (a.rope.mode * 2 + (split ? 1 : 0)) {
    case 0: hipLaunchKernelGGL((prefill_kernel<1, 0>), g, b1, 0, stream, a); break;
    case 1: hipLaunchKernelGGL((prefill_kernel<2, 0>), g, b2, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<1, 1>), g, b1, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((prefill_kernel<2, 1>), g, b2, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<1, 2>), g, b1, 0, stream, a); break;
    case 5: hipLaunchKernelGGL((prefill_kernel<2, 2>), g, b2, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace diffattn
