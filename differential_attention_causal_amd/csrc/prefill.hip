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
// loaded, and a wave skips tiles past its own diagonal.  Two launch shapes:
//   - one group (4 waves): the default; two workgroups share a CU, and a grid
//     larger than the chip balances itself in longest-first order;
//   - two groups (8 waves) that take alternate tiles of the causal range
//     (group 0 the even ones, group 1 the odd ones), each with its own softmax
//     states and accumulators, merged through LDS at the end.  For a grid that
//     fits on the chip in one round, this halves the run time of the longest
//     query blocks, which would otherwise finish alone.
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
__device__ __forceinline__ u32x2 load8(const uint16_t* p) { return *reinterpret_cast<const u32x2*>(p); }

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
  if constexpr (kRope != 0) {
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

// kGroups wave groups of four waves share a workgroup's 128 queries and split
// its key tiles.  Two waves per SIMD (<= 256 VGPRs each): one wave's softmax
// VALU work overlaps the other's matrix products.
// kRope: the rotary embedding mode (0 none, 1 split-half, 2 interleaved),
// fixed at compile time so the plain kernel carries none of its registers.
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
  if constexpr (kRope != 0) {
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
  if constexpr (kRope == 0) stage_dma_k(a, kb1, kb2, soff, smem, tile0 * kBN, kend, tid);
  stage_load<kRope>(st, a, kb1, kb2, vbase, soff, tile0 * kBN, kend, tid);
  stage_store<kRope>(st, smem, tid, rope_tab);
  if constexpr (kRope == 0) wait_dma();
  __syncthreads();

  for (int it = 0; it < nsteps; ++it) {
    char* cur = smem + (it & 1) * kStage;
    char* nxt = smem + ((it + 1) & 1) * kStage;
    const bool more = it + 1 < nsteps;
    if (more) {
      if constexpr (kRope == 0) stage_dma_k(a, kb1, kb2, soff, nxt, (tile0 + (it + 1) * kGroups) * kBN, kend, tid);
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
    if constexpr (kRope == 0) wait_dma();
    __syncthreads();
  }

  // Fold group 1's states into group 0 (the stage memory is free: the last
  // loop iteration ended with a barrier after every read of it).
  if constexpr (kGroups == 2) {
    merge_map(smem, grp, wq, lane, wave_live, m1, l1, O1);
    merge_map(smem, grp, wq, lane, wave_live, m2, l2, O2);
  }
  if (grp != 0 || !wave_live) return;

  // Combine the two maps, then GroupNorm over the 128 channels of the query.
  // Lane (hf, lq) holds channels 32cb + 8(i/4) + 4hf + i%4; its partner lane
  // (lane ^ 32) holds the other 64.
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
  const dim3 g((unsigned)grid), b1(64 * kGroupWaves), b2(64 * kGroupWaves * 2);
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
