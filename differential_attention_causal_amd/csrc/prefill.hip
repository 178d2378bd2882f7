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
#include "prefill_tiles.h"

namespace diffattn {
namespace {

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
    if (tid < 32) rope_tab[tid] = rope_phase_at(a.rope, tid);
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
  // most four tiles before the diagonal: the streaming kernel (window.hip).
  if (prefill_window_kernel_fits(a)) return launch_prefill_window(a, stream);
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
