// Sliding-window causal differential-attention prefill for gfx950 (MI355X).
//
// Same result as the plain prefill kernels restricted to the window: query i
// sees keys i-W+1 .. i (the Motif 3 summary's sliding-window layers, section
// 2.1, with 128-token windows, section "Practical Implications").  Tile
// geometry, staging, products, mask and epilogue are the prefill kernels'
// (prefill_tiles.h); this file holds the streaming schedule.
#include "prefill_tiles.h"

namespace diffattn {
namespace {

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

// kRope: the keys arrive already rotated, as fp16 (the workspace pre-pass),
// and each block's queries turn at their positions once loaded; the score
// products then take fp16 operands, as in the other prefill kernels.
template <bool kRope>
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

  // Prologue: lambda, the first block's queries and the four tiles of its
  // first step, all loads issued before the first V store (one round trip).
  const float lam = head_lambda(a, head);
  load_q(qb0);
  {
    Staged st4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = 4 * qb0 - d + i;
      if (k < 0) continue;
      stage_dma_k(a, kb1, kb2, soff, slot(k), k * kBN, a.T, tid);
      stage_load<0>(st4[i], a, kb1, kb2, vbase, soff, k * kBN, a.T, tid);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = 4 * qb0 - d + i;
      if (k >= 0) sw_store_v(st4[i], slot(k), tid);
    }
  }
  wait_dma();
  __syncthreads();
  // With pre-rotated keys, a block's queries turn once they have landed (here
  // for the first block, in the epilogue before it for the others), as fp16.
  // The lane half goes in through an empty asm, which keeps the compiler from
  // hoisting the lanes' selected phases (32 registers) out of the block loop,
  // where they would stay live through every step (about 100 spilled
  // registers).
  auto rotate_q = [&](int qb) {
    if constexpr (kRope) {
      int h = hf;
      asm volatile("" : "+v"(h));
      rope_query_lean(qa, qb2, h, a.rope.pos0 + (uint32_t)(qb * kBM + 32 * wave + lq), a.rope.mode, a.rope);
    }
  };
  rotate_q(qb0);

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
      const int j = t0 + wave;
      const bool act = wave_live && j >= 0;
      const char* kt = slot(j < 0 ? 0 : j);
      f32x16 s1 = f32x16{}, s2 = f32x16{};
      if (act) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int off = lq * kKRow + (((2 * k + hf) ^ ksw) << 4);
          const bf16x8 k1v = *reinterpret_cast<const bf16x8*>(kt + off);
          const bf16x8 k2v = *reinterpret_cast<const bf16x8*>(kt + kKBytes + off);
          if constexpr (kRope) {
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, k1v), __builtin_bit_cast(f16x8, qa[k]),
                                                        s1, 0, 0, 0);
            s2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, k2v),
                                                        __builtin_bit_cast(f16x8, qb2[k]), s2, 0, 0, 0);
          } else {
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k1v, qa[k], s1, 0, 0, 0);
            s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k2v, qb2[k], s2, 0, 0, 0);
          }
        }
      }
      // The next tile's loads go out after the score products: a wait for the
      // query registers before the first product (which the compiler places
      // conservatively) then has nothing newer in flight to wait for.
      __builtin_amdgcn_sched_barrier(0);
      if (pf >= 0) load_kv(pf);
      __builtin_amdgcn_sched_barrier(0);
      if (act) {
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
    // Epilogue.  The next block's queries (unconditionally: rows at or past
    // T read as zero, and no second set of query registers is needed) and
    // the lane's two gains go out first and are waited for once the two maps
    // are combined, before any store.  Left to the compiler, the wait for the
    // queries would sit before the next block's first product, where it
    // would also cover each step's tile prefetch; a gain load after a store
    // would wait for that store.
    const bool more = qb + 1 < qb1;
    load_q(qb + 1);
    const f32x2 gl = load_lane_gain(a, head, lane);
    if (wave_live) combine_maps(lam, l1 + __shfl_xor(l1, 32), l2 + __shfl_xor(l2, 32), O1, O2);
    wait_vm<0>();
    if (more) rotate_q(qb + 1);
    if (wave_live) norm_store_g(a, b, head, q, hf, O1, LaneGain{gl.x, gl.y, hf});
    if (more) {
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

bool prefill_window_kernel_fits(const PrefillArgs& a) {
  return a.window > 0 && (a.rope.mode == 0 || a.keys_rotated) && a.o1n == nullptr &&
         (a.window - 1 + kBN - 1) / kBN <= 4;
}

hipError_t launch_prefill_window(const PrefillArgs& a, hipStream_t stream) {
  if (!prefill_window_kernel_fits(a)) return hipErrorInvalidValue;
  const int nqb = (a.T + kBM - 1) / kBM;
  const int64_t chunks = (nqb + kSwBlocks - 1) / kSwBlocks;
  const dim3 grid((unsigned)(chunks * a.B * a.H));
  if (a.rope.mode != 0) return launch_kernel(prefill_swa_kernel<true>, grid, dim3(256), stream, a);
  return launch_kernel(prefill_swa_kernel<false>, grid, dim3(256), stream, a);
}

}  // namespace diffattn
