// Grouped differential attention with token-wise lambda and an output gate,
// for gfx950 (picx.dev summary of the Motif 3 report, section 2.2):
//   H_h = softmax(Q_h K_h^T * scale) V_h    causally, for every head h
//   D_s = H_s - lambda_t,s * H_(nS + s / g)  for signal head s (Repeat_g)
//   out_s = sigmoid(G_s) * D_s              (or D_s without a gate)
// Each head is one softmax map with its own values, so a noise head's map is
// computed once and shared by its g signal heads.  Two launches: every head's
// causal attention (normalised outputs to an fp32 workspace), longest query
// blocks first across all heads, then an elementwise kernel that forms D and
// applies the gate.
//
// The single-map kernel follows the prefill's layout: a workgroup owns 128
// queries of one (b, head), a wave 32 of them; S^T = K Q^T on
// v_mfma_f32_32x32x16_bf16 with Q^T in registers, lane-local online softmax
// (softmax_step), O^T = V^T P^T on v_mfma_f32_32x32x16_f16 with P in fp16 and
// V converted to fp16 on staging.  Key tiles reach LDS by buffer-load DMA.  A
// grid that fits on the chip in one round uses two groups of four waves that
// take alternate key tiles and merge at the end, in the prefill's ping-pong
// form (grouped_pp_kernel); larger grids use four-wave workgroups.
#include "kernels.h"
#include "tile.h"

namespace diffattn {
namespace {

constexpr int kBM = 128, kBN = 32;
constexpr int kKRow = kDqk * 2;
constexpr int kKBytes = kBN * kKRow;   // 4 KiB K tile
constexpr int kVRow = (kBN + 8) * 2;   // 80-byte V^T rows
constexpr int kVBytes = kDv * kVRow;   // 10 KiB
constexpr int kStage = kKBytes + kVBytes;

// V tile -> registers: thread t loads keys 4(t%8) .. +3, channels 4(t/8) .. +3.
__device__ __forceinline__ void load_vt(u32x2 (&w)[4], const uint16_t* vb, int64_t st, int k0, int kend, int tid) {
  const int kg = tid & 7, cg = tid >> 3;
  const __amdgpu_buffer_rsrc_t r = rows_rsrc(vb, st, k0, kend, kDv);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = __builtin_amdgcn_raw_buffer_load_b64(r, (uint32_t)(((4 * kg + i) * st + 4 * cg) * 2), 0, 0);
}

// ... -> LDS as fp16 V^T rows (channel-major, keys in kVPos order).
__device__ __forceinline__ void store_vt(const u32x2 (&w)[4], char* vt, int tid) {
  const int kg = tid & 7, cg = tid >> 3;
  char* d = vt + kVPos(kg) * 8;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int word = c >> 1;
    f16x4 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = (_Float16)((c & 1) ? bf16_hi(w[i][word]) : bf16_lo(w[i][word]));
    *reinterpret_cast<f16x4*>(d + (4 * cg + c) * kVRow) = h;
  }
}

template <int kGroups>
__global__ void __launch_bounds__(256 * kGroups) __attribute__((amdgpu_waves_per_eu(2, 2)))
grouped_attn_kernel(GroupedArgs a) {
  constexpr int kSmem = kGroups == 1 ? 2 * kStage : (4 * kStage > kMergeBytes ? 4 * kStage : kMergeBytes);
  __shared__ __attribute__((aligned(16))) char smem[kSmem];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, hf = lane >> 5, lq = lane & 31;
  const int grp = wave / 4, wq = wave % 4;
  const int nqb = (a.T + kBM - 1) / kBM, BH = a.B * a.nH;
  const int qb = nqb - 1 - (int)(blockIdx.x / BH);  // longest rows first
  const int bh = (int)(blockIdx.x % BH), head = bh % a.nH, b = bh / a.nH;
  const int q_first = qb * kBM + 32 * wq, q = q_first + lq;
  const bool wave_live = q_first < a.T, ok = q < a.T;
  const int ntiles = min(qb * (kBM / kBN) + kBM / kBN, (a.T + kBN - 1) / kBN);
  const int nsteps = (ntiles + kGroups - 1) / kGroups;
  const int kend = min(a.T, ntiles * kBN);
  const int last_tile = q_first / kBN;

  bf16x8 qa[4];
  {
    const uint16_t* p = a.q + (int64_t)b * a.sq.b + (int64_t)q * a.sq.t + (int64_t)head * a.sq.h + 8 * hf;
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[s] = ok ? *reinterpret_cast<const bf16x8*>(p + 16 * s) : bf16x8{};
  }
  const uint16_t* kb = a.k + (int64_t)b * a.sk.b + (int64_t)head * a.sk.h;
  const uint16_t* vb = a.v + (int64_t)b * a.sv.b + (int64_t)head * a.sv.h;
  // Threads 256t .. 256t+255 stage tile t of a step (group t's tile).  DMA:
  // thread fetches key row (tid%256)/8, logical chunk (tid%8) ^ kSwz(row).
  const int st_tile = tid / 256, tt = tid % 256, kr = tt >> 3;
  const uint32_t koff = (uint32_t)((kr * a.sk.t + 8 * ((tt & 7) ^ kSwz(kr))) * 2);

  f32x16 O[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  float m = kNoMax, l = 0.f;
  const float c = a.c;
  const int ksw = kSwz(lq);

  u32x2 vw[4];
  auto issue = [&](int step, char* st) {
    const int k0 = (step * kGroups + st_tile) * kBN;
    char* tile = st + st_tile * kStage;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rows_rsrc(kb, a.sk.t, k0, kend, kDqk),
                                             (lds_ptr_t)(tile + (tt >> 6) * 1024), 16, koff, 0, 0, 0);
    load_vt(vw, vb, a.sv.t, k0, kend, tt);
  };
  auto store = [&](char* st) { store_vt(vw, st + st_tile * kStage + kKBytes, tt); };
  issue(0, smem);
  store(smem);
  wait_dma();
  __syncthreads();

  for (int it = 0; it < nsteps; ++it) {
    char* cur = smem + (it & 1) * kGroups * kStage;
    char* nxt = smem + ((it + 1) & 1) * kGroups * kStage;
    const bool more = it + 1 < nsteps;
    if (more) issue(it + 1, nxt);
    const int j = it * kGroups + grp;
    if (wave_live && j <= last_tile) {
      const char* kt = cur + grp * kStage;
      f32x16 s = f32x16{};
#pragma unroll
      for (int k = 0; k < 4; ++k)
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(kt + lq * kKRow + (((2 * k + hf) ^ ksw) << 4)), qa[k], s, 0, 0, 0);
      if (j == last_tile) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (8 * (i >> 2) + 4 * hf + (i & 3) > lq) s[i] = -__builtin_inff();
      }
      f16x8 pa, pb;
      softmax_step(s, c, m, l, O, pa, pb);
      const char* vt = kt + kKBytes + lq * kVRow + hf * 16;
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(*reinterpret_cast<const f16x8*>(vt + cb * 32 * kVRow), pa,
                                                       O[cb], 0, 0, 0);
        O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(*reinterpret_cast<const f16x8*>(vt + cb * 32 * kVRow + 32),
                                                       pb, O[cb], 0, 0, 0);
      }
    }
    if (more) store(nxt);
    wait_dma();
    __syncthreads();
  }
  if constexpr (kGroups == 2) merge_map(smem, grp, wq, lane, wave_live, m, l, O);
  if (grp != 0) return;

  // Lane (hf, lq) holds channels 32cb + 8(i/4) + 4hf + i%4 of query lq; the
  // partner lane (lane ^ 32) the other 64, and half of the sum.
  l += __shfl_xor(l, 32);
  if (!ok) return;
  const float r = 1.0f / l;
  float* dst = a.hw + (((int64_t)b * a.T + q) * a.nH + head) * kDv;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = O[cb][4 * r4 + i] * r;
      *reinterpret_cast<f32x4*>(dst + 32 * cb + 8 * r4 + 4 * hf) = o;
    }
}

// Ping-pong split-key form of the single-map kernel (the prefill's ping-pong
// kernel with one map and per-head values): two groups of four waves on the
// same 128 queries take alternate key tiles, group 1 one phase behind group
// 0, so on every SIMD one wave's matrix phase (O += V P of its tile, then
// S = K Q^T of its next) runs beside the other wave's vector phase (softmax,
// V staging).  Keys come by DMA two steps ahead from buffer resources fixed
// for the kernel (the host keeps a head's key span under 2^31 bytes), values
// one step ahead through registers.  Workgroup r * B*nH + bh runs query-block
// rows r and nqb - 1 - r of (b, head) = bh back to back.
constexpr int kGStage = 2 * kStage;  // one step: a tile for each group
constexpr int kGSmem = 2 * kGStage > kMergeBytes ? 2 * kGStage : kMergeBytes;

__device__ __forceinline__ void gpp_block(const GroupedArgs& a, char* smem, int item) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / 4, wq = wave % 4;
  const int lane = tid & 63, hf = lane >> 5, lq = lane & 31, rt = tid & 255;
  const int nqb = (a.T + kBM - 1) / kBM, BH = a.B * a.nH;
  const int qb = nqb - 1 - item / BH;
  const int bh = item % BH, head = bh % a.nH, b = bh / a.nH;
  const int q_first = qb * kBM + 32 * wq, q = q_first + lq;
  const bool wave_live = q_first < a.T, ok = q < a.T;
  const int ntiles = min(qb * (kBM / kBN) + kBM / kBN, (a.T + kBN - 1) / kBN);
  const int nsteps = (ntiles + 1) / 2;
  const int kend = min(a.T, ntiles * kBN);
  const int last_tile = q_first / kBN;
  auto live = [&](int j) { return wave_live && j <= last_tile; };

  bf16x8 qa[4];
  {
    const uint16_t* p = a.q + (int64_t)b * a.sq.b + (int64_t)q * a.sq.t + (int64_t)head * a.sq.h + 8 * hf;
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[s] = ok ? *reinterpret_cast<const bf16x8*>(p + 16 * s) : bf16x8{};
  }
  const uint16_t* kb = a.k + (int64_t)b * a.sk.b + (int64_t)head * a.sk.h;
  const uint16_t* vb = a.v + (int64_t)b * a.sv.b + (int64_t)head * a.sv.h;
  const __amdgpu_buffer_rsrc_t rk = rows_rsrc(kb, a.sk.t, 0, kend, kDqk);
  const __amdgpu_buffer_rsrc_t rv = rows_rsrc(vb, a.sv.t, 0, kend, kDv);
  const uint32_t ks = (uint32_t)(a.sk.t * 2), vs = (uint32_t)(a.sv.t * 2);
  // DMA: thread rt of the group fetches key row rt / 8, logical chunk
  // (rt % 8) ^ kSwz(row), landing at chunk position rt of the group's tile.
  const int kr = rt >> 3;
  const uint32_t koff = (uint32_t)((kr * a.sk.t + 8 * ((rt & 7) ^ kSwz(kr))) * 2);
  // V loads: keys 4(rt % 8) .. +3, channels 4(rt / 8) .. +3 (see load_vt).
  const uint32_t voff = (uint32_t)((4 * (rt & 7) * a.sv.t + 4 * (rt >> 3)) * 2);
  auto key0 = [&](int x) { return (2 * x + grp) * kBN; };
  char* const slot0 = smem + grp * kStage;
  auto dma_k = [&](char* slot, int k0) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(slot + wq * 1024), 16, koff + (uint32_t)k0 * ks, 0, 0,
                                             0);
  };
  u32x2 vw[4];
  auto load_v = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) vw[i] = __builtin_amdgcn_raw_buffer_load_b64(rv, voff + (uint32_t)(k0 + i) * vs, 0, 0);
  };

  f32x16 O[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  float m = kNoMax, l = 0.f;
  const float c = a.c;
  const int ksw = kSwz(lq);
  auto scores = [&](const char* kt) {
    f32x16 s = f32x16{};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *reinterpret_cast<const bf16x8*>(kt + lq * kKRow + (((2 * k + hf) ^ ksw) << 4)), qa[k], s, 0, 0, 0);
    return s;
  };
  auto mask = [&](f32x16& s, int j) {
    if (j == last_tile) {
      // key row 8(i/4) + 4hf + i%4 of tile j is key 32j + row: visible iff <= q
      const int hi = q - j * kBN - 4 * hf;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + (i & 3) > hi) s[i] = -__builtin_inff();
    }
  };
  // O += V^T P for channel blocks cb, cb + 1 (consecutive products on
  // different accumulators).
  auto pv_pair = [&](const char* kt, int cb, const f16x8& pa, const f16x8& pb) {
    const char* vt = kt + kKBytes + lq * kVRow + hf * 16 + cb * 32 * kVRow;
    const f16x8 a0 = *reinterpret_cast<const f16x8*>(vt), b0 = *reinterpret_cast<const f16x8*>(vt + 32 * kVRow);
    O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, pa, O[cb], 0, 0, 0);
    O[cb + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0, pa, O[cb + 1], 0, 0, 0);
    const f16x8 a1 = *reinterpret_cast<const f16x8*>(vt + 32),
                b1 = *reinterpret_cast<const f16x8*>(vt + 32 * kVRow + 32);
    O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, pb, O[cb], 0, 0, 0);
    O[cb + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b1, pb, O[cb + 1], 0, 0, 0);
  };

  // Prologue: tile 0 complete in slot 0, K(1) in slot 1, V(1) in registers.
  dma_k(slot0, key0(0));
  load_v(key0(0));
  dma_k(slot0 + kGStage, key0(1));
  store_vt(vw, slot0 + kKBytes, rt);
  load_v(key0(1));
  wait_vm<4>();
  wait_lds();
  phase_barrier();
  f16x8 pa, pb;
  if (live(grp)) {
    f32x16 s = scores(slot0);
    mask(s, grp);
    softmax_step(s, c, m, l, O, pa, pb);
  }
  // Every wave is done reading slot 0's keys before step 0 refills them.
  phase_barrier();
  if (grp == 1) phase_barrier();  // group 1 starts one phase late

  for (int it = 0; it < nsteps; ++it) {
    char* cur = smem + (it & 1) * kGStage + grp * kStage;
    char* nxt = smem + ((it + 1) & 1) * kGStage + grp * kStage;
    const int j = 2 * it + grp;
    const bool next = it + 1 < nsteps && live(j + 2);
    // Matrix phase.
    __builtin_amdgcn_s_setprio(1);
    f32x16 s;
    const bool lj = live(j);
    if (lj) pv_pair(cur, 0, pa, pb);
    // K(it + 2) into slot it % 2 (unconditional: past the last tile the
    // loads read zeros into a slot nobody reads again).
    __builtin_amdgcn_sched_barrier(0);
    dma_k(slot0 + (it & 1) * kGStage, key0(it + 2));
    __builtin_amdgcn_sched_barrier(0);
    if (lj) pv_pair(cur, 2, pa, pb);
    if (next) s = scores(nxt);
    __builtin_amdgcn_s_setprio(0);
    phase_barrier();
    // Vector phase.
    if (it + 1 < nsteps) store_vt(vw, nxt + kKBytes, rt);
    load_v(key0(it + 2));
    if (next) {
      mask(s, j + 2);
      softmax_step(s, c, m, l, O, pa, pb);
    }
    wait_vm<4>();  // K(it + 2) has landed; only the four V(it + 2) loads may be in flight
    wait_lds();    // V(it + 1) stored
    phase_barrier();
  }
  if (grp == 0) phase_barrier();
  wait_vm<0>();  // the zero-filling loads past the last tile, before the merge reuses LDS
  __syncthreads();

  merge_map(smem, grp, wq, lane, wave_live, m, l, O);
  if (grp != 0) return;
  l += __shfl_xor(l, 32);
  if (!ok) return;
  const float r = 1.0f / l;
  float* dst = a.hw + (((int64_t)b * a.T + q) * a.nH + head) * kDv;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = O[cb][4 * r4 + i] * r;
      *reinterpret_cast<f32x4*>(dst + 32 * cb + 8 * r4 + 4 * hf) = o;
    }
}

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
grouped_pp_kernel(GroupedArgs a) {
  // One LDS object: no per-object alias scopes, so the compiler adds no waits
  // of its own for the key DMA before LDS reads (the explicit ones order them).
  __shared__ __attribute__((aligned(16))) char smem[kGSmem];
  const int BH = a.B * a.nH;
  const int nqb = (a.T + kBM - 1) / kBM;
  const int r = (int)blockIdx.x / BH, bh = (int)blockIdx.x % BH;
  gpp_block(a, smem, (int)blockIdx.x);
  if (nqb - 1 - r > r) {
    __syncthreads();  // the first block's epilogue is done with LDS
    gpp_block(a, smem, (nqb - 1 - r) * BH + bh);
  }
}

// The same ping-pong form with fp16 V^T tiles (vtiles.hip): keys and values
// both come by DMA, and no V conversion is left in the key loop.
// Each group cycles through kVtGSlots slots: tile x sits in slot x % kVtGSlots,
// K(x + kVtGSlots) goes into slot x's key half in the matrix phase of step x
// (K(x) was read in the step before) and V(x + kVtGSlots) into its value half
// in the vector phase (the matrix phase has read V(x)).  Workgroups run
// query-block rows r and nqb - 1 - r of one (b, head) back to back.
constexpr int kVtGTile = kKBytes + kVtTileBytes;  // a group's key and V^T tiles
constexpr int kVtGStage = 2 * kVtGTile;             // one slot of both groups
constexpr int kVtGSlots = 4;
constexpr int kVtGSmem = kVtGSlots * kVtGStage > kMergeBytes ? kVtGSlots * kVtGStage : kMergeBytes;
// Vector-memory instructions issued after K(x + 2) by the time the vector
// phase of step x ends: V(x + 2), then K(y), V(y) for y = x + 3 .. x + slots
// (one key instruction, two value instructions per tile).
constexpr int kVtGYounger = 2 + 3 * (kVtGSlots - 2);

__device__ __forceinline__ void gppvt_block(const GroupedArgs& a, char* smem, int item) {
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave / 4, wq = wave % 4;
  const int lane = tid & 63, hf = lane >> 5, lq = lane & 31, rt = tid & 255;
  const int nqb = (a.T + kBM - 1) / kBM, BH = a.B * a.nH;
  const int qb = nqb - 1 - item / BH;
  const int bh = item % BH, head = bh % a.nH, b = bh / a.nH;
  const int q_first = qb * kBM + 32 * wq, q = q_first + lq;
  const bool wave_live = q_first < a.T, ok = q < a.T;
  const int ntiles = min(qb * (kBM / kBN) + kBM / kBN, (a.T + kBN - 1) / kBN);
  const int nsteps = (ntiles + 1) / 2;
  const int kend = min(a.T, ntiles * kBN);
  const int last_tile = q_first / kBN;
  auto live = [&](int j) { return wave_live && j <= last_tile; };

  const uint16_t* kb = a.k + (int64_t)b * a.sk.b + (int64_t)head * a.sk.h;
  const __amdgpu_buffer_rsrc_t rk = rows_rsrc(kb, a.sk.t, 0, kend, kDqk);
  const __amdgpu_buffer_rsrc_t rvt = vt_tiles_rsrc(a.vt, (int64_t)b * a.nH + head, a.T);
  const uint32_t ks = (uint32_t)(a.sk.t * 2);
  // DMA: thread rt of the group fetches key row rt / 8, logical chunk
  // (rt % 8) ^ kSwz(row), landing at chunk position rt of the group's tile.
  const int kr = rt >> 3;
  const uint32_t koff = (uint32_t)((kr * a.sk.t + 8 * ((rt & 7) ^ kSwz(kr))) * 2);
  auto key0 = [&](int x) { return (2 * x + grp) * kBN; };  // first key of the group's tile of step x
  char* const slot0 = smem + grp * kVtGTile;
  auto slot = [&](int x) { return slot0 + (x % kVtGSlots) * kVtGStage; };
  auto dma_k = [&](int x) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(slot(x) + wq * 1024), 16, koff + (uint32_t)key0(x) * ks,
                                             0, 0, 0);
  };
  auto dma_v = [&](int x) { dma_vt(rvt, slot(x) + kKBytes, 2 * x + grp, wq, lane); };

  // Prologue: the first three tiles' DMAs go out first, the queries load
  // under their latency, then the rest of the slots fill; the wait leaves
  // only V(1) .. V(slots - 1) and K(2) .. K(slots - 1) in flight.
  dma_k(0);
  dma_v(0);
  dma_k(1);
  bf16x8 qa[4];
  {
    const uint16_t* p = a.q + (int64_t)b * a.sq.b + (int64_t)q * a.sq.t + (int64_t)head * a.sq.h + 8 * hf;
#pragma unroll
    for (int s = 0; s < 4; ++s) qa[s] = ok ? *reinterpret_cast<const bf16x8*>(p + 16 * s) : bf16x8{};
  }
  dma_v(1);
#pragma unroll
  for (int x = 2; x < kVtGSlots; ++x) {
    dma_k(x);
    dma_v(x);
  }
  wait_vm<kVtGYounger>();
  wait_lds();
  phase_barrier();

  f32x16 O[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  float m = kNoMax, l = 0.f;
  const float c = a.c;
  const int ksw = kSwz(lq);
  auto scores = [&](const char* kt) {
    f32x16 s = f32x16{};
#pragma unroll
    for (int k = 0; k < 4; ++k)
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *reinterpret_cast<const bf16x8*>(kt + lq * kKRow + (((2 * k + hf) ^ ksw) << 4)), qa[k], s, 0, 0, 0);
    return s;
  };
  auto mask = [&](f32x16& s, int j) {
    if (j == last_tile) {
      // key row 8(i/4) + 4hf + i%4 of tile j is key 32j + row: visible iff <= q
      const int hi = q - j * kBN - 4 * hf;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + (i & 3) > hi) s[i] = -__builtin_inff();
    }
  };
  // O += V^T P for channel blocks cb, cb + 1 (consecutive products on
  // different accumulators).
  auto pv_pair = [&](const char* st, int cb, const f16x8& pa, const f16x8& pb) {
    const char* vt = st + kKBytes;
    const f16x8 a0 = vt_operand(vt, lq, hf, cb, 0), b0 = vt_operand(vt, lq, hf, cb + 1, 0);
    O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a0, pa, O[cb], 0, 0, 0);
    O[cb + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b0, pa, O[cb + 1], 0, 0, 0);
    const f16x8 a1 = vt_operand(vt, lq, hf, cb, 1), b1 = vt_operand(vt, lq, hf, cb + 1, 1);
    O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a1, pb, O[cb], 0, 0, 0);
    O[cb + 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b1, pb, O[cb + 1], 0, 0, 0);
  };

  // The ping-pong from the first tile: group 0 takes its first scores, then
  // its softmax beside group 1's first scores, then its step 0 matrix phase
  // beside group 1's first softmax.  Each group reads its slot 0's keys
  // before the barrier that precedes their refill.
  f16x8 pa, pb;
  {
    const bool l0 = live(grp);
    f32x16 s;
    if (grp == 0 && l0) s = scores(slot(0));
    phase_barrier();
    if (grp == 1 && l0) s = scores(slot(0));
    if (grp == 0 && l0) {
      mask(s, 0);
      softmax_step(s, c, m, l, O, pa, pb);
    }
    phase_barrier();
    if (grp == 1) {
      if (l0) {
        mask(s, 1);
        softmax_step(s, c, m, l, O, pa, pb);
      }
      phase_barrier();  // group 0's step 0 matrix phase is done
    }
  }

  for (int it = 0; it < nsteps; ++it) {
    char* cur = slot(it);
    char* nxt = slot(it + 1);
    const int j = 2 * it + grp;
    const bool next = it + 1 < nsteps && live(j + 2);
    // Matrix phase (raised issue priority: its products go first whenever
    // both waves of a SIMD are ready).
    __builtin_amdgcn_s_setprio(1);
    f32x16 s;
    const bool lj = live(j);
    if (lj) pv_pair(cur, 0, pa, pb);
    // K(it + slots) into slot it's key half, issued once the first products
    // are queued.  Unconditional: past the last tile the loads read zeros
    // into a slot nobody reads again, and the wait counts stay the same on
    // every iteration.
    __builtin_amdgcn_sched_barrier(0);
    dma_k(it + kVtGSlots);
    __builtin_amdgcn_sched_barrier(0);
    if (lj) pv_pair(cur, 2, pa, pb);
    if (next) s = scores(nxt);
    __builtin_amdgcn_s_setprio(0);
    phase_barrier();
    // Vector phase: V(it + slots) into slot it's value half (every wave of
    // the group has read V(it)), then the softmax of the next tile.
    dma_v(it + kVtGSlots);
    if (next) {
      mask(s, j + 2);
      softmax_step(s, c, m, l, O, pa, pb);
    }
    wait_vm<kVtGYounger>();  // K(it + 2) and V(it + 1) have landed
    phase_barrier();
  }
  if (grp == 0) phase_barrier();
  wait_vm<0>();  // the zero-filling loads past the last tile, before the merge reuses LDS
  __syncthreads();

  merge_map(smem, grp, wq, lane, wave_live, m, l, O);
  if (grp != 0) return;
  l += __shfl_xor(l, 32);
  if (!ok) return;
  const float r = 1.0f / l;
  float* dst = a.hw + (((int64_t)b * a.T + q) * a.nH + head) * kDv;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      f32x4 o;
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = O[cb][4 * r4 + i] * r;
      *reinterpret_cast<f32x4*>(dst + 32 * cb + 8 * r4 + 4 * hf) = o;
    }
}

__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2)))
grouped_ppvt_kernel(GroupedArgs a) {
  // One LDS object: no per-object alias scopes, so the compiler adds no waits
  // of its own for the DMAs before LDS reads (the explicit ones order them).
  __shared__ __attribute__((aligned(16))) char smem[kVtGSmem];
  const int BH = a.B * a.nH;
  const int nqb = (a.T + kBM - 1) / kBM;
  const int rows = (nqb + 1) / 2;
  // Workgroup w runs on XCD w % 8.  With B * nH a multiple of 8, XCD x takes
  // heads x, x + 8, ... one after another, every row of a head before the
  // next, so its L2 holds the keys and values of few heads at a time.
  const int w = (int)blockIdx.x;
  int r, bh;
  if (BH % 8 == 0) {
    const int xcd = w & 7, s = w >> 3;
    bh = (s / rows) * 8 + xcd;
    r = s % rows;
  } else {
    r = w / BH;
    bh = w % BH;
  }
  gppvt_block(a, smem, r * BH + bh);
  if (nqb - 1 - r > r) {
    __syncthreads();  // the first block's epilogue is done with LDS
    gppvt_block(a, smem, (nqb - 1 - r) * BH + bh);
  }
}

// out_s = sigmoid(G_s) * (H_s - lambda_t,s * H_(nS + s / g)): 32 threads per
// (b, t, s) row, four channels each.
__global__ void __launch_bounds__(256) grouped_combine_kernel(GroupedArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);  // (b * T + t) * nS + s
  if (row >= (int64_t)a.B * a.T * a.nS) return;
  const int ch = 4 * (threadIdx.x & 31);
  const int s = (int)(row % a.nS);
  const int64_t bt = row / a.nS;
  const f32x4 hs = *reinterpret_cast<const f32x4*>(a.hw + (bt * a.nH + s) * kDv + ch);
  const f32x4 hn = *reinterpret_cast<const f32x4*>(a.hw + (bt * a.nH + a.nS + s / a.g) * kDv + ch);
  const float lam = a.lam[row];
  f32x4 y;
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = hs[i] - lam * hn[i];
  if (a.gate) {
    const u32x2 gw = *reinterpret_cast<const u32x2*>(a.gate + row * kDv + ch);
    const float gv[4] = {bf16_lo(gw.x), bf16_hi(gw.x), bf16_lo(gw.y), bf16_hi(gw.y)};
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] *= 1.0f / (1.0f + __builtin_amdgcn_exp2f(-gv[i] * 1.4426950408889634f));
  }
  if (a.out_f32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + row * kDv + ch) = y;
  } else {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const bf16x4 yb = {(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
    *reinterpret_cast<bf16x4*>(static_cast<uint16_t*>(a.out) + row * kDv + ch) = yb;
  }
}

}  // namespace

hipError_t launch_grouped(const GroupedArgs& a, hipStream_t stream) {
  const int64_t nqb = (a.T + kBM - 1) / kBM;
  const int64_t grid = nqb * a.B * a.nH;
  const int64_t cus = device_cu_count();
  const int64_t pairs = (nqb + 1) / 2 * a.B * a.nH;
  // The V^T form's workgroups all carry equal work (a long block with a
  // short one), so its grid must fill its rounds (a last round nearly empty
  // costs a whole round), and its pre-pass (V read and written once) pays
  // off against a one-round grid of the register-staged ping-pong kernel
  // only for long sequences.  Measured, 16 heads: B=1, T=16384 1071 against
  // 1285 us (four-wave kernel); B=1, T=4096 97.7 against 95.3 us; B=4,
  // T=1100 (288 pairs: two rounds, the second an eighth full) 81 against 57.
  const int64_t rounds = (pairs + cus - 1) / cus;
  const bool filled = pairs * 10 >= rounds * cus * 9;
  const bool one_round = grid <= 2 * cus;
  hipError_t e;
  if (a.vt != nullptr && filled && (!one_round || a.T >= 8192)) {
    if ((e = launch_vtiles(make_vtiles_args(a.v, a.sv, a.B, a.T, a.nH, const_cast<uint16_t*>(a.vt)), stream)) !=
        hipSuccess)
      return e;
    e = launch_kernel(grouped_ppvt_kernel, dim3((unsigned)pairs), dim3(512), stream, a);
  } else if (one_round) {
    // The register-staged ping-pong form addresses a head's key and value
    // rows from one buffer base with 32-bit offsets (up to about T + 192 rows).
    const int64_t row_max = a.sk.t > a.sv.t ? a.sk.t : a.sv.t;
    if ((int64_t)(a.T + 256) * row_max * 2 < (int64_t(1) << 31))
      e = launch_kernel(grouped_pp_kernel, dim3((unsigned)pairs), dim3(512), stream, a);
    else
      e = launch_kernel(grouped_attn_kernel<2>, dim3((unsigned)grid), dim3(512), stream, a);
  } else {
    e = launch_kernel(grouped_attn_kernel<1>, dim3((unsigned)grid), dim3(256), stream, a);
  }
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)a.B * a.T * a.nS;
  return launch_kernel(grouped_combine_kernel, dim3((unsigned)((rows + 7) / 8)), dim3(256), stream, a);
}

}  // namespace diffattn
