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
// take alternate key tiles and merge at the end (as the prefill does).
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
  const int64_t grid = (int64_t)((a.T + kBM - 1) / kBM) * a.B * a.nH;
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  if (grid <= 2 * (int64_t)cus)
    hipLaunchKernelGGL(grouped_attn_kernel<2>, dim3((unsigned)grid), dim3(512), 0, stream, a);
  else
    hipLaunchKernelGGL(grouped_attn_kernel<1>, dim3((unsigned)grid), dim3(256), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows = (int64_t)a.B * a.T * a.nS;
  hipLaunchKernelGGL(grouped_combine_kernel, dim3((unsigned)((rows + 7) / 8)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace diffattn
