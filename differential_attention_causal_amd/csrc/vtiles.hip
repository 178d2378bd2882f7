// The prefill's value tiles, converted and transposed once: V (bf16, [B, T,
// H, 128]) -> per (b, h) and 32-key tile an 8 KiB fp16 V^T tile laid out
// exactly as the prefill kernels hold it in LDS, so that they move it with
// buffer loads into LDS (no registers, no conversion in the key loop).
//
// Tile layout: row c (channel, 0..127) is 64 bytes = 32 keys.  Key
// k = 16s + 8m + 4h + r (s, m, h in {0, 1}, r in 0..3) sits at position
// 16s + 8h + 4m + r: the keys lane half h of a 32x32 score accumulator holds,
// in its register order, are then one 16-byte chunk (chunk 2s + h) of the row.
// Chunk j of row c is stored at chunk j ^ ((c >> 2) & 3), so the 16-byte reads
// of 16 consecutive rows (one per lane) at the same logical chunk touch 16
// distinct bank groups.  Keys at or past T are zero (their probabilities are
// zero, and zero values keep 0 * v finite).
#include "kernels.h"
#include "rope.h"
#include "tile.h"

namespace diffattn {
namespace {

constexpr int kThreads = 256;

// 16-byte accesses both ways with the transposition in LDS.  Loads: thread t takes the 16-byte chunk (t % 16) (channels
// 8 (t % 16) .. + 7) of key rows 2 (t / 16) and 2 (t / 16) + 1, a key pair
// that sits at adjacent positions of the tile (position bit 0 is key bit 0),
// so each of its channels becomes one 4-byte word of two fp16 keys, written
// into LDS at [channel][key position] (rows padded to 68 bytes: the words a
// wave writes at once fall on distinct banks but for pairs of channels 64
// apart).  Then each thread reads back two 16-byte output chunks (eight keys
// of one channel, four 4-byte reads) and stores them to consecutive
// addresses.
constexpr int kLdsRow = 68;  // bytes per channel row in LDS: 64 + 4 of padding

// Loads of tile g (flattened over (b, h, tile)) by thread t of the 256 of a
// workgroup: key rows kr, kr + 1 of the tile, channels ch0 .. ch0 + 7.
__device__ __forceinline__ void vtiles_load(const VTilesArgs& a, int64_t g, int t, u32x4 (&w)[2]) {
  const int j = (int)(g % a.ntiles);
  const int64_t bh = g / a.ntiles;
  const int h = (int)(bh % a.H);
  const int b = (int)(bh / a.H);
  const uint16_t* src = a.v + (int64_t)b * a.sv.b + (int64_t)h * a.sv.h;
  const int kr = 2 * (t >> 4), ch0 = 8 * (t & 15);  // key rows kr, kr + 1 of the tile; first channel
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int key = 32 * j + kr + u;
    w[u] = key < a.T ? *reinterpret_cast<const u32x4*>(src + (int64_t)key * a.sv.t + ch0) : u32x4{0, 0, 0, 0};
  }
}

// The loaded rows into lds (kDv * kLdsRow bytes, 16-byte aligned) as fp16
// words of two keys.
__device__ __forceinline__ void vtiles_transpose(const u32x4 (&w)[2], int t, char* lds) {
  const int kr = 2 * (t >> 4), ch0 = 8 * (t & 15);
  // position of key kr in its row: bits 2 and 3 swapped (see the file header); kr + 1 follows it
  const int pos = (kr & 16) | ((kr & 4) << 1) | ((kr & 8) >> 1) | (kr & 3);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // channels ch0 + 2i (low halves) and ch0 + 2i + 1 (high halves) of both keys
    const f16x2 lo = {(_Float16)bf16_lo(w[0][i]), (_Float16)bf16_lo(w[1][i])};
    const f16x2 hi = {(_Float16)bf16_hi(w[0][i]), (_Float16)bf16_hi(w[1][i])};
    *reinterpret_cast<f16x2*>(lds + (ch0 + 2 * i) * kLdsRow + pos * 2) = lo;
    *reinterpret_cast<f16x2*>(lds + (ch0 + 2 * i + 1) * kLdsRow + pos * 2) = hi;
  }
}

// Tile g's output chunks from lds (after a barrier) to the workspace.
__device__ __forceinline__ void vtiles_store(const VTilesArgs& a, int64_t g, int t, const char* lds) {
  char* dst = reinterpret_cast<char*>(a.out) + g * kVtTileBytes;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int q = t + 256 * u;                   // output chunk: row q / 4, stored chunk q % 4
    const int row = q >> 2;
    const int lc = (q & 3) ^ ((row >> 2) & 3);   // the logical chunk stored there
    const uint32_t* r = reinterpret_cast<const uint32_t*>(lds + row * kLdsRow + lc * 16);
    *reinterpret_cast<u32x4*>(dst + q * 16) = u32x4{r[0], r[1], r[2], r[3]};
  }
}

// Tile g by the 256 threads of one workgroup.
__device__ __forceinline__ void vtiles_tile(const VTilesArgs& a, int64_t g, int t, char* lds) {
  u32x4 w[2];
  vtiles_load(a, g, t, w);
  vtiles_transpose(w, t, lds);
  __syncthreads();
  vtiles_store(a, g, t, lds);
}

// Two tiles per workgroup, every load of both issued before the first
// conversion (one workgroup per tile: 46.0 against 42.8 us at B=8, T=4096,
// H=16; the same bytes).
constexpr int kTilesPerGroup = 2;
__global__ void __launch_bounds__(kThreads) vtiles_kernel(VTilesArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[kTilesPerGroup][kDv * kLdsRow];
  const int64_t tiles = (int64_t)a.B * a.H * a.ntiles;
  const int t = (int)threadIdx.x;
  u32x4 w[kTilesPerGroup][2];
#pragma unroll
  for (int x = 0; x < kTilesPerGroup; ++x) {
    const int64_t g = (int64_t)blockIdx.x * kTilesPerGroup + x;
    vtiles_load(a, g < tiles ? g : tiles - 1, t, w[x]);  // a last odd tile loads a valid tile twice
  }
#pragma unroll
  for (int x = 0; x < kTilesPerGroup; ++x) vtiles_transpose(w[x], t, lds[x]);
  __syncthreads();
#pragma unroll
  for (int x = 0; x < kTilesPerGroup; ++x) {
    const int64_t g = (int64_t)blockIdx.x * kTilesPerGroup + x;
    if (g < tiles) vtiles_store(a, g, t, lds[x]);
  }
}

// Both workspace pre-passes of a rotary prefill in one launch: workgroups
// below rope_blocks rotate the keys (32 key vectors each), the rest build one
// V^T tile each.  The two share no data, so one launch lets their memory
// traffic overlap and saves the gap between two launches; each workgroup
// computes exactly what the separate kernels compute.
struct PrepassArgs {
  RopeKeysArgs r;
  VTilesArgs t;
  int64_t rope_blocks;
};

__global__ void __launch_bounds__(kThreads) prepass_kernel(PrepassArgs p) {
  __shared__ __attribute__((aligned(16))) char lds[kDv * kLdsRow];
  const int64_t g = blockIdx.x;
  if (g < p.rope_blocks) {
    uint64_t* tab = reinterpret_cast<uint64_t*>(lds);
    if (threadIdx.x < 32) tab[threadIdx.x] = rope_phase_at(p.r.rope, (int)threadIdx.x);
    __syncthreads();
    rope_keys_block(p.r, g, (int)threadIdx.x, tab);
  } else {
    vtiles_tile(p.t, g - p.rope_blocks, (int)threadIdx.x, lds);
  }
}

}  // namespace

hipError_t launch_vtiles(const VTilesArgs& a, hipStream_t stream) {
  const int64_t tiles = (int64_t)a.B * a.H * a.ntiles;
  return launch_kernel(vtiles_kernel, dim3((unsigned)((tiles + kTilesPerGroup - 1) / kTilesPerGroup)),
                       dim3(kThreads), stream, a);
}

hipError_t launch_prepass(const RopeKeysArgs& r, const VTilesArgs& t, hipStream_t stream) {
  PrepassArgs p{r, t, ((int64_t)r.B * r.T * r.H + 31) / 32};
  const int64_t tiles = (int64_t)t.B * t.H * t.ntiles;
  return launch_kernel(prepass_kernel, dim3((unsigned)(p.rope_blocks + tiles)), dim3(kThreads), stream, p);
}

}  // namespace diffattn
