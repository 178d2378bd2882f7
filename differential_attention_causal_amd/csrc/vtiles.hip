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
#include "tile.h"

namespace diffattn {
namespace {

constexpr int kThreads = 256;

// One workgroup per tile.  Thread t converts keys 4kg .. 4kg+3 (kg = t % 8) of
// channels 4cg .. 4cg+3 (cg = t / 8): four 8-byte loads, four 8-byte stores of
// four keys of one channel each.  A wave's stores cover eight 64-byte rows.
__global__ void __launch_bounds__(kThreads) vtiles_kernel(VTilesArgs a) {
  const int64_t g = blockIdx.x;
  const int j = (int)(g % a.ntiles);
  const int64_t bh = g / a.ntiles;
  const int h = (int)(bh % a.H);
  const int b = (int)(bh / a.H);
  const int t = threadIdx.x, kg = t & 7, cg = t >> 3;
  const uint16_t* src = a.v + (int64_t)b * a.sv.b + (int64_t)h * a.sv.h + 4 * cg;
  u32x2 w[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int key = 32 * j + 4 * kg + r;
    w[r] = key < a.T ? *reinterpret_cast<const u32x2*>(src + (int64_t)key * a.sv.t) : u32x2{0, 0};
  }
  float e[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    e[r][0] = bf16_lo(w[r].x);
    e[r][1] = bf16_hi(w[r].x);
    e[r][2] = bf16_lo(w[r].y);
    e[r][3] = bf16_hi(w[r].y);
  }
  char* dst = reinterpret_cast<char*>(a.out) + g * kVtTileBytes;
  const int pos4 = kVPos(kg);  // position of the four keys, in units of 4
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int row = 4 * cg + c;
    const int chunk = (pos4 >> 1) ^ ((row >> 2) & 3);
    f16x4 hv = {(_Float16)e[0][c], (_Float16)e[1][c], (_Float16)e[2][c], (_Float16)e[3][c]};
    *reinterpret_cast<f16x4*>(dst + row * 64 + chunk * 16 + (pos4 & 1) * 8) = hv;
  }
}

}  // namespace

hipError_t launch_vtiles(const VTilesArgs& a, hipStream_t stream) {
  const int64_t tiles = (int64_t)a.B * a.H * a.ntiles;
  return launch_kernel(vtiles_kernel, dim3((unsigned)tiles), dim3(kThreads), stream, a);
}

}  // namespace diffattn
