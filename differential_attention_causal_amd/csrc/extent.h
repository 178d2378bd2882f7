// Byte extent of the rows a buffer resource covers.  Plain C++ (no HIP types),
// so the host-side tests compile it with a host compiler as well.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define DIFFATTN_HD __host__ __device__
#else
#define DIFFATTN_HD
#endif

namespace diffattn {

// num_records of a raw buffer resource over rows k0 .. kend-1 (row stride
// `stride` 16-bit elements, `row` elements used per row): the bytes from row
// k0's start to the end of row kend-1, 0 for no rows.  The field holds 32 bits;
// a longer extent is clamped to 2^32 - 1.  Loads through such a resource stay
// within 32 rows of k0 (a tile), which the library's stride limit keeps far
// below 2^32 bytes, so clamping never hides a valid row, and a tile that ends
// past kend lies within the last 32 rows, where the extent is exact.
DIFFATTN_HD inline uint32_t rows_extent_bytes(int64_t stride, int k0, int kend, int row) {
  if (kend <= k0) return 0;
  const int64_t bytes = ((int64_t)(kend - k0 - 1) * stride + row) * 2;
  return bytes >= (int64_t)0xFFFFFFFF ? 0xFFFFFFFFu : (uint32_t)bytes;
}

}  // namespace diffattn
