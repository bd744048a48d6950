// take (Nx_quant API docs, take): the rows (or whole matrices) of a packed part at given positions,
// copied as bytes with no value decoded; a position outside [0, src_rows) gives a zero row.  The
// caller gathers each part of a weight (codes, scales, biases, blocks) with its own row size.
// Workgroup (i, part) copies up to 32 KiB of output row i: 16-byte units when the row size and
// both buffers allow it, else 4-byte units, else bytes.
#include "device_common.hpp"
#include "launch.hpp"

namespace ql {
namespace {

constexpr int64_t kTakePart = 32768;  // bytes of a row per workgroup

template <int UNIT>
__global__ __launch_bounds__(256) void take_kernel(const int64_t* __restrict__ pos, int64_t parts,
                                                   const uint8_t* __restrict__ src, int64_t src_rows,
                                                   int64_t row_bytes, uint8_t* __restrict__ dst) {
  const int64_t i = blockIdx.x / parts;
  const int64_t part = blockIdx.x - i * parts;
  const int64_t p = pos[i];
  const bool in = p >= 0 && p < src_rows;
  const int64_t b0 = part * kTakePart;
  const int64_t b1 = min(row_bytes, b0 + kTakePart);
  uint8_t* d = dst + i * row_bytes;
  const uint8_t* sr = src + (in ? p : 0) * row_bytes;  // not read when out of range
  if (in) {  // uniform over the workgroup: the source is read only for a position in range
    for (int64_t b = b0 + (int64_t)threadIdx.x * UNIT; b < b1; b += 256 * UNIT) {
      if constexpr (UNIT == 16)
        *(u32x4_t*)(d + b) = *(const u32x4_t*)(sr + b);
      else if constexpr (UNIT == 4)
        *(uint32_t*)(d + b) = *(const uint32_t*)(sr + b);
      else
        d[b] = sr[b];
    }
  } else {
    for (int64_t b = b0 + (int64_t)threadIdx.x * UNIT; b < b1; b += 256 * UNIT) {
      if constexpr (UNIT == 16)
        *(u32x4_t*)(d + b) = u32x4_t{0u, 0u, 0u, 0u};
      else if constexpr (UNIT == 4)
        *(uint32_t*)(d + b) = 0u;
      else
        d[b] = 0;
    }
  }
}

}  // namespace

hipError_t launch_take(const int64_t* pos, int64_t n_pos, const void* src, int64_t src_rows, int64_t row_bytes,
                       void* dst, hipStream_t s) {
  const int64_t parts = (row_bytes + kTakePart - 1) / kTakePart;
  const unsigned grid = (unsigned)(n_pos * parts);
  const uintptr_t a = (uintptr_t)src | (uintptr_t)dst | (uintptr_t)row_bytes;
  if ((a & 15) == 0)
    take_kernel<16><<<grid, 256, 0, s>>>(pos, parts, (const uint8_t*)src, src_rows, row_bytes, (uint8_t*)dst);
  else if ((a & 3) == 0)
    take_kernel<4><<<grid, 256, 0, s>>>(pos, parts, (const uint8_t*)src, src_rows, row_bytes, (uint8_t*)dst);
  else
    take_kernel<1><<<grid, 256, 0, s>>>(pos, parts, (const uint8_t*)src, src_rows, row_bytes, (uint8_t*)dst);
  return hipGetLastError();
}

}  // namespace ql
