// Internal launchers called by the C ABI layer after host validation.  Each returns the
// hipError_t of its launch(es).  Shapes are already checked: kernels may assume them.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

// Device problem descriptor of one GEMV (mirrors ql_problem without the per-list constants).
struct GemvDesc {
  const void* x;
  const uint32_t* packed;
  const void* scales;
  const void* biases;
  const void* layer_bias;
  void* y;
  int64_t m, n, k;
  int32_t bits, group_size;
};

// GEMV work split: lanes_per_row lanes of a wave share a row, each streaming 16-byte chunks
// of packed words; each lane keeps rows_per_lane rows in flight; rows_per_wg rows go to one
// 256-thread (4-wave) workgroup.  Shared by the host (grid size) and the kernel.
struct GemvGeom {
  int lanes_per_row;    // largest power of two <= 64 dividing the 16-byte chunks of a row
  int chunks_per_lane;  // chunks of a row / lanes_per_row
  int rows_per_lane;
  int rows_per_wg;      // 4 waves * (64 / lanes_per_row) * rows_per_lane
};
// Template row count M_T (1, 2, 4 or 8) a GEMV of m rows runs with.
__host__ __device__ inline int gemv_mt(int64_t m) { return m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : 8; }
__host__ __device__ inline int gemv_rows_per_lane(int mt) { return mt <= 2 ? 4 : 2; }
__host__ __device__ inline GemvGeom gemv_geometry(int64_t k, int bits, int mt) {
  GemvGeom g;
  const int64_t chunks = k * bits / 128;
  int L = 64;
  while (L > 1 && (chunks % L) != 0) L >>= 1;
  g.lanes_per_row = L;
  g.chunks_per_lane = (int)(chunks / L);
  g.rows_per_lane = gemv_rows_per_lane(mt);
  g.rows_per_wg = 4 * (64 / L) * g.rows_per_lane;
  return g;
}

hipError_t launch_quantize(const float* w, int64_t n, int64_t k, int bits, int g, int pdt, uint32_t* packed,
                           void* scales, void* biases, hipStream_t s);
hipError_t launch_dequant_affine(const uint32_t* packed, const void* scales, const void* biases, int pdt,
                                 int64_t rows, int64_t k, int bits, int g, void* out, int odt, hipStream_t s);
hipError_t launch_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k, void* out,
                                int odt, hipStream_t s);
hipError_t launch_dequant_q8_0(const uint8_t* blocks, int64_t rows, int64_t k, void* out, int odt, hipStream_t s);

// One GEMV (desc passed by value) or a device table of `count` descs with tile prefix
// `tile_start[count+1]` (all descs of the table share m, bits and group size).
hipError_t launch_gemv(const GemvDesc& single, const GemvDesc* table, const int64_t* tile_start, int count,
                       int64_t total_tiles, int m, int bits, int xdt, int pdt, int ydt, hipStream_t s);

hipError_t launch_gemm(const void* x, int xdt, int64_t m, int64_t k, const uint32_t* packed, const void* scales,
                       const void* biases, int pdt, int64_t n, int bits, int g, const void* layer_bias, void* y,
                       int ydt, void* ws, hipStream_t s);
size_t gemm_workspace_bytes(int64_t m, int64_t k, int g);

hipError_t launch_route(const int64_t* ids, int64_t n_pos, int64_t e, int32_t* offsets, int32_t* perm,
                        hipStream_t s);
hipError_t launch_apply_experts(int fmt, const void* w0, const void* w1, int64_t e, int64_t n, int64_t k,
                                const int64_t* ids, int64_t n_pos, const void* x, int xdt, int64_t pos_per_row,
                                void* y, int ydt, int32_t* offsets, int32_t* perm, hipStream_t s);

}  // namespace ql
