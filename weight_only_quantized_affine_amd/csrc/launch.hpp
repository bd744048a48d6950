// Internal launchers called by the C ABI layer after host validation.  Each returns the
// hipError_t of its launch(es).  Shapes are already checked: kernels may assume them.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

// Device problem descriptor of one GEMV (mirrors ql_problem plus the host-chosen batch count).
struct GemvDesc {
  const void* x;
  const uint32_t* packed;
  const void* scales;
  const void* biases;
  const void* layer_bias;
  void* y;
  int64_t m, n, k;
  int32_t bits, group_size;
  int32_t batches;  // row batches per workgroup (see GemvGeom)
  int32_t pad_;
};
// Tile of a problem list: problem index in the device table and tile index inside the problem.
struct GemvTile {
  int32_t prob;
  int32_t local;
};

// GEMV work split: a row is cut into 16-byte chunks of packed words; lanes_per_row lanes of a
// wave share a row, each streaming chunks and holding GEMV_ROWS_PER_LANE rows; a 256-thread
// (4-wave) workgroup walks `batches` sets of 4 * (64 / lanes_per_row) * GEMV_ROWS_PER_LANE rows.
// Shared by the host (grid, tiles) and the kernel.
#ifndef GEMV_ROWS_PER_LANE
#define GEMV_ROWS_PER_LANE 2
#endif
#ifndef GEMV_WG_BYTES
#define GEMV_WG_BYTES 65536
#endif
struct GemvGeom {
  int chunks;           // 16-byte chunks per row
  int lanes_per_row;    // largest power of two <= 64 dividing `chunks`
  int chunks_per_lane;  // chunks / lanes_per_row
  int batches;
  int64_t rows_per_wg;  // 4 waves * (64 / lanes_per_row) * GEMV_ROWS_PER_LANE * batches
};
// Template row count M_T (1, 2, 4 or 8) a GEMV of m rows runs with.
__host__ __device__ inline int gemv_mt(int64_t m) { return m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : 8; }
__host__ __device__ inline GemvGeom gemv_geometry(int64_t k, int bits, int batches) {
  GemvGeom g;
  const int64_t row_bytes = k * bits / 8;
  g.chunks = (int)(row_bytes / 16);
  int L = 64;
  while (L > 1 && (g.chunks % L) != 0) L >>= 1;
  g.lanes_per_row = L;
  g.chunks_per_lane = g.chunks / L;
  g.batches = batches;
  g.rows_per_wg = (int64_t)4 * (64 / L) * GEMV_ROWS_PER_LANE * batches;
  return g;
}
// Host choice of the batch count: about GEMV_WG_BYTES of packed words per workgroup, fewer
// batches when `min_tiles` workgroups would otherwise not be reached.
inline int gemv_batches(int64_t n, int64_t k, int bits, int64_t min_tiles) {
  const GemvGeom g1 = gemv_geometry(k, bits, 1);
  const int64_t set_bytes = g1.rows_per_wg * (k * bits / 8);
  int nb = set_bytes > 0 ? (int)((GEMV_WG_BYTES + set_bytes / 2) / set_bytes) : 1;
  nb = nb < 1 ? 1 : (nb > 32 ? 32 : nb);
  while (nb > 1 && (n + g1.rows_per_wg * nb - 1) / (g1.rows_per_wg * nb) < min_tiles) --nb;
  return nb;
}
// LDS pitch (16-bit elements) of a 16-byte chunk of x (128 / bits values): padded by 8 against
// bank conflicts for up to 2 rows of x, unpadded for more (so that 8 rows of k = 3072 fit).
__host__ __device__ constexpr int gemv_x_pitch(int mt, int bits) { return 128 / bits + (mt <= 2 ? 8 : 0); }
// Dynamic LDS of a GEMV launch: x chunks, their sums and the layer-bias rows; x is kept in LDS
// (xlds) when it fits in 64 KiB, else read from memory by every lane.
struct GemvLds {
  size_t bytes;
  int xlds;
};
GemvLds gemv_lds(int64_t k, int bits, int64_t mt, int batches);

hipError_t launch_quantize(const float* w, int64_t n, int64_t k, int bits, int g, int pdt, uint32_t* packed,
                           void* scales, void* biases, hipStream_t s);
hipError_t launch_dequant_affine(const uint32_t* packed, const void* scales, const void* biases, int pdt,
                                 int64_t rows, int64_t k, int bits, int g, void* out, int odt, hipStream_t s);
hipError_t launch_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k, void* out,
                                int odt, hipStream_t s);
hipError_t launch_dequant_q8_0(const uint8_t* blocks, int64_t rows, int64_t k, void* out, int odt, hipStream_t s);

// One GEMV (desc passed by value, table == NULL) or `grid` tiles of a device problem table
// (all problems of one launch share the row-count template of m and bits).
hipError_t launch_gemv(const GemvDesc& single, const GemvDesc* table, const GemvTile* tiles, int64_t grid, int m,
                       int bits, int xdt, int pdt, int ydt, size_t lds_bytes, int xlds, bool g2, hipStream_t s);

hipError_t launch_gemm(const void* x, int xdt, int64_t m, int64_t k, const uint32_t* packed, const void* scales,
                       const void* biases, int pdt, int64_t n, int bits, int g, const void* layer_bias, void* y,
                       int ydt, void* ws, hipStream_t s);
size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int g);

hipError_t launch_route(const int64_t* ids, int64_t n_pos, int64_t e, int32_t* offsets, int32_t* perm,
                        hipStream_t s);
hipError_t launch_apply_experts(int fmt, const void* w0, const void* w1, int64_t e, int64_t n, int64_t k,
                                const int64_t* ids, int64_t n_pos, const void* x, int xdt, int64_t pos_per_row,
                                void* y, int ydt, int32_t* offsets, int32_t* perm, hipStream_t s);

}  // namespace ql
