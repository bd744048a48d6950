// Internal launchers called by the C ABI layer after host validation.  Each returns the
// hipError_t of its launch(es).  Shapes are already checked: kernels may assume them.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

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

// Matrix-core GEMV (2- to 6- or 8-bit codes, k a multiple of 128): a wave owns 16 * GEMV_MF_RS weight
// rows and walks them in u-blocks of 128 codes (64 or 128 bytes of each row); GEMV_MF_NU u-blocks
// make one pipeline step.  A 256-thread workgroup walks `batches` sets of 64 * GEMV_MF_RS rows.
#ifndef GEMV_MF_NU
#define GEMV_MF_NU 2
#endif
#ifndef GEMV_MF_WG_BYTES
#define GEMV_MF_WG_BYTES 32768  // packed bytes per workgroup the batch count aims at (one x row)
#endif
#ifndef GEMV_MF_WG_BYTES_M8
#define GEMV_MF_WG_BYTES_M8 262144  // the same for 5 to 8 x rows (staging x costs more per workgroup)
#endif
#ifndef GEMV_MF_WG_BYTES_M8_B8
#define GEMV_MF_WG_BYTES_M8_B8 524288  // the same for 5 to 8 x rows of 8-bit codes
#endif
#ifndef GEMV_MF_LDS_MAX
#define GEMV_MF_LDS_MAX (80 * 1024)  // LDS of one workgroup (two fit a compute unit)
#endif
#ifndef GEMV_MF_RS
#define GEMV_MF_RS 1
#endif
#ifndef GEMV_MF_NB
#define GEMV_MF_NB 2  // step buffers of the load pipeline
#endif
#ifndef GEMV_MF_NB_M8
#define GEMV_MF_NB_M8 4  // the same for 5 to 8 x rows
#endif
#ifndef GEMV_MF_SCHED
#define GEMV_MF_SCHED 1
#endif
#ifndef GEMV_MF_MINB
#define GEMV_MF_MINB 1  // waves per SIMD the register allocation must allow
#endif
#ifndef GEMV_MF_AUX
#define GEMV_MF_AUX 0  // cache policy bits of the weight-word loads
#endif
#ifndef GEMV_MF_SU
#define GEMV_MF_SU 4  // 16-byte chunks of x a thread loads at once when it stages x
#endif
#ifndef GEMV_MF_SU_M8
#define GEMV_MF_SU_M8 8  // the same with 5 to 8 x rows
#endif
#ifndef GEMV_MF_LINES
#define GEMV_MF_LINES 1  // 4-bit codes, 5 to 8 x rows: whole 128-byte lines per load, regrouped through LDS
#endif
#ifndef GEMV_MF_LAUX
#define GEMV_MF_LAUX 2  // cache policy bits of those loads (non-temporal: each line is read once)
#endif
// A wave's regrouping area: its 16 rows x 128 bytes as two 1 KB halves (rows 0-7, rows 8-15),
// the second 128 bytes after the first's end so that the two halves' lanes meet different banks.
constexpr int kGemvMfRegroupBytes = 2304;
constexpr int kGemvMfHalfOff = 1152;
__host__ __device__ constexpr bool gemv_mf_lines(int bits, int mt) {
  return GEMV_MF_LINES && bits == 4 && mt >= 8 && GEMV_MF_NU == 2 && GEMV_MF_RS == 1;
}
struct GemvMfGeom {
  int ublocks;        // k / 128
  int steps_per_row;  // ceil(ublocks / GEMV_MF_NU)
  int kpad;           // steps_per_row * GEMV_MF_NU * 128: x rows are zero-padded to this length
  int batches;
  int64_t rows_per_wg;
};
__host__ __device__ inline GemvMfGeom gemv_mf_geometry(int64_t k, int batches) {
  GemvMfGeom g;
  g.ublocks = (int)(k / 128);
  g.steps_per_row = (g.ublocks + GEMV_MF_NU - 1) / GEMV_MF_NU;
  g.kpad = g.steps_per_row * GEMV_MF_NU * 128;
  g.batches = batches;
  g.rows_per_wg = (int64_t)64 * GEMV_MF_RS * batches;
  return g;
}
// Groups of a u-block (1 when the group spans it) and the x rows one matrix-core pass serves.
__host__ __device__ constexpr int gemv_mf_gu(int g) { return g >= 128 ? 1 : 128 / g; }
// LDS of a matrix-core GEMV launch, in this order: mt x rows and one zero row of kpad + 8
// elements; the table of x sums (one float per u-block and accumulator row); the x row factors
// (8 floats); the workgroup's scales, then its biases (16 bits per row and group, as in memory);
// for 4-bit codes and 5 to 8 x rows, each wave's regrouping area (16-byte aligned).
struct GemvMfLds {
  size_t xsum_off, xscale_off, param_off, bias_off, regroup_off, bytes;
};
__host__ __device__ inline GemvMfLds gemv_mf_lds(int64_t k, int mt, int g, int batches, int bits) {
  const GemvMfGeom geo = gemv_mf_geometry(k, batches);
  GemvMfLds r;
  r.xsum_off = ((size_t)(mt + 1) * (geo.kpad + 8) * 2 + 15) / 16 * 16;
  r.xscale_off = r.xsum_off + (size_t)geo.steps_per_row * GEMV_MF_NU * 16 * 4;
  r.param_off = r.xscale_off + 32;
  r.bias_off = r.param_off + (size_t)geo.rows_per_wg * (k / g) * 2;
  r.regroup_off = (r.bias_off + (size_t)geo.rows_per_wg * (k / g) * 2 + 15) / 16 * 16;
  r.bytes = r.regroup_off + (gemv_mf_lines(bits, mt) ? (size_t)4 * kGemvMfRegroupBytes : 0);
  return r;
}
#ifndef GEMV_MF_ENABLE
#define GEMV_MF_ENABLE 1
#endif
// Whether a problem takes the matrix-core GEMV: 2- to 6- or 8-bit codes, group size 32, 64 or 128, k a
// multiple of 128 with an even number of groups per row, scales and biases 4-byte aligned, at
// most 16 accumulator rows (rows of x times groups per u-block) and the LDS of one batch within
// GEMV_MF_LDS_MAX.
inline bool gemv_mf_eligible(int64_t m, int64_t k, int bits, int g, const void* scales, const void* biases) {
  if (!GEMV_MF_ENABLE || bits < 2 || bits > 8 || bits == 7 || k < 128 || k % 128 != 0 || (g != 32 && g != 64 && g != 128))
    return false;
  if ((k / g) % 2 != 0 || ((uintptr_t)scales | (uintptr_t)biases) % 4 != 0) return false;
  const int mt = gemv_mt(m);
  return mt * gemv_mf_gu(g) <= 16 && gemv_mf_lds(k, mt, g, 1, bits).bytes <= GEMV_MF_LDS_MAX;
}
// Batches per workgroup: about GEMV_MF_WG_BYTES (GEMV_MF_WG_BYTES_M8 for mt = 8) of packed words,
// fewer when `min_tiles` workgroups would otherwise not be reached or the LDS would pass
// GEMV_MF_LDS_MAX.
int gemv_mf_batches(int64_t n, int64_t k, int bits, int g, int mt, int64_t min_tiles);

hipError_t launch_quantize(const float* w, int64_t n, int64_t k, int bits, int g, int pdt, uint32_t* packed,
                           void* scales, void* biases, hipStream_t s);
hipError_t launch_dequant_affine(const uint32_t* packed, const void* scales, const void* biases, int pdt,
                                 int64_t rows, int64_t k, int bits, int g, void* out, int odt, hipStream_t s);
hipError_t launch_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k, void* out,
                                int odt, hipStream_t s);
hipError_t launch_dequant_mxfp4_blocks(const uint8_t* blocks, int64_t rows, int64_t k, void* out, int odt,
                                       hipStream_t s);
hipError_t launch_quantize_q8_0(const float* w, int64_t rows, int64_t k, uint8_t* blocks, hipStream_t s);
hipError_t launch_take(const int64_t* pos, int64_t n_pos, const void* src, int64_t src_rows, int64_t row_bytes,
                       void* dst, hipStream_t s);
hipError_t launch_transcode_gptq(const uint32_t* qweight, const uint32_t* qzeros, const void* scales, int pdt,
                                 int64_t k, int64_t n, int bits, int g, int v1, uint32_t* packed, void* scales_out,
                                 void* biases_out, hipStream_t s);
hipError_t launch_transcode_gptq_planar(const uint32_t* qweight, const uint32_t* qzeros, const void* scales, int pdt,
                                        int64_t k, int64_t n, int bits, int g, uint32_t* packed, void* scales_out,
                                        void* biases_out, hipStream_t s);
hipError_t launch_transcode_awq(const uint32_t* qweight, const uint32_t* qzeros, const void* scales, int pdt,
                                int64_t k, int64_t n, int bits, int g, uint32_t* packed, void* scales_out,
                                void* biases_out, hipStream_t s);
// Q4_K (block_bytes 144) or Q6_K (210) blocks [rows, k/256 * block_bytes] -> out [rows, k].
hipError_t launch_dequant_kquant(int block_bytes, const uint8_t* blocks, int64_t rows, int64_t k, void* out, int odt,
                                 hipStream_t s);
hipError_t launch_dequant_q8_0(const uint8_t* blocks, int64_t rows, int64_t k, void* out, int odt, hipStream_t s);

// One GEMV (desc passed by value, table == NULL) or `grid` tiles of a device problem table
// (all problems of one launch share the row-count template of m and bits).
// Copies `bytes` of host memory to device memory `dst` (4-byte aligned) through kernel arguments:
// asynchronous on `s`, the host memory may be reused when the call returns.
hipError_t launch_upload(const void* host, size_t bytes, void* dst, hipStream_t s);
hipError_t launch_gemv(const GemvDesc& single, const GemvDesc* table, const GemvTile* tiles, int64_t grid, int m,
                       int bits, int xdt, int pdt, int ydt, size_t lds_bytes, int xlds, bool g2, hipStream_t s);
// The same for the matrix-core GEMV; every problem of the launch has `bits` and group size `g`.
hipError_t launch_gemv_mf(const GemvDesc& single, const GemvDesc* table, const GemvTile* tiles, int64_t grid, int m,
                          int bits, int g, int xdt, int pdt, int ydt, size_t lds_bytes, hipStream_t s);

hipError_t launch_gemm(const void* x, int xdt, int64_t m, int64_t k, const uint32_t* packed, const void* scales,
                       const void* biases, int pdt, int64_t n, int bits, int g, const void* layer_bias, void* y,
                       int ydt, void* ws, hipStream_t s);
size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int bits, int g);
// One weight of a grouped GEMM (mirrors ql_gemm_weight).
struct GemmWeight {
  const uint32_t* packed;
  const void* scales;
  const void* biases;
  const void* layer_bias;
  void* y;
  int64_t n;
};
size_t gemm_grouped_workspace_bytes(int64_t m, int64_t k, const GemmWeight* w, int count, int bits, int g);
hipError_t launch_gemm_grouped(const void* x, int xdt, int64_t m, int64_t k, const GemmWeight* w, int count, int pdt,
                               int bits, int g, int ydt, void* ws, hipStream_t s);

// Affine widths whose rows are read as a bitstream of 32-code chunks (BITS words each) rather
// than by whole codes per word: 2, 3, 5 and 6 bits.
constexpr bool is_stream_bits(int bits) { return bits == 2 || bits == 3 || bits == 5 || bits == 6; }

// GEMV at the bitstream widths, m <= 8 rows of x.
struct GemvStreamArgs {
  const void* x;  // [m, k], x dtype; 16-byte aligned
  int m;
  int64_t k;
  const uint32_t* packed;
  const void* scales;
  const void* biases;
  int64_t n;
  int g;
  const void* layer_bias;  // [n] in x's dtype, or NULL
  void* y;                 // [m, n]
  int ydt, bits, xdt, pdt;
};
hipError_t launch_gemv_stream(const GemvStreamArgs& a, hipStream_t s);
// A problem list of bitstream GEMVs (every problem: `bits`, k % 128 == 0, m <= 8); tiles as
// stream_quad_tile_rows gives them; lds from stream_quad_lds (the largest over the list).
hipError_t launch_gemv_stream_table(const GemvDesc* table, const GemvTile* tiles, int64_t grid, int m, int bits,
                                    int xdt, int pdt, int ydt, size_t lds, hipStream_t s);

// Geometry of the bitstream GEMV for k % 128 == 0 (shared by the host plan and the kernels):
// x slices of ks values (plus 16 bytes of padding per 128) in at most 64 KiB of LDS; lanes per
// row group from the 128-code quads of a row; weight rows per lane group by x rows (mt).
constexpr int kStreamLdsBytes = 65536;
inline int stream_quad_ks(int64_t k, int mt) {
  const int64_t cap = kStreamLdsBytes / 2 / mt * 16 / 17 / 128 * 128;
  return (int)(k < 128 ? 128 : (k < cap ? k : cap));
}
inline size_t stream_quad_lds(int64_t k, int mt) {
  const int ks = stream_quad_ks(k, mt);
  return (size_t)mt * (size_t)(ks + ks / 16) * 2;
}
inline int stream_quad_lg(int64_t k, int mt) {
  const int64_t nq = std::max<int64_t>(1, std::min<int64_t>(k, stream_quad_ks(k, mt)) / 128);
  int lg = 8;
  for (int cand = 16; cand <= 64; cand *= 2)
    if (nq % cand == 0 || nq >= 4 * cand) lg = cand;
  return lg;
}
constexpr int stream_quad_rows(int mt) { return mt >= 8 ? 1 : (mt >= 4 ? 2 : 4); }
inline int64_t stream_quad_tile_rows(int64_t k, int mt) {
  return 4 * (64 / stream_quad_lg(k, mt)) * stream_quad_rows(mt);
}

hipError_t launch_route(const int64_t* ids, int64_t n_pos, int64_t e, int32_t* offsets, int32_t* perm,
                        hipStream_t s);
// The MXFP4 routed apply, after routing: offsets, permutation and expert order as launch_apply_experts
// computes them.
hipError_t launch_experts_mx(const uint8_t* codes, const uint8_t* scales, int64_t e, int64_t n, int64_t k,
                             const int32_t* offsets, const int32_t* perm, const int32_t* order, const uint16_t* x,
                             int xdt, int64_t x_rows, int64_t pos_per_row, void* y, int ydt, hipStream_t s);
hipError_t launch_experts_q8(const uint8_t* blocks, int64_t e, int64_t n, int64_t k, const int32_t* offsets,
                             const int32_t* perm, const int32_t* order, const float* xfac, const uint16_t* x,
                             int xdt, int64_t x_rows, int64_t pos_per_row, void* y, int ydt, hipStream_t s);
// The Q4_K (fmt 4) / Q6_K (fmt 5) routed apply, after routing.
hipError_t launch_experts_kq(int fmt, const uint8_t* blocks, int64_t e, int64_t n, int64_t k, const int32_t* offsets,
                             const int32_t* perm, const int32_t* order, const uint16_t* x, int xdt, int64_t x_rows,
                             int64_t pos_per_row, void* y, int ydt, hipStream_t s);
hipError_t launch_apply_experts(int fmt, const void* w0, const void* w1, int64_t e, int64_t n, int64_t k,
                                const int64_t* ids, int64_t n_pos, const void* x, int xdt, int64_t pos_per_row,
                                void* y, int ydt, int32_t* offsets, int32_t* perm, int32_t* order, float* xfac,
                                hipStream_t s);

}  // namespace ql
