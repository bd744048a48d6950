// Host-side geometry and dispatch of the decode GEMVs; the kernels are in gemv_impl.hpp (vector
// ALU) and gemv_mfma.hpp (matrix cores), their instantiations in gemv_m{1,2,4,8}.hip.
#include "launch.hpp"

#include <algorithm>
#include <cstring>

namespace ql {

// Launchers of the per-row-count instantiations (gemv_m{1,2,4,8}.hip).
hipError_t launch_gemv_m1(const GemvDesc&, const GemvDesc*, const GemvTile*, int64_t, size_t, int, bool, int, int, int,
                          int, hipStream_t);
hipError_t launch_gemv_m2(const GemvDesc&, const GemvDesc*, const GemvTile*, int64_t, size_t, int, bool, int, int, int,
                          int, hipStream_t);
hipError_t launch_gemv_m4(const GemvDesc&, const GemvDesc*, const GemvTile*, int64_t, size_t, int, bool, int, int, int,
                          int, hipStream_t);
hipError_t launch_gemv_m8(const GemvDesc&, const GemvDesc*, const GemvTile*, int64_t, size_t, int, bool, int, int, int,
                          int, hipStream_t);

hipError_t launch_gemv_mf_m1(const GemvDesc&, const GemvDesc*, const GemvTile*, int64_t, size_t, int, int, int, int,
                             int, hipStream_t);
hipError_t launch_gemv_mf_m2(const GemvDesc&, const GemvDesc*, const GemvTile*, int64_t, size_t, int, int, int, int,
                             int, hipStream_t);
hipError_t launch_gemv_mf_m4(const GemvDesc&, const GemvDesc*, const GemvTile*, int64_t, size_t, int, int, int, int,
                             int, hipStream_t);
hipError_t launch_gemv_mf_m8(const GemvDesc&, const GemvDesc*, const GemvTile*, int64_t, size_t, int, int, int, int,
                             int, hipStream_t);

int gemv_mf_batches(int64_t n, int64_t k, int bits, int g, int mt, int64_t min_tiles) {
  const int64_t rows = gemv_mf_geometry(k, 1).rows_per_wg;
  const int64_t set_bytes = rows * (k * bits / 8);
  const int64_t target = mt >= 8 ? (bits == 8 ? GEMV_MF_WG_BYTES_M8_B8 : GEMV_MF_WG_BYTES_M8) : GEMV_MF_WG_BYTES;
  int nb = set_bytes > 0 ? (int)((target + set_bytes / 2) / set_bytes) : 1;
  nb = nb < 1 ? 1 : (nb > 32 ? 32 : nb);
  while (nb > 1 &&
         ((n + rows * nb - 1) / (rows * nb) < min_tiles || gemv_mf_lds(k, mt, g, nb, bits).bytes > GEMV_MF_LDS_MAX))
    --nb;
  return nb;
}

hipError_t launch_gemv_mf(const GemvDesc& single, const GemvDesc* table, const GemvTile* tiles, int64_t grid, int m,
                          int bits, int g, int xdt, int pdt, int ydt, size_t lds_bytes, hipStream_t s) {
  switch (gemv_mt(m)) {
    case 1: return launch_gemv_mf_m1(single, table, tiles, grid, lds_bytes, bits, g, xdt, pdt, ydt, s);
    case 2: return launch_gemv_mf_m2(single, table, tiles, grid, lds_bytes, bits, g, xdt, pdt, ydt, s);
    case 4: return launch_gemv_mf_m4(single, table, tiles, grid, lds_bytes, bits, g, xdt, pdt, ydt, s);
    default: return launch_gemv_mf_m8(single, table, tiles, grid, lds_bytes, bits, g, xdt, pdt, ydt, s);
  }
}

GemvLds gemv_lds(int64_t k, int bits, int64_t mt, int batches) {
  const GemvGeom g = gemv_geometry(k, bits, batches);
  const int64_t lb = g.rows_per_wg * 4;
  const int64_t xb = mt * g.chunks * (gemv_x_pitch((int)mt, bits) * 2 + 4);
  GemvLds r;
  r.xlds = (xb + lb) <= 64 * 1024 ? 1 : 0;
  r.bytes = (size_t)((r.xlds ? xb : 0) + lb);
  return r;
}

hipError_t launch_gemv(const GemvDesc& single, const GemvDesc* table, const GemvTile* tiles, int64_t grid, int m,
                       int bits, int xdt, int pdt, int ydt, size_t lds_bytes, int xlds, bool g2, hipStream_t s) {
  switch (gemv_mt(m)) {
    case 1: return launch_gemv_m1(single, table, tiles, grid, lds_bytes, xlds, g2, bits, xdt, pdt, ydt, s);
    case 2: return launch_gemv_m2(single, table, tiles, grid, lds_bytes, xlds, g2, bits, xdt, pdt, ydt, s);
    case 4: return launch_gemv_m4(single, table, tiles, grid, lds_bytes, xlds, g2, bits, xdt, pdt, ydt, s);
    default: return launch_gemv_m8(single, table, tiles, grid, lds_bytes, xlds, g2, bits, xdt, pdt, ydt, s);
  }
}

// The problem table of a list travels to the device inside kernel arguments, kUploadWords words
// per launch: the runtime copies a launch's arguments when it is enqueued, so the host image may
// be released as soon as the call returns, and the upload is ordered on the stream like any
// launch (no host wait; it can be captured into a graph).
constexpr int kUploadWords = 496;  // 1984 bytes of payload per launch, well inside the argument limit
struct UploadChunk {
  uint32_t w[kUploadWords];
};
__global__ __launch_bounds__(256) void upload_words_kernel(UploadChunk c, int nwords, uint32_t* __restrict__ dst) {
  for (int i = threadIdx.x; i < nwords; i += 256) dst[i] = c.w[i];
}

hipError_t launch_upload(const void* host, size_t bytes, void* dst, hipStream_t s) {
  const uint8_t* src = (const uint8_t*)host;
  const size_t words = (bytes + 3) / 4;
  for (size_t w0 = 0; w0 < words; w0 += kUploadWords) {
    const int nw = (int)std::min<size_t>(kUploadWords, words - w0);
    UploadChunk c{};
    const size_t b0 = w0 * 4, nb = std::min<size_t>((size_t)nw * 4, bytes - b0);
    memcpy(c.w, src + b0, nb);
    upload_words_kernel<<<1, 256, 0, s>>>(c, nw, (uint32_t*)dst + w0);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ql
