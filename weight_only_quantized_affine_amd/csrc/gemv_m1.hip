// Instantiations of the decode GEMVs for row-count template 1 (see gemv_impl.hpp and gemv_mfma.hpp).
#include "gemv_mfma.hpp"

namespace ql {
hipError_t launch_gemv_m1(const GemvDesc& single, const GemvDesc* table, const GemvTile* tiles, int64_t grid,
                         size_t lds, int xlds, bool g2, int bits, int xdt, int pdt, int ydt, hipStream_t s) {
  return gemv_detail::launch_m<1>(single, table, tiles, grid, lds, xlds, g2, bits, xdt, pdt, ydt, s);
}
hipError_t launch_gemv_mf_m1(const GemvDesc& single, const GemvDesc* table, const GemvTile* tiles, int64_t grid,
                            size_t lds, int bits, int g, int xdt, int pdt, int ydt, hipStream_t s) {
  return gemv_detail::launch_mf_m<1>(single, table, tiles, grid, lds, bits, g, xdt, pdt, ydt, s);
}
}  // namespace ql
