// Instantiations of the decode GEMV for row-count template 4 (see gemv_impl.hpp).
#include "gemv_impl.hpp"

namespace ql {
hipError_t launch_gemv_m4(const GemvDesc& single, const GemvDesc* table, const GemvTile* tiles, int64_t grid,
                         size_t lds, int xlds, bool g2, int bits, int xdt, int pdt, int ydt, hipStream_t s) {
  return gemv_detail::launch_m<4>(single, table, tiles, grid, lds, xlds, g2, bits, xdt, pdt, ydt, s);
}
}  // namespace ql
