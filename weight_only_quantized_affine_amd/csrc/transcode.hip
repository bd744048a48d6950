// GPTQ (continuous layout) to MLX affine rows (GPTQModel wiki "MLX Apple Silicon", Packed layouts
// and exact transcoding; GPTQModel "Packing Formats and Compatibility", GPTQ and GPTQ_V2).
//   qweight [K*b/32, N]: the codes of output column n as one little-endian b-bit stream down the
//   input axis; qzeros [G, N*b/32]: group g's zeros as one stream along the outputs; scales [G, N].
// The affine row of output n is the same b-bit stream of the same codes, so the packed words are
// qweight transposed word for word; scales transpose to [N, G]; the additive bias is
// -zero * scale, exact in fp32 (zero < 2^8, scale of at most 11 significant bits) and rounded
// once to the scale dtype.  v1 checkpoints store zero - 1.
#include "device_common.hpp"
#include "launch.hpp"

namespace ql {
namespace {

constexpr int TT = 64;  // transpose tile (words)

// dst[c][r] = src[r][c] for src [rows, cols]; 64 x 64 tiles through LDS (one padding word per row).
__global__ __launch_bounds__(256) void transpose_words_kernel(const uint32_t* __restrict__ src, int64_t rows,
                                                              int64_t cols, uint32_t* __restrict__ dst) {
  __shared__ uint32_t tile[TT][TT + 1];
  const int64_t tiles_c = (cols + TT - 1) / TT;
  const int64_t r0 = (int64_t)(blockIdx.x / tiles_c) * TT, c0 = (int64_t)(blockIdx.x % tiles_c) * TT;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;  // 64 x 4
  for (int i = ty; i < TT; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    tile[i][tx] = (r < rows && c < cols) ? src[r * cols + c] : 0u;
  }
  __syncthreads();
  for (int i = ty; i < TT; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;
    if (c < cols && r < rows) dst[c * rows + r] = tile[tx][i];
  }
}

// One lane per (output n, group g), g fastest: the zero is bits [b n, b n + b) of row g of qzeros.
template <typename PT>
__global__ __launch_bounds__(256) void gptq_params_kernel(const uint32_t* __restrict__ qzeros,
                                                          const uint16_t* __restrict__ scales, int64_t n, int groups,
                                                          int bits, int v1, uint16_t* __restrict__ scales_out,
                                                          uint16_t* __restrict__ biases_out) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n * groups) return;
  const int64_t o = t / groups;
  const int g = (int)(t - o * groups);
  const uint32_t* zrow = qzeros + (int64_t)g * (n * bits / 32);
  const int64_t pos = o * bits;
  const int64_t wi = pos >> 5;
  const int sh = (int)(pos & 31);
  uint32_t z = zrow[wi] >> sh;
  if (sh + bits > 32) z |= zrow[wi + 1] << (32 - sh);  // the zero continues in the next word
  z &= (1u << bits) - 1u;
  const int zero = (int)z + (v1 ? 1 : 0);
  const uint16_t sb = scales[(int64_t)g * n + o];
  // -(zero * scale): the product is exact and rounding to nearest even is symmetric, so the bias
  // is the product's 16-bit pattern with its sign bit flipped (zero = 0 gives -0, as IEEE
  // negation does).  The empty asm keeps the flip an integer operation: as a float negation the
  // compiler folds it into a mixed-precision fma with a +0 addend, which turns -0 into +0.
  float prod = (float)zero * param_to_f32<PT>(sb);  // exact (a plain product: -0 kept)
  asm volatile("" : "+v"(prod));
  uint32_t pbits = f32_to_bits<PT>(prod);
  asm volatile("" : "+v"(pbits));
  scales_out[t] = sb;
  biases_out[t] = (uint16_t)(pbits ^ 0x8000u);
}

}  // namespace

hipError_t launch_transcode_gptq(const uint32_t* qweight, const uint32_t* qzeros, const void* scales, int pdt,
                                 int64_t k, int64_t n, int bits, int g, int v1, uint32_t* packed, void* scales_out,
                                 void* biases_out, hipStream_t s) {
  const int64_t rows = k * bits / 32;
  const int64_t tiles = ((rows + TT - 1) / TT) * ((n + TT - 1) / TT);
  transpose_words_kernel<<<(unsigned)tiles, 256, 0, s>>>(qweight, rows, n, packed);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int groups = (int)(k / g);
  const unsigned nb = (unsigned)((n * groups + 255) / 256);
  if (pdt == DT_BF16)
    gptq_params_kernel<BF16><<<nb, 256, 0, s>>>(qzeros, (const uint16_t*)scales, n, groups, bits, v1,
                                                (uint16_t*)scales_out, (uint16_t*)biases_out);
  else
    gptq_params_kernel<F16><<<nb, 256, 0, s>>>(qzeros, (const uint16_t*)scales, n, groups, bits, v1,
                                               (uint16_t*)scales_out, (uint16_t*)biases_out);
  return hipGetLastError();
}

}  // namespace ql
