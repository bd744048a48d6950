// GPTQ (continuous layout) to MLX affine rows (GPTQModel wiki "MLX Apple Silicon", Packed layouts
// and exact transcoding; GPTQModel "Packing Formats and Compatibility", GPTQ and GPTQ_V2).
//   qweight [K*b/32, N]: the codes of output column n as one little-endian b-bit stream down the
//   input axis; qzeros [G, N*b/32]: group g's zeros as one stream along the outputs; scales [G, N].
// The affine row of output n is the same b-bit stream of the same codes, so the packed words are
// qweight transposed word for word; scales transpose to [N, G]; the additive bias is
// -zero * scale, exact in fp32 (zero < 2^8, scale of at most 11 significant bits) and rounded
// once to the scale dtype.  v1 checkpoints store zero - 1.
//
// GPTQ_P ("Packing Formats and Compatibility", GPTQ_P) keeps GPTQ's tensors but stores every 32
// codes as b adjacent words of bit planes, low plane first (widths: the powers of two that make
// up b, largest first; fields least significant first inside a plane), with true zero points.
// At 2, 4 and 8 bits the single plane is GPTQ's continuous word, so those widths take the GPTQ
// path; at 3, 5, 6 and 7 bits a workgroup stages 16 blocks x 64 columns of qweight in LDS and
// rewrites each (column, block) as the affine row's continuous words (8-bit words for 7 bits).
//
// AWQ GEMM (same pages, AWQ GEMM row and ParoQuant; "Packing Formats and Compatibility", AWQ GEMM)
// packs the other axis: qweight [K, N*b/32] holds each input row's codes as one b-bit stream
// along the outputs, qzeros [G, N*b/32] the true zeros the same way, and at 4 bits the nibbles
// of a word hold, from the low one up, columns 0, 2, 4, 6, 1, 3, 5, 7 of the word's 8.  The
// affine rows need the codes along the inputs, so the codes themselves are transposed: a
// workgroup decodes a 128 x 128 tile of codes into LDS (one byte each, the lane order undone)
// and writes it back as 128 row streams.  A 7-bit source keeps its code values in 8-bit rows.
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

// Field i (0..31) of the planar block at w (bits words): each plane's field shifted past the
// planes below it.
__device__ __forceinline__ uint32_t planar_field(const uint32_t* __restrict__ w, int i, int bits) {
  uint32_t v = 0u;
  int first = 0, off = 0;
#pragma unroll
  for (int wp = 8; wp >= 1; wp >>= 1) {
    if (!(bits & wp)) continue;
    const int pos = i * wp;
    v |= ((w[first + (pos >> 5)] >> (pos & 31)) & ((1u << wp) - 1u)) << off;
    first += wp;
    off += wp;
  }
  return v;
}

// One lane per (output n, group g), g fastest: the zero is bits [b n, b n + b) of row g of qzeros.
// With awq4 the zeros are 4-bit AWQ words: column c of a word's 8 sits in nibble slot
// (c >> 1) | ((c & 1) << 2), the inverse of the lane order 0, 2, 4, 6, 1, 3, 5, 7.  With planar
// the row is GPTQ_P blocks: the zero is field n % 32 of the block at word b (n / 32).
template <typename PT>
__global__ __launch_bounds__(256) void gptq_params_kernel(const uint32_t* __restrict__ qzeros,
                                                          const uint16_t* __restrict__ scales, int64_t n, int groups,
                                                          int bits, int v1, int awq4, int planar,
                                                          uint16_t* __restrict__ scales_out,
                                                          uint16_t* __restrict__ biases_out) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n * groups) return;
  const int64_t o = t / groups;
  const int g = (int)(t - o * groups);
  const uint32_t* zrow = qzeros + (int64_t)g * (n * bits / 32);
  const int c = (int)(o & 7);
  const int64_t slot = awq4 ? ((o & ~(int64_t)7) | (c >> 1) | ((c & 1) << 2)) : o;
  const int64_t pos = slot * bits;
  const int64_t wi = pos >> 5;
  const int sh = (int)(pos & 31);
  uint32_t z;
  if (planar) {
    z = planar_field(zrow + (o >> 5) * bits, (int)(o & 31), bits);
  } else {
    z = zrow[wi] >> sh;
    if (sh + bits > 32) z |= zrow[wi + 1] << (32 - sh);  // the zero continues in the next word
    z &= (1u << bits) - 1u;
  }
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

hipError_t launch_params(const uint32_t* qzeros, const void* scales, int pdt, int64_t n, int groups, int bits, int v1,
                         int awq4, int planar, void* scales_out, void* biases_out, hipStream_t s) {
  const unsigned nb = (unsigned)((n * groups + 255) / 256);
  if (pdt == DT_BF16)
    gptq_params_kernel<BF16><<<nb, 256, 0, s>>>(qzeros, (const uint16_t*)scales, n, groups, bits, v1, awq4, planar,
                                                (uint16_t*)scales_out, (uint16_t*)biases_out);
  else
    gptq_params_kernel<F16><<<nb, 256, 0, s>>>(qzeros, (const uint16_t*)scales, n, groups, bits, v1, awq4, planar,
                                               (uint16_t*)scales_out, (uint16_t*)biases_out);
  return hipGetLastError();
}

constexpr int PKB = 16;  // planar tile: 16 blocks of 32 codes (512 inputs) x 64 output columns

// Tile (k0, n0): word rows k0 / 32 * B .. + 16 B of qweight, columns n0 .. n0 + 63, into LDS (one
// padding word per row); then item (column c, block kb) decodes its B words and writes the TB
// words of target row n0 + c from word (k0 / 32 + kb) TB.  k is a multiple of 32, so a block is
// wholly inside or outside the matrix.
template <int B, int TB>
__global__ __launch_bounds__(256) void planar_codes_kernel(const uint32_t* __restrict__ qweight, int64_t k, int64_t n,
                                                           uint32_t* __restrict__ packed) {
  __shared__ uint32_t tile[PKB * B][65];
  const int64_t tiles_n = (n + 63) / 64;
  const int64_t k0 = (int64_t)(blockIdx.x / tiles_n) * (32 * PKB), n0 = (int64_t)(blockIdx.x % tiles_n) * 64;
  const int64_t src_rows = k / 32 * B, row0 = k0 / 32 * B, dst_words = k / 32 * TB;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int r = ty; r < PKB * B; r += 4) {
    const int64_t wr = row0 + r, c = n0 + tx;
    tile[r][tx] = (wr < src_rows && c < n) ? qweight[wr * n + c] : 0u;
  }
  __syncthreads();
  for (int it = threadIdx.x; it < 64 * PKB; it += 256) {
    const int c = it / PKB, kb = it % PKB;
    if (n0 + c >= n || k0 + 32 * kb >= k) continue;
    uint32_t w[B];
#pragma unroll
    for (int i = 0; i < B; ++i) w[i] = tile[kb * B + i][c];
    uint32_t o[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) o[i] = 0u;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t v = planar_field(w, j, B);
      const int pos = j * TB, wi = pos >> 5, sh = pos & 31;
      o[wi] |= v << sh;
      if (sh + TB > 32) o[wi + 1] |= v >> (32 - sh);
    }
    uint32_t* dst = packed + (n0 + c) * dst_words + (k0 / 32 + kb) * TB;
#pragma unroll
    for (int i = 0; i < TB; ++i) dst[i] = o[i];
  }
}

template <int B, int TB>
hipError_t launch_planar_codes(const uint32_t* qweight, int64_t k, int64_t n, uint32_t* packed, hipStream_t s) {
  const int64_t tiles = ((k + 32 * PKB - 1) / (32 * PKB)) * ((n + 63) / 64);
  planar_codes_kernel<B, TB><<<(unsigned)tiles, 256, 0, s>>>(qweight, k, n, packed);
  return hipGetLastError();
}

constexpr int AT = 128;       // AWQ code tile: 128 input rows x 128 output columns
constexpr int AP = AT + 4;    // LDS pitch of a tile row (bytes)

// Tile (k0, n0) of the code matrix [k, n]: source row r's columns n0 .. n0 + 127 are the
// 4 * SB words from word n0 * SB / 32 of that row (n0 is a multiple of 128, so whole words);
// target row n0 + c's codes k0 .. k0 + 127 are the 4 * TB words from word k0 * TB / 32 of it.
// k and n are multiples of 32, so every 32-code block is wholly inside or outside the matrix.
template <int SB, int TB>
__global__ __launch_bounds__(256) void awq_codes_kernel(const uint32_t* __restrict__ qweight, int64_t k, int64_t n,
                                                        uint32_t* __restrict__ packed) {
  __shared__ uint8_t tile[AT * AP];
  const int64_t tiles_n = (n + AT - 1) / AT;
  const int64_t k0 = (int64_t)(blockIdx.x / tiles_n) * AT, n0 = (int64_t)(blockIdx.x % tiles_n) * AT;
  const int64_t src_words = n * SB / 32, dst_words = k * TB / 32;
  // 1. decode: item = (tile row r, 32-column block cb); four consecutive lanes read one row's
  //    4 * SB consecutive words
  for (int it = threadIdx.x; it < AT * 4; it += 256) {
    const int r = it >> 2, cb = it & 3;
    if (k0 + r >= k || n0 + 32 * cb >= n) continue;
    const uint32_t* src = qweight + (k0 + r) * src_words + (n0 + 32 * cb) * SB / 32;
    uint32_t w[SB];
#pragma unroll
    for (int i = 0; i < SB; ++i) w[i] = src[i];
    uint8_t* dst = tile + r * AP + 32 * cb;
#pragma unroll
    for (int slot = 0; slot < 32; ++slot) {
      constexpr uint32_t mask = (1u << SB) - 1u;
      const int pos = slot * SB, wi = pos >> 5, sh = pos & 31;
      uint32_t v = w[wi] >> sh;
      if (sh + SB > 32) v |= w[wi + 1] << (32 - sh);
      // at 4 bits, nibble slot s of a word holds column ((s & 3) << 1) | (s >> 2) of its 8
      const int col = SB == 4 ? ((slot & ~7) | ((slot & 3) << 1) | ((slot >> 2) & 1)) : slot;
      dst[col] = (uint8_t)(v & mask);
    }
  }
  __syncthreads();
  // 2. pack: item = (tile column c, 32-row block kb); four consecutive lanes write one target
  //    row's 4 * TB consecutive words
  for (int it = threadIdx.x; it < AT * 4; it += 256) {
    const int c = it >> 2, kb = it & 3;
    if (n0 + c >= n || k0 + 32 * kb >= k) continue;
    uint32_t w[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) w[i] = 0u;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const uint32_t v = tile[(32 * kb + j) * AP + c];
      const int pos = j * TB, wi = pos >> 5, sh = pos & 31;
      w[wi] |= v << sh;
      if (sh + TB > 32) w[wi + 1] |= v >> (32 - sh);
    }
    uint32_t* dst = packed + (n0 + c) * dst_words + (k0 + 32 * kb) * TB / 32;
#pragma unroll
    for (int i = 0; i < TB; ++i) dst[i] = w[i];
  }
}

template <int SB, int TB>
hipError_t launch_awq_codes(const uint32_t* qweight, int64_t k, int64_t n, uint32_t* packed, int64_t tiles,
                            hipStream_t s) {
  awq_codes_kernel<SB, TB><<<(unsigned)tiles, 256, 0, s>>>(qweight, k, n, packed);
  return hipGetLastError();
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
  return launch_params(qzeros, scales, pdt, n, groups, bits, v1, 0, 0, scales_out, biases_out, s);
}

hipError_t launch_transcode_gptq_planar(const uint32_t* qweight, const uint32_t* qzeros, const void* scales, int pdt,
                                        int64_t k, int64_t n, int bits, int g, uint32_t* packed, void* scales_out,
                                        void* biases_out, hipStream_t s) {
  hipError_t e = hipSuccess;
  switch (bits) {
    case 2:
    case 4:
    case 8: {  // one plane: GPTQ's continuous words
      const int64_t rows = k * bits / 32;
      const int64_t tiles = ((rows + TT - 1) / TT) * ((n + TT - 1) / TT);
      transpose_words_kernel<<<(unsigned)tiles, 256, 0, s>>>(qweight, rows, n, packed);
      e = hipGetLastError();
      break;
    }
    case 3: e = launch_planar_codes<3, 3>(qweight, k, n, packed, s); break;
    case 5: e = launch_planar_codes<5, 5>(qweight, k, n, packed, s); break;
    case 6: e = launch_planar_codes<6, 6>(qweight, k, n, packed, s); break;
    case 7: e = launch_planar_codes<7, 8>(qweight, k, n, packed, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return launch_params(qzeros, scales, pdt, n, (int)(k / g), bits, 0, 0, 1, scales_out, biases_out, s);
}

hipError_t launch_transcode_awq(const uint32_t* qweight, const uint32_t* qzeros, const void* scales, int pdt,
                                int64_t k, int64_t n, int bits, int g, uint32_t* packed, void* scales_out,
                                void* biases_out, hipStream_t s) {
  const int64_t tiles = ((k + AT - 1) / AT) * ((n + AT - 1) / AT);
  hipError_t e = hipSuccess;
  switch (bits) {
    case 2: e = launch_awq_codes<2, 2>(qweight, k, n, packed, tiles, s); break;
    case 3: e = launch_awq_codes<3, 3>(qweight, k, n, packed, tiles, s); break;
    case 4: e = launch_awq_codes<4, 4>(qweight, k, n, packed, tiles, s); break;
    case 5: e = launch_awq_codes<5, 5>(qweight, k, n, packed, tiles, s); break;
    case 6: e = launch_awq_codes<6, 6>(qweight, k, n, packed, tiles, s); break;
    case 7: e = launch_awq_codes<7, 8>(qweight, k, n, packed, tiles, s); break;
    case 8: e = launch_awq_codes<8, 8>(qweight, k, n, packed, tiles, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  return launch_params(qzeros, scales, pdt, n, (int)(k / g), bits, 0, bits == 4 ? 1 : 0, 0, scales_out, biases_out,
                       s);
}

}  // namespace ql
