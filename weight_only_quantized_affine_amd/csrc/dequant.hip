// dequant (Nx_quant API docs, Products: dequant): every weight as its float32 value, rounded
// once to the output dtype.  Affine: value = fl32(code*scale + bias) (GPTQModel wiki "MLX Apple
// Silicon", Concepts).  MXFP4: e2m1 code * 2^(s-127) (Nx_quant Weights, Mxfp4).  Q8_0: d*q
// (Nx_quant Weights, Q8_0).  Elementwise and HBM-bound: each lane turns one 16-byte chunk of
// packed data (or one 34-byte Q8_0 block) into its values and writes them out contiguously.
#include "device_common.hpp"
#include "launch.hpp"

namespace ql {
namespace {

__device__ __forceinline__ void store8(void* out, int64_t i0, const float* v, int odt) {
  if (odt == DT_F32) {
    f32x4_t a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
    *(f32x4_t*)((float*)out + i0) = a;
    *(f32x4_t*)((float*)out + i0 + 4) = b;
  } else {
    uint32_t h[8];
    if (odt == DT_BF16) {
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = f32_to_bf16_bits(v[j]);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) h[j] = f32_to_f16_bits(v[j]);
    }
    u32x4_t p = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
    *(u32x4_t*)((uint16_t*)out + i0) = p;
  }
}

template <int BITS, typename PT>
__global__ __launch_bounds__(256) void dequant_affine_kernel(const uint32_t* __restrict__ packed,
                                                             const uint16_t* __restrict__ scales,
                                                             const uint16_t* __restrict__ biases, int64_t rows,
                                                             int64_t k, int g, void* __restrict__ out, int odt) {
  constexpr int PER = 128 / BITS;  // values per 16-byte chunk
  const int64_t chunks_per_row = k / PER;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * chunks_per_row) return;
  const int64_t row = t / chunks_per_row;
  const int64_t c = t - row * chunks_per_row;
  const int64_t k0 = c * PER;
  const int64_t gi = row * (k / g) + k0 / g;  // a chunk never straddles a group (g >= 32)
  const float s = param_to_f32<PT>(scales[gi]);
  const float b = param_to_f32<PT>(biases[gi]);
  u32x4_t w = load16(packed + row * (k * BITS / 32) + c * 4);
  float v[PER];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int i = 0; i < 32 / BITS; ++i) {
      uint32_t q = (w[j] >> (BITS * i)) & ((1u << BITS) - 1);
      v[j * (32 / BITS) + i] = __builtin_fmaf((float)q, s, b);  // q*s is exact: one rounding
    }
  }
  const int64_t o = row * k + k0;
#pragma unroll
  for (int j = 0; j < PER / 8; ++j) store8(out, o + 8 * j, v + 8 * j, odt);
}

// Bitstream widths (2, 3, 5, 6): each lane turns one 32-code chunk (BITS words) into 32 values.
template <int BITS, typename PT>
__global__ __launch_bounds__(256) void dequant_stream_kernel(const uint32_t* __restrict__ packed,
                                                             const uint16_t* __restrict__ scales,
                                                             const uint16_t* __restrict__ biases, int64_t rows,
                                                             int64_t k, int g, void* __restrict__ out, int odt) {
  const int64_t chunks_per_row = k / 32;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * chunks_per_row) return;
  const int64_t row = t / chunks_per_row;
  const int64_t c = t - row * chunks_per_row;
  const int64_t k0 = c * 32;
  const int64_t gi = row * (k / g) + k0 / g;  // a chunk never straddles a group (g >= 32)
  const float s = param_to_f32<PT>(scales[gi]);
  const float b = param_to_f32<PT>(biases[gi]);
  const uint32_t* src = packed + row * (k / 32 * BITS) + c * BITS;
  uint32_t w[BITS];
#pragma unroll
  for (int j = 0; j < BITS; ++j) w[j] = src[j];
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = __builtin_fmaf((float)stream_code<BITS>(w, i), s, b);  // one rounding
  const int64_t o = row * k + k0;
#pragma unroll
  for (int j = 0; j < 4; ++j) store8(out, o + 8 * j, v + 8 * j, odt);
}

template <int BITS>
void launch_dequant_stream(const uint32_t* packed, const uint16_t* sc, const uint16_t* bi, int pdt, int64_t rows,
                           int64_t k, int g, void* out, int odt, hipStream_t s) {
  const unsigned nb = (unsigned)((rows * (k / 32) + 255) / 256);
  if (pdt == DT_BF16)
    dequant_stream_kernel<BITS, BF16><<<nb, 256, 0, s>>>(packed, sc, bi, rows, k, g, out, odt);
  else
    dequant_stream_kernel<BITS, F16><<<nb, 256, 0, s>>>(packed, sc, bi, rows, k, g, out, odt);
}

// 2^(s-127) as an fp32 value (s = 0 gives the subnormal 2^-127); s == 255 is NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  if (s == 0) return __uint_as_float(0x00400000u);
  if (s == 255) return __uint_as_float(0x7fc00000u);
  return __uint_as_float(s << 23);
}

__global__ __launch_bounds__(256) void dequant_mxfp4_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales, int64_t rows,
                                                            int64_t k, void* __restrict__ out, int odt) {
  // Twice the e2m1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 (OCP Microscaling Formats, named by the
  // Nx_quant page) as 4-bit fields of one word, indexed by the code's low three bits.
  const uint32_t twice_mag = 0xC8643210u;
  const int64_t blocks_per_row = k / 32;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * blocks_per_row) return;
  const int64_t row = t / blocks_per_row;
  const int64_t blk = t - row * blocks_per_row;
  const float half_p2 = 0.5f * e8m0_to_f32(scales[row * blocks_per_row + blk]);  // exact
  u32x4_t w = load16(codes + row * (k / 2) + blk * 16);
  float v[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t c = (w[j] >> (4 * i)) & 15u;  // value 2m in byte m's low nibble, 2m+1 in its high one
      float m = (float)((twice_mag >> (4 * (c & 7u))) & 15u) * half_p2;  // exact, inf past fp32, or NaN
      v[j * 8 + i] = __uint_as_float(__float_as_uint(m) | ((c & 8u) << 28));
    }
  }
  const int64_t o = row * k + blk * 32;
#pragma unroll
  for (int j = 0; j < 4; ++j) store8(out, o + 8 * j, v + 8 * j, odt);
}

// MXFP4 in GGUF's blocks (Nx_quant Weights, Mxfp4_blocks): per 32 values the E8M0 scale byte,
// then 16 bytes, byte j holding value j in its low nibble and value j + 16 in its high one.  One
// 17-byte block per lane (byte loads: blocks are not aligned), decoded as in the split layout.
__global__ __launch_bounds__(256) void dequant_mxfp4_blocks_kernel(const uint8_t* __restrict__ blocks, int64_t rows,
                                                                   int64_t k, void* __restrict__ out, int odt) {
  const uint32_t twice_mag = 0xC8643210u;  // twice the e2m1 magnitudes, as above
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * (k / 32)) return;
  const uint8_t* bp = blocks + t * 17;
  const float half_p2 = 0.5f * e8m0_to_f32(bp[0]);
  float v[32];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t b = bp[1 + j];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t c = (b >> (4 * h)) & 15u;
      const float m = (float)((twice_mag >> (4 * (c & 7u))) & 15u) * half_p2;
      v[16 * h + j] = __uint_as_float(__float_as_uint(m) | ((c & 8u) << 28));
    }
  }
  const int64_t o = t * 32;  // rows of k values: block t covers values 32 t .. 32 t + 31
#pragma unroll
  for (int j = 0; j < 4; ++j) store8(out, o + 8 * j, v + 8 * j, odt);
}

__global__ __launch_bounds__(256) void dequant_q8_0_kernel(const uint8_t* __restrict__ blocks, int64_t rows,
                                                           int64_t k, void* __restrict__ out, int odt) {
  const int64_t blocks_per_row = k / 32;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * blocks_per_row) return;
  // 34-byte blocks are 2-byte aligned: read 17 half-words.
  const uint16_t* bp = (const uint16_t*)(blocks + t * 34);
  const float d = f16_bits_to_f32(bp[0]);
  float v[32];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    uint32_t h = bp[1 + j];
    v[2 * j] = d * (float)(int8_t)(h & 0xffu);
    v[2 * j + 1] = d * (float)(int8_t)(h >> 8);
  }
  const int64_t row = t / blocks_per_row;
  const int64_t blk = t - row * blocks_per_row;
  const int64_t o = row * k + blk * 32;
#pragma unroll
  for (int j = 0; j < 4; ++j) store8(out, o + 8 * j, v + 8 * j, odt);
}

// Q4_K (Nx_quant Weights, Q4_K; the layout of ggml's block_q4_K): per 256 values a 144-byte block of
// fp16 d and dmin, 12 bytes of 6-bit scales and mins (sub-block j < 4: low 6 bits of bytes j and
// j + 4; j >= 4: low / high nibble of byte j + 4 under the top two bits of bytes j - 4 / j) and 128
// bytes of quants (values 64 c + i and 64 c + 32 + i in the low / high nibble of quant byte 32 c + i).
// One lane per sub-block of 32 values: value = (d*sc)*q - dmin*m, the products exact in fp32 and one
// rounding at the subtraction.
__global__ __launch_bounds__(256) void dequant_q4_k_kernel(const uint8_t* __restrict__ blocks, int64_t rows,
                                                           int64_t k, void* __restrict__ out, int odt) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * (k / 256) * 8) return;
  const int64_t b = t >> 3;
  const int j = (int)(t & 7);
  const uint8_t* bp = blocks + b * 144;
  const u32x4_t hdr = *(const u32x4_t*)bp;  // d, dmin, scale bytes 0..11 (blocks are 16-byte aligned)
  auto sbyte = [&](int i) __attribute__((always_inline)) { return (hdr[1 + (i >> 2)] >> (8 * (i & 3))) & 0xffu; };
  uint32_t sc, mn;
  if (j < 4) {
    sc = sbyte(j) & 63u;
    mn = sbyte(j + 4) & 63u;
  } else {
    sc = (sbyte(j + 4) & 15u) | ((sbyte(j - 4) >> 6) << 4);
    mn = (sbyte(j + 4) >> 4) | ((sbyte(j) >> 6) << 4);
  }
  const float ds = f16_bits_to_f32(hdr[0] & 0xffffu) * (float)sc;   // exact
  const float dm = f16_bits_to_f32(hdr[0] >> 16) * (float)mn;       // exact
  const u32x4_t q0 = *(const u32x4_t*)(bp + 16 + 32 * (j >> 1));
  const u32x4_t q1 = *(const u32x4_t*)(bp + 32 + 32 * (j >> 1));
  const int sh = 4 * (j & 1);
  float v[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t w = i < 16 ? q0[i >> 2] : q1[(i - 16) >> 2];
    const uint32_t q = (w >> (8 * (i & 3) + sh)) & 15u;
    v[i] = ds * (float)q - dm;  // ds*q is exact: the only rounding is the subtraction's
  }
  const int64_t o = b * 256 + 32 * j;  // rows of k values hold k / 256 blocks each
#pragma unroll
  for (int i = 0; i < 4; ++i) store8(out, o + 8 * i, v + 8 * i, odt);
}

// Q6_K (Nx_quant Weights, Q6_K; the layout of ggml's block_q6_K): per 256 values a 210-byte block of
// 128 bytes of low 4 bits, 64 bytes of high 2 bits, 16 int8 sub-block scales and fp16 d.  Value
// 128 h + 32 g + l (l < 32) takes its low bits from byte 64 h + 32 (g % 2) + l (low nibble for g < 2,
// high for g >= 2) and its high bits from bits 2g, 2g + 1 of byte 128 + 32 h + l; its scale is byte
// 192 + (value / 16).  One lane per (h, g): value = (d*sc)*(q - 32), exact in fp32 (0 * -32 = -0).
__global__ __launch_bounds__(256) void dequant_q6_k_kernel(const uint8_t* __restrict__ blocks, int64_t rows,
                                                           int64_t k, void* __restrict__ out, int odt) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= rows * (k / 256) * 8) return;
  const int64_t b = t >> 3;
  const int h = (int)((t >> 2) & 1), g = (int)(t & 3);
  const uint16_t* bp = (const uint16_t*)(blocks + b * 210);  // blocks are 2-byte aligned
  const float d = f16_bits_to_f32(bp[104]);
  const uint32_t sw = bp[96 + 4 * h + g];  // scale bytes 192 + 8 h + 2 g and the next
  const float s0 = d * (float)(int8_t)(sw & 0xffu), s1 = d * (float)(int8_t)(sw >> 8);  // exact
  const int lo_sh = 4 * (g >> 1), hi_sh = 2 * g;
  float v[32];
#pragma unroll
  for (int l2 = 0; l2 < 16; ++l2) {  // two values (l = 2 l2, 2 l2 + 1) per half-word
    const uint32_t lo = bp[32 * h + 16 * (g & 1) + l2];
    const uint32_t hi = bp[64 + 16 * h + l2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int l = 2 * l2 + e;
      const int q = (int)((((lo >> (8 * e)) >> lo_sh) & 15u) | ((((hi >> (8 * e)) >> hi_sh) & 3u) << 4));
      v[l] = (l < 16 ? s0 : s1) * (float)(q - 32);
    }
  }
  const int64_t o = b * 256 + 128 * h + 32 * g;
#pragma unroll
  for (int i = 0; i < 4; ++i) store8(out, o + 8 * i, v + 8 * i, odt);
}

}  // namespace

hipError_t launch_dequant_affine(const uint32_t* packed, const void* scales, const void* biases, int pdt,
                                 int64_t rows, int64_t k, int bits, int g, void* out, int odt, hipStream_t s) {
  const int64_t total = rows * (k * bits / 128);
  const unsigned nb = (unsigned)((total + 255) / 256);
  const uint16_t* sc = (const uint16_t*)scales;
  const uint16_t* bi = (const uint16_t*)biases;
  if (bits == 2)
    launch_dequant_stream<2>(packed, sc, bi, pdt, rows, k, g, out, odt, s);
  else if (bits == 3)
    launch_dequant_stream<3>(packed, sc, bi, pdt, rows, k, g, out, odt, s);
  else if (bits == 5)
    launch_dequant_stream<5>(packed, sc, bi, pdt, rows, k, g, out, odt, s);
  else if (bits == 6)
    launch_dequant_stream<6>(packed, sc, bi, pdt, rows, k, g, out, odt, s);
  else if (bits == 4 && pdt == DT_BF16)
    dequant_affine_kernel<4, BF16><<<nb, 256, 0, s>>>(packed, sc, bi, rows, k, g, out, odt);
  else if (bits == 4)
    dequant_affine_kernel<4, F16><<<nb, 256, 0, s>>>(packed, sc, bi, rows, k, g, out, odt);
  else if (pdt == DT_BF16)
    dequant_affine_kernel<8, BF16><<<nb, 256, 0, s>>>(packed, sc, bi, rows, k, g, out, odt);
  else
    dequant_affine_kernel<8, F16><<<nb, 256, 0, s>>>(packed, sc, bi, rows, k, g, out, odt);
  return hipGetLastError();
}

hipError_t launch_dequant_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k, void* out,
                                int odt, hipStream_t s) {
  const int64_t total = rows * (k / 32);
  dequant_mxfp4_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(codes, scales, rows, k, out, odt);
  return hipGetLastError();
}

hipError_t launch_dequant_mxfp4_blocks(const uint8_t* blocks, int64_t rows, int64_t k, void* out, int odt,
                                       hipStream_t s) {
  const int64_t total = rows * (k / 32);
  dequant_mxfp4_blocks_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(blocks, rows, k, out, odt);
  return hipGetLastError();
}

hipError_t launch_dequant_q8_0(const uint8_t* blocks, int64_t rows, int64_t k, void* out, int odt, hipStream_t s) {
  const int64_t total = rows * (k / 32);
  dequant_q8_0_kernel<<<(unsigned)((total + 255) / 256), 256, 0, s>>>(blocks, rows, k, out, odt);
  return hipGetLastError();
}

}  // namespace ql

namespace ql {
hipError_t launch_dequant_kquant(int fmt_bytes, const uint8_t* blocks, int64_t rows, int64_t k, void* out, int odt,
                                 hipStream_t s) {
  const int64_t total = rows * (k / 256) * 8;
  const unsigned nb = (unsigned)((total + 255) / 256);
  if (fmt_bytes == 144)
    dequant_q4_k_kernel<<<nb, 256, 0, s>>>(blocks, rows, k, out, odt);
  else
    dequant_q6_k_kernel<<<nb, 256, 0, s>>>(blocks, rows, k, out, odt);
  return hipGetLastError();
}
}  // namespace ql
