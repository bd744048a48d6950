// Affine group quantize + pack (MLX affine storage: code*scale + additive bias, codes packed
// low bits first into uint32 words, scales/biases [n, k/g]; GPTQModel wiki "MLX Apple
// Silicon", Concepts and Packed layouts; gguf2mlx-stream section 01).
//
// One lane owns 8 consecutive weights of a row: one packed word at 4 bits, two at 8 bits, and at
// the bitstream widths (2, 3, 5, 6 bits) a quarter of a 32-code chunk of BITS words.
// The g/8 lanes of a group are consecutive in the wave, so the group min/max is a butterfly
// over g/8 lanes.  HBM traffic per weight: 4 B read, bits/8 B + 4/g B written.
#include "device_common.hpp"
#include "launch.hpp"

namespace ql {
namespace {

// Monotone integer key of an fp32 value under the IEEE total order (-0 < +0).
__device__ __forceinline__ int32_t order_key(float f) {
  int32_t i = __float_as_int(f);
  return i ^ ((i >> 31) & 0x7fffffff);
}
__device__ __forceinline__ float from_order_key(int32_t i) { return __int_as_float(i ^ ((i >> 31) & 0x7fffffff)); }

template <int BITS, typename PT>
__global__ __launch_bounds__(256) void quantize_kernel(const float* __restrict__ w, int64_t n, int64_t k, int g,
                                                       uint32_t* __restrict__ packed, uint16_t* __restrict__ scales,
                                                       uint16_t* __restrict__ biases) {
  const int64_t lanes_per_row = k >> 3;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = n * lanes_per_row;
  // Lanes past the end still take part in the shuffles (their group is wholly past the end
  // because totals are multiples of g/8), they only skip loads and stores.
  const bool live = t < total;
  const int64_t tt = live ? t : total - 1;
  const int64_t row = tt / lanes_per_row;
  const int64_t c8 = tt - row * lanes_per_row;
  const float* src = w + row * k + c8 * 8;
  f32x4_t a = *(const f32x4_t*)src;
  f32x4_t b = *(const f32x4_t*)(src + 4);
  float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  int32_t kmin = order_key(v[0]), kmax = kmin;
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    int32_t key = order_key(v[i]);
    kmin = min(kmin, key);
    kmax = max(kmax, key);
  }
  const int lpg = g >> 3;  // lanes per group: 4, 8 or 16
  for (int off = 1; off < lpg; off <<= 1) {
    kmin = min(kmin, __shfl_xor(kmin, off));
    kmax = max(kmax, __shfl_xor(kmax, off));
  }
  const float mn = from_order_key(kmin);
  const float mx = from_order_key(kmax);
  const float levels = (float)((1 << BITS) - 1);
  const float s32 = __fdiv_rn(mx - mn, levels);
  const uint32_t sbits = f32_to_bits<PT>(s32);
  const uint32_t bbits = f32_to_bits<PT>(mn);
  const float s = param_to_f32<PT>(sbits);
  const float bb = param_to_f32<PT>(bbits);
  uint32_t q[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float tq = __fdiv_rn(v[i] - bb, s);
    float r = __builtin_rintf(tq);
    r = r > levels ? levels : r;
    r = r > 0.0f ? r : 0.0f;  // also maps NaN to 0
    q[i] = (s == 0.0f) ? 0u : (uint32_t)r;
  }
  if constexpr (is_stream_bits(BITS)) {
    // Bitstream widths: the 4 lanes of a 32-code chunk (consecutive lanes, c8 % 4 = 0..3) hold
    // 8 * BITS consecutive bits of the chunk's stream each; every lane gathers all four parts
    // and writes the chunk's words w with w % 4 == c8 % 4.
    uint64_t mine = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) mine |= (uint64_t)q[i] << (BITS * i);
    const int base = (int)(threadIdx.x & 63) & ~3;
    uint64_t part[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)mine, base + j);
      const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(mine >> 32), base + j);
      part[j] = (uint64_t)lo | ((uint64_t)hi << 32);
    }
    if (!live) return;
    const int j0 = (int)(c8 & 3);
    uint32_t* dst = packed + row * (k / 32 * BITS) + (c8 >> 2) * BITS;
#pragma unroll
    for (int wi = 0; wi < BITS; ++wi) {
      if (wi % 4 != j0) continue;
      // stream bits [32 wi, 32 wi + 32): part j covers [8 BITS j, 8 BITS (j + 1))
      uint32_t word = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 8 * BITS * j - 32 * wi;  // where part j starts relative to the word
        if (d >= 32 || d + 8 * BITS <= 0) continue;
        word |= d >= 0 ? (uint32_t)(part[j] << d) : (uint32_t)(part[j] >> (-d));
      }
      dst[wi] = word;
    }
  }
  if (!live) return;
  if constexpr (is_stream_bits(BITS)) {
  } else if (BITS == 4) {
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) word |= q[i] << (4 * i);
    packed[row * (k >> 3) + c8] = word;
  } else {
    uint32_t w0 = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
    uint32_t w1 = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
    u32x2_t pr = {w0, w1};
    *(u32x2_t*)(packed + row * (k >> 2) + c8 * 2) = pr;
  }
  if ((c8 & (lpg - 1)) == 0) {
    const int64_t gi = row * (k / g) + (c8 * 8) / g;
    scales[gi] = (uint16_t)sbits;
    biases[gi] = (uint16_t)bbits;
  }
}

// quantize_q8_0 (Nx_quant API docs, quantize_q8_0): per block of 32 fp32 values, d = amax / 127
// stored as fp16 (nearest), quants round(v * (1/d)) half away from zero with 1/d from the fp32 d,
// products in fp32.  Non-finite rules: d == 0 or 1/d infinite -> zero bytes; a block holding an
// infinity and no NaN -> d = +inf, quants 0; a block holding a NaN -> d = the fp16 quiet NaN
// 0x7E00, quants 0.  Eight lanes per block (4 values each, one 16-byte load), reduced by shuffles.
__global__ __launch_bounds__(256) void quantize_q8_0_kernel(const float* __restrict__ w, int64_t nblocks,
                                                            uint8_t* __restrict__ blocks) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t b = t >> 3;
  const int j = (int)(t & 7);
  const bool live = b < nblocks;  // the 8 lanes of a block are live together
  const int64_t bb = live ? b : nblocks - 1;
  const f32x4_t v = *(const f32x4_t*)(w + bb * 32 + 4 * j);
  float am = 0.0f;
  int has_nan = 0, has_inf = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    has_nan |= v[e] != v[e];
    has_inf |= __builtin_isinf(v[e]) ? 1 : 0;
    am = fmaxf(am, fabsf(v[e]));  // a NaN is skipped here and handled by the flags
  }
#pragma unroll
  for (int off = 1; off < 8; off <<= 1) {
    am = fmaxf(am, __shfl_xor(am, off));
    has_nan |= __shfl_xor(has_nan, off);
    has_inf |= __shfl_xor(has_inf, off);
  }
  const bool finite = !has_nan && !has_inf;
  const float d = __fdiv_rn(am, 127.0f);
  const float inv = d == 0.0f ? 0.0f : __fdiv_rn(1.0f, d);
  const bool zero = !finite || d == 0.0f || __builtin_isinf(inv);
  uint32_t qb[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) qb[e] = zero ? 0u : ((uint32_t)(int32_t)roundf(v[e] * inv) & 0xffu);
  uint32_t d_bits = (finite && !zero) ? f32_to_f16_bits(d) : 0u;
  if (has_inf) d_bits = 0x7C00u;
  if (has_nan) d_bits = 0x7E00u;
  if (!live) return;
  uint16_t* o = (uint16_t*)(blocks + bb * 34);  // 34-byte blocks: 2-byte aligned
  if (j == 0) o[0] = (uint16_t)d_bits;
  o[1 + 2 * j] = (uint16_t)(qb[0] | (qb[1] << 8));
  o[2 + 2 * j] = (uint16_t)(qb[2] | (qb[3] << 8));
}

}  // namespace

hipError_t launch_quantize_q8_0(const float* w, int64_t rows, int64_t k, uint8_t* blocks, hipStream_t s) {
  const int64_t nblocks = rows * (k / 32);
  quantize_q8_0_kernel<<<(unsigned)((nblocks * 8 + 255) / 256), 256, 0, s>>>(w, nblocks, blocks);
  return hipGetLastError();
}

hipError_t launch_quantize(const float* w, int64_t n, int64_t k, int bits, int g, int pdt, uint32_t* packed,
                           void* scales, void* biases, hipStream_t s) {
  const int64_t total = n * (k >> 3);
  const unsigned blocks = (unsigned)((total + 255) / 256);
  uint16_t* sc = (uint16_t*)scales;
  uint16_t* bi = (uint16_t*)biases;
#define QL_QUANT_STREAM(B)                                                              \
  if (bits == B) {                                                                      \
    if (pdt == DT_BF16)                                                                 \
      quantize_kernel<B, BF16><<<blocks, 256, 0, s>>>(w, n, k, g, packed, sc, bi);      \
    else                                                                                \
      quantize_kernel<B, F16><<<blocks, 256, 0, s>>>(w, n, k, g, packed, sc, bi);       \
    return hipGetLastError();                                                           \
  }
  QL_QUANT_STREAM(2)
  QL_QUANT_STREAM(3)
  QL_QUANT_STREAM(5)
  QL_QUANT_STREAM(6)
#undef QL_QUANT_STREAM
  if (bits == 4 && pdt == DT_BF16)
    quantize_kernel<4, BF16><<<blocks, 256, 0, s>>>(w, n, k, g, packed, sc, bi);
  else if (bits == 4)
    quantize_kernel<4, F16><<<blocks, 256, 0, s>>>(w, n, k, g, packed, sc, bi);
  else if (pdt == DT_BF16)
    quantize_kernel<8, BF16><<<blocks, 256, 0, s>>>(w, n, k, g, packed, sc, bi);
  else
    quantize_kernel<8, F16><<<blocks, 256, 0, s>>>(w, n, k, g, packed, sc, bi);
  return hipGetLastError();
}

}  // namespace ql
