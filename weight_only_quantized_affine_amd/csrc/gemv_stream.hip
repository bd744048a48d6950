// Decode GEMV on affine rows at the bitstream widths (2, 3, 5 or 6 bits; GPTQModel wiki "MLX Apple
// Silicon", Concepts and Packed layouts and exact transcoding; Nx_quant API docs, Products: apply):
//   y[m, n] = sum_k x[m, k] * (q[n, k] * s[n, k/g] + b[n, k/g]),   fp32 accumulation.
// A row's 32-code chunk (BITS words) lies in one group (g >= 32), so per chunk
//   sum_i x_i (q_i s + b) = s * sum_i x_i q_i + b * sum_i x_i,
// with the codes exact in fp32 and one fp32 product-sum per (x row, chunk).
//
// Work split: 256 threads (4 waves); wave w takes the R weight rows 4R * block + R w .. + R - 1,
// its lanes the chunks along k (lane, lane + 64, ...), so the x values of a chunk are read once
// from LDS for R rows.  x (MT rows, 16-bit) is staged in LDS in slices of at most 32 KiB / MT
// values; every lane keeps R x MT partial sums, reduced over the wave at the end.
#include "device_common.hpp"
#include "launch.hpp"

namespace ql {
namespace {

constexpr int kStreamLdsBytes = 65536;  // x slice: MT rows of ks 16-bit values

template <typename XT> __device__ __forceinline__ float xval(uint32_t b);
template <> __device__ __forceinline__ float xval<BF16>(uint32_t b) { return bf16_bits_to_f32(b); }
template <> __device__ __forceinline__ float xval<F16>(uint32_t b) { return f16_bits_to_f32(b); }

template <int BITS, typename XT, typename PT, int MT, int R>
__global__ __launch_bounds__(256) void gemv_stream_kernel(const uint16_t* __restrict__ x, int m, int64_t k,
                                                          const uint32_t* __restrict__ packed,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint16_t* __restrict__ biases, int64_t n, int g,
                                                          const uint16_t* __restrict__ layer_bias, void* __restrict__ y,
                                                          int ydt, int ks) {
  extern __shared__ __attribute__((aligned(16))) uint16_t sx[];  // [MT][ks]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row0 = (int64_t)blockIdx.x * (4 * R) + (int64_t)wave * R;
  const int64_t wpr = k / 32 * BITS;  // words per weight row
  const int groups = (int)(k / g);
  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[r][j] = 0.0f;
  // rows past n read row n - 1 (never stored)
  int64_t wrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) wrow[r] = min(row0 + r, n - 1);

  for (int64_t k0 = 0; k0 < k; k0 += ks) {
    const int kn = (int)min((int64_t)ks, k - k0);
    __syncthreads();  // every wave is done with the previous slice
    // stage x[:, k0 .. k0 + kn) as 16-byte pieces; x rows past m are zeros
    const int pieces = kn / 8;
    for (int i = tid; i < MT * pieces; i += 256) {
      const int j = i / pieces, c = i - j * pieces;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (j < m) v = load16(x + (int64_t)j * k + k0 + 8 * c);
      *(u32x4_t*)(sx + j * ks + 8 * c) = v;
    }
    __syncthreads();
    const int nch = kn / 32;
    const int64_t c0 = k0 / 32;
    for (int c = lane; c < nch; c += 64) {
      uint32_t w[R][BITS];
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int i = 0; i < BITS; ++i) w[r][i] = packed[wrow[r] * wpr + (c0 + c) * BITS + i];
      float p[R][MT], xs[MT];
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        xs[j] = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) p[r][j] = 0.0f;
      }
      // 8 codes at a time: one 16-byte LDS read per x row
#pragma unroll
      for (int q8 = 0; q8 < 4; ++q8) {
        float xv[MT][8];
#pragma unroll
        for (int j = 0; j < MT; ++j) {
          const u32x4_t v = *(const u32x4_t*)(sx + j * ks + 32 * c + 8 * q8);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xv[j][2 * e] = xval<XT>(v[e] & 0xffffu);
            xv[j][2 * e + 1] = xval<XT>(v[e] >> 16);
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) xs[j] += xv[j][e];
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float qv = (float)stream_code<BITS>(w[r], 8 * q8 + e);
#pragma unroll
            for (int j = 0; j < MT; ++j) p[r][j] = __builtin_fmaf(xv[j][e], qv, p[r][j]);
          }
      }
      const int gi = (int)((k0 + 32 * c) / g);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float s = param_to_f32<PT>(scales[wrow[r] * groups + gi]);
        const float b = param_to_f32<PT>(biases[wrow[r] * groups + gi]);
#pragma unroll
        for (int j = 0; j < MT; ++j) acc[r][j] = __builtin_fmaf(s, p[r][j], __builtin_fmaf(b, xs[j], acc[r][j]));
      }
    }
  }
  // wave sums, then lane 0 writes its rows
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < MT; ++j)
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) acc[r][j] += __shfl_xor(acc[r][j], off);
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = row0 + r;
      if (row >= n) continue;
      const float add = layer_bias ? xval<XT>(layer_bias[row]) : 0.0f;  // x's dtype
#pragma unroll
      for (int j = 0; j < MT; ++j)
        if (j < m) store_out(y, (int64_t)j * n + row, acc[r][j] + add, ydt);
    }
  }
}

// rows per wave: enough workgroups to spread over the chip (at least 512 when n allows), at most
// R x MT = 16 partial sums per lane and R <= 8
template <int BITS, typename XT, typename PT, int MT, int RR>
void launch_r(const GemvStreamArgs& a, int ks, size_t lds, hipStream_t s) {
  gemv_stream_kernel<BITS, XT, PT, MT, RR><<<(unsigned)((a.n + 4 * RR - 1) / (4 * RR)), 256, lds, s>>>(
      (const uint16_t*)a.x, a.m, a.k, a.packed, (const uint16_t*)a.scales, (const uint16_t*)a.biases, a.n, a.g,
      (const uint16_t*)a.layer_bias, a.y, a.ydt, ks);
}

template <int BITS, typename XT, typename PT, int MT>
hipError_t launch_mt(const GemvStreamArgs& a, hipStream_t s) {
  const int ks = (int)std::max<int64_t>(32, std::min<int64_t>(a.k, kStreamLdsBytes / 2 / MT / 32 * 32));
  const size_t lds = (size_t)MT * (size_t)ks * 2;
  constexpr int rmax = 16 / MT < 8 ? 16 / MT : 8;
  int r = 1;
  while (r * 2 <= rmax && (a.n + 8 * r - 1) / (8 * r) >= 512) r *= 2;
  if (r == 1) launch_r<BITS, XT, PT, MT, 1>(a, ks, lds, s);
  if constexpr (rmax >= 2) if (r == 2) launch_r<BITS, XT, PT, MT, 2>(a, ks, lds, s);
  if constexpr (rmax >= 4) if (r == 4) launch_r<BITS, XT, PT, MT, 4>(a, ks, lds, s);
  if constexpr (rmax >= 8) if (r == 8) launch_r<BITS, XT, PT, MT, 8>(a, ks, lds, s);
  return hipGetLastError();
}

template <int BITS, typename XT, typename PT>
hipError_t launch_b(const GemvStreamArgs& a, hipStream_t s) {
  if (a.m <= 1) return launch_mt<BITS, XT, PT, 1>(a, s);
  if (a.m <= 2) return launch_mt<BITS, XT, PT, 2>(a, s);
  if (a.m <= 4) return launch_mt<BITS, XT, PT, 4>(a, s);
  return launch_mt<BITS, XT, PT, 8>(a, s);
}

template <int BITS>
hipError_t launch_bits(const GemvStreamArgs& a, hipStream_t s) {
  if (a.xdt == DT_BF16)
    return a.pdt == DT_BF16 ? launch_b<BITS, BF16, BF16>(a, s) : launch_b<BITS, BF16, F16>(a, s);
  return a.pdt == DT_BF16 ? launch_b<BITS, F16, BF16>(a, s) : launch_b<BITS, F16, F16>(a, s);
}

}  // namespace

hipError_t launch_gemv_stream(const GemvStreamArgs& a, hipStream_t s) {
  switch (a.bits) {
    case 2:
      return launch_bits<2>(a, s);
    case 3:
      return launch_bits<3>(a, s);
    case 5:
      return launch_bits<5>(a, s);
    case 6:
      return launch_bits<6>(a, s);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace ql
