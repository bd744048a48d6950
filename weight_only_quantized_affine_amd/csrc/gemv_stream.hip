// Decode GEMV on affine rows at the bitstream widths (2, 3, 5 or 6 bits; GPTQModel wiki "MLX Apple
// Silicon", Concepts and Packed layouts and exact transcoding; Nx_quant API docs, Products: apply):
//   y[m, n] = sum_k x[m, k] * (q[n, k] * s[n, k/g] + b[n, k/g]),   fp32 accumulation.
// A row's 32-code chunk (BITS words) lies in one group (g >= 32), so per chunk
//   sum_i x_i (q_i s + b) = s * sum_i x_i q_i + b * sum_i x_i.
// The sums run on v_dot2 (two 16-bit products, fp32 accumulation) with x pairs straight from LDS
// and code pairs made in registers, both exact: with bf16 x a code is the bf16 128 + q (exact for
// q < 128), so the pair sum is P + 128 X and the chunk adds s (P + 128 X) + (b - 128 s) X; with
// fp16 x a code is the fp16 subnormal q 2^-24 (its bits are q), so the pair sum is P 2^-24.
// X = sum_i x_i is a dot with (1, 1).
//
// Work split: 256 threads (4 waves).  A wave's lanes form groups of LG lanes (8 to 64: no more
// than a row has chunks); a group takes R weight rows and strides over their chunks, so every x
// pair read from LDS feeds R rows.  A workgroup covers 4 (64 / LG) R rows per pass and makes
// `passes` passes when x fits in LDS whole (x staged once); otherwise x goes through LDS in
// slices of ks values and the workgroup makes one pass.  Partial sums are reduced over each group
// at the end of a pass.
#include "device_common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace ql {
namespace {

typedef __attribute__((ext_vector_type(2))) uint16_t u16x2_t;

__device__ __forceinline__ uint32_t vgpr_const(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}


template <typename XT> __device__ __forceinline__ float xval(uint32_t b);
template <> __device__ __forceinline__ float xval<BF16>(uint32_t b) { return bf16_bits_to_f32(b); }
template <> __device__ __forceinline__ float xval<F16>(uint32_t b) { return f16_bits_to_f32(b); }

// Rows of x per kernel (MT) -> weight rows per lane group (R): at most 16 partial sums.
constexpr int stream_rows(int mt) { return mt >= 8 ? 2 : (mt >= 4 ? 4 : 8); }

template <int BITS, typename XT, int MT>
__global__ __launch_bounds__(256) void gemv_stream_kernel(const uint16_t* __restrict__ x, int m, int64_t k,
                                                          const uint32_t* __restrict__ packed,
                                                          const uint16_t* __restrict__ scales,
                                                          const uint16_t* __restrict__ biases, int pbf16, int64_t n,
                                                          int g, const uint16_t* __restrict__ layer_bias,
                                                          void* __restrict__ y, int ydt, int ks, int lg, int passes) {
  constexpr int R = stream_rows(MT);
  constexpr bool BX = std::is_same<XT, BF16>::value;
  constexpr uint32_t MAGIC = BX ? 0x43004300u : 0u;    // bf16 128 in both halves (fp16: none)
  constexpr uint32_t ONES = BX ? 0x3F803F80u : 0x3C003C00u;  // (1, 1)
  extern __shared__ __attribute__((aligned(16))) uint16_t sx[];  // [MT][ks]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / lg, cl = lane - sub * lg;
  const int rpp = 4 * (64 / lg) * R;  // rows per workgroup pass
  const int64_t wpr = k / 32 * BITS;  // words per weight row
  const int groups = (int)(k / g);
  const bool one_slice = k <= ks;

  auto stage = [&](int64_t k0, int kn) {
    const int pieces = kn / 8;
    for (int i = tid; i < MT * pieces; i += 256) {
      const int j = i / pieces, c = i - j * pieces;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (j < m) v = load16(x + (int64_t)j * k + k0 + 8 * c);  // x rows past m are zeros
      *(u32x4_t*)(sx + j * ks + 8 * c) = v;
    }
  };
  if (one_slice) {
    stage(0, (int)k);
    __syncthreads();
  }

  for (int pass = 0; pass < passes; ++pass) {
    const int64_t row0 = ((int64_t)blockIdx.x * passes + pass) * rpp + (int64_t)(wave * (64 / lg) + sub) * R;
    if (row0 - (int64_t)(wave * (64 / lg) + sub) * R >= n) break;  // the workgroup's rows are done
    int64_t wrow[R];  // rows past n read row n - 1 (never stored)
#pragma unroll
    for (int r = 0; r < R; ++r) wrow[r] = min(row0 + r, n - 1);
    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < MT; ++j) acc[r][j] = 0.0f;

    for (int64_t k0 = 0; k0 < k; k0 += ks) {
      const int kn = (int)min((int64_t)ks, k - k0);
      if (!one_slice) {
        __syncthreads();  // every wave is done with the previous slice
        stage(k0, kn);
        __syncthreads();
      }
      const int nch = kn / 32;
      const int c0 = (int)(k0 / 32);
      for (int c = cl; c < nch; c += lg) {
        uint32_t w[R][BITS];
        float sc[R], bc[R];
        const int gi = (c0 + c) * 32 / g;
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
          for (int i = 0; i < BITS; ++i) w[r][i] = packed[wrow[r] * wpr + (int64_t)(c0 + c) * BITS + i];
          const uint32_t sb = scales[wrow[r] * groups + gi], bb = biases[wrow[r] * groups + gi];
          sc[r] = pbf16 ? bf16_bits_to_f32(sb) : f16_bits_to_f32(sb);
          bc[r] = pbf16 ? bf16_bits_to_f32(bb) : f16_bits_to_f32(bb);
        }
        float p[R][MT], xs[MT];
#pragma unroll
        for (int j = 0; j < MT; ++j) {
          xs[j] = 0.0f;
#pragma unroll
          for (int r = 0; r < R; ++r) p[r][j] = 0.0f;
        }
#pragma unroll
        for (int q8 = 0; q8 < 4; ++q8) {
          u32x4_t xq[MT];  // x values 8 q8 .. 8 q8 + 7 of the chunk, as 4 pairs
#pragma unroll
          for (int j = 0; j < MT; ++j) {
            xq[j] = *(const u32x4_t*)(sx + j * ks + 32 * c + 8 * q8);
#pragma unroll
            for (int e = 0; e < 4; ++e) xs[j] = dot2(XT(), xq[j][e], ONES, xs[j]);
          }
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 8 * q8 + 2 * e;
              const uint32_t pr = (stream_code<BITS>(w[r], i) | MAGIC) | (stream_code<BITS>(w[r], i + 1) << 16);
#pragma unroll
              for (int j = 0; j < MT; ++j) p[r][j] = dot2(XT(), xq[j][e], pr, p[r][j]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const float sp = BX ? sc[r] : sc[r] * 16777216.0f;  // fp16 codes carry 2^-24
          const float bx = BX ? __builtin_fmaf(-128.0f, sc[r], bc[r]) : bc[r];
#pragma unroll
          for (int j = 0; j < MT; ++j) acc[r][j] = __builtin_fmaf(sp, p[r][j], __builtin_fmaf(bx, xs[j], acc[r][j]));
        }
      }
    }
    // group sums, then the group's first lane writes its rows
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < MT; ++j)
        for (int off = lg >> 1; off >= 1; off >>= 1) acc[r][j] += __shfl_xor(acc[r][j], off);
    if (cl == 0) {
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
}

// k a multiple of 128: each lane takes 4 consecutive chunks of a row (128 codes, BITS 16-byte
// loads) per step, R rows at a time (up to 4 x BITS loads of 16 bytes in flight per lane); the
// scale and bias of each group the 4 chunks meet are loaded once.  Same arithmetic as above.
// table != NULL: a problem list; workgroup b takes tile tiles[b] (problem, row tile): the
// problem's arguments come from its descriptor (lane group width in `batches`), one pass of
// 4 (64 / lg) R rows, ks = min(k, ks) for that problem.
template <int BITS, typename XT, int MT, int R>
__global__ __launch_bounds__(256) void gemv_quad_kernel(const uint16_t* __restrict__ x, int m, int64_t k,
                                                        const uint32_t* __restrict__ packed,
                                                        const uint16_t* __restrict__ scales,
                                                        const uint16_t* __restrict__ biases, int pbf16, int64_t n,
                                                        int g, const uint16_t* __restrict__ layer_bias,
                                                        void* __restrict__ y, int ydt, int ks, int lg, int passes,
                                                        const GemvDesc* __restrict__ table,
                                                        const GemvTile* __restrict__ tiles) {
  int64_t first_row;
  if (table) {
    const GemvTile t = tiles[blockIdx.x];
    const GemvDesc& d = table[t.prob];
    x = (const uint16_t*)d.x;
    m = (int)d.m;
    k = d.k;
    packed = d.packed;
    scales = (const uint16_t*)d.scales;
    biases = (const uint16_t*)d.biases;
    n = d.n;
    g = d.group_size;
    layer_bias = (const uint16_t*)d.layer_bias;
    y = d.y;
    lg = d.batches;
    passes = 1;
    ks = (int)max((int64_t)128, min(k, (int64_t)ks));
    first_row = (int64_t)t.local * (4 * (64 / lg) * R);
  } else {
    first_row = (int64_t)blockIdx.x * passes * (4 * (64 / lg) * R);
  }
  constexpr bool BX = std::is_same<XT, BF16>::value;
  constexpr uint32_t MAGIC = BX ? 0x43004300u : 0u;
  constexpr uint32_t ONES = BX ? 0x3F803F80u : 0x3C003C00u;
  // the 2- and 3-bit pair masks and the offset in VGPRs once (the VOP3 forms, v_and_or_b32 among them,
  // take no literal operand)
  const uint32_t kMask2 = vgpr_const(0x00030003u), kMagic = vgpr_const(MAGIC);
  const uint32_t kMask3 = vgpr_const(0x00070007u);
  // x row j, value v at sx[j * pitch + v + 8 (v / 128)]: 16 bytes of padding after every 128
  // values, so that the lanes of a group (quads 256 bytes apart) read distinct banks
  extern __shared__ __attribute__((aligned(16))) uint16_t sx[];
  const int pitch = ks + ks / 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int sub = lane / lg, cl = lane - sub * lg;
  const int rpp = 4 * (64 / lg) * R;
  const int64_t wpr = k / 32 * BITS;
  const int groups = (int)(k / g);
  const bool one_slice = k <= ks;

  auto stage = [&](int64_t k0, int kn) {
    const int pieces = kn / 8;
    for (int i = tid; i < MT * pieces; i += 256) {
      const int j = i / pieces, c = i - j * pieces;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (j < m) v = load16(x + (int64_t)j * k + k0 + 8 * c);
      *(u32x4_t*)(sx + j * pitch + 8 * c + 8 * (c >> 4)) = v;
    }
  };
  if (one_slice) {
    stage(0, (int)k);
    __syncthreads();
  }

  for (int pass = 0; pass < passes; ++pass) {
    const int64_t base = first_row + (int64_t)pass * rpp;
    if (base >= n) break;  // uniform over the workgroup
    const int64_t row0 = base + (int64_t)(wave * (64 / lg) + sub) * R;
    int64_t wrow[R];
#pragma unroll
    for (int r = 0; r < R; ++r) wrow[r] = min(row0 + r, n - 1);
    float acc[R][MT];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < MT; ++j) acc[r][j] = 0.0f;

    for (int64_t k0 = 0; k0 < k; k0 += ks) {
      const int kn = (int)min((int64_t)ks, k - k0);
      if (!one_slice) {
        __syncthreads();
        stage(k0, kn);
        __syncthreads();
      }
      const int nq = kn / 128;
      for (int qd = cl; qd < nq; qd += lg) {
        const int64_t q0 = k0 / 128 + qd;  // quad of the row
        u32x4_t w[R][BITS];
        float sc[R][4], bc[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
          for (int i = 0; i < BITS; ++i) w[r][i] = load16(packed + wrow[r] * wpr + q0 * (4 * BITS) + 4 * i);
          // chunk cc starts a group when 32 cc is a multiple of g (always for cc == 0)
#pragma unroll
          for (int cc = 0; cc < 4; ++cc) {
            if (cc == 0 || (32 * cc) % g == 0) {
              const int64_t gi = wrow[r] * groups + (q0 * 128 + 32 * cc) / g;
              const uint32_t sb = scales[gi], bb = biases[gi];
              sc[r][cc] = pbf16 ? bf16_bits_to_f32(sb) : f16_bits_to_f32(sb);
              bc[r][cc] = pbf16 ? bf16_bits_to_f32(bb) : f16_bits_to_f32(bb);
            } else {
              sc[r][cc] = sc[r][cc - 1];
              bc[r][cc] = bc[r][cc - 1];
            }
          }
        }
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          float p[R][MT], xs[MT];
#pragma unroll
          for (int j = 0; j < MT; ++j) {
            xs[j] = 0.0f;
#pragma unroll
            for (int r = 0; r < R; ++r) p[r][j] = 0.0f;
          }
#pragma unroll
          for (int q8 = 0; q8 < 4; ++q8) {
            u32x4_t xq[MT];
#pragma unroll
            for (int j = 0; j < MT; ++j) {
              xq[j] = *(const u32x4_t*)(sx + j * pitch + qd * 136 + 32 * cc + 8 * q8);
#pragma unroll
              for (int e = 0; e < 4; ++e) xs[j] = dot2(XT(), xq[j][e], ONES, xs[j]);
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
              uint32_t cw[BITS];  // the chunk's words
#pragma unroll
              for (int i = 0; i < BITS; ++i) cw[i] = w[r][(cc * BITS + i) >> 2][(cc * BITS + i) & 3];
              if constexpr (BITS == 2) {
                // the 8 codes of k-step q8 are one 16-bit half of a word: copied into both halves,
                // one packed 16-bit shift per pair puts code 2e in the low half and 2e + 1 in the
                // high one, and one and-or masks them and adds the offset
                const uint32_t wd = cw[q8 >> 1];
                const uint32_t hw = (q8 & 1) ? (wd >> 16) : (wd & 0xffffu);
                const u16x2_t both = __builtin_bit_cast(u16x2_t, hw | (hw << 16));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const u16x2_t sh = {(uint16_t)(4 * e), (uint16_t)(4 * e + 2)};
                  const uint32_t pr = (__builtin_bit_cast(uint32_t, both >> sh) & kMask2) | kMagic;
#pragma unroll
                  for (int j = 0; j < MT; ++j) p[r][j] = dot2(XT(), xq[j][e], pr, p[r][j]);
                }
              } else if constexpr (BITS == 3) {
                // two pairs (12 bits) start at bit 6 (2 e) of the stream: one 16-bit window of the
                // chunk (funnel shift), copied into both halves, serves both; per pair one packed
                // shift and one and-or as above
#pragma unroll
                for (int e2 = 0; e2 < 2; ++e2) {
                  const int pos = 3 * (8 * q8 + 4 * e2);
                  const int wi = pos >> 5, sh = pos & 31;
                  // only the window's 12 low bits are used: the next word is read only when they
                  // cross into it (it then exists: pos + 12 <= 96)
                  const uint32_t win =
                      sh + 12 <= 32 ? (cw[wi] >> sh) : ((cw[wi] >> sh) | (cw[wi + 1] << (32 - sh)));
                  const u16x2_t both = __builtin_bit_cast(u16x2_t, (win & 0xffffu) | (win << 16));
#pragma unroll
                  for (int h = 0; h < 2; ++h) {
                    const u16x2_t shv = {(uint16_t)(6 * h), (uint16_t)(6 * h + 3)};
                    const uint32_t pr = (__builtin_bit_cast(uint32_t, both >> shv) & kMask3) | kMagic;
#pragma unroll
                    for (int j = 0; j < MT; ++j) p[r][j] = dot2(XT(), xq[j][2 * e2 + h], pr, p[r][j]);
                  }
                }
              } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  const int i = 8 * q8 + 2 * e;
                  const uint32_t pr = (stream_code<BITS>(cw, i) | MAGIC) | (stream_code<BITS>(cw, i + 1) << 16);
#pragma unroll
                  for (int j = 0; j < MT; ++j) p[r][j] = dot2(XT(), xq[j][e], pr, p[r][j]);
                }
              }
            }
          }
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float sp = BX ? sc[r][cc] : sc[r][cc] * 16777216.0f;
            const float bx = BX ? __builtin_fmaf(-128.0f, sc[r][cc], bc[r][cc]) : bc[r][cc];
#pragma unroll
            for (int j = 0; j < MT; ++j)
              acc[r][j] = __builtin_fmaf(sp, p[r][j], __builtin_fmaf(bx, xs[j], acc[r][j]));
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < MT; ++j)
        for (int off = lg >> 1; off >= 1; off >>= 1) acc[r][j] += __shfl_xor(acc[r][j], off);
    if (cl == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int64_t row = row0 + r;
        if (row >= n) continue;
        const float add = layer_bias ? xval<XT>(layer_bias[row]) : 0.0f;
#pragma unroll
        for (int j = 0; j < MT; ++j)
          if (j < m) store_out(y, (int64_t)j * n + row, acc[r][j] + add, ydt);
      }
    }
  }
}

template <int BITS, typename XT, int MT, int R>
void launch_quad_r(const GemvStreamArgs& a, int ks, size_t lds, int lg, int64_t rows_per_pass, hipStream_t s) {
  const int64_t row_groups = (a.n + rows_per_pass - 1) / rows_per_pass;
  int passes = 1;
  if (a.k <= ks)
    while (passes < 8 && (row_groups + 2 * passes - 1) / (2 * passes) >= 1024) passes *= 2;
  const int64_t grid = (row_groups + passes - 1) / passes;
  gemv_quad_kernel<BITS, XT, MT, R><<<(unsigned)grid, 256, lds, s>>>(
      (const uint16_t*)a.x, a.m, a.k, a.packed, (const uint16_t*)a.scales, (const uint16_t*)a.biases,
      a.pdt == DT_BF16, a.n, a.g, (const uint16_t*)a.layer_bias, a.y, a.ydt, ks, lg, passes, nullptr, nullptr);
}

template <int BITS, typename XT, int MT>
hipError_t launch_quad(const GemvStreamArgs& a, hipStream_t s) {
  const int ks = stream_quad_ks(a.k, MT);
  const size_t lds = stream_quad_lds(a.k, MT);
  int lg = stream_quad_lg(a.k, MT);
  // rows per lane group: at most 8 partial sums; while the chip would get fewer than 512
  // workgroups, fewer rows per group, then wider groups
  constexpr int rmax = stream_quad_rows(MT);
  int r = rmax;
  auto wgs = [&](int rr, int l) { return (a.n + 4 * (64 / l) * rr - 1) / (4 * (64 / l) * rr); };
  while (wgs(r, lg) < 512) {
    if (r > 1)
      r /= 2;
    else if (lg < 64)
      lg *= 2;
    else
      break;
  }
  if (r == 4) {
    if constexpr (rmax >= 4) launch_quad_r<BITS, XT, MT, 4>(a, ks, lds, lg, 4 * (64 / lg) * 4, s);
  } else if (r == 2) {
    if constexpr (rmax >= 2) launch_quad_r<BITS, XT, MT, 2>(a, ks, lds, lg, 4 * (64 / lg) * 2, s);
  } else {
    launch_quad_r<BITS, XT, MT, 1>(a, ks, lds, lg, 4 * (64 / lg), s);
  }
  return hipGetLastError();
}

template <int BITS, typename XT, int MT>
hipError_t launch_mt(const GemvStreamArgs& a, hipStream_t s) {
  if (a.k % 128 == 0 && a.k > 0) return launch_quad<BITS, XT, MT>(a, s);
  const int ks = (int)std::max<int64_t>(32, std::min<int64_t>(a.k, kStreamLdsBytes / 2 / MT / 32 * 32));
  const size_t lds = (size_t)MT * (size_t)ks * 2;
  // lanes per row group: no more than the chunks of a row (up to 64), whole chunk rounds when possible
  const int64_t nch = std::max<int64_t>(1, std::min<int64_t>(a.k, ks) / 32);
  int lg = 8;
  for (int cand = 16; cand <= 64; cand *= 2)
    if (nch % cand == 0 || nch >= 4 * cand) lg = cand;
  const int64_t rpp = 4 * (64 / lg) * stream_rows(MT);
  const int64_t row_groups = (a.n + rpp - 1) / rpp;
  // several passes per workgroup (x staged once) while at least 1024 workgroups remain
  int passes = 1;
  if (a.k <= ks)
    while (passes < 8 && (row_groups + 2 * passes - 1) / (2 * passes) >= 1024) passes *= 2;
  const int64_t grid = (row_groups + passes - 1) / passes;
  gemv_stream_kernel<BITS, XT, MT><<<(unsigned)grid, 256, lds, s>>>(
      (const uint16_t*)a.x, a.m, a.k, a.packed, (const uint16_t*)a.scales, (const uint16_t*)a.biases,
      a.pdt == DT_BF16, a.n, a.g, (const uint16_t*)a.layer_bias, a.y, a.ydt, ks, lg, passes);
  return hipGetLastError();
}

template <int BITS, typename XT>
hipError_t launch_b(const GemvStreamArgs& a, hipStream_t s) {
  if (a.m <= 1) return launch_mt<BITS, XT, 1>(a, s);
  if (a.m <= 2) return launch_mt<BITS, XT, 2>(a, s);
  if (a.m <= 4) return launch_mt<BITS, XT, 4>(a, s);
  return launch_mt<BITS, XT, 8>(a, s);
}

template <int BITS>
hipError_t launch_bits(const GemvStreamArgs& a, hipStream_t s) {
  return a.xdt == DT_BF16 ? launch_b<BITS, BF16>(a, s) : launch_b<BITS, F16>(a, s);
}

template <int BITS, typename XT, int MT>
hipError_t launch_table_mt(const GemvDesc* table, const GemvTile* tiles, int64_t grid, int pbf16, int ydt,
                           size_t lds, hipStream_t s) {
  constexpr int R = stream_quad_rows(MT);
  gemv_quad_kernel<BITS, XT, MT, R><<<(unsigned)grid, 256, lds, s>>>(
      nullptr, 0, 0, nullptr, nullptr, nullptr, pbf16, 0, 32, nullptr, nullptr, ydt,
      stream_quad_ks(int64_t(1) << 40, MT), 8, 1, table, tiles);
  return hipGetLastError();
}

template <int BITS, typename XT>
hipError_t launch_table_b(const GemvDesc* table, const GemvTile* tiles, int64_t grid, int m, int pbf16, int ydt,
                          size_t lds, hipStream_t s) {
  if (m <= 1) return launch_table_mt<BITS, XT, 1>(table, tiles, grid, pbf16, ydt, lds, s);
  if (m <= 2) return launch_table_mt<BITS, XT, 2>(table, tiles, grid, pbf16, ydt, lds, s);
  if (m <= 4) return launch_table_mt<BITS, XT, 4>(table, tiles, grid, pbf16, ydt, lds, s);
  return launch_table_mt<BITS, XT, 8>(table, tiles, grid, pbf16, ydt, lds, s);
}

template <int BITS>
hipError_t launch_table_bits(const GemvDesc* table, const GemvTile* tiles, int64_t grid, int m, int xdt, int pdt,
                             int ydt, size_t lds, hipStream_t s) {
  return xdt == DT_BF16 ? launch_table_b<BITS, BF16>(table, tiles, grid, m, pdt == DT_BF16, ydt, lds, s)
                        : launch_table_b<BITS, F16>(table, tiles, grid, m, pdt == DT_BF16, ydt, lds, s);
}

}  // namespace

hipError_t launch_gemv_stream_table(const GemvDesc* table, const GemvTile* tiles, int64_t grid, int m, int bits,
                                    int xdt, int pdt, int ydt, size_t lds, hipStream_t s) {
  switch (bits) {
    case 2:
      return launch_table_bits<2>(table, tiles, grid, m, xdt, pdt, ydt, lds, s);
    case 3:
      return launch_table_bits<3>(table, tiles, grid, m, xdt, pdt, ydt, lds, s);
    case 5:
      return launch_table_bits<5>(table, tiles, grid, m, xdt, pdt, ydt, lds, s);
    case 6:
      return launch_table_bits<6>(table, tiles, grid, m, xdt, pdt, ydt, lds, s);
    default:
      return hipErrorInvalidValue;
  }
}

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
