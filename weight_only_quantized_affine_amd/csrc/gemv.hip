// Decode GEMV on affine-quantized weights: y[m,n] = x[m,k] . (code*scale + bias)^T, fp32
// accumulation, one rounding to the output dtype (Nx_quant API docs, Products: apply; GPTQModel
// wiki "MLX Apple Silicon", Executing MLX qlinear kernels: packed weights consumed directly,
// FP32 accumulation, activation-dtype output).  HBM-bound: the packed words are streamed once.
//
// Data flow per lane: a row's packed words are split into 16-byte chunks (32 codes at 4 bits,
// 16 at 8 bits, always inside one group since g >= 32); lanes_per_row consecutive lanes read
// consecutive chunks (coalesced 128-bit loads) and each lane keeps rows_per_lane rows in
// flight.  Codes become exact 16-bit floats with bit operations only:
//   4-bit, bf16 x: (w >> 4i) & 0x000F000F | 0x43004300 -> two bf16 values 128 + q
//   4-bit, f16 x:  ... | 0x64006400 -> two f16 values 1024 + q
//   8-bit, bf16 x: v_cvt_f32_ubyte{0..3} + v_cvt_pk_bf16_f32 -> q exactly
//   8-bit, f16 x:  (w >> 8i) & 0x00FF00FF | 0x64006400 -> 1024 + q
// and v_dot2 sums code*x pairs in fp32.  Per chunk, with P = sum x*(off + q) and X = sum x:
//   y += s * (P - off*X) + b * X,
// which is sum x*(q*s + b) exactly up to fp32 rounding.  The x pairs are permuted once per chunk
// to match the order the unpacking produces.  The lanes of a row then reduce with shuffles.
#include "device_common.hpp"
#include "launch.hpp"

namespace ql {
namespace {

template <typename XT> struct XTraits;
template <> struct XTraits<BF16> {
  static constexpr uint32_t kMagic4 = 0x43004300u;  // bf16 128.0 in both halves
  static constexpr float kOff4 = 128.0f;
  static constexpr uint32_t kOnes = 0x3F803F80u;
};
template <> struct XTraits<F16> {
  static constexpr uint32_t kMagic4 = 0x64006400u;  // f16 1024.0 in both halves
  static constexpr float kOff4 = 1024.0f;
  static constexpr uint32_t kOnes = 0x3C003C00u;
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};  // exact for the small integers used here
  return __builtin_bit_cast(uint32_t, v);
}

// Codes of one 16-byte chunk -> x-ordered operand pairs for v_dot2 (NP = 16 pairs at 4 bits,
// 8 pairs at 8 bits), and the matching permutation of x.
template <int BITS, typename XT> struct Unpack;

template <typename XT> struct Unpack<4, XT> {
  static constexpr int NP = 16;
  static constexpr float kOff = XTraits<XT>::kOff4;
  __device__ __forceinline__ static void codes(const u32x4_t& w, uint32_t* t) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = w[j];
      t[4 * j + 0] = (v & 0x000F000Fu) | XTraits<XT>::kMagic4;          // codes 0, 4
      t[4 * j + 1] = ((v >> 4) & 0x000F000Fu) | XTraits<XT>::kMagic4;   // codes 1, 5
      t[4 * j + 2] = ((v >> 8) & 0x000F000Fu) | XTraits<XT>::kMagic4;   // codes 2, 6
      t[4 * j + 3] = ((v >> 12) & 0x000F000Fu) | XTraits<XT>::kMagic4;  // codes 3, 7
    }
  }
  // x of the chunk (32 values = four 16-byte loads) into pairs (x0,x4),(x1,x5),(x2,x6),(x3,x7) per 8.
  __device__ __forceinline__ static void xpairs(const uint16_t* xrow, int64_t k0, uint32_t* p) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      u32x4_t u = load16(xrow + k0 + 8 * j);
      p[4 * j + 0] = perm(u[2], u[0], 0x05040100u);
      p[4 * j + 1] = perm(u[2], u[0], 0x07060302u);
      p[4 * j + 2] = perm(u[3], u[1], 0x05040100u);
      p[4 * j + 3] = perm(u[3], u[1], 0x07060302u);
    }
  }
};

template <> struct Unpack<8, BF16> {
  static constexpr int NP = 8;
  static constexpr float kOff = 0.0f;
  __device__ __forceinline__ static void codes(const u32x4_t& w, uint32_t* t) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = w[j];
      t[2 * j + 0] = pack_bf16((float)(v & 0xffu), (float)((v >> 8) & 0xffu));
      t[2 * j + 1] = pack_bf16((float)((v >> 16) & 0xffu), (float)(v >> 24));
    }
  }
  __device__ __forceinline__ static void xpairs(const uint16_t* xrow, int64_t k0, uint32_t* p) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4_t u = load16(xrow + k0 + 8 * j);
      p[4 * j + 0] = u[0];
      p[4 * j + 1] = u[1];
      p[4 * j + 2] = u[2];
      p[4 * j + 3] = u[3];
    }
  }
};

template <> struct Unpack<8, F16> {
  static constexpr int NP = 8;
  static constexpr float kOff = 1024.0f;
  __device__ __forceinline__ static void codes(const u32x4_t& w, uint32_t* t) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = w[j];
      t[2 * j + 0] = (v & 0x00FF00FFu) | 0x64006400u;         // codes 0, 2
      t[2 * j + 1] = ((v >> 8) & 0x00FF00FFu) | 0x64006400u;  // codes 1, 3
    }
  }
  __device__ __forceinline__ static void xpairs(const uint16_t* xrow, int64_t k0, uint32_t* p) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      u32x4_t u = load16(xrow + k0 + 8 * j);
      p[4 * j + 0] = perm(u[1], u[0], 0x05040100u);  // x0, x2
      p[4 * j + 1] = perm(u[1], u[0], 0x07060302u);  // x1, x3
      p[4 * j + 2] = perm(u[3], u[2], 0x05040100u);  // x4, x6
      p[4 * j + 3] = perm(u[3], u[2], 0x07060302u);  // x5, x7
    }
  }
};

template <typename T> __device__ __forceinline__ float x_to_f32(uint32_t b);
template <> __device__ __forceinline__ float x_to_f32<BF16>(uint32_t b) { return bf16_bits_to_f32(b); }
template <> __device__ __forceinline__ float x_to_f32<F16>(uint32_t b) { return f16_bits_to_f32(b); }

template <int MT, int BITS, typename XT, typename PT>
__global__ __launch_bounds__(256) void gemv_kernel(GemvDesc single, const GemvDesc* __restrict__ table,
                                                   const int64_t* __restrict__ tile_start, int count, int ydt) {
  using U = Unpack<BITS, XT>;
  constexpr int NP = U::NP;
  constexpr int R = (MT <= 2) ? 4 : 2;  // == gemv_rows_per_lane(MT)
  constexpr int CK = 128 / BITS;        // k-values per 16-byte chunk

  GemvDesc d;
  int64_t tile = blockIdx.x;
  if (count == 0) {
    d = single;
  } else {
    int lo = 0, hi = count - 1;  // last problem whose first tile <= tile
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (tile_start[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    d = table[lo];
    tile -= tile_start[lo];
  }
  const GemvGeom geo = gemv_geometry(d.k, BITS, MT);
  const int L = geo.lanes_per_row;
  const int P = 64 / L;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int rg = lane / L;
  const int li = lane - rg * L;
  const int64_t n = d.n, k = d.k;
  const int64_t groups = k / d.group_size;
  const int gshift = __builtin_ctz((unsigned)d.group_size);
  const int64_t words_per_row = k * BITS / 32;
  const int64_t row_base = tile * geo.rows_per_wg + (int64_t)wave * P * R + rg;

  const uint32_t* __restrict__ pk = d.packed;
  const uint16_t* __restrict__ sc = (const uint16_t*)d.scales;
  const uint16_t* __restrict__ bi = (const uint16_t*)d.biases;
  const uint16_t* __restrict__ xb = (const uint16_t*)d.x;
  const int m = (int)d.m;

  int64_t rows[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    int64_t rr = row_base + (int64_t)r * P;
    rows[r] = rr < n ? rr : n - 1;  // clamp loads; stores check the true row
  }

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[r][j] = 0.0f;

  for (int i = 0; i < geo.chunks_per_lane; ++i) {
    const int64_t c = li + (int64_t)i * L;
    const int64_t k0 = c * CK;
    const int64_t gi = k0 >> gshift;
    u32x4_t wv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) wv[r] = load16(pk + rows[r] * words_per_row + c * 4);
    float s[R], b[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      s[r] = param_to_f32<PT>(sc[rows[r] * groups + gi]);
      b[r] = param_to_f32<PT>(bi[rows[r] * groups + gi]);
    }
    uint32_t xp[MT][NP];
    float xs[MT];
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int jj = j < m ? j : 0;  // rows past m read row 0 and are never stored
      U::xpairs(xb + (int64_t)jj * k, k0, xp[j]);
      float t = 0.0f;
#pragma unroll
      for (int p = 0; p < NP; ++p) t = dot2(XT{}, xp[j][p], XTraits<XT>::kOnes, t);
      xs[j] = t;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      uint32_t t[NP];
      U::codes(wv[r], t);
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        float p = 0.0f;
#pragma unroll
        for (int q = 0; q < NP; ++q) p = dot2(XT{}, t[q], xp[j][q], p);
        const float pq = __builtin_fmaf(-U::kOff, xs[j], p);  // sum x*q
        acc[r][j] = __builtin_fmaf(s[r], pq, __builtin_fmaf(b[r], xs[j], acc[r][j]));
      }
    }
  }

  // Reduce over the L lanes of each row (butterfly inside aligned groups of L lanes).
  for (int off = 1; off < L; off <<= 1) {
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int j = 0; j < MT; ++j) acc[r][j] += __shfl_xor(acc[r][j], off);
  }
  if (li == 0) {
    const uint16_t* lb = (const uint16_t*)d.layer_bias;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = row_base + (int64_t)r * P;
      if (row >= n) continue;
      const float add = lb ? x_to_f32<XT>(lb[row]) : 0.0f;
#pragma unroll
      for (int j = 0; j < MT; ++j)
        if (j < m) store_out(d.y, (int64_t)j * n + row, acc[r][j] + add, ydt);
    }
  }
}

template <int MT, int BITS, typename XT, typename PT>
hipError_t launch_t(const GemvDesc& single, const GemvDesc* table, const int64_t* tile_start, int count,
                    int64_t total_tiles, int ydt, hipStream_t s) {
  gemv_kernel<MT, BITS, XT, PT><<<(unsigned)total_tiles, 256, 0, s>>>(single, table, tile_start, count, ydt);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_m(const GemvDesc& single, const GemvDesc* table, const int64_t* tile_start, int count,
                    int64_t total_tiles, int bits, int xdt, int pdt, int ydt, hipStream_t s) {
  const bool xb = xdt == DT_BF16, pb = pdt == DT_BF16;
  if (bits == 4) {
    if (xb && pb) return launch_t<MT, 4, BF16, BF16>(single, table, tile_start, count, total_tiles, ydt, s);
    if (xb) return launch_t<MT, 4, BF16, F16>(single, table, tile_start, count, total_tiles, ydt, s);
    if (pb) return launch_t<MT, 4, F16, BF16>(single, table, tile_start, count, total_tiles, ydt, s);
    return launch_t<MT, 4, F16, F16>(single, table, tile_start, count, total_tiles, ydt, s);
  }
  if (xb && pb) return launch_t<MT, 8, BF16, BF16>(single, table, tile_start, count, total_tiles, ydt, s);
  if (xb) return launch_t<MT, 8, BF16, F16>(single, table, tile_start, count, total_tiles, ydt, s);
  if (pb) return launch_t<MT, 8, F16, BF16>(single, table, tile_start, count, total_tiles, ydt, s);
  return launch_t<MT, 8, F16, F16>(single, table, tile_start, count, total_tiles, ydt, s);
}

}  // namespace

hipError_t launch_gemv(const GemvDesc& single, const GemvDesc* table, const int64_t* tile_start, int count,
                       int64_t total_tiles, int m, int bits, int xdt, int pdt, int ydt, hipStream_t s) {
  switch (gemv_mt(m)) {
    case 1: return launch_m<1>(single, table, tile_start, count, total_tiles, bits, xdt, pdt, ydt, s);
    case 2: return launch_m<2>(single, table, tile_start, count, total_tiles, bits, xdt, pdt, ydt, s);
    case 4: return launch_m<4>(single, table, tile_start, count, total_tiles, bits, xdt, pdt, ydt, s);
    default: return launch_m<8>(single, table, tile_start, count, total_tiles, bits, xdt, pdt, ydt, s);
  }
}

}  // namespace ql
