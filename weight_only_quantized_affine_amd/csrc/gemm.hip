// Prefill GEMM on affine-quantized weights with the CDNA4 matrix cores:
//   y[m,n] = sum_g s[n,g] * sum_{k in g} x[m,k] q[n,k]  +  sum_g b[n,g] * X[m,g],
// where X[m,g] = sum_{k in g} x[m,k].  This is the block-scaled contraction of the Nx_quant API
// docs (Products: apply; a tensor-core product scales each block's partial sum): the codes enter
// the bf16/f16 MFMA as exact small values, each group's fp32 partial sum is multiplied by its
// fp32 scale, and the additive bias of the MLX affine storage (GPTQModel wiki "MLX Apple
// Silicon", Concepts) enters through X, which a pre-pass computes.  No weight value is ever
// rounded to 16 bits, so the result carries fp32 accumulation error only.
//
// Encodings of a code q as an MFMA operand (exact):
//   4 bits: 1 + q/16, i.e. bits 0x3F80 | q << 3 (bf16) or 0x3C00 | q << 6 (f16); then
//           sum x*(1 + q/16) = X + P/16, so  s*P = 16s*P' - 16s*X  and -16s joins the bias.
//   8 bits: q itself (v_cvt_f32_ubyte + pack).
// The X-terms X*(b - 16s) are one extra MFMA per two groups: A = the bf16 hi/lo split of X,
// B = the bf16 hi/lo split of b and of -16s.
//
// Tiling: 256 threads (4 waves, 2x2), workgroup tile 128 (m) x 128 (n) x 64 (k), each wave a
// 64x64 block of 2x2 v_mfma_f32_32x32x16 tiles.  A and packed B tiles are double-buffered in
// LDS; the B codes stay packed in LDS and each wave unpacks its own fragments in registers.
// MFMA operand layout (32x32x16): lane l supplies row/column l%32 and k-slots 8*(l/32)..+7;
// the result register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#include "device_common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace ql {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int A_PITCH = BK + 8;  // bf16 elements per LDS row of A (padding against bank conflicts)

template <int BITS> struct BTile {
  static constexpr int ROW_BYTES = BK * BITS / 8;  // 32 or 64
  static constexpr int PITCH = ROW_BYTES + 16;     // bytes per LDS row of B
};

// ---------------------------------------------------------------- pre-pass: group sums of x

template <typename XT>
__global__ __launch_bounds__(256) void xsum_kernel(const uint16_t* __restrict__ x, int64_t m, int64_t k, int g,
                                                   uint32_t* __restrict__ xs) {
  const int64_t groups = k / g;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= m * groups) return;
  const int64_t row = t / groups, gi = t - row * groups;
  const uint16_t* p = x + row * k + gi * g;
  float s = 0.0f;
  const uint32_t ones = std::is_same<XT, BF16>::value ? 0x3F803F80u : 0x3C003C00u;
  for (int j = 0; j < g; j += 8) {
    u32x4_t u = load16(p + j);
#pragma unroll
    for (int q = 0; q < 4; ++q) s = dot2(XT{}, u[q], ones, s);
  }
  const uint32_t hi = f32_to_bf16_bits(s);
  const uint32_t lo = f32_to_bf16_bits(s - bf16_bits_to_f32(hi));
  xs[t] = hi | (lo << 16);
}

// ---------------------------------------------------------------- code unpacking

template <int BITS, typename XT> struct Codes;
// 4-bit: word j -> 4 operand registers holding codes (0,4),(1,5),(2,6),(3,7) as 1 + q/16.
template <> struct Codes<4, BF16> {
  __device__ __forceinline__ static void unpack(uint32_t w, uint32_t* r) {
    r[0] = ((w << 3) & 0x00780078u) | 0x3F803F80u;
    r[1] = ((w >> 1) & 0x00780078u) | 0x3F803F80u;
    r[2] = ((w >> 5) & 0x00780078u) | 0x3F803F80u;
    r[3] = ((w >> 9) & 0x00780078u) | 0x3F803F80u;
  }
};
template <> struct Codes<4, F16> {
  __device__ __forceinline__ static void unpack(uint32_t w, uint32_t* r) {
    r[0] = ((w << 6) & 0x03C003C0u) | 0x3C003C00u;
    r[1] = ((w << 2) & 0x03C003C0u) | 0x3C003C00u;
    r[2] = ((w >> 2) & 0x03C003C0u) | 0x3C003C00u;
    r[3] = ((w >> 6) & 0x03C003C0u) | 0x3C003C00u;
  }
};
// 8-bit: two words -> codes 0..7 in order, exact.
template <> struct Codes<8, BF16> {
  __device__ __forceinline__ static void unpack2(uint32_t w0, uint32_t w1, uint32_t* r) {
    bf16x2_t a = {(__bf16)(float)(w0 & 0xffu), (__bf16)(float)((w0 >> 8) & 0xffu)};
    bf16x2_t b = {(__bf16)(float)((w0 >> 16) & 0xffu), (__bf16)(float)(w0 >> 24)};
    bf16x2_t c = {(__bf16)(float)(w1 & 0xffu), (__bf16)(float)((w1 >> 8) & 0xffu)};
    bf16x2_t d = {(__bf16)(float)((w1 >> 16) & 0xffu), (__bf16)(float)(w1 >> 24)};
    r[0] = __builtin_bit_cast(uint32_t, a);
    r[1] = __builtin_bit_cast(uint32_t, b);
    r[2] = __builtin_bit_cast(uint32_t, c);
    r[3] = __builtin_bit_cast(uint32_t, d);
  }
};
template <> struct Codes<8, F16> {
  __device__ __forceinline__ static void unpack2(uint32_t w0, uint32_t w1, uint32_t* r) {
    f16x2_t a = {(_Float16)(float)(w0 & 0xffu), (_Float16)(float)((w0 >> 8) & 0xffu)};
    f16x2_t b = {(_Float16)(float)((w0 >> 16) & 0xffu), (_Float16)(float)(w0 >> 24)};
    f16x2_t c = {(_Float16)(float)(w1 & 0xffu), (_Float16)(float)((w1 >> 8) & 0xffu)};
    f16x2_t d = {(_Float16)(float)((w1 >> 16) & 0xffu), (_Float16)(float)(w1 >> 24)};
    r[0] = __builtin_bit_cast(uint32_t, a);
    r[1] = __builtin_bit_cast(uint32_t, b);
    r[2] = __builtin_bit_cast(uint32_t, c);
    r[3] = __builtin_bit_cast(uint32_t, d);
  }
};

__device__ __forceinline__ f32x16_t mfma(BF16, const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ f32x16_t mfma(F16, const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                0, 0);
}

// Permute 8 consecutive 16-bit x values to the order the 4-bit unpacking yields: x0,x4,x1,x5,x2,x6,x3,x7.
__device__ __forceinline__ u32x4_t perm8(const u32x4_t& u) {
  u32x4_t r;
  r[0] = perm(u[2], u[0], 0x05040100u);
  r[1] = perm(u[2], u[0], 0x07060302u);
  r[2] = perm(u[3], u[1], 0x05040100u);
  r[3] = perm(u[3], u[1], 0x07060302u);
  return r;
}

// Split an fp32 value into bf16 hi + lo (hi = RNE(v), lo = RNE(v - hi)).
__device__ __forceinline__ void split_bf16(float v, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_bits(v);
  lo = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
}

// k-value of MFMA slot j (0..7) of lane half h at k-step t (0..3) of a 64-wide k-tile:
//   16t + 8h + j, so every 16-wide k-step lies inside one group for g in {32, 64, 128}.
// The packed words a lane needs are rearranged in LDS so each lane reads them with one or two
// 16-byte LDS loads: 4-bit rows hold words [0,2,4,6 | 1,3,5,7], 8-bit rows hold
// [0,1,4,5,8,9,12,13 | 2,3,6,7,10,11,14,15].
template <int BITS, int G, typename XT, typename PT>
__global__ __launch_bounds__(256) void gemm_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                   const uint32_t* __restrict__ packed,
                                                   const uint16_t* __restrict__ scales,
                                                   const uint16_t* __restrict__ biases, int64_t N,
                                                   const uint16_t* __restrict__ layer_bias, void* __restrict__ y,
                                                   int ydt, const uint32_t* __restrict__ xsum) {
  using BT = BTile<BITS>;
  constexpr float kFold = BITS == 4 ? 16.0f : 1.0f;  // partial sums of 1 + q/16 carry q/16
  constexpr int SPG = G / 16;                         // 16-wide k-steps per group: 2, 4 or 8
  constexpr int BW = BITS == 4 ? 4 : 8;               // words a lane reads per k-tile
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][BM * A_PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * BT::PITCH];
  __shared__ float sS[2][BN][2];  // kFold * scale of the groups of k-steps {0,1} and {2,3}

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int l32 = lane & 31, h = lane >> 5;

  const int64_t m_tiles = (M + BM - 1) / BM;
  const int64_t mt = blockIdx.x % m_tiles;
  const int64_t nt = blockIdx.x / m_tiles;
  const int64_t m0 = mt * BM, n0 = nt * BN;
  const int64_t groups = K / G;
  const int64_t KT = (K + BK - 1) / BK;
  const int64_t words_per_row = K * BITS / 32;

  // Global -> register staging of one k-tile.
  // A: thread -> row tid/2, 32 k-values (4 x 16 B) at (tid&1)*32.
  const int a_row = tid >> 1, a_half = tid & 1;
  const int64_t a_grow = m0 + a_row < M ? m0 + a_row : M - 1;
  // B and scales: threads 0..127 each take one row of the tile.
  const bool b_thread = tid < BN;
  const int64_t b_grow = n0 + tid < N ? n0 + tid : N - 1;

  u32x4_t ra[4];
  u32x4_t rb[BITS == 4 ? 2 : 4];
  float rs[2];

  auto load_tile = [&](int64_t kt) {
    const int64_t k0 = kt * BK;
    const bool full = k0 + BK <= K;  // else k-values [k0+32, k0+64) lie past K (K % 64 == 32)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t kk = k0 + a_half * 32 + 8 * j;
      if (full || kk < K)
        ra[j] = load16(x + a_grow * K + kk);
      else
        ra[j] = u32x4_t{0, 0, 0, 0};
    }
    if (b_thread) {
      const int64_t wi = k0 * BITS / 32;
#pragma unroll
      for (int j = 0; j < (BITS == 4 ? 2 : 4); ++j) {
        if (full || j < (BITS == 4 ? 1 : 2))
          rb[j] = load16(packed + b_grow * words_per_row + wi + 4 * j);
        else
          rb[j] = u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int64_t kq = k0 + 32 * q;
        rs[q] = kq < K ? kFold * param_to_f32<PT>(scales[b_grow * groups + kq / G]) : 0.0f;
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* a = &sA[buf][a_row * A_PITCH + a_half * 32];
#pragma unroll
    for (int j = 0; j < 4; ++j) *(u32x4_t*)(a + 8 * j) = BITS == 4 ? perm8(ra[j]) : ra[j];
    if (b_thread) {
      uint8_t* b = &sB[buf][tid * BT::PITCH];
      if (BITS == 4) {
        // words w0..w7 -> [w0,w2,w4,w6 | w1,w3,w5,w7]
        *(u32x4_t*)(b) = u32x4_t{rb[0][0], rb[0][2], rb[1][0], rb[1][2]};
        *(u32x4_t*)(b + 16) = u32x4_t{rb[0][1], rb[0][3], rb[1][1], rb[1][3]};
      } else {
        // words w0..w15 -> [w0,w1,w4,w5,w8,w9,w12,w13 | w2,w3,w6,w7,w10,w11,w14,w15]
        *(u32x4_t*)(b) = u32x4_t{rb[0][0], rb[0][1], rb[1][0], rb[1][1]};
        *(u32x4_t*)(b + 16) = u32x4_t{rb[2][0], rb[2][1], rb[3][0], rb[3][1]};
        *(u32x4_t*)(b + 32) = u32x4_t{rb[0][2], rb[0][3], rb[1][2], rb[1][3]};
        *(u32x4_t*)(b + 48) = u32x4_t{rb[2][2], rb[2][3], rb[3][2], rb[3][3]};
      }
      sS[buf][tid][0] = rs[0];
      sS[buf][tid][1] = rs[1];
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
  f32x16_t P[2][2];
  const f32x16_t zero16 = {0.0f};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int64_t kt = 0; kt < KT; ++kt) {
    const int buf = (int)(kt & 1);
    if (kt + 1 < KT) load_tile(kt + 1);

    // A fragments: 2 row-tiles x 4 k-steps; lane (row l32, half h) reads 16 B at k-offset 16t + 8h.
    u32x4_t af[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        af[rt][t] = *(const u32x4_t*)&sA[buf][(wm * 64 + rt * 32 + l32) * A_PITCH + 16 * t + 8 * h];
    // B words of this lane: column l32 of each col-tile, its half h of the rearranged row.
    u32x4_t bw[2][BW / 4];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int j = 0; j < BW / 4; ++j)
        bw[ct][j] = *(const u32x4_t*)&sB[buf][(wn * 64 + ct * 32 + l32) * BT::PITCH + h * (BW * 4) + 16 * j];

    // For G == 128 a group spans two k-tiles: it starts on even tiles only.
    const bool even_tile = (G < 128) || ((kt & 1) == 0);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bool first = (G < 128) ? (t % SPG == 0) : (t == 0 && even_tile);
      const bool last = (G < 128) ? ((t + 1) % SPG == 0) : (t == 3 && !even_tile);
      u32x4_t bf[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        uint32_t r[4];
        if (BITS == 4)
          Codes<4, XT>::unpack(bw[ct][0][t], r);
        else
          Codes<8, XT>::unpack2(bw[ct][t >> 1][2 * (t & 1)], bw[ct][t >> 1][2 * (t & 1) + 1], r);
        bf[ct] = u32x4_t{r[0], r[1], r[2], r[3]};
      }
      if (first) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) P[rt][ct] = mfma(XT{}, af[rt][t], bf[ct], zero16);
      } else {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) P[rt][ct] = mfma(XT{}, af[rt][t], bf[ct], P[rt][ct]);
      }
      if (last) {
        // group complete: fold its partial sums with the group's scale (one per output column)
        const int q = t >> 1;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          const float sc = sS[buf][wn * 64 + ct * 32 + l32][q];
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[rt][ct][r] = __builtin_fmaf(sc, P[rt][ct][r], acc[rt][ct][r]);
        }
      }
    }

    if (kt + 1 < KT) store_tile(buf ^ 1);
    __syncthreads();
  }

  // X-terms: sum_g X[m,g] * (b[n,g] - kFold*s[n,g]) as bf16 hi/lo products, two groups per MFMA
  // (lane half h takes group 2p + h; slots: Xhi*bhi, Xhi*blo, Xlo*bhi, Xlo*blo, same with c).
  {
    int64_t arow[2], bcol[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int64_t r = m0 + wm * 64 + rt * 32 + l32;
      arow[rt] = r < M ? r : M - 1;
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int64_t c = n0 + wn * 64 + ct * 32 + l32;
      bcol[ct] = c < N ? c : N - 1;
    }
    for (int64_t p = 0; p < (groups + 1) / 2; ++p) {
      const int64_t gi = 2 * p + h;
      const bool live = gi < groups;
      u32x4_t ab[2], bb[2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        const uint32_t v = live ? xsum[arow[rt] * groups + gi] : 0u;
        const uint32_t xh = v & 0xffffu, xl = v >> 16;
        const uint32_t hh = xh | (xh << 16), ll = xl | (xl << 16);
        ab[rt] = u32x4_t{hh, ll, hh, ll};
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        uint32_t bh = 0, bl = 0, ch = 0, cl = 0;
        if (live) {
          const float bv = param_to_f32<PT>(biases[bcol[ct] * groups + gi]);
          const float cv = BITS == 4 ? -kFold * param_to_f32<PT>(scales[bcol[ct] * groups + gi]) : 0.0f;
          split_bf16(bv, bh, bl);
          split_bf16(cv, ch, cl);
        }
        bb[ct] = u32x4_t{bh | (bl << 16), bh | (bl << 16), ch | (cl << 16), ch | (cl << 16)};
      }
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[rt][ct] = mfma(BF16{}, ab[rt], bb[ct], acc[rt][ct]);
    }
  }

  // Epilogue: lane holds column l32 of each 32x32 tile, rows 8*(r/4) + 4*h + (r%4).
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int64_t col = n0 + wn * 64 + ct * 32 + l32;
    if (col >= N) continue;
    const float add = layer_bias ? (std::is_same<XT, BF16>::value ? bf16_bits_to_f32(layer_bias[col])
                                                                  : f16_bits_to_f32(layer_bias[col]))
                                 : 0.0f;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + rt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (row < M) store_out(y, row * N + col, acc[rt][ct][r] + add, ydt);
      }
  }
}

template <int BITS, typename XT, typename PT>
hipError_t launch_t(const void* x, int64_t m, int64_t k, const uint32_t* packed, const void* scales,
                    const void* biases, int64_t n, int g, const void* layer_bias, void* y, int ydt, void* ws,
                    hipStream_t s) {
  const int64_t groups = k / g;
  const int64_t total = m * groups;
  xsum_kernel<XT><<<(unsigned)((total + 255) / 256), 256, 0, s>>>((const uint16_t*)x, m, k, g, (uint32_t*)ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  const uint16_t* xx = (const uint16_t*)x;
  const uint16_t* sc = (const uint16_t*)scales;
  const uint16_t* bi = (const uint16_t*)biases;
  const uint16_t* lb = (const uint16_t*)layer_bias;
  const uint32_t* xs = (const uint32_t*)ws;
  if (g == 32)
    gemm_kernel<BITS, 32, XT, PT><<<(unsigned)tiles, 256, 0, s>>>(xx, m, k, packed, sc, bi, n, lb, y, ydt, xs);
  else if (g == 64)
    gemm_kernel<BITS, 64, XT, PT><<<(unsigned)tiles, 256, 0, s>>>(xx, m, k, packed, sc, bi, n, lb, y, ydt, xs);
  else
    gemm_kernel<BITS, 128, XT, PT><<<(unsigned)tiles, 256, 0, s>>>(xx, m, k, packed, sc, bi, n, lb, y, ydt, xs);
  return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(int64_t m, int64_t k, int g) { return (size_t)(m * (k / g)) * 4u; }

hipError_t launch_gemm(const void* x, int xdt, int64_t m, int64_t k, const uint32_t* packed, const void* scales,
                       const void* biases, int pdt, int64_t n, int bits, int g, const void* layer_bias, void* y,
                       int ydt, void* ws, hipStream_t s) {
  const bool xb = xdt == DT_BF16, pb = pdt == DT_BF16;
  if (bits == 4) {
    if (xb && pb) return launch_t<4, BF16, BF16>(x, m, k, packed, scales, biases, n, g, layer_bias, y, ydt, ws, s);
    if (xb) return launch_t<4, BF16, F16>(x, m, k, packed, scales, biases, n, g, layer_bias, y, ydt, ws, s);
    if (pb) return launch_t<4, F16, BF16>(x, m, k, packed, scales, biases, n, g, layer_bias, y, ydt, ws, s);
    return launch_t<4, F16, F16>(x, m, k, packed, scales, biases, n, g, layer_bias, y, ydt, ws, s);
  }
  if (xb && pb) return launch_t<8, BF16, BF16>(x, m, k, packed, scales, biases, n, g, layer_bias, y, ydt, ws, s);
  if (xb) return launch_t<8, BF16, F16>(x, m, k, packed, scales, biases, n, g, layer_bias, y, ydt, ws, s);
  if (pb) return launch_t<8, F16, BF16>(x, m, k, packed, scales, biases, n, g, layer_bias, y, ydt, ws, s);
  return launch_t<8, F16, F16>(x, m, k, packed, scales, biases, n, g, layer_bias, y, ydt, ws, s);
}

}  // namespace ql
