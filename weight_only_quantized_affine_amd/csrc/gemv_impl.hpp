// Decode GEMV on affine-quantized weights: y[m,n] = x[m,k] . (code*scale + bias)^T, fp32
// accumulation, one rounding to the output dtype (Nx_quant API docs, Products: apply; GPTQModel
// wiki "MLX Apple Silicon", Executing MLX qlinear kernels: packed weights consumed directly,
// FP32 accumulation, activation-dtype output).  HBM-bound: the packed words are streamed once.
//
// Work split: a row's packed words are cut into 16-byte chunks (32 codes at 4 bits, 16 at 8
// bits, always inside one group since g >= 32); lanes_per_row (L) consecutive lanes read
// consecutive chunks, so every 128-bit load instruction of a wave reads contiguous memory; each
// lane holds R rows, and a 256-thread workgroup walks `batches` sets of 4 waves x (64/L) x R
// rows.  The loads of the next steps are issued before the current step is computed.  x is
// staged once per workgroup in LDS, already in the order the unpacking needs, with its
// per-chunk sums.
//
// Codes become exact 16-bit floats with bit operations only:
//   4-bit, bf16 x: (w >> 4i) & 0x000F000F | 0x43004300 -> two bf16 values 128 + q
//   4-bit, f16 x:  ... | 0x64006400 -> two f16 values 1024 + q
//   8-bit, bf16 x: v_cvt_f32_ubyte{0..3} + v_cvt_pk_bf16_f32 -> q exactly
//   8-bit, f16 x:  (w >> 8i) & 0x00FF00FF | 0x64006400 -> 1024 + q
// and v_dot2 sums code*x pairs in fp32.  Per chunk, with P = sum x*(off + q) and X = sum x:
//   y += s * (P - off*X) + b * X,
// i.e. sum x*(q*s + b) up to fp32 rounding.  The L lanes of a row then reduce with DPP and
// swizzle lane moves.
#pragma once
#include "device_common.hpp"
#include "launch.hpp"

namespace ql {
namespace gemv_detail {

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

// Codes of one 16-byte chunk -> operand pairs for v_dot2 (NP = 16 pairs at 4 bits, 8 at 8 bits),
// and the permutation of 8 consecutive x values that matches the pair order.
template <int BITS, typename XT> struct Unpack;

// A 32-bit constant placed in a VGPR once.  The VOP3 encodings of this target take no literal
// operand, so shift-and-mask-and-or only folds into one v_and_or_b32 when the mask and the magic
// bits are registers.
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

template <typename XT> struct Unpack<4, XT> {
  static constexpr int NP = 16;
  static constexpr float kOff = XTraits<XT>::kOff4;
  static constexpr uint32_t kMask = 0x000F000Fu, kMagic = XTraits<XT>::kMagic4;
  // mk, mg: kMask and kMagic held in registers (see vconst)
  __device__ __forceinline__ static void codes(const u32x4_t& w, uint32_t* t, uint32_t mk, uint32_t mg) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = w[j];
      t[4 * j + 0] = (v & mk) | mg;          // codes 0, 4
      t[4 * j + 1] = ((v >> 4) & mk) | mg;   // codes 1, 5
      t[4 * j + 2] = ((v >> 8) & mk) | mg;   // codes 2, 6
      t[4 * j + 3] = ((v >> 12) & mk) | mg;  // codes 3, 7
    }
  }
  // x0..x7 -> (x0,x4),(x1,x5),(x2,x6),(x3,x7)
  __device__ __forceinline__ static u32x4_t xperm(const u32x4_t& u) {
    return u32x4_t{perm(u[2], u[0], 0x05040100u), perm(u[2], u[0], 0x07060302u), perm(u[3], u[1], 0x05040100u),
                   perm(u[3], u[1], 0x07060302u)};
  }
};

// 2-bit codes, two words (codes 0..15, 16..31) -> operand pairs as at 4 bits: product t takes the
// codes 8t..8t+7 (bytes 2t, 2t+1 of the lane's 8), which one byte permute places in the low bytes
// of the two halves, so that a shift by 2p and the mask give codes (8t+p, 8t+p+4).
template <typename XT> struct Unpack<2, XT> {
  static constexpr int NP = 16;
  static constexpr float kOff = XTraits<XT>::kOff4;
  static constexpr uint32_t kMask = 0x00030003u, kMagic = XTraits<XT>::kMagic4;
  __device__ __forceinline__ static void codes(const u32x4_t& w, uint32_t* t, uint32_t mk, uint32_t mg) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = perm(0u, w[j >> 1], (j & 1) ? 0x0C030C02u : 0x0C010C00u);
      t[4 * j + 0] = (v & mk) | mg;         // codes 8j + 0, 8j + 4
      t[4 * j + 1] = ((v >> 2) & mk) | mg;  // codes 8j + 1, 8j + 5
      t[4 * j + 2] = ((v >> 4) & mk) | mg;  // codes 8j + 2, 8j + 6
      t[4 * j + 3] = ((v >> 6) & mk) | mg;  // codes 8j + 3, 8j + 7
    }
  }
  __device__ __forceinline__ static u32x4_t xperm(const u32x4_t& u) { return Unpack<4, XT>::xperm(u); }
};

// 3-bit codes, three words (the lane's 96 bits) -> operand pairs as at 4 bits: the 24 bits of
// codes 8t..8t+7 (one funnel shift) are split 12 + 12 into the two 16-bit halves, so that a shift
// by 3p and the mask give codes (8t+p, 8t+p+4); bits above a half's 12 are never selected.
template <typename XT> struct Unpack<3, XT> {
  static constexpr int NP = 16;
  static constexpr float kOff = XTraits<XT>::kOff4;
  static constexpr uint32_t kMask = 0x00070007u, kMagic = XTraits<XT>::kMagic4;
  __device__ __forceinline__ static void codes(const u32x4_t& w, uint32_t* t, uint32_t mk, uint32_t mg) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t u = j == 0   ? w[0]
                         : j == 1 ? __builtin_amdgcn_alignbit(w[1], w[0], 24)
                         : j == 2 ? __builtin_amdgcn_alignbit(w[2], w[1], 16)
                                  : w[2] >> 8;
      const uint32_t v = (u & 0xFFFFu) | ((u << 4) & 0xFFFF0000u);
      t[4 * j + 0] = (v & mk) | mg;         // codes 8j + 0, 8j + 4
      t[4 * j + 1] = ((v >> 3) & mk) | mg;  // codes 8j + 1, 8j + 5
      t[4 * j + 2] = ((v >> 6) & mk) | mg;  // codes 8j + 2, 8j + 6
      t[4 * j + 3] = ((v >> 9) & mk) | mg;  // codes 8j + 3, 8j + 7
    }
  }
  __device__ __forceinline__ static u32x4_t xperm(const u32x4_t& u) { return Unpack<4, XT>::xperm(u); }
};

// 5-bit codes, five words (a: words 0..3, b: word 4) -> operand pairs as at 4 bits: the 40 bits
// of codes 8t..8t+7 give two 32-bit windows (funnel shifts at bits 40t and 40t + 10) whose low
// half keeps its first two codes and whose high half takes its bits 20..35 (shift by 4), so
// that shifts by 0 and 5 with the mask give codes (8t+p, 8t+p+4).
template <typename XT> struct Unpack<5, XT> {
  static constexpr int NP = 16;
  static constexpr float kOff = XTraits<XT>::kOff4;
  static constexpr uint32_t kMask = 0x001F001Fu, kMagic = XTraits<XT>::kMagic4;
  __device__ __forceinline__ static void codes2(const u32x4_t& a, const u32x4_t& b, uint32_t* t, uint32_t mk,
                                                uint32_t mg) {
    const uint32_t w[5] = {a[0], a[1], a[2], a[3], b[0]};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int o = 40 * j + 10 * hf, i = o / 32, sh = o % 32;  // constants after unrolling
        const uint32_t u = sh == 0 ? w[i] : i + 1 < 5 ? __builtin_amdgcn_alignbit(w[i + 1 < 5 ? i + 1 : 4], w[i], sh)
                                                      : w[i] >> sh;
        const uint32_t v = (u & 0xFFFFu) | ((u >> 4) & 0xFFFF0000u);
        t[4 * j + 2 * hf + 0] = (v & mk) | mg;         // codes 8j + 2hf, 8j + 2hf + 4
        t[4 * j + 2 * hf + 1] = ((v >> 5) & mk) | mg;  // codes 8j + 2hf + 1, 8j + 2hf + 5
      }
    }
  }
  __device__ __forceinline__ static u32x4_t xperm(const u32x4_t& u) { return Unpack<4, XT>::xperm(u); }
};

// 6-bit codes, six words (a: words 0..3, b: words 4, 5) -> operand pairs as at 4 bits: the six
// bytes c0..c5 of codes 8t..8t+7 give two byte permutes, (c0 c1 c3 c4) and (c1 c2 c4 c5), whose
// shifts by 0, 6 and by 4, 10 with the mask give codes (8t+p, 8t+p+4).  (bf16 128 + q and fp16
// 1024 + q stay exact for q < 64.)
template <typename XT> struct Unpack<6, XT> {
  static constexpr int NP = 16;
  static constexpr float kOff = XTraits<XT>::kOff4;
  static constexpr uint32_t kMask = 0x003F003Fu, kMagic = XTraits<XT>::kMagic4;
  __device__ __forceinline__ static void codes2(const u32x4_t& a, const u32x4_t& b, uint32_t* t, uint32_t mk,
                                                uint32_t mg) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = j == 0 ? a[0] : j == 1 ? a[1] : j == 2 ? a[3] : b[0];
      const uint32_t hi = j == 0 ? a[1] : j == 1 ? a[2] : j == 2 ? b[0] : b[1];
      const uint32_t pa = perm(hi, lo, (j & 1) ? 0x06050302u : 0x04030100u);
      const uint32_t pb = perm(hi, lo, (j & 1) ? 0x07060403u : 0x05040201u);
      t[4 * j + 0] = (pa & mk) | mg;          // codes 8j + 0, 8j + 4
      t[4 * j + 1] = ((pa >> 6) & mk) | mg;   // codes 8j + 1, 8j + 5
      t[4 * j + 2] = ((pb >> 4) & mk) | mg;   // codes 8j + 2, 8j + 6
      t[4 * j + 3] = ((pb >> 10) & mk) | mg;  // codes 8j + 3, 8j + 7
    }
  }
  __device__ __forceinline__ static u32x4_t xperm(const u32x4_t& u) { return Unpack<4, XT>::xperm(u); }
};

template <> struct Unpack<8, BF16> {
  static constexpr int NP = 8;
  static constexpr float kOff = 0.0f;
  static constexpr uint32_t kMask = 0u, kMagic = 0u;
  __device__ __forceinline__ static void codes(const u32x4_t& w, uint32_t* t, uint32_t, uint32_t) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = w[j];
      t[2 * j + 0] = pack_bf16((float)(v & 0xffu), (float)((v >> 8) & 0xffu));
      t[2 * j + 1] = pack_bf16((float)((v >> 16) & 0xffu), (float)(v >> 24));
    }
  }
  __device__ __forceinline__ static u32x4_t xperm(const u32x4_t& u) { return u; }
};

template <> struct Unpack<8, F16> {
  static constexpr int NP = 8;
  static constexpr float kOff = 1024.0f;
  static constexpr uint32_t kMask = 0x00FF00FFu, kMagic = 0x64006400u;
  __device__ __forceinline__ static void codes(const u32x4_t& w, uint32_t* t, uint32_t mk, uint32_t mg) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t v = w[j];
      t[2 * j + 0] = (v & mk) | mg;         // codes 0, 2
      t[2 * j + 1] = ((v >> 8) & mk) | mg;  // codes 1, 3
    }
  }
  // x0..x7 -> (x0,x2),(x1,x3),(x4,x6),(x5,x7)
  __device__ __forceinline__ static u32x4_t xperm(const u32x4_t& u) {
    return u32x4_t{perm(u[1], u[0], 0x05040100u), perm(u[1], u[0], 0x07060302u), perm(u[3], u[2], 0x05040100u),
                   perm(u[3], u[2], 0x07060302u)};
  }
};

template <typename T> __device__ __forceinline__ float x_to_f32(uint32_t b);
template <> __device__ __forceinline__ float x_to_f32<BF16>(uint32_t b) { return bf16_bits_to_f32(b); }
template <> __device__ __forceinline__ float x_to_f32<F16>(uint32_t b) { return f16_bits_to_f32(b); }

// Sum over aligned groups of L lanes (L a power of two <= 64); every lane gets its group's sum.
__device__ __forceinline__ float dpp_add(float v, int ctrl_sel) {
  // ctrl_sel: 0 = quad xor 1, 1 = quad xor 2, 2 = half-row mirror, 3 = row mirror
  int iv = __float_as_int(v), r;
  if (ctrl_sel == 0)
    r = __builtin_amdgcn_update_dpp(iv, iv, 0xB1, 0xF, 0xF, false);
  else if (ctrl_sel == 1)
    r = __builtin_amdgcn_update_dpp(iv, iv, 0x4E, 0xF, 0xF, false);
  else if (ctrl_sel == 2)
    r = __builtin_amdgcn_update_dpp(iv, iv, 0x141, 0xF, 0xF, false);
  else
    r = __builtin_amdgcn_update_dpp(iv, iv, 0x140, 0xF, 0xF, false);
  return v + __int_as_float(r);
}
__device__ __forceinline__ float group_sum(float v, int L) {
  if (L >= 2) v = dpp_add(v, 0);
  if (L >= 4) v = dpp_add(v, 1);
  if (L >= 8) v = dpp_add(v, 2);
  if (L >= 16) v = dpp_add(v, 3);
  if (L >= 32) v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));  // xor 16
  if (L >= 64) v += __shfl_xor(v, 32);
  return v;
}

// Buffer resource over `bytes` bytes at `base` (raw buffer, 32-bit offsets; loads past the end
// return zero without touching memory, stores past the end are dropped).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int nr = bytes < 0x7fffffff ? (int)bytes : 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nr, 0x00020000);
}

template <typename T> using gptr = const __attribute__((address_space(1))) T*;

constexpr int R = GEMV_ROWS_PER_LANE;  // rows per lane per step
constexpr int kOOB = 0x7ffffff0;       // a buffer offset past every resource

// Loads of one step: R rows x one 16-byte chunk, and the rows' scale and bias of the chunk's group.
struct StepBuf {
  u32x4_t w[R];
  uint32_t s[R], b[R];
};

template <int MT, int BITS, typename XT, typename PT, bool XLDS>
__global__ __launch_bounds__(256) void gemv_kernel(GemvDesc single, const GemvDesc* __restrict__ table,
                                                   const GemvTile* __restrict__ tiles, int ydt) {
  using U = Unpack<BITS, XT>;
  constexpr int NP = U::NP;       // operand pairs per 16-byte chunk
  const uint32_t mk = vconst(U::kMask), mg = vconst(U::kMagic);
  constexpr int CK = 128 / BITS;  // k-values per chunk
  constexpr int CP = gemv_x_pitch(MT, BITS);  // LDS pitch of a chunk of x (16-bit elements)
  extern __shared__ __attribute__((aligned(16))) uint16_t sx[];

  GemvDesc d;
  int64_t tile;
  if (table == nullptr) {
    d = single;
    tile = blockIdx.x;
  } else {
    const GemvTile tt = tiles[blockIdx.x];
    d = table[tt.prob];
    tile = tt.local;
  }
  const int64_t n = d.n, k = d.k;
  const int m = (int)d.m;
  const GemvGeom geo = gemv_geometry(k, BITS, d.batches);
  const int L = geo.lanes_per_row;
  const int P = 64 / L;
  const int CPL = geo.chunks_per_lane;
  const int cpl = CPL > 0 ? CPL : 1;  // k == 0 has no chunks (and no steps)
  const int C = geo.chunks;           // 16-byte chunks per row
  const int row_bytes = C * 16;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rg = lane / L, li = lane - rg * L;
  const int groups = (int)(k / d.group_size);
  const int gshift = __builtin_ctz((unsigned)d.group_size);
  const int rows_per_set = 4 * P * R;
  const int steps = geo.batches * CPL;
  const int64_t wg_row = tile * geo.rows_per_wg;
  const int64_t rows_left = n - wg_row;
  const int esz = ydt == DT_F32 ? 4 : 2;
  // Offsets are relative to the workgroup's first row (32-bit); the resources end at the last
  // row of the matrix, so rows past n read zeros and store nothing.
  const __amdgpu_buffer_rsrc_t rw = make_rsrc((const uint8_t*)d.packed + wg_row * row_bytes, rows_left * row_bytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc((const uint16_t*)d.scales + wg_row * groups, rows_left * groups * 2);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc((const uint16_t*)d.biases + wg_row * groups, rows_left * groups * 2);
  const int lrow0 = wave * P * R + rg;  // this lane's first row, relative to the workgroup

  auto step_of = [&](int st, int& b, int& i) __attribute__((always_inline)) {
    b = st / cpl;
    i = st - b * cpl;
  };
  auto issue = [&](int st, StepBuf& q) __attribute__((always_inline)) {
    int b, i;
    step_of(st, b, i);
    const bool live = st < steps;
    const int c = li + i * L;
    const int gi = (c * CK) >> gshift;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int lr = lrow0 + b * rows_per_set + r * P;
      // packed words, scales and biases are read once: non-temporal loads (cache policy nt)
      q.w[r] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, live ? lr * row_bytes + 16 * c : kOOB, 0, 2));
      q.s[r] = __builtin_amdgcn_raw_buffer_load_b16(rs, live ? (lr * groups + gi) * 2 : kOOB, 0, 2);
      q.b[r] = __builtin_amdgcn_raw_buffer_load_b16(rb, live ? (lr * groups + gi) * 2 : kOOB, 0, 2);
    }
  };

  // Two step buffers in ping-pong: the loads of step s+1 are issued before step s is computed.
  StepBuf bufA, bufB;
  issue(0, bufA);

  // -- LDS: x (m rows) as chunks of CK values at (j*C + c)*CP, permuted per 8 values; each chunk's
  //    sum of x at sX[j*C + c]; the workgroup's layer-bias rows at sLB.
  float* sX = (float*)(sx + (XLDS ? (size_t)MT * C * CP : 0));
  float* sLB = sX + (XLDS ? MT * C : 0);
  {
    gptr<uint16_t> lbg = (gptr<uint16_t>)d.layer_bias;
    for (int t = threadIdx.x; t < geo.rows_per_wg; t += 256)
      sLB[t] = (lbg && t < rows_left) ? x_to_f32<XT>(lbg[wg_row + t]) : 0.0f;
  }
  if (XLDS) {
    gptr<uint16_t> xg = (gptr<uint16_t>)d.x;
    for (int t = threadIdx.x; t < m * C; t += 256) {
      const int j = t / C, c = t - j * C;
      float xsum = 0.0f;
#pragma unroll
      for (int q = 0; q < CK / 8; ++q) {
        const u32x4_t u = *(gptr<u32x4_t>)(xg + (int64_t)j * k + (int64_t)c * CK + 8 * q);
#pragma unroll
        for (int e = 0; e < 4; ++e) xsum = dot2(XT{}, u[e], XTraits<XT>::kOnes, xsum);
        *(u32x4_t*)&sx[(j * C + c) * CP + 8 * q] = U::xperm(u);
      }
      sX[t] = xsum;
    }
  }
  __syncthreads();

  float acc[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int j = 0; j < MT; ++j) acc[r][j] = 0.0f;

  const __amdgpu_buffer_rsrc_t ry = make_rsrc(d.y, (int64_t)m * n * esz);
  // End of a batch: reduce over the L lanes of each row; lane li == 0 of each row stores (all
  // lanes issue the stores, the others with an out-of-range offset).
  auto finish_batch = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int lr = lrow0 + b * rows_per_set + r * P;
      const bool own = li == 0 && lr < rows_left;
      const float add = sLB[lr];
#pragma unroll
      for (int j = 0; j < MT; ++j) {
        const float v = group_sum(acc[r][j], L) + add;
        const int64_t e = (int64_t)j * n + wg_row + lr;
        const int off = (own && j < m) ? (int)(e * esz) : kOOB;
        if (esz == 4)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ry, off, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b16(
              (uint16_t)(ydt == DT_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v)), ry, off, 0, 0);
        acc[r][j] = 0.0f;
      }
    }
  };

  // The codes of the R rows are unpacked once; each row of x is then read (LDS or memory) and
  // dotted with all R of them, so the live registers do not grow with MT.
  auto compute = [&](int i, const StepBuf& q) __attribute__((always_inline)) {
    const int c = li + i * L;
    uint32_t t[R][NP];
    float sr[R], br[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      U::codes(q.w[r], t[r], mk, mg);
      sr[r] = param_to_f32<PT>(q.s[r]);
      br[r] = param_to_f32<PT>(q.b[r]);
    }
#pragma unroll
    for (int j = 0; j < MT; ++j) {
      const int jj = j < m ? j : 0;  // rows past m reuse row 0 and are never stored
      uint32_t xp[NP];
      float xs;
      if (XLDS) {
#pragma unroll
        for (int e = 0; e < NP / 4; ++e) {
          const u32x4_t u = *(const u32x4_t*)&sx[(jj * C + c) * CP + 8 * e];
          xp[4 * e + 0] = u[0];
          xp[4 * e + 1] = u[1];
          xp[4 * e + 2] = u[2];
          xp[4 * e + 3] = u[3];
        }
        xs = sX[jj * C + c];
      } else {
        gptr<uint16_t> xg = (gptr<uint16_t>)d.x;
        float tsum = 0.0f;
#pragma unroll
        for (int e = 0; e < NP / 4; ++e) {
          const u32x4_t raw = *(gptr<u32x4_t>)(xg + (int64_t)jj * k + (int64_t)c * CK + 8 * e);
#pragma unroll
          for (int z = 0; z < 4; ++z) tsum = dot2(XT{}, raw[z], XTraits<XT>::kOnes, tsum);
          const u32x4_t u = U::xperm(raw);
          xp[4 * e + 0] = u[0];
          xp[4 * e + 1] = u[1];
          xp[4 * e + 2] = u[2];
          xp[4 * e + 3] = u[3];
        }
        xs = tsum;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
        for (int e = 0; e < NP; e += 2) {
          p0 = dot2(XT{}, t[r][e], xp[e], p0);
          p1 = dot2(XT{}, t[r][e + 1], xp[e + 1], p1);
        }
        const float pq = __builtin_fmaf(-U::kOff, xs, p0 + p1);  // sum x*q
        acc[r][j] = __builtin_fmaf(sr[r], pq, __builtin_fmaf(br[r], xs, acc[r][j]));
      }
    }
  };

  // Every load is issued on every path (past the end with an out-of-range offset), so the wait
  // counts are the same whichever way a branch goes.
  auto run = [&](int st, const StepBuf& q) __attribute__((always_inline)) {
    if (st < steps) {
      int b, i;
      step_of(st, b, i);
      compute(i, q);
      if (i == CPL - 1) finish_batch(b);
    }
  };
  for (int s0 = 0; s0 < steps; s0 += 2) {
    issue(s0 + 1, bufB);
    run(s0, bufA);
    issue(s0 + 2, bufA);
    run(s0 + 1, bufB);
  }
  if (steps == 0)  // k == 0: the product is the layer bias (or zero)
    for (int bb = 0; bb < geo.batches; ++bb) finish_batch(bb);
}

template <int MT, int BITS, typename XT, typename PT>
hipError_t launch_t(const GemvDesc& single, const GemvDesc* table, const GemvTile* tiles, int64_t grid,
                    size_t lds_bytes, int xlds, bool g2, int ydt, hipStream_t s) {
  (void)g2;
  const unsigned gd = (unsigned)grid;
  if (xlds)
    gemv_kernel<MT, BITS, XT, PT, true><<<gd, 256, lds_bytes, s>>>(single, table, tiles, ydt);
  else
    gemv_kernel<MT, BITS, XT, PT, false><<<gd, 256, lds_bytes, s>>>(single, table, tiles, ydt);
  return hipGetLastError();
}

template <int MT>
inline hipError_t launch_m(const GemvDesc& single, const GemvDesc* table, const GemvTile* tiles, int64_t grid,
                    size_t lds, int xlds, bool g2, int bits, int xdt, int pdt, int ydt, hipStream_t s) {
  const bool xb = xdt == DT_BF16, pb = pdt == DT_BF16;
  if (bits == 4) {
    if (xb && pb) return launch_t<MT, 4, BF16, BF16>(single, table, tiles, grid, lds, xlds, g2, ydt, s);
    if (xb) return launch_t<MT, 4, BF16, F16>(single, table, tiles, grid, lds, xlds, g2, ydt, s);
    if (pb) return launch_t<MT, 4, F16, BF16>(single, table, tiles, grid, lds, xlds, g2, ydt, s);
    return launch_t<MT, 4, F16, F16>(single, table, tiles, grid, lds, xlds, g2, ydt, s);
  }
  if (xb && pb) return launch_t<MT, 8, BF16, BF16>(single, table, tiles, grid, lds, xlds, false, ydt, s);
  if (xb) return launch_t<MT, 8, BF16, F16>(single, table, tiles, grid, lds, xlds, false, ydt, s);
  if (pb) return launch_t<MT, 8, F16, BF16>(single, table, tiles, grid, lds, xlds, false, ydt, s);
  return launch_t<MT, 8, F16, F16>(single, table, tiles, grid, lds, xlds, false, ydt, s);
}

}  // namespace gemv_detail
}  // namespace ql
