// Decode GEMV on the matrix cores for affine codes of 2 to 6 and 8 bits: y[m,n] = x[m,k] . (code*scale +
// bias)^T, fp32 accumulation, one rounding to the output dtype -- the product of gemv_impl.hpp
// (Nx_quant API docs, Products: apply; GPTQModel wiki "MLX Apple Silicon", Executing MLX qlinear
// kernels), with the code-times-x sums done by v_mfma_f32_16x16x32 instead of v_dot2.
//
// One product D = A.B takes a 16x32 A and a 32x16 B (lane l: row or column l%16, k-slots
// 8*(l/16)..+7; D: column l%16, rows 4*(l/16)..+3).  B is 16 weight rows, one per column: every
// lane reads 32 codes of its row (8 bytes at 2 bits, 12 at 3, 16 at 4, 20 at 5, 24 at 6, 32 at 8), and codes 8t..8t+7 of them are its
// k-slots in product t, so four products cover a u-block of 128 codes of 16 rows.  A carries x: its row i serves one
// (x row, group of the u-block) pair, with x in the k-slots of that group and zeros in the others,
// so accumulator row i collects that group's sum of x*code for that x row.  Each u-block ends with
// the fold of every accumulator element with its group's scale and bias,
//   acc += s * (D - off*X) + b * X,   X = that group's sum of x,
// the codes entering as 16-bit floats off + q (exact), so that D - off*X is the group's sum of
// x*q: 2- to 6-bit codes as bf16 128 + q with bf16 x and as f16 1024 + q with f16 x; 8-bit codes always
// as f16 1024 + q (bf16 has too few bits for 128 + q), with bf16 x converted to f16 after an exact
// power-of-two scaling per x row that brings max |x| into [2^14, 2^15) (every bf16 value of that
// row within 2^31 of the maximum converts exactly); the row's factor is applied at the end.
//
// x is staged once per workgroup in LDS, permuted to the order the code unpacking gives, with a
// zero row that the lanes of non-matching (row, group) pairs read, and the table of group sums.
// The workgroup's scales and biases are copied once, coalesced, into LDS by DMA (reading them
// per u-block and lane touches 16 rows' cache lines per instruction).  Weight words are read with
// a plain cache policy: a 128-byte line is consumed by two consecutive u-blocks.
#pragma once
#include "gemv_impl.hpp"

#include <type_traits>

namespace ql {
namespace gemv_detail {

template <typename XT> struct MfOp;
template <> struct MfOp<BF16> {
  __device__ __forceinline__ static f32x4_t mma(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                   0, 0, 0);
  }
};
template <> struct MfOp<F16> {
  __device__ __forceinline__ static f32x4_t mma(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
  }
};

// Low (hi = false) or high half of a word of two 16-bit parameters, as fp32.
template <typename PT> __device__ __forceinline__ float half_param(uint32_t w, bool hi);
template <> __device__ __forceinline__ float half_param<BF16>(uint32_t w, bool hi) {
  return __uint_as_float(hi ? (w & 0xffff0000u) : (w << 16));
}
template <> __device__ __forceinline__ float half_param<F16>(uint32_t w, bool hi) {
  return f16_bits_to_f32(hi ? (w >> 16) : (w & 0xffffu));
}

constexpr int MNU = GEMV_MF_NU;  // u-blocks per step
constexpr int MRS = GEMV_MF_RS;  // 16-row sets per wave

// Loads of one step: per row set and u-block, the lane's 32 codes (WPB = 1 or 2 16-byte loads).
template <int WPB> struct MfBuf {
  u32x4_t w[MRS][MNU][WPB];
};

// The scales and biases of the u-block's groups for one row, from the two LDS arrays that hold
// the workgroup's rows as they lie in memory (G = 32: four groups, two words of each; 64: two
// groups, one word; 128: one group, one 16-bit value in the low half).
template <int G> struct MfParams;
template <> struct MfParams<32> {
  uint32_t s[2], b[2];
  __device__ __forceinline__ void load(const uint8_t* ps, const uint8_t* pb) {
    const u32x2_t ts = *(const u32x2_t*)ps, tb = *(const u32x2_t*)pb;
    s[0] = ts[0], s[1] = ts[1], b[0] = tb[0], b[1] = tb[1];
  }
};
template <> struct MfParams<64> {
  uint32_t s[1], b[1];
  __device__ __forceinline__ void load(const uint8_t* ps, const uint8_t* pb) {
    s[0] = *(const uint32_t*)ps, b[0] = *(const uint32_t*)pb;
  }
};
template <> struct MfParams<128> {
  uint32_t s[1], b[1];
  __device__ __forceinline__ void load(const uint8_t* ps, const uint8_t* pb) {
    s[0] = *(const uint16_t*)ps, b[0] = *(const uint16_t*)pb;
  }
};

typedef __attribute__((address_space(3))) void mf_lds_void;

template <int MT, int G, typename XT, typename PT, int BITS>
__global__ __launch_bounds__(256, GEMV_MF_MINB) void gemv_mf_kernel(GemvDesc single, const GemvDesc* __restrict__ table,
                                                      const GemvTile* __restrict__ tiles, int ydt) {
  // CT: the 16-bit type of the products' operands; x is converted (and scaled) to it when it differs
  using CT = typename std::conditional<BITS == 8, F16, XT>::type;
  constexpr bool kConvX = !std::is_same<CT, XT>::value;
  // loads per row and u-block: one of 8, 12 or 16 bytes at 2, 3 or 4 bits; 16 + 4 at 5; 16 + 8 at 6;
  // 16 + 16 at 8
  constexpr int WPB = BITS >= 5 ? 2 : 1;
  constexpr int LB = 4 * BITS;                   // bytes of the lane's 32 codes
  using U = Unpack<BITS, CT>;
  constexpr int GU = gemv_mf_gu(G);                // groups per u-block
  constexpr int NR = MT * GU < 4 ? MT * GU : 4;    // accumulator registers a lane folds
  constexpr int GW = 128 / GU;                     // x values of one accumulator row per u-block
  constexpr float kOff = U::kOff;
  const uint32_t mk = vconst(U::kMask), mg = vconst(U::kMagic);
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
  const GemvMfGeom geo = gemv_mf_geometry(k, d.batches);
  const int UB = geo.ublocks, SR = geo.steps_per_row, KP = geo.kpad, XP = KP + 8;
  const int groups = (int)(k / G);
  const int row_bytes = (int)(k * BITS / 8);
  const int steps = geo.batches * SR;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int j = lane & 15, h = lane >> 4;
  const int64_t wg_row = tile * geo.rows_per_wg;
  const int64_t rows_left = n - wg_row;
  const int esz = ydt == DT_F32 ? 4 : 2;
  // Offsets are relative to the workgroup's first row; the resources end at the matrix's last
  // row, so rows past n read zeros.  Within a row the u-block offset (uniform) is clamped to the
  // row's last u-block: a step past the row end re-reads real words, whose products meet zeros.
  const __amdgpu_buffer_rsrc_t rw = make_rsrc((const uint8_t*)d.packed + wg_row * row_bytes, rows_left * row_bytes);
  const __amdgpu_buffer_rsrc_t rsc = make_rsrc((const uint16_t*)d.scales + wg_row * groups, rows_left * groups * 2);
  const __amdgpu_buffer_rsrc_t rbi = make_rsrc((const uint16_t*)d.biases + wg_row * groups, rows_left * groups * 2);
  const int lrow0 = wave * 16 * MRS + j;  // this lane's weight row in row set 0 of batch 0
  constexpr int kSetRows = 64 * MRS;       // rows of one batch of the workgroup

  // 4-bit codes, 5 to 8 x rows (whose loads run three steps ahead): a step's 16 rows x 128 bytes
  // (u-blocks 2i, 2i + 1) are read by two loads that each cover 8 whole 128-byte lines,
  // non-temporally (lane 8q + p of half f reads 16-byte chunk (p - q) mod 8 of row 8f + q: the
  // rotation spreads the chunks one product reads over the LDS banks); before the products the
  // wave regroups them through its LDS area into the product layout (lane (j, h) of u-block u:
  // row j, chunk 4u + h).  Rows past n read zeros; a u-block past the row's last is clamped to
  // it, as below.
  constexpr bool kLines = gemv_mf_lines(BITS, MT);
  auto issue = [&](int st, MfBuf<WPB>& q) __attribute__((always_inline)) {
    const int b = st / SR, i = st - b * SR;
    const bool live = st < steps;
    if constexpr (kLines) {
      const int qr = lane >> 3, c = ((lane & 7) - qr) & 7;
      const int ub = min(2 * i + (c >> 2), UB - 1);
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int lr = wave * 16 + b * kSetRows + 8 * f + qr;
        const uint32_t off = live ? (uint32_t)(lr * row_bytes + ub * 64 + 16 * (c & 3)) : (uint32_t)kOOB;
        q.w[0][f][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)off, 0, GEMV_MF_LAUX));
      }
      return;
    }
#pragma unroll
    for (int rs = 0; rs < MRS; ++rs) {
      const int lr = lrow0 + b * kSetRows + rs * 16;
      // unsigned, so that the second load's vw + 16 past the end wraps instead of overflowing; an
      // offset at or past 0x7ffffff0 stays outside every resource (they are below 2^31 bytes)
      const uint32_t vw = live ? (uint32_t)(lr * row_bytes + LB * h) : (uint32_t)kOOB;
#pragma unroll
      for (int u = 0; u < MNU; ++u) {
        const int ub = min(i * MNU + u, UB - 1);
        if constexpr (BITS == 2) {
          const u32x2_t t2 =
              __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rw, (int)vw, ub * 4 * LB, GEMV_MF_AUX));
          q.w[rs][u][0] = u32x4_t{t2[0], t2[1], 0u, 0u};
        } else if constexpr (BITS == 5) {  // 20 bytes at a 4-byte aligned offset
          q.w[rs][u][0] =
              __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)vw, ub * 4 * LB, GEMV_MF_AUX));
          q.w[rs][u][1] = u32x4_t{__builtin_amdgcn_raw_buffer_load_b32(rw, (int)(vw + 16u), ub * 4 * LB, GEMV_MF_AUX), 0u, 0u, 0u};
        } else if constexpr (BITS == 6) {  // 24 bytes at an 8-byte aligned offset
          q.w[rs][u][0] =
              __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)vw, ub * 4 * LB, GEMV_MF_AUX));
          const u32x2_t t2 =
              __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rw, (int)(vw + 16u), ub * 4 * LB, GEMV_MF_AUX));
          q.w[rs][u][1] = u32x4_t{t2[0], t2[1], 0u, 0u};
        } else if constexpr (BITS == 3) {  // 12 bytes at a 4-byte aligned offset
          const auto t3 = __builtin_amdgcn_raw_buffer_load_b96(rw, (int)vw, ub * 4 * LB, GEMV_MF_AUX);
          q.w[rs][u][0] = u32x4_t{t3[0], t3[1], t3[2], 0u};
        } else {
#pragma unroll
          for (int c = 0; c < WPB; ++c)
            q.w[rs][u][c] = __builtin_bit_cast(
                u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(vw + 16u * c), ub * 4 * LB, GEMV_MF_AUX));
        }
      }
    }
  };

  // NB step buffers in rotation: the loads of step s + NB - 1 are issued before step s is computed.
  constexpr int NB = MT >= 8 ? GEMV_MF_NB_M8 : GEMV_MF_NB;
  MfBuf<WPB> buf[NB];
#pragma unroll
  for (int t = 0; t < NB - 1; ++t) issue(t, buf[t]);

  // -- LDS: MT rows of x, each KP values at pitch XP, permuted per 8 values as the codes unpack;
  //    then a zero row; then the sums X[ub][i] of accumulator row i's x values in u-block ub;
  //    then the workgroup's scales, then its biases, each `groups` 16-bit values per row; then,
  //    for 4-bit codes and 5 to 8 x rows, each wave's regrouping area.
  const GemvMfLds lay = gemv_mf_lds(k, MT, G, d.batches, BITS);
  float* xsum = (float*)((uint8_t*)sx + lay.xsum_off);
  float* xscale = (float*)((uint8_t*)sx + lay.xscale_off);
  uint8_t* sps = (uint8_t*)sx + lay.param_off;
  uint8_t* spb = (uint8_t*)sx + lay.bias_off;
  {
    // The scales and biases of the rows of the workgroup that exist (groups / 2 words per row,
    // contiguous in memory) are copied HBM -> LDS by DMA, 64 words per wave instruction, every
    // pass in flight at once and no registers held: the x staging below issues its loads behind
    // them, so both take one round trip.  The wait before the barrier below lands them.
    const int pw = (int)((rows_left < geo.rows_per_wg ? rows_left : geo.rows_per_wg) * groups / 2);
    for (int i0 = wave * 64; i0 < pw; i0 += 256)
      if (i0 + lane < pw) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, (mf_lds_void*)(sps + 4 * i0), 4, 4 * (i0 + lane), 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rbi, (mf_lds_void*)(spb + 4 * i0), 4, 4 * (i0 + lane), 0, 0, 0);
      }
  }
  gptr<uint16_t> xg = (gptr<uint16_t>)d.x;
  const int c8n = KP / 8;
  // x is staged MSU chunks of 8 values per thread at a time, their loads issued together (one
  // round trip per MSU chunks); chunk t is (x row t / c8n, values 8 (t % c8n) ..), zero past m or k
  constexpr int MSU = MT >= 8 ? GEMV_MF_SU_M8 : GEMV_MF_SU;
  auto load_x = [&](int t, int total) __attribute__((always_inline)) {
    const int xr = t / c8n, c8 = t - xr * c8n;
    u32x4_t r = {0u, 0u, 0u, 0u};
    if (t < total && xr < m && c8 * 8 < k) r = *(gptr<u32x4_t>)(xg + (int64_t)xr * k + 8 * c8);
    return r;
  };
  // bf16 x into f16 products: per x row the factor 2^-t that brings max |x| into [2^14, 2^15)
  // (t clamped to [-100, 100]; 2^t is kept for the end)
  float xmul[MT];
  if constexpr (kConvX) {
    __shared__ uint32_t s_amax[MT];
    if (threadIdx.x < MT) s_amax[threadIdx.x] = 0u;
    __syncthreads();
    for (int t0 = threadIdx.x; t0 < MT * c8n; t0 += 256 * MSU) {
      u32x4_t raw[MSU];
#pragma unroll
      for (int u = 0; u < MSU; ++u) raw[u] = load_x(t0 + 256 * u, MT * c8n);
#pragma unroll
      for (int u = 0; u < MSU; ++u) {
        const int t = t0 + 256 * u, xr = t / c8n;
        uint32_t a = 0u;
#pragma unroll
        for (int e = 0; e < 4; ++e) a = max(a, max(raw[u][e] & 0x7fffu, (raw[u][e] >> 16) & 0x7fffu));
        if (t < MT * c8n && xr < m) atomicMax(&s_amax[xr], a);  // |x| of bf16 bits orders as the integer bits
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < MT; ++r) {
      const uint32_t a = s_amax[r];
      const int e = (int)(a >> 7) - 127;  // a in [2^e, 2^(e+1)) for a normal value
      const int t = a == 0u ? 0 : min(100, max(-100, e - 14));
      xmul[r] = __builtin_ldexpf(1.0f, -t);
      if (threadIdx.x == 0) xscale[r] = __builtin_ldexpf(1.0f, t);
    }
  }
  {
    // One thread per 8 values: stage them, and sum them with the GW/8 neighbours of the same
    // accumulator row and u-block (aligned lane groups; (MT+1) * KP/8 is a multiple of 16).
    constexpr int GL = GW / 8;  // lanes per x sum: 16, 8 or 4
    const int total = (MT + 1) * c8n;
    for (int t0 = threadIdx.x; t0 < total; t0 += 256 * MSU) {
      u32x4_t raws[MSU];
#pragma unroll
      for (int u = 0; u < MSU; ++u) raws[u] = load_x(t0 + 256 * u, total);
#pragma unroll
      for (int u = 0; u < MSU; ++u) {
      const int t = t0 + 256 * u;
      if (t >= total) break;
      const int xr = t / c8n, c8 = t - xr * c8n;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (xr < m && c8 * 8 < k) {
        u32x4_t raw = raws[u];
        if constexpr (kConvX) {
          float f = 1.0f;
#pragma unroll
          for (int r = 0; r < MT; ++r)
            if (xr == r) f = xmul[r];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const _Float16 lo = (_Float16)(__uint_as_float(raw[e] << 16) * f);
            const _Float16 hi = (_Float16)(__uint_as_float(raw[e] & 0xffff0000u) * f);
            raw[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
          }
        }
        v = U::xperm(raw);
      }
      *(u32x4_t*)&sx[xr * XP + 8 * c8] = v;
      float sum = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) sum = dot2(CT{}, v[e], XTraits<CT>::kOnes, sum);
      sum = group_sum(sum, GL);
      const int ub = c8 >> 4, gp = (c8 & 15) / GL;
      if (xr < MT && (c8 & (GL - 1)) == 0) xsum[ub * 16 + xr * GU + gp] = sum;
      }
    }
    // accumulator rows past MT * GU have no x row: zero sums
    for (int t = threadIdx.x; t < SR * MNU * (16 - MT * GU); t += 256) {
      const int ub = t / (16 - MT * GU), i = MT * GU + t - ub * (16 - MT * GU);
      xsum[ub * 16 + i] = 0.0f;
    }
  }
  // this wave's parameter copies have landed (vmcnt 0; expcnt and lgkmcnt left alone), then the
  // barrier publishes every wave's
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();

  // A row of this lane is j: x row j / GU, group slot j % GU; its k-slots (quadrant h) lie in
  // group slot (32 h) / G of the u-block.  Lanes whose pair does not match read the zero row.
  const int xra = j / GU, gpa = j - xra * GU;
  const int gph = G >= 128 ? 0 : (32 * h) / G;
  const bool amatch = xra < m && gpa == gph;
  const uint8_t* abase = (const uint8_t*)sx + ((amatch ? xra : MT) * XP + 32 * h) * 2;
  const uint8_t* xbase = (const uint8_t*)xsum + 16 * h;  // X[ub][4h .. 4h+3]

  float acc[MRS][4];
#pragma unroll
  for (int rs = 0; rs < MRS; ++rs)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[rs][r] = 0.0f;

  const __amdgpu_buffer_rsrc_t ry = make_rsrc(d.y, (int64_t)m * n * esz);
  gptr<uint16_t> lbg = (gptr<uint16_t>)d.layer_bias;
  // End of a batch: lane (j, h) holds accumulator rows 4h..4h+3 of column j, i.e. x rows
  // 4h/GU + p, each the sum of GU registers.
  auto finish_batch = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int rs = 0; rs < MRS; ++rs) {
      const int lr = lrow0 + b * kSetRows + rs * 16;
      const bool rowok = lr < rows_left;
      const float add = (lbg && rowok) ? x_to_f32<XT>(lbg[wg_row + lr]) : 0.0f;
#pragma unroll
      for (int p = 0; p < NR / GU; ++p) {
        const int xr = (4 * h) / GU + p;
        float v = 0.0f;
#pragma unroll
        for (int e = 0; e < GU; ++e) v += acc[rs][p * GU + e];
        if constexpr (kConvX) v *= xscale[xr < MT ? xr : 0];
        v += add;
        const int64_t el = (int64_t)xr * n + wg_row + lr;
        const int off = (rowok && xr < m) ? (int)(el * esz) : kOOB;
        if (esz == 4)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ry, off, 0, 0);
        else
          __builtin_amdgcn_raw_buffer_store_b16(
              (uint16_t)(ydt == DT_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v)), ry, off, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[rs][r] = 0.0f;
    }
  };

  auto compute = [&](int b, int i, const MfBuf<WPB>& q) __attribute__((always_inline)) {
    // this lane's (row, group) index at u-block i * MNU, per row set
    const int pe = (lrow0 + b * kSetRows) * groups + i * MNU * GU;
#pragma unroll
    for (int u = 0; u < MNU; ++u) {
      const int ub = i * MNU + u;  // past UB the x rows and sums are zero
      u32x4_t a[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = *(const u32x4_t*)(abase + ub * 256 + 16 * t);
      const f32x4_t X = *(const f32x4_t*)(xbase + ub * 64);
#pragma unroll
      for (int rs = 0; rs < MRS; ++rs) {
        // 16 operand words: product t takes words 4t .. 4t+3 (codes 8t .. 8t+7 of the lane's 32)
        uint32_t c[16];
        if constexpr (BITS == 5 || BITS == 6) {
          U::codes2(q.w[rs][u][0], q.w[rs][u][1], c, mk, mg);
        } else {
#pragma unroll
          for (int w = 0; w < WPB; ++w) U::codes(q.w[rs][u][w], c + (16 / WPB) * w, mk, mg);
        }
        f32x4_t D = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < 4; ++t) D = MfOp<CT>::mma(a[t], u32x4_t{c[4 * t], c[4 * t + 1], c[4 * t + 2], c[4 * t + 3]}, D);
        // past UB the words of the row's last u-block stand in (finite; they meet zeros)
        MfParams<G> pr;
        const int e = pe + rs * 16 * groups + min(u, UB - 1 - i * MNU) * GU;
        pr.load(sps + 2 * e, spb + 2 * e);
        float sv[GU < NR ? GU : NR], bv[GU < NR ? GU : NR];
#pragma unroll
        for (int gp = 0; gp < (GU < NR ? GU : NR); ++gp) {
          sv[gp] = half_param<PT>(pr.s[gp / 2], gp % 2 == 1);
          bv[gp] = half_param<PT>(pr.b[gp / 2], gp % 2 == 1);
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const float pq = __builtin_fmaf(-kOff, X[r], D[r]);  // sum x*q of the group
          acc[rs][r] = __builtin_fmaf(sv[r % GU], pq, __builtin_fmaf(bv[r % GU], X[r], acc[rs][r]));
        }
      }
    }
  };

  uint8_t* sre = (uint8_t*)sx + lay.regroup_off + wave * kGemvMfRegroupBytes;
  auto run = [&](int st, const MfBuf<WPB>& q) __attribute__((always_inline)) {
    if (st < steps) {
      const int b = st / SR, i = st - b * SR;
      if constexpr (kLines) {
        // the wave's LDS accesses run in order: the previous step's reads of the area are done
#pragma unroll
        for (int f = 0; f < 2; ++f) *(u32x4_t*)(sre + f * kGemvMfHalfOff + 16 * lane) = q.w[0][f][0];
        MfBuf<WPB> r;
        const int q7 = j & 7;
        const uint8_t* sb = sre + (j >> 3) * kGemvMfHalfOff + 128 * q7;
#pragma unroll
        for (int u = 0; u < MNU; ++u) r.w[0][u][0] = *(const u32x4_t*)(sb + 16 * ((4 * u + h + q7) & 7));
        compute(b, i, r);
      } else {
        compute(b, i, q);
      }
      if (i == SR - 1) finish_batch(b);
    }
  };
  for (int s0 = 0; s0 < steps; s0 += NB) {
#pragma unroll
    for (int t = 0; t < NB; ++t) {
      issue(s0 + t + NB - 1, buf[(t + NB - 1) % NB]);
      if (GEMV_MF_SCHED) __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the products
      run(s0 + t, buf[t]);
    }
  }
}

template <int MT, int G, typename XT, typename PT, int BITS>
hipError_t launch_mf_t(const GemvDesc& single, const GemvDesc* table, const GemvTile* tiles, int64_t grid,
                       size_t lds_bytes, int ydt, hipStream_t s) {
  gemv_mf_kernel<MT, G, XT, PT, BITS><<<(unsigned)grid, 256, lds_bytes, s>>>(single, table, tiles, ydt);
  return hipGetLastError();
}

template <int MT, int G, int BITS>
hipError_t launch_mf_g(const GemvDesc& single, const GemvDesc* table, const GemvTile* tiles, int64_t grid,
                       size_t lds, int xdt, int pdt, int ydt, hipStream_t s) {
  const bool xb = xdt == DT_BF16, pb = pdt == DT_BF16;
  if (xb && pb) return launch_mf_t<MT, G, BF16, BF16, BITS>(single, table, tiles, grid, lds, ydt, s);
  if (xb) return launch_mf_t<MT, G, BF16, F16, BITS>(single, table, tiles, grid, lds, ydt, s);
  if (pb) return launch_mf_t<MT, G, F16, BF16, BITS>(single, table, tiles, grid, lds, ydt, s);
  return launch_mf_t<MT, G, F16, F16, BITS>(single, table, tiles, grid, lds, ydt, s);
}

template <int MT, int BITS>
hipError_t launch_mf_b(const GemvDesc& single, const GemvDesc* table, const GemvTile* tiles, int64_t grid,
                       size_t lds, int g, int xdt, int pdt, int ydt, hipStream_t s) {
  if (g == 128) return launch_mf_g<MT, 128, BITS>(single, table, tiles, grid, lds, xdt, pdt, ydt, s);
  if (g == 64) return launch_mf_g<MT, 64, BITS>(single, table, tiles, grid, lds, xdt, pdt, ydt, s);
  if constexpr (MT * gemv_mf_gu(32) <= 16) {
    if (g == 32) return launch_mf_g<MT, 32, BITS>(single, table, tiles, grid, lds, xdt, pdt, ydt, s);
  }
  return hipErrorInvalidValue;
}

template <int MT>
hipError_t launch_mf_m(const GemvDesc& single, const GemvDesc* table, const GemvTile* tiles, int64_t grid,
                       size_t lds, int bits, int g, int xdt, int pdt, int ydt, hipStream_t s) {
  if (bits == 8) return launch_mf_b<MT, 8>(single, table, tiles, grid, lds, g, xdt, pdt, ydt, s);
  if (bits == 4) return launch_mf_b<MT, 4>(single, table, tiles, grid, lds, g, xdt, pdt, ydt, s);
  if (bits == 2) return launch_mf_b<MT, 2>(single, table, tiles, grid, lds, g, xdt, pdt, ydt, s);
  if (bits == 3) return launch_mf_b<MT, 3>(single, table, tiles, grid, lds, g, xdt, pdt, ydt, s);
  if (bits == 6) return launch_mf_b<MT, 6>(single, table, tiles, grid, lds, g, xdt, pdt, ydt, s);
  if (bits == 5) return launch_mf_b<MT, 5>(single, table, tiles, grid, lds, g, xdt, pdt, ydt, s);
  return hipErrorInvalidValue;
}

}  // namespace gemv_detail
}  // namespace ql
