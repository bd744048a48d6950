// Decode GEMV on the matrix cores for 4-bit affine codes: y[m,n] = x[m,k] . (code*scale + bias)^T,
// fp32 accumulation, one rounding to the output dtype -- the product of gemv_impl.hpp (Nx_quant
// API docs, Products: apply; GPTQModel wiki "MLX Apple Silicon", Executing MLX qlinear kernels),
// with the code-times-x sums done by v_mfma_f32_16x16x32 instead of v_dot2.
//
// One product D = A.B takes a 16x32 A and a 32x16 B (lane l: row or column l%16, k-slots
// 8*(l/16)..+7; D: column l%16, rows 4*(l/16)..+3).  B is 16 weight rows, one per column: every
// lane reads 16 bytes (32 codes) of its row, and word t of them is its k-slots in product t, so
// four products cover a u-block of 128 codes of 16 rows.  A carries x: its row i serves one
// (x row, group of the u-block) pair, with x in the k-slots of that group and zeros in the others,
// so accumulator row i collects that group's sum of x*code for that x row.  Each u-block ends with
// the fold of every accumulator element with its group's scale and bias,
//   acc += s * (D - off*X) + b * X,   X = that group's sum of x,
// the codes entering as 16-bit floats off + q (off = 128 for bf16 x, 1024 for f16 x; exact), so
// that D - off*X is the group's sum of x*q.
//
// x is staged once per workgroup in LDS, permuted to the order the code unpacking gives, with a
// zero row that the lanes of non-matching (row, group) pairs read, and the table of group sums.
// The workgroup's scales and biases are read once, coalesced, into LDS (reading them per u-block
// and lane touches 16 rows' cache lines per instruction).  Weight words are read with a plain
// cache policy: a 128-byte line is consumed by two consecutive u-blocks.
#pragma once
#include "gemv_impl.hpp"

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

// Loads of one step: per row set and u-block, the lane's 16 bytes of codes.
struct MfBuf {
  u32x4_t w[MRS][MNU];
};

// The (scale | bias << 16) words of the u-block's groups for one row, from LDS (G = 32: four
// groups; 64: two; 128: one).
template <int G> struct MfParams;
template <> struct MfParams<32> {
  uint32_t v[4];
  __device__ __forceinline__ void load(const uint8_t* p) {
    const u32x4_t t = *(const u32x4_t*)p;
    v[0] = t[0], v[1] = t[1], v[2] = t[2], v[3] = t[3];
  }
};
template <> struct MfParams<64> {
  uint32_t v[2];
  __device__ __forceinline__ void load(const uint8_t* p) {
    const u32x2_t t = *(const u32x2_t*)p;
    v[0] = t[0], v[1] = t[1];
  }
};
template <> struct MfParams<128> {
  uint32_t v[1];
  __device__ __forceinline__ void load(const uint8_t* p) { v[0] = *(const uint32_t*)p; }
};

template <int MT, int G, typename XT, typename PT>
__global__ __launch_bounds__(256, GEMV_MF_MINB) void gemv_mf_kernel(GemvDesc single, const GemvDesc* __restrict__ table,
                                                      const GemvTile* __restrict__ tiles, int ydt) {
  using U = Unpack<4, XT>;
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
  const int row_bytes = (int)(k / 2);
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

  auto issue = [&](int st, MfBuf& q) __attribute__((always_inline)) {
    const int b = st / SR, i = st - b * SR;
    const bool live = st < steps;
#pragma unroll
    for (int rs = 0; rs < MRS; ++rs) {
      const int lr = lrow0 + b * kSetRows + rs * 16;
      const int vw = live ? lr * row_bytes + 16 * h : kOOB;
#pragma unroll
      for (int u = 0; u < MNU; ++u) {
        const int ub = min(i * MNU + u, UB - 1);
        q.w[rs][u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, vw, ub * 64, GEMV_MF_AUX));
      }
    }
  };

  // NB step buffers in rotation: the loads of step s + NB - 1 are issued before step s is computed.
  constexpr int NB = GEMV_MF_NB;
  MfBuf buf[NB];
#pragma unroll
  for (int t = 0; t < NB - 1; ++t) issue(t, buf[t]);

  // -- LDS: MT rows of x, each KP values at pitch XP, permuted per 8 values as the codes unpack;
  //    then a zero row; then the sums X[ub][i] of accumulator row i's x values in u-block ub;
  //    then the workgroup's scales and biases as (scale | bias << 16) words, `groups` per row.
  const GemvMfLds lay = gemv_mf_lds(k, MT, G, d.batches);
  float* xsum = (float*)((uint8_t*)sx + lay.xsum_off);
  uint8_t* sp = (uint8_t*)sx + lay.param_off;
  {
    // rows of the workgroup that exist, times groups / 2 words of scales (and of biases); read
    // coalesced, a group count per row that is even keeps every word inside one array
    const int64_t prow = rows_left < geo.rows_per_wg ? rows_left : geo.rows_per_wg;
    const int pw = (int)(prow * groups / 2);
    for (int t = threadIdx.x; t < pw; t += 256) {
      const uint32_t sw = __builtin_amdgcn_raw_buffer_load_b32(rsc, 4 * t, 0, 0);
      const uint32_t bw = __builtin_amdgcn_raw_buffer_load_b32(rbi, 4 * t, 0, 0);
      *(u32x2_t*)(sp + 8 * t) = u32x2_t{perm(bw, sw, 0x05040100u), perm(bw, sw, 0x07060302u)};
    }
  }
  {
    // One thread per 8 values: stage them, and sum them with the GW/8 neighbours of the same
    // accumulator row and u-block (aligned lane groups; (MT+1) * KP/8 is a multiple of 16).
    gptr<uint16_t> xg = (gptr<uint16_t>)d.x;
    const int c8n = KP / 8;
    constexpr int GL = GW / 8;  // lanes per x sum: 16, 8 or 4
    for (int t = threadIdx.x; t < (MT + 1) * c8n; t += 256) {
      const int xr = t / c8n, c8 = t - xr * c8n;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (xr < m && c8 * 8 < k) {
        const u32x4_t raw = *(gptr<u32x4_t>)(xg + (int64_t)xr * k + 8 * c8);
        v = U::xperm(raw);
      }
      *(u32x4_t*)&sx[xr * XP + 8 * c8] = v;
      float sum = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) sum = dot2(XT{}, v[e], XTraits<XT>::kOnes, sum);
      sum = group_sum(sum, GL);
      const int ub = c8 >> 4, gp = (c8 & 15) / GL;
      if (xr < MT && (c8 & (GL - 1)) == 0) xsum[ub * 16 + xr * GU + gp] = sum;
    }
    // accumulator rows past MT * GU have no x row: zero sums
    for (int t = threadIdx.x; t < SR * MNU * (16 - MT * GU); t += 256) {
      const int ub = t / (16 - MT * GU), i = MT * GU + t - ub * (16 - MT * GU);
      xsum[ub * 16 + i] = 0.0f;
    }
  }
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
        float v = add;
#pragma unroll
        for (int e = 0; e < GU; ++e) v += acc[rs][p * GU + e];
        const int xr = (4 * h) / GU + p;
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

  auto compute = [&](int b, int i, const MfBuf& q) __attribute__((always_inline)) {
    // this lane's parameter words of u-block i * MNU, per row set
    const uint8_t* pb = sp + ((lrow0 + b * kSetRows) * groups + i * MNU * GU) * 4;
#pragma unroll
    for (int u = 0; u < MNU; ++u) {
      const int ub = i * MNU + u;  // past UB the x rows and sums are zero
      u32x4_t a[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) a[t] = *(const u32x4_t*)(abase + ub * 256 + 16 * t);
      const f32x4_t X = *(const f32x4_t*)(xbase + ub * 64);
#pragma unroll
      for (int rs = 0; rs < MRS; ++rs) {
        uint32_t c[16];
        U::codes(q.w[rs][u], c, mk, mg);
        f32x4_t D = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < 4; ++t) D = MfOp<XT>::mma(a[t], u32x4_t{c[4 * t], c[4 * t + 1], c[4 * t + 2], c[4 * t + 3]}, D);
        // past UB the words of the row's last u-block stand in (finite; they meet zeros)
        MfParams<G> pr;
        pr.load(pb + (rs * 16 * groups + min(u, UB - 1 - i * MNU) * GU) * 4);
        float sv[GU < NR ? GU : NR], bv[GU < NR ? GU : NR];
#pragma unroll
        for (int gp = 0; gp < (GU < NR ? GU : NR); ++gp) {
          sv[gp] = half_param<PT>(pr.v[gp], false);
          bv[gp] = half_param<PT>(pr.v[gp], true);
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          const float pq = __builtin_fmaf(-kOff, X[r], D[r]);  // sum x*q of the group
          acc[rs][r] = __builtin_fmaf(sv[r % GU], pq, __builtin_fmaf(bv[r % GU], X[r], acc[rs][r]));
        }
      }
    }
  };

  auto run = [&](int st, const MfBuf& q) __attribute__((always_inline)) {
    if (st < steps) {
      const int b = st / SR, i = st - b * SR;
      compute(b, i, q);
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

template <int MT, int G, typename XT, typename PT>
hipError_t launch_mf_t(const GemvDesc& single, const GemvDesc* table, const GemvTile* tiles, int64_t grid,
                       size_t lds_bytes, int ydt, hipStream_t s) {
  gemv_mf_kernel<MT, G, XT, PT><<<(unsigned)grid, 256, lds_bytes, s>>>(single, table, tiles, ydt);
  return hipGetLastError();
}

template <int MT, int G>
hipError_t launch_mf_g(const GemvDesc& single, const GemvDesc* table, const GemvTile* tiles, int64_t grid,
                       size_t lds, int xdt, int pdt, int ydt, hipStream_t s) {
  const bool xb = xdt == DT_BF16, pb = pdt == DT_BF16;
  if (xb && pb) return launch_mf_t<MT, G, BF16, BF16>(single, table, tiles, grid, lds, ydt, s);
  if (xb) return launch_mf_t<MT, G, BF16, F16>(single, table, tiles, grid, lds, ydt, s);
  if (pb) return launch_mf_t<MT, G, F16, BF16>(single, table, tiles, grid, lds, ydt, s);
  return launch_mf_t<MT, G, F16, F16>(single, table, tiles, grid, lds, ydt, s);
}

template <int MT>
hipError_t launch_mf_m(const GemvDesc& single, const GemvDesc* table, const GemvTile* tiles, int64_t grid,
                       size_t lds, int g, int xdt, int pdt, int ydt, hipStream_t s) {
  if (g == 128) return launch_mf_g<MT, 128>(single, table, tiles, grid, lds, xdt, pdt, ydt, s);
  if (g == 64) return launch_mf_g<MT, 64>(single, table, tiles, grid, lds, xdt, pdt, ydt, s);
  if constexpr (MT * gemv_mf_gu(32) <= 16) {
    if (g == 32) return launch_mf_g<MT, 32>(single, table, tiles, grid, lds, xdt, pdt, ydt, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace gemv_detail
}  // namespace ql
