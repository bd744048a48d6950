// Routed apply for Q8_0 experts (Nx_quant API docs, Products: apply_experts; Nx_quant Weights:
// Q8_0): y[p, :] = x[p / pos_per_row, :] . W_{ids[p]}^T in fp32 with W = d * q per 32-value block.
// The routing (offsets, permutation, expert order) and the per-row factors of x are computed by
// experts.hip.
//
// Each weight is dequantized once, in registers, to fp16: d * q rounded once (2^-12 relative; d is
// an fp16 and q an int8, so the product has up to 18 significant bits), and x enters as fp16 after
// an exact power-of-two scaling per x row that brings max |x| into [2^14, 2^15).  The products run
// on v_mfma_f32_16x16x32_f16 with fp32 accumulation; the row factor is applied at the end.  fp16 x
// enters as it is (factor 1).  A block
// scale |d| > 511.75 could overflow fp16 (|d q| > 65504): a workgroup that meets one recomputes its
// outputs in fp32 from the blocks directly (slow, exact up to fp32 rounding).
#include "experts_common.hpp"

namespace ql {
namespace {
using namespace ex_detail;

// One workgroup of 8 waves per (expert, 256 weight rows), in decreasing order of the experts'
// position counts; wave w owns two column tiles of 16 weight rows and all the chunk's positions
// (up to 96: MS m-subtiles of 16).  k-tiles are 128 wide (4 blocks of 136 bytes per row): lane
// quadrant q takes block 4 kt + q of its row, a 36-byte window from the aligned word at or below
// the block; the four lanes of a row read the tile's 136 bytes.  x rows go straight into QNS LDS
// stages, QNS - 1 k-tiles ahead, and are converted to fp16 in place once they have landed; the
// weight windows go into a ring of QNS register buffers.
#ifndef EXPERTS_Q8_CONV_AHEAD
#define EXPERTS_Q8_CONV_AHEAD 1  // convert x one k-tile ahead, one barrier per k-tile
#endif
constexpr int QBK = 128, QMC = 96, QCT = 2, QW = 8, QBN = QW * 16 * QCT, QNS = 3;

struct Q8Buf {
  u32x4_t a[QCT], b[QCT];  // bytes 0..31 of the window
  uint32_t c[QCT];         // bytes 32..35 (zero past the end of the blocks: see `tail`)
};

__device__ __forceinline__ f32x4_t mfma16_f16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                0, 0, 0);
}

// Four int8 codes (one word, k order) times d -> f16 pairs (q0 d, q1 d) and (q2 d, q3 d), each
// rounded once: the bytes q + 128 become the f16 values 1024 + q + 128 (exponent bits 0x64 above
// each byte), minus 1152 gives q exactly, times d rounds once.
__device__ __forceinline__ void q8_dequant(uint32_t w, f16x2_t d2, uint32_t& lo, uint32_t& hi) {
  const uint32_t u = w ^ 0x80808080u;
  const f16x2_t off = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  const f16x2_t a = __builtin_bit_cast(f16x2_t, perm(0x64646464u, u, 0x04010400u)) + off;
  const f16x2_t b = __builtin_bit_cast(f16x2_t, perm(0x64646464u, u, 0x04030402u)) + off;
  lo = __builtin_bit_cast(uint32_t, a * d2);
  hi = __builtin_bit_cast(uint32_t, b * d2);
}

// x stage: row r holds 16 chunks of 8 values, chunk c at slot c ^ (r % 16) (as experts_mx.hip).
template <int MS, bool XF16>
__device__ __forceinline__ void q8_chunk(const int32_t* __restrict__ sPos, const float* __restrict__ sXinv,
                                         const float* __restrict__ sXs, int* __restrict__ sFlag, int rows,
                                         uint8_t* const* stg, __amdgpu_buffer_rsrc_t rsX,
                                         __amdgpu_buffer_rsrc_t rsW, int64_t K, int64_t N, int64_t ncol0,
                                         const uint32_t* wa, const uint32_t* wsh, uint32_t wend, uint32_t tail,
                                         int64_t pos_per_row, void* __restrict__ y, int ydt) {
  constexpr int CPW = (MS + 1) / 2;                // x copies per wave and k-tile
  constexpr int NW = 3 * QCT;                      // weight loads per lane and k-tile
  constexpr int L = NW + (QNS - 2) * (CPW + NW);  // loads issued after x(kt) when kt is due
  static_assert(L < 64, "vmcnt range");
  // the copies of a k-tile (1 KB each, at (QW i + w) KB), the converted chunks and the output
  // blocks (2 KB per wave) stay inside one stage
  static_assert(QW * CPW * 1024 <= QMC * QBK * 2, "x copies past the stage");
  static_assert(16 * 16 * MS * 16 <= QMC * QBK * 2, "converted chunks past the stage");
  static_assert(QW * 2048 <= QMC * QBK * 2, "output blocks past the stage");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j16 = lane & 15, q = lane >> 4;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int KT = (int)((K + QBK - 1) / QBK);
  const int kint = (int)K;

  uint32_t xoff[CPW];
  int xc[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int r = (QW * i + wave) * 4 + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    const int32_t pos = sPos[r < rows ? r : 0];
    xoff[i] = (uint32_t)(((int64_t)(pos / pos_per_row) * K + 8 * c) * 2);
    xc[i] = c;
  }
  auto copy_x = [&](int kt, uint8_t* stage) __attribute__((always_inline)) {
    const int k0 = kt * QBK;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const uint32_t v = k0 + 8 * xc[i] < kint ? xoff[i] : kExOOB;  // zeros past K
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsX, (lds_void*)(stage + (QW * i + wave_u) * 1024), 16, v,
                                               (uint32_t)(k0 * 2), 0, 0);
    }
  };
  // bf16 x of a stage -> f16 times the row's factor (exact for every value within 2^31 of the row's
  // maximum), in place; 16 * 16 * MS chunks of 8 values over the 512 threads
  auto convert_x = [&](uint8_t* stage) __attribute__((always_inline)) {
#pragma unroll
    for (int i0 = 0; i0 < 16 * 16 * MS; i0 += QW * 64) {
      const int i = i0 + tid;
      if (i < 16 * 16 * MS) {
        const float f = sXinv[i >> 4];
        u32x4_t v = *(const u32x4_t*)(stage + i * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const _Float16 lo = (_Float16)(__uint_as_float(v[e] << 16) * f);
          const _Float16 hi = (_Float16)(__uint_as_float(v[e] & 0xffff0000u) * f);
          v[e] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
        }
        *(u32x4_t*)(stage + i * 16) = v;
      }
    }
  };
  auto load_w = [&](int kt, Q8Buf& wb) __attribute__((always_inline)) {
    const uint32_t so = (uint32_t)(kt * 136);
#pragma unroll
    for (int ct = 0; ct < QCT; ++ct) {
      wb.a[ct] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsW, wa[ct], so, 0));
      wb.b[ct] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsW, wa[ct] + 16, so, 0));
      wb.c[ct] = __builtin_amdgcn_raw_buffer_load_b32(rsW, wa[ct] + 32, so, 0);
    }
  };

  f32x4_t acc[QCT][MS];
#pragma unroll
  for (int ct = 0; ct < QCT; ++ct)
#pragma unroll
    for (int i = 0; i < MS; ++i) acc[ct][i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  bool big = false;  // a block scale that could overflow fp16

  // k-slots: MFMA slot s of lane quadrant q at k-step t reads k = 32q + 8t + s of the tile, i.e. x
  // chunk 4q + t and codes 8t .. 8t+7 of the lane's block.
  auto compute = [&](int kt, const uint8_t* stage, const Q8Buf& wb) __attribute__((always_inline)) {
    const bool kin = kt * QBK + 32 * q < kint;
    uint32_t cw[QCT][8];
    f16x2_t d2[QCT];
#pragma unroll
    for (int ct = 0; ct < QCT; ++ct) {
      // the word at byte 32 passes the end of the blocks only for the last block of all (sh = 0),
      // whose last two codes `tail` holds
      const uint32_t w8 = wa[ct] + (uint32_t)(kt * 136) + 36u > wend ? tail : wb.c[ct];
      const uint32_t w[9] = {wb.a[ct][0], wb.a[ct][1], wb.a[ct][2], wb.a[ct][3], wb.b[ct][0], wb.b[ct][1],
                             wb.b[ct][2], wb.b[ct][3], w8};
      const uint32_t sh = wsh[ct];  // 0 or 2: d at bytes sh, sh+1, codes from byte sh + 2
#pragma unroll
      for (int i = 0; i < 8; ++i)
        cw[ct][i] = (uint32_t)(((((uint64_t)w[i + 1]) << 32) | w[i]) >> (8 * (sh + 2)));
      const uint32_t db = kin ? (w[0] >> (8 * sh)) & 0xffffu : 0u;  // past K: d = 0
      big |= (db & 0x7fffu) > 0x5fffu;
      const _Float16 d = __builtin_bit_cast(_Float16, (uint16_t)db);
      d2[ct] = f16x2_t{d, d};
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4_t af[MS];
#pragma unroll
      for (int rt = 0; rt < MS; ++rt) {
        const int r = rt * 16 + j16;
        af[rt] = *(const u32x4_t*)(stage + (r * 16 + ((4 * q + t) ^ j16)) * 16);
      }
#pragma unroll
      for (int ct = 0; ct < QCT; ++ct) {
        uint32_t b0, b1, b2, b3;
        q8_dequant(cw[ct][2 * t], d2[ct], b0, b1);
        q8_dequant(cw[ct][2 * t + 1], d2[ct], b2, b3);
        const u32x4_t bf = {b0, b1, b2, b3};
#pragma unroll
        for (int rt = 0; rt < MS; ++rt) acc[ct][rt] = mfma16_f16(af[rt], bf, acc[ct][rt]);
      }
    }
  };

  Q8Buf wbr[QNS];
#if EXPERTS_Q8_CONV_AHEAD
  // One k-tile kt: wait until this wave's copies of x(kt + 1) have landed (and the weights of kt),
  // barrier (every wave's copies of x(kt + 1) are in LDS, and every wave is done with step kt - 1:
  // the products of kt - 1 and the conversion of x(kt)), copy x(kt + 2) into the stage kt - 1
  // freed, products of kt, convert x(kt + 1) in place while other waves issue their products,
  // load the weights of kt + 3 into the ring slot just consumed.  One barrier per k-tile; x is
  // copied one k-tile ahead of its conversion.
  auto step2 = [&](int kt, const uint8_t* cur, uint8_t* next, uint8_t* refill, Q8Buf& wb) __attribute__((always_inline)) {
    ex_wait_vmcnt<NW>();
    __builtin_amdgcn_s_barrier();
    copy_x(kt + 2 < KT ? kt + 2 : KT - 1, refill);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (kt < KT) compute(kt, cur, wb);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!XF16) {
      if (kt + 1 < KT) convert_x(next);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this thread's conversions are in LDS
      asm volatile("" ::: "memory");
    }
    __builtin_amdgcn_sched_barrier(0);
    load_w(kt + QNS < KT ? kt + QNS : KT - 1, wb);
    asm volatile("" ::: "memory");
  };
  copy_x(0, stg[0]);
  asm volatile("" ::: "memory");
  load_w(0, wbr[0]);
  asm volatile("" ::: "memory");
  copy_x(1 < KT ? 1 : KT - 1, stg[1]);
  asm volatile("" ::: "memory");
  load_w(1 < KT ? 1 : KT - 1, wbr[1]);
  load_w(2 < KT ? 2 : KT - 1, wbr[2]);
  asm volatile("" ::: "memory");
  ex_wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();  // x(0) of every wave is in LDS
  if constexpr (!XF16) {
    convert_x(stg[0]);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);
    asm volatile("" ::: "memory");
  }
#pragma unroll
  for (int j = 0; j < QNS; ++j) step2(j, stg[j], stg[(j + 1) % QNS], stg[(j + 2) % QNS], wbr[j]);
  for (int kt = QNS; kt < KT; kt += QNS) {
#pragma unroll
    for (int j = 0; j < QNS; ++j) step2(kt + j, stg[j], stg[(j + 1) % QNS], stg[(j + 2) % QNS], wbr[j]);
  }
#else
  // One k-tile: wait for its x copies and weights, barrier (every wave is done with the stage the
  // copies below refill), copy x of kt + QNS - 1, convert this tile's x, barrier, compute, load the
  // weights of kt + QNS into the ring slot just consumed.  Steps past the last tile (completing a
  // round) load clamped tiles and compute nothing.
  auto step = [&](int kt, uint8_t* cur, uint8_t* refill, Q8Buf& wb) __attribute__((always_inline)) {
    ex_wait_vmcnt<L>();
    __builtin_amdgcn_s_barrier();
    copy_x(kt + QNS - 1 < KT ? kt + QNS - 1 : KT - 1, refill);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (!XF16) {  // fp16 x is staged as it is
      if (kt < KT) convert_x(cur);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this thread's conversions are in LDS
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kt < KT) compute(kt, cur, wb);
    __builtin_amdgcn_sched_barrier(0);
    load_w(kt + QNS < KT ? kt + QNS : KT - 1, wb);
    asm volatile("" ::: "memory");
  };

#pragma unroll
  for (int t = 0; t < QNS - 1; ++t) {
    copy_x(t < KT ? t : KT - 1, stg[t]);
    asm volatile("" ::: "memory");
    load_w(t < KT ? t : KT - 1, wbr[t]);
    asm volatile("" ::: "memory");
  }
  load_w(QNS - 1 < KT ? QNS - 1 : KT - 1, wbr[QNS - 1]);
  asm volatile("" ::: "memory");
#pragma unroll
  for (int j = 0; j < QNS; ++j) step(j, stg[j], stg[(j + QNS - 1) % QNS], wbr[j]);
  for (int kt = QNS; kt < KT; kt += QNS) {
#pragma unroll
    for (int j = 0; j < QNS; ++j) step(kt + j, stg[j], stg[(j + QNS - 1) % QNS], wbr[j]);
  }
#endif
  ex_wait_vmcnt<0>();  // no copy may still be writing LDS
  if (big) *sFlag = 1;
  __syncthreads();     // every wave is done with the stages: stage 0 now holds the output blocks

  // store: lane holds weight row ncol0 + 16 ct for positions 4q + r of each m-subtile, times the
  // position's x row factor; through LDS as in experts_mx.hip when y rows are 16-byte aligned
  const int esz = ydt == DT_F32 ? 4 : 2;
  if (N % 8 == 0 && ((uintptr_t)y & 15) == 0) {
    uint8_t* wbuf = stg[0] + wave * 2048;
    const int rb = 32 * esz;           // bytes of a staged row (32 columns)
    const int nch = 16 * rb / 16;      // 16-byte chunks of a block: 64 or 128
    const int64_t col0 = ncol0 - j16;  // the wave's first column
#pragma unroll
    for (int rt = 0; rt < MS; ++rt) {
#pragma unroll
      for (int ct = 0; ct < QCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          uint8_t* dst = wbuf + (4 * q + r) * rb + (16 * ct + j16) * esz;
          const float v = acc[ct][rt][r] * sXs[rt * 16 + 4 * q + r];
          if (esz == 4)
            *(float*)dst = v;
          else
            *(uint16_t*)dst = (uint16_t)(ydt == DT_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v));
        }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the block is in LDS for every lane
      asm volatile("" ::: "memory");
      for (int i = lane; i < nch; i += 64) {
        const int row = i / (rb / 16), c = i - row * (rb / 16);
        const int rr = rt * 16 + row;
        const int64_t col = col0 + c * (16 / esz);
        if (rr < rows && col < N)
          *(u32x4_t*)((uint8_t*)y + ((int64_t)sPos[rr] * N + col) * esz) = *(const u32x4_t*)(wbuf + i * 16);
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xc07f);  // the reads are done before the next block is written
      asm volatile("" ::: "memory");
    }
  } else {
#pragma unroll
    for (int ct = 0; ct < QCT; ++ct) {
      const int64_t ncol = ncol0 + 16 * ct;
      if (ncol >= N) continue;
#pragma unroll
      for (int rt = 0; rt < MS; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = rt * 16 + 4 * q + r;
          if (rr < rows) store_out(y, (int64_t)sPos[rr] * N + ncol, acc[ct][rt][r] * sXs[rr], ydt);
        }
    }
  }
}

template <bool XF16>
__global__ __launch_bounds__(512, 1) void experts_q8_kernel(const uint8_t* __restrict__ blocks, int64_t e, int64_t N,
                                                            int64_t K, const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ perm_pos,
                                                            const int32_t* __restrict__ order,
                                                            const float* __restrict__ xfac,
                                                            const uint16_t* __restrict__ x, int64_t x_rows,
                                                            int64_t pos_per_row, void* __restrict__ y, int ydt) {
  static_assert(QNS == 3, "the stage arrays below");
  __shared__ __attribute__((aligned(16))) uint8_t st0[QMC * QBK * 2];
  __shared__ __attribute__((aligned(16))) uint8_t st1[QMC * QBK * 2];
  __shared__ __attribute__((aligned(16))) uint8_t st2[QMC * QBK * 2];
  __shared__ int32_t sPos[QMC];
  __shared__ float sXinv[QMC], sXs[QMC];
  __shared__ int sFlag;
  uint8_t* const stg[QNS] = {st0, st1, st2};

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j16 = lane & 15;
  const int64_t n_tiles = (N + QBN - 1) / QBN;
  const int64_t rank = blockIdx.x / n_tiles;
  const int64_t nt = blockIdx.x - rank * n_tiles;
  const int64_t ex = order[rank];
  const int32_t off = offsets[ex];
  const int32_t cnt = offsets[ex + 1] - off;
  if (cnt <= 0) return;

  const int64_t row_bytes = (K / 32) * 34;
  const __amdgpu_buffer_rsrc_t rsX = ex_rsrc(x, x_rows * K * 2);
  const __amdgpu_buffer_rsrc_t rsW = ex_rsrc(blocks, e * N * row_bytes);
  // the last two code bytes of all blocks (an aligned word past the end would read zero)
  const uint32_t wend = (uint32_t)(e * N * row_bytes);
  const uint32_t tail = __builtin_amdgcn_raw_buffer_load_b16(rsW, wend - 2u, 0, 0);
  // this lane's weight rows (ncol0 + 16 ct; past N the last row stands in): the aligned word at or
  // below its block in the first k-tile, and the block's offset in it
  const int64_t ncol0 = nt * QBN + wave * (16 * QCT) + j16;
  uint32_t wa[QCT], wsh[QCT];
#pragma unroll
  for (int ct = 0; ct < QCT; ++ct) {
    const int64_t wrow = ex * N + min(ncol0 + 16 * ct, N - 1);
    const int64_t o = wrow * row_bytes + 34 * (lane >> 4);
    wa[ct] = (uint32_t)(o & ~(int64_t)3);
    wsh[ct] = (uint32_t)(o & 3);
  }
  for (int32_t mc = 0; mc < cnt; mc += QMC) {
    const int rows = min(QMC, cnt - mc);
    __syncthreads();  // previous chunk's readers of sPos and of the stages are done
    if (tid < QMC) {
      const int32_t pos = tid < rows ? perm_pos[off + mc + tid] : perm_pos[off + mc];
      sPos[tid] = tid < rows ? pos : -1;
      sXinv[tid] = XF16 ? 1.0f : xfac[2 * (pos / pos_per_row)];
      sXs[tid] = XF16 ? 1.0f : xfac[2 * (pos / pos_per_row) + 1];
    }
    if (tid == 0) sFlag = 0;
    __syncthreads();
    switch ((rows + 15) >> 4) {
#define QL_Q8_CASE(ms)                                                                                             \
  case ms:                                                                                                         \
    q8_chunk<ms, XF16>(sPos, sXinv, sXs, &sFlag, rows, stg, rsX, rsW, K, N, ncol0, wa, wsh, wend, tail, pos_per_row, y, \
                       ydt);                                                                                        \
    break;
      QL_Q8_CASE(1)
      QL_Q8_CASE(2)
      QL_Q8_CASE(3)
      QL_Q8_CASE(4)
      QL_Q8_CASE(5)
      default:
        q8_chunk<6, XF16>(sPos, sXinv, sXs, &sFlag, rows, stg, rsX, rsW, K, N, ncol0, wa, wsh, wend, tail, pos_per_row, y,
                          ydt);
        break;
#undef QL_Q8_CASE
    }
    __syncthreads();
    if (sFlag) {
      // a block scale beyond the fp16 range of d * q: these outputs again, in fp32 from the blocks
      for (int i = tid; i < rows * QBN; i += QW * 64) {
        const int rr = i / QBN;
        const int64_t col = nt * QBN + (i - rr * QBN);
        if (col >= N) continue;
        const uint8_t* wr = blocks + (ex * N + col) * row_bytes;
        const uint16_t* xr = x + (int64_t)(sPos[rr] / pos_per_row) * K;
        float acc = 0.0f;
        for (int64_t b = 0; b < K / 32; ++b) {
          const uint8_t* blk = wr + 34 * b;
          float part = 0.0f;
          for (int jj = 0; jj < 32; ++jj)
            part = __builtin_fmaf(XF16 ? f16_bits_to_f32(xr[32 * b + jj]) : bf16_bits_to_f32(xr[32 * b + jj]),
                                  (float)(int8_t)blk[2 + jj], part);
          acc = __builtin_fmaf(f16_bits_to_f32((uint32_t)blk[0] | ((uint32_t)blk[1] << 8)), part, acc);
        }
        store_out(y, (int64_t)sPos[rr] * N + col, acc, ydt);
      }
    }
  }
}

}  // namespace

hipError_t launch_experts_q8(const uint8_t* blocks, int64_t e, int64_t n, int64_t k, const int32_t* offsets,
                             const int32_t* perm, const int32_t* order, const float* xfac, const uint16_t* x,
                             int xdt, int64_t x_rows, int64_t pos_per_row, void* y, int ydt, hipStream_t s) {
  const int64_t grid = e * ((n + QBN - 1) / QBN);
  if (xdt == DT_F16)
    experts_q8_kernel<true><<<(unsigned)grid, QW * 64, 0, s>>>(blocks, e, n, k, offsets, perm, order, nullptr, x,
                                                                x_rows, pos_per_row, y, ydt);
  else
    experts_q8_kernel<false><<<(unsigned)grid, QW * 64, 0, s>>>(blocks, e, n, k, offsets, perm, order, xfac, x, x_rows,
                                                                 pos_per_row, y, ydt);
  return hipGetLastError();
}

}  // namespace ql
