// Routed apply for MXFP4 experts (Nx_quant API docs, Products: apply_experts; Nx_quant Weights:
// MXFP4): y[p, :] = x[p / pos_per_row, :] . W_{ids[p]}^T in fp32, the codes decoded while summing.
// The routing (offsets, permutation and expert order) is computed by experts.hip.
//
// MXFP4 in GGUF's blocks (Nx_quant Weights, Mxfp4_blocks: per 32 values the scale byte, then 16
// bytes, byte j holding value j in its low nibble and value j + 16 in its high one) takes the same
// kernel (BLK): each lane reads the 17-byte block from the aligned 20-byte window around it,
// takes the scale byte and regroups the nibbles into the split layout's order (byte i holding
// values 2i and 2i + 1), then decodes as above.
#include "experts_common.hpp"

namespace ql {
namespace {
using namespace ex_detail;

// ---------------------------------------------------------------- MXFP4, 48 weight rows per wave
//
// One workgroup of 8 waves per (expert, 384 weight rows), taken in decreasing order of the experts'
// position counts; wave w owns three column tiles of 16 weight rows and all the chunk's positions
// (up to 96: MS m-subtiles of 16), and multiplies with v_mfma_f32_16x16x32_bf16 (lane l: row or
// column l%16, k-slots 8*(l/16)..+7; D: column l%16, rows 4*(l/16)..+3), so that every x fragment
// read from LDS feeds three products and every decoded code fragment MS.  k-tiles are 128 wide: a
// lane reads 16 bytes (one 32-value block) of its row per tile, and the four lanes of a row read 64
// consecutive bytes, half a cache line, in one instruction.  The gathered x rows go straight into
// XNS LDS stages, XNS - 1 k-tiles ahead, shared by the 8 waves; each lane's code words go into a
// ring of XNS register buffers, XNS k-tiles ahead (one in-order counter, as in experts_kernel).
// The workgroup's scale bytes (all k) are read once into LDS, coalesced, when they fit
// (SCL_LDS); otherwise each lane loads its block's byte with its codes.
#ifndef EXPERTS_MX_MC
#define EXPERTS_MX_MC 96  // positions per chunk (a multiple of 16, at most 96)
#endif
#ifndef EXPERTS_MX_SCL_MAX
#define EXPERTS_MX_SCL_MAX (48 * 1024)  // LDS bytes for the staged scale bytes
#endif
#ifndef EXPERTS_MX_SCL16
#define EXPERTS_MX_SCL16 1  // stage the scale bytes 16 per lane (else 4)
#endif
#ifndef EXPERTS_MX_MINB
#define EXPERTS_MX_MINB 1  // workgroups per compute unit the register allocation must allow
#endif
constexpr int XBK = 128, XMC = EXPERTS_MX_MC, XCT = 3, XW = 8, XBN = XW * 16 * XCT, XNS = 3;
constexpr int XSCL_MAX = EXPERTS_MX_SCL_MAX;

struct MxBuf {
  u32x4_t c[XCT];   // this lane's 32 codes (block 4 kt + q of its row), per column tile; BLK: the
                    // first 16 bytes of the aligned window holding the block
  uint32_t s[XCT];  // that block's scale byte (per-lane loads only); BLK: the window's last word
};

// GGUF block -> split layout: from the 20-byte window w (block at byte sh, 0 <= sh < 4) the scale
// byte and the code words of the split layout (word t: values 8t .. 8t + 7, byte i of it holding
// values 8t + 2i and 8t + 2i + 1 in its low and high nibble).  The block's byte j (j < 16) holds
// values j and j + 16, so words 0 and 1 gather low nibbles, words 2 and 3 high ones.
__device__ __forceinline__ void gguf_block_to_split(const u32x4_t& w03, uint32_t w4, uint32_t sh, uint32_t& scale,
                                                    u32x4_t& codes) {
  const uint32_t w[5] = {w03[0], w03[1], w03[2], w03[3], w4};
  scale = (w[0] >> (8 * sh)) & 0xffu;
  uint32_t b[4];  // block bytes 1 .. 16 as four words
#pragma unroll
  for (int t = 0; t < 4; ++t) b[t] = (uint32_t)(((((uint64_t)w[t + 1]) << 32) | w[t]) >> (8 * (sh + 1)));
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    // nibbles of bytes 8 (t % 2) .. + 7: low ones for t < 2, high ones for t >= 2
    const int sft = t < 2 ? 0 : 4;
    const uint32_t n0 = (b[2 * (t & 1)] >> sft) & 0x0f0f0f0fu, n1 = (b[2 * (t & 1) + 1] >> sft) & 0x0f0f0f0fu;
    // pairs of neighbouring nibbles into one byte: bytes 0 and 2 of (n | n >> 4)
    const uint32_t p0 = n0 | (n0 >> 4), p1 = n1 | (n1 >> 4);
    codes[t] = perm(p1, p0, 0x06040200u);
  }
}

__device__ __forceinline__ f32x4_t mfma16_bf16(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Output block of one chunk: lane holds weight row ncol0 + 16 ct (column j16 of its tile) for
// positions 4q + r of each m-subtile.  When every y row is 16-byte aligned (N a multiple of 8), each
// m-subtile goes through this wave's 3 KB of stage 0 (16 positions x 48 columns) so that every lane
// writes 16 contiguous bytes of one y row (y 16-byte aligned); otherwise element by element.
// ESZ = bytes per output element.
template <int MS, int ESZ>
__device__ __forceinline__ void mx_store(const f32x4_t (&acc)[XCT][MS], const int32_t* __restrict__ sPos, int rows,
                                         uint8_t* const* stg, int64_t N, int64_t ncol0, void* __restrict__ y,
                                         int ydt) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j16 = lane & 15, q = lane >> 4;
  auto bits = [&](float v) __attribute__((always_inline)) {
    return (uint32_t)(ydt == DT_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v));
  };
  if (N % 8 == 0 && ((uintptr_t)y & 15) == 0) {
    // 3 KB per wave: in stage 0, and in stage 1 for the waves that stage 0 cannot hold
    constexpr int kStageBytes = XMC * XBK * 2, kFit = kStageBytes / 3072;
    uint8_t* wbuf = wave < kFit ? stg[0] + wave * 3072 : stg[1] + (wave - kFit) * 3072;
    constexpr int rb = 48 * ESZ;          // bytes of a staged row
    constexpr int nch = 16 * rb / 16;     // 16-byte chunks of a block: 96 or 192
    const int64_t col0 = ncol0 - j16;     // the wave's first column
#pragma unroll
    for (int rt = 0; rt < MS; ++rt) {
#pragma unroll
      for (int ct = 0; ct < XCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          uint8_t* dst = wbuf + (4 * q + r) * rb + (16 * ct + j16) * ESZ;
          if constexpr (ESZ == 4)
            *(float*)dst = acc[ct][rt][r];
          else
            *(uint16_t*)dst = (uint16_t)bits(acc[ct][rt][r]);
        }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the block is in LDS for every lane
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i0 = 0; i0 < nch; i0 += 64) {
        const int i = i0 + lane;
        const int row = i / (rb / 16), c = i - row * (rb / 16);
        const int rr = rt * 16 + row;
        const int64_t col = col0 + c * (16 / ESZ);
        if (i < nch && rr < rows && col < N)
          *(u32x4_t*)((uint8_t*)y + ((int64_t)sPos[rr] * N + col) * ESZ) = *(const u32x4_t*)(wbuf + i * 16);
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xc07f);  // the reads are done before the next block is written
      asm volatile("" ::: "memory");
    }
  } else {
#pragma unroll
    for (int ct = 0; ct < XCT; ++ct) {
      const int64_t ncol = ncol0 + 16 * ct;
      if (ncol >= N) continue;
#pragma unroll
      for (int rt = 0; rt < MS; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = rt * 16 + 4 * q + r;
          if (rr < rows) {
            uint8_t* p = (uint8_t*)y + ((int64_t)sPos[rr] * N + ncol) * ESZ;
            if constexpr (ESZ == 4)
              *(float*)p = acc[ct][rt][r];
            else
              *(uint16_t*)p = (uint16_t)bits(acc[ct][rt][r]);
          }
        }
    }
  }
}

// 8 fp16 values (one x fragment) -> bf16 fragments hi and lo with hi + lo equal to them exactly: hi
// keeps the top 8 significant bits of each (its fp32 pattern cut to 16 bits), lo = x - hi holds the
// other 3 at most, exact in bf16 (fp16's exponent range lies inside bf16's).
__device__ __forceinline__ void split_f16(const u32x4_t& v, u32x4_t& hi, u32x4_t& lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float f0 = f16_bits_to_f32(v[e] & 0xffffu), f1 = f16_bits_to_f32(v[e] >> 16);
    const uint32_t h0 = __float_as_uint(f0) & 0xffff0000u, h1 = __float_as_uint(f1) & 0xffff0000u;
    const uint32_t l0 = __float_as_uint(f0 - __uint_as_float(h0)), l1 = __float_as_uint(f1 - __uint_as_float(h1));
    hi[e] = (h0 >> 16) | h1;
    lo[e] = (l0 >> 16) | (l1 & 0xffff0000u);
  }
}

// x stage: row r holds 16 chunks of 8 values (k-tile 128), chunk c at slot c ^ (r % 16), so that the
// 16 rows of one fragment read hit 16 distinct bank groups.  fp16 x (XF16) is staged as it is and
// each fragment goes through the products twice, as its bf16 hi and lo parts.
template <int MS, bool SCL_LDS, bool XF16, bool BLK>
__device__ __forceinline__ void mx_chunk(const int32_t* __restrict__ sPos, int rows, uint8_t* const* stg,
                                         const uint8_t* __restrict__ sScl, __amdgpu_buffer_rsrc_t rsX,
                                         __amdgpu_buffer_rsrc_t rsW, __amdgpu_buffer_rsrc_t rsS, int64_t K, int64_t N,
                                         int64_t ncol0, const uint32_t* wo, const uint32_t* so, int64_t pos_per_row,
                                         void* __restrict__ y, int ydt) {
  constexpr int CPW = (MS + 1) / 2;                // x copies per wave and k-tile (32 rows per copy round)
  constexpr int NW = BLK ? 5 * XCT : (SCL_LDS ? XCT : 2 * XCT);  // weight loads per lane and k-tile
  constexpr int L = NW + (XNS - 2) * (CPW + NW);  // loads issued after x(kt) when kt is due
  static_assert(L < 64, "vmcnt range");
  // the copies of a k-tile (1 KB each, at (XW i + w) KB) stay inside one stage, the output blocks (3 KB
  // per wave) inside stages 0 and 1
  static_assert(XW * CPW * 1024 <= XMC * XBK * 2, "x copies past the stage");
  static_assert(XW * 3072 <= 2 * XMC * XBK * 2, "output blocks past stages 0 and 1");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j16 = lane & 15, q = lane >> 4;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int KT = (int)((K + XBK - 1) / XBK);
  const int kint = (int)K;

  // x copies: copy i (0..CPW-1) of wave w covers chunk rows (8i + w)*4 .. +3; lane l -> row + l/16,
  // slot l%16 (chunk (l%16) ^ (row % 16)).  Rows past the chunk copy its first position (never
  // stored).
  uint32_t xoff[CPW];
  int xc[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int r = (XW * i + wave) * 4 + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    const int32_t pos = sPos[r < rows ? r : 0];
    xoff[i] = (uint32_t)(((int64_t)(pos / pos_per_row) * K + 8 * c) * 2);
    xc[i] = c;
  }
  auto copy_x = [&](int kt, uint8_t* stage) __attribute__((always_inline)) {
    const int k0 = kt * XBK;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const uint32_t v = k0 + 8 * xc[i] < kint ? xoff[i] : kExOOB;  // zeros past K
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsX, (lds_void*)(stage + (XW * i + wave_u) * 1024), 16, v,
                                               (uint32_t)(k0 * 2), 0, 0);
    }
  };
  auto load_w = [&](int kt, MxBuf& wb) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < XCT; ++ct) {
      if constexpr (BLK) {
        // the aligned 20-byte window of block 4 kt + q (4 blocks = 68 bytes per k-tile, so the block's
        // place in its window is the same on every tile): wo = window offset in tile 0, so = place;
        // the word that the end of all blocks cuts is rebuilt from bytes (sScl holds it, see below)
#pragma unroll
        for (int i = 0; i < 5; ++i) {
          const uint32_t a = wo[ct] + (uint32_t)(kt * 68) + 4u * i;
          uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(rsW, a, 0, 0);
          if (a == *(const uint32_t*)sScl) v = *(const uint32_t*)(sScl + 4);
          if (i < 4)
            wb.c[ct][i] = v;
          else
            wb.s[ct] = v;
        }
      } else {
        wb.c[ct] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsW, wo[ct], (uint32_t)(kt * 64), 0));
        if constexpr (!SCL_LDS) wb.s[ct] = __builtin_amdgcn_raw_buffer_load_b8(rsS, so[ct], (uint32_t)(kt * 4), 0);
      }
    }
  };

  f32x4_t acc[XCT][MS];
#pragma unroll
  for (int ct = 0; ct < XCT; ++ct)
#pragma unroll
    for (int i = 0; i < MS; ++i) acc[ct][i] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // k-slots: MFMA slot s of lane quadrant q at k-step t reads k = 32q + 8t + s of the tile, i.e.
  // x chunk 4q + t and code word t of the lane's 16 bytes.
  auto compute = [&](int kt, const uint8_t* stage, const MxBuf& wb) __attribute__((always_inline)) {
    // the block scale 2^(s-127) as fp32 (s = 0: the subnormal 2^-127), NaN for s = 255, 0 past K
    const bool kin = kt * XBK + 32 * q < kint;
    float scl[XCT];
    u32x4_t cw[XCT];
#pragma unroll
    for (int ct = 0; ct < XCT; ++ct) {
      uint32_t sb;
      if constexpr (BLK)
        gguf_block_to_split(wb.c[ct], wb.s[ct], so[ct], sb, cw[ct]);
      else if constexpr (SCL_LDS)
        sb = sScl[so[ct] + 4 * kt];
      else
        sb = wb.s[ct] & 0xffu;
      if constexpr (!BLK) cw[ct] = wb.c[ct];
      scl[ct] = !kin ? 0.0f : __uint_as_float(sb == 255u ? 0x7fc00000u : (sb == 0u ? 0x00400000u : sb << 23));
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      u32x4_t af[MS], al[XF16 ? MS : 1];
#pragma unroll
      for (int rt = 0; rt < MS; ++rt) {
        const int r = rt * 16 + j16;
        af[rt] = *(const u32x4_t*)(stage + (r * 16 + ((4 * q + t) ^ j16)) * 16);
        if constexpr (XF16) split_f16(af[rt], af[rt], al[rt]);
      }
#pragma unroll
      for (int ct = 0; ct < XCT; ++ct) {
        const u32x4_t bf = decode_mxfp4(cw[ct][t], scl[ct]);
#pragma unroll
        for (int rt = 0; rt < MS; ++rt) {
          acc[ct][rt] = mfma16_bf16(af[rt], bf, acc[ct][rt]);
          if constexpr (XF16) acc[ct][rt] = mfma16_bf16(al[rt], bf, acc[ct][rt]);
        }
      }
    }
  };

  MxBuf wbr[XNS];
  // One k-tile: wait for its x copies and weights, barrier (every wave is done with the stage the
  // copies below refill), copy x of kt + XNS - 1, compute, load the weights of kt + XNS into the
  // ring slot just consumed.  Steps past the last tile (completing a round) load clamped tiles and
  // compute nothing.
  auto step = [&](int kt, const uint8_t* cur, uint8_t* refill, MxBuf& wb) __attribute__((always_inline)) {
    ex_wait_vmcnt<L>();
    __builtin_amdgcn_s_barrier();
    copy_x(kt + XNS - 1 < KT ? kt + XNS - 1 : KT - 1, refill);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (kt < KT) compute(kt, cur, wb);
    __builtin_amdgcn_sched_barrier(0);
    load_w(kt + XNS < KT ? kt + XNS : KT - 1, wb);
    asm volatile("" ::: "memory");
  };

#pragma unroll
  for (int t = 0; t < XNS - 1; ++t) {
    copy_x(t < KT ? t : KT - 1, stg[t]);
    asm volatile("" ::: "memory");
    load_w(t < KT ? t : KT - 1, wbr[t]);
    asm volatile("" ::: "memory");
  }
  load_w(XNS - 1 < KT ? XNS - 1 : KT - 1, wbr[XNS - 1]);
  asm volatile("" ::: "memory");
#pragma unroll
  for (int j = 0; j < XNS; ++j) step(j, stg[j], stg[(j + XNS - 1) % XNS], wbr[j]);
  for (int kt = XNS; kt < KT; kt += XNS) {
#pragma unroll
    for (int j = 0; j < XNS; ++j) step(kt + j, stg[j], stg[(j + XNS - 1) % XNS], wbr[j]);
  }
  ex_wait_vmcnt<0>();  // no copy may still be writing LDS
  __syncthreads();     // every wave is done with the stages: stages 0 and 1 now hold the output blocks

  // store: the output dtype is dispatched once, outside the loops
  if (ydt == DT_F32)
    mx_store<MS, 4>(acc, sPos, rows, stg, N, ncol0, y, DT_F32);
  else if (ydt == DT_BF16)
    mx_store<MS, 2>(acc, sPos, rows, stg, N, ncol0, y, DT_BF16);
  else
    mx_store<MS, 2>(acc, sPos, rows, stg, N, ncol0, y, DT_F16);
}

// The chunk's m-subtile count as a template argument: the smallest MS >= rows / 16.
template <int MS, bool SCL_LDS, bool XF16, bool BLK>
__device__ __forceinline__ void mx_chunks(const int32_t* __restrict__ sPos, int rows, uint8_t* const* stg,
                                          const uint8_t* __restrict__ sScl, __amdgpu_buffer_rsrc_t rsX,
                                          __amdgpu_buffer_rsrc_t rsW, __amdgpu_buffer_rsrc_t rsS, int64_t K,
                                          int64_t N, int64_t ncol0, const uint32_t* wo, const uint32_t* so,
                                          int64_t pos_per_row, void* __restrict__ y, int ydt) {
  if constexpr (MS < XMC / 16) {
    if (rows > 16 * MS) {
      mx_chunks<MS + 1, SCL_LDS, XF16, BLK>(sPos, rows, stg, sScl, rsX, rsW, rsS, K, N, ncol0, wo, so, pos_per_row, y,
                                            ydt);
      return;
    }
  }
  mx_chunk<MS, SCL_LDS, XF16, BLK>(sPos, rows, stg, sScl, rsX, rsW, rsS, K, N, ncol0, wo, so, pos_per_row, y, ydt);
}

template <bool SCL_LDS, bool XF16, bool BLK>
__global__ __launch_bounds__(512, EXPERTS_MX_MINB) void experts_mx_kernel(const uint8_t* __restrict__ codes,
                                                            const uint8_t* __restrict__ scales, int64_t e, int64_t N,
                                                            int64_t K, const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ perm_pos,
                                                            const int32_t* __restrict__ order,
                                                            const uint16_t* __restrict__ x, int64_t x_rows,
                                                            int64_t pos_per_row, void* __restrict__ y, int ydt) {
  static_assert(XNS == 3, "the stage arrays below");
  __shared__ __attribute__((aligned(16))) uint8_t st0[XMC * XBK * 2];
  __shared__ __attribute__((aligned(16))) uint8_t st1[XMC * XBK * 2];
  __shared__ __attribute__((aligned(16))) uint8_t st2[XMC * XBK * 2];
  __shared__ int32_t sPos[XMC];
  extern __shared__ uint32_t sScl32[];  // the scale bytes of the workgroup's rows (SCL_LDS)
  uint8_t* const stg[XNS] = {st0, st1, st2};

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int j16 = lane & 15;
  const int64_t n_tiles = (N + XBN - 1) / XBN;
  const int64_t rank = blockIdx.x / n_tiles;
  const int64_t nt = blockIdx.x - rank * n_tiles;
  const int64_t ex = order[rank];
  const int32_t off = offsets[ex];
  const int32_t cnt = offsets[ex + 1] - off;
  if (cnt <= 0) return;

  const __amdgpu_buffer_rsrc_t rsX = ex_rsrc(x, x_rows * K * 2);
  const int64_t wtotal = BLK ? e * N * (K / 32) * 17 : e * N * (K / 2);
  const __amdgpu_buffer_rsrc_t rsW = ex_rsrc(codes, wtotal);
  const __amdgpu_buffer_rsrc_t rsS = ex_rsrc(scales, BLK ? 0 : e * N * (K / 32));
  // this lane's weight rows of the expert, one per column tile (ncol0 + 16 ct; past N the last row
  // stands in): byte offsets of its 16 code bytes in the first k-tile, and of its block's scale
  // byte (in the staged LDS copy, or in the scales array)
  const int64_t ncol0 = nt * XBN + wave * (16 * XCT) + j16;
  const int64_t sbase = (ex * N + nt * XBN) * (K / 32);  // first scale byte of the workgroup's rows
  const int ssh = (int)(sbase & 3);
  uint32_t wo[XCT], so[XCT];
#pragma unroll
  for (int ct = 0; ct < XCT; ++ct) {
    const int64_t wrow = ex * N + min(ncol0 + 16 * ct, N - 1);
    if constexpr (BLK) {  // the aligned window of block q of the row, and the block's place in it
      const int64_t o = wrow * (K / 32) * 17 + 17 * (lane >> 4);
      wo[ct] = (uint32_t)(o & ~(int64_t)3);
      so[ct] = (uint32_t)(o & 3);
    } else {
      wo[ct] = (uint32_t)(wrow * (K / 2) + 16 * (lane >> 4));
      so[ct] = SCL_LDS ? (uint32_t)(ssh + (wrow - ex * N - nt * XBN) * (K / 32) + (lane >> 4))
                       : (uint32_t)(wrow * (K / 32) + (lane >> 4));
    }
  }
  if constexpr (BLK) {
    // the word that the end of all blocks cuts (a word load past the end reads zero): its offset
    // and its bytes, for load_w; 0xffffffff when the blocks end on a word boundary
    if (tid == 0) {
      uint32_t a = 0xffffffffu, w = 0u;
      if (wtotal & 3) {
        a = (uint32_t)(wtotal & ~(int64_t)3);
        for (int i = 0; i < (int)(wtotal & 3); ++i) w |= __builtin_amdgcn_raw_buffer_load_b8(rsW, a + i, 0, 0) << (8 * i);
      }
      sScl32[0] = a;
      sScl32[1] = w;
    }
  }
  if constexpr (SCL_LDS) {
    // rows of the tile that exist, K/32 bytes each, from the aligned word at or below the first:
    // copied HBM -> LDS by DMA, 64 words per wave instruction, all in flight at once (a load-store
    // loop through registers would wait out one round trip per pass); the chunk loop's first
    // barrier, after the wait below, publishes them
    const int64_t live = min((int64_t)XBN, N - nt * XBN);
    const uint32_t a0 = (uint32_t)(sbase - ssh);
    if (EXPERTS_MX_SCL16) {
      // 16 bytes per lane: the last chunk may copy up to 15 bytes past the tile's scale bytes into
      // the rest of the 1 KB-rounded allocation (bytes past every scale read zero)
      const int nd = (int)((ssh + live * (K / 32) + 15) / 16);
      for (int i0 = wave * 64; i0 < nd; i0 += XW * 64)
        if (i0 + lane < nd)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsS, (lds_void*)(sScl32 + 4 * i0), 16, a0 + 16u * (i0 + lane), 0, 0,
                                                   0);
    } else {
      const int nd = (int)((ssh + live * (K / 32) + 3) / 4);
      for (int i0 = wave * 64; i0 < nd; i0 += XW * 64)
        if (i0 + lane < nd)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rsS, (lds_void*)(sScl32 + i0), 4, a0 + 4u * (i0 + lane), 0, 0, 0);
    }
    ex_wait_vmcnt<0>();
  }
  const uint8_t* sScl = (const uint8_t*)sScl32;
  for (int32_t mc = 0; mc < cnt; mc += XMC) {
    const int rows = min(XMC, cnt - mc);
    __syncthreads();  // previous chunk's readers of sPos are done (and the scale bytes are staged)
    if (tid < XMC) sPos[tid] = tid < rows ? perm_pos[off + mc + tid] : -1;
    __syncthreads();
    mx_chunks<1, SCL_LDS, XF16, BLK>(sPos, rows, stg, sScl, rsX, rsW, rsS, K, N, ncol0, wo, so, pos_per_row, y, ydt);
  }
}

}  // namespace

hipError_t launch_experts_mx(const uint8_t* codes, const uint8_t* scales, int64_t e, int64_t n, int64_t k,
                             const int32_t* offsets, const int32_t* perm, const int32_t* order, const uint16_t* x,
                             int xdt, int64_t x_rows, int64_t pos_per_row, void* y, int ydt, hipStream_t s) {
  const unsigned grid = (unsigned)(e * ((n + XBN - 1) / XBN));
  // the staged scale bytes (from the aligned word at or below the first), rounded up to whole
  // 1 KB copies when they are copied 16 bytes per lane
  const size_t scl = EXPERTS_MX_SCL16 ? (size_t)((3 + XBN * (k / 32) + 1023) / 1024 * 1024)
                                      : (size_t)((3 + XBN * (k / 32) + 3) / 4 * 4);
  const bool blk = scales == nullptr;  // GGUF blocks: codes holds the 17-byte blocks
  const bool in_lds = !blk && scl <= (size_t)XSCL_MAX;
  const bool h = xdt == DT_F16;
#define QL_MX_LAUNCH(L, H, B)                                                                                       \
  experts_mx_kernel<L, H, B><<<grid, XW * 64, L ? scl : (B ? 8 : 0), s>>>(codes, scales, e, n, k, offsets, perm,    \
                                                                          order, x, x_rows, pos_per_row, y, ydt)
  if (blk && h)
    QL_MX_LAUNCH(false, true, true);
  else if (blk)
    QL_MX_LAUNCH(false, false, true);
  else if (in_lds && h)
    QL_MX_LAUNCH(true, true, false);
  else if (in_lds)
    QL_MX_LAUNCH(true, false, false);
  else if (h)
    QL_MX_LAUNCH(false, true, false);
  else
    QL_MX_LAUNCH(false, false, false);
#undef QL_MX_LAUNCH
  return hipGetLastError();
}

}  // namespace ql
