// Routing and routed apply (Nx_quant API docs, Products: apply_experts): each position's x row
// through the expert its id names, zeros for ids out of [0, e), a row's bits independent of the
// other positions' experts.  Weights in MXFP4 (codes + E8M0 scales apart) or Q8_0 blocks
// (Nx_quant Weights), decoded while summing (no stored decoded weight).
//
// route_kernel: workgroup j counts all ids in LDS (its offset and the experts' order by count),
// then writes the positions with id j in increasing order: a stable counting sort, identical on
// every run.
//
// experts_kernel: one workgroup per (expert, 128 weight rows); its 4 waves own 32 weight rows
// each and loop over the expert's positions in chunks of up to 96 (m-subtiles of 32) and over k
// in tiles of 64.  The gathered x rows go straight from memory into five LDS stages four k-tiles
// ahead (shared by the waves); each lane loads its weight row's words into registers five
// k-tiles ahead and decodes them there.
//   MXFP4: a byte of codes becomes a bf16 pair with the scaled conversion of CDNA4, which applies
//          the block scale 2^(s-127) exactly (NaN for s == 255).
//   Q8_0:  int8 codes become exact bf16; each 32-block's fp32 partial sum is scaled by its d.
#include "experts_common.hpp"

namespace ql {
namespace {
using namespace ex_detail;

// ---------------------------------------------------------------- routing

// Workgroup j: an LDS histogram of all ids gives expert j's offset (the counts below j) and its
// rank among the experts by count (larger counts first, ties by index); then the positions with
// id j are written in increasing order (wave ballots + an LDS prefix over the 16 waves), so the
// permutation is a stable counting sort, identical on every run.  With `order`, order[rank] = j.
// With `y`, the workgroup also zeroes the output rows of the positions of its share
// [j n_pos / e, (j+1) n_pos / e) whose id is out of [0, e); with `xfac`, it writes the power-of-two
// factors of its share of the x rows (for f16 products).  1024 threads: one pass per 1024 ids.
__global__ __launch_bounds__(1024) void route_kernel(const int64_t* __restrict__ ids, int64_t n_pos, int64_t e,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ perm_out,
                                                     int32_t* __restrict__ order, void* __restrict__ y, int64_t n,
                                                     int ydt, const uint16_t* __restrict__ x, int64_t x_rows,
                                                     int64_t K, float* __restrict__ xfac) {
  extern __shared__ int32_t s_hist[];  // e counts
  __shared__ int32_t s_wave[16];
  __shared__ int32_t s_red[2][16];
  const int64_t j = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int64_t i = tid; i < e; i += 1024) s_hist[i] = 0;
  __syncthreads();
  for (int64_t p = tid; p < n_pos; p += 1024) {
    const int64_t v = ids[p];
    if (v >= 0 && v < e) atomicAdd(&s_hist[v], 1);
  }
  __syncthreads();
  const int32_t cj = s_hist[j];
  int32_t below = 0, ahead = 0;
  for (int64_t i = tid; i < e; i += 1024) {
    const int32_t ci = s_hist[i];
    below += i < j ? ci : 0;
    ahead += (ci > cj || (ci == cj && i < j)) ? 1 : 0;
  }
  for (int off = 32; off >= 1; off >>= 1) {
    below += __shfl_xor(below, off);
    ahead += __shfl_xor(ahead, off);
  }
  if (lane == 0) {
    s_red[0][wave] = below;
    s_red[1][wave] = ahead;
  }
  __syncthreads();
  int32_t base = 0, rank = 0;
  for (int w = 0; w < 16; ++w) {
    base += s_red[0][w];
    rank += s_red[1][w];
  }
  if (tid == 0) {
    offsets[j] = base;
    if (j == e - 1) offsets[e] = base + cj;
    if (order) order[rank] = (int32_t)j;
  }
  int32_t running = 0;
  for (int64_t p0 = 0; p0 < n_pos; p0 += 1024) {
    const int64_t p = p0 + tid;
    const bool hit = p < n_pos && ids[p] == j;
    const uint64_t bal = __ballot(hit);
    const int32_t in_wave = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_wave[wave] = __popcll(bal);
    __syncthreads();
    int32_t before = running, total = 0;
    for (int w = 0; w < 16; ++w) {
      const int32_t c = s_wave[w];
      before += w < wave ? c : 0;
      total += c;
    }
    if (hit) perm_out[base + before + in_wave] = (int32_t)p;
    running += total;
    __syncthreads();
  }
  if (y) {
    // positions of this workgroup's share whose id is out of range, 1024 at a time: listed in LDS
    // (in any order), then their rows zeroed by all threads
    const int64_t esz = ydt == DT_F32 ? 4 : 2;
    int32_t* s_dead = s_hist;  // the histogram is no longer read
    for (int64_t pb = j * n_pos / e; pb < (j + 1) * n_pos / e; pb += 1024) {
      if (tid == 0) s_red[0][0] = 0;
      __syncthreads();
      const int64_t p = pb + tid;
      if (p < (j + 1) * n_pos / e) {
        const int64_t v = ids[p];
        if (v < 0 || v >= e) s_dead[atomicAdd(&s_red[0][0], 1)] = tid;
      }
      __syncthreads();
      const int nd = s_red[0][0];
      for (int d = 0; d < nd; ++d) {
        uint16_t* row = (uint16_t*)((uint8_t*)y + (pb + s_dead[d]) * n * esz);
        for (int64_t i = tid; i < n * esz / 2; i += 1024) row[i] = 0;
      }
      __syncthreads();
    }
  }
  if (xfac) {
    // bf16 x rows: the factors 2^-t and 2^t with max |x| 2^-t in [2^14, 2^15) (t = 0 for a zero
    // row, clamped to [-100, 100]); one wave per row, rows spread over all workgroups' waves
    for (int64_t r = j * 16 + wave; r < x_rows; r += e * 16) {
      uint32_t a = 0u;
      const uint16_t* xr = x + r * K;
      for (int64_t i = 8 * lane; i < K; i += 512) {
        const u32x4_t v = *(const u32x4_t*)(xr + i);  // K % 32 == 0 and x 16-byte aligned
#pragma unroll
        for (int c = 0; c < 4; ++c) a = max(a, max(v[c] & 0x7fffu, (v[c] >> 16) & 0x7fffu));
      }
      for (int off = 32; off >= 1; off >>= 1) a = max(a, (uint32_t)__shfl_xor((int)a, off));
      if (lane == 0) {
        const int t = a == 0u ? 0 : min(100, max(-100, (int)(a >> 7) - 127 - 14));
        xfac[2 * r] = __builtin_ldexpf(1.0f, -t);
        xfac[2 * r + 1] = __builtin_ldexpf(1.0f, t);
      }
    }
  }
}

// Zero every output row (no expert, or k == 0: every product is empty).
__global__ __launch_bounds__(256) void zero_rows_kernel(int64_t n, void* __restrict__ y, int ydt) {
  const int64_t p = blockIdx.x;
  const int64_t esz = ydt == DT_F32 ? 4 : 2;
  uint8_t* row = (uint8_t*)y + p * n * esz;
  for (int64_t i = threadIdx.x; i < n * esz / 2; i += 256) ((uint16_t*)row)[i] = 0;
}

// ---------------------------------------------------------------- routed apply

constexpr int EBK = 64, EMC = 96;  // k / positions per chunk (up to 3 m-subtiles of 32)
constexpr int ENS = 5;              // LDS stages of x (k-tiles in flight: ENS - 1)

enum : int { FMT_MXFP4 = 1, FMT_Q8_0 = 2 };

// 32-row column tiles per wave and weight rows per workgroup (4 waves).
#ifndef EX_MXFP4_CT
#define EX_MXFP4_CT 1
#endif
template <int FMT> constexpr int ex_ct() { return FMT == FMT_MXFP4 ? EX_MXFP4_CT : 1; }
template <int FMT> constexpr int ex_bn() { return 128 * ex_ct<FMT>(); }

__device__ __forceinline__ f32x16_t mfma_bf16(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// x tile swizzle: chunk c (8 values) of row r sits at 16-byte slot r*8 + (c ^ xswz(r)); keeps the
// fragment reads of 8 and of 16 consecutive rows on distinct banks.
__device__ __forceinline__ int ex_xswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Two int8 values (low bytes of a and b) -> packed bf16 pair, exact.
__device__ __forceinline__ uint32_t pack2_bf16_i8(uint32_t a, uint32_t b) {
  bf16x2_t v = {(__bf16)(float)(int32_t)(int8_t)a, (__bf16)(float)(int32_t)(int8_t)b};
  return __builtin_bit_cast(uint32_t, v);
}

// Weight words of one lane for one k-tile, loaded into registers three tiles ahead.
//   MXFP4: 16 bytes of codes (32 values); the scale bytes of the workgroup's rows sit in LDS.
//   Q8_0:  for each of the tile's two blocks, a 4-byte aligned window of 20 bytes holding the
//          lane's 16 code bytes (shift sh) and the block's fp16 d.
template <int FMT> struct WBuf;
template <> struct WBuf<FMT_MXFP4> {
  static constexpr int LOADS = 1;
  u32x4_t c;
};
template <> struct WBuf<FMT_Q8_0> {
  static constexpr int LOADS = 6;
  u32x4_t c[2];
  uint32_t c4[2];
  uint32_t d[2];
};

// k-slots: MXFP4 (32 codes per block, one scale per lane half): MFMA slot j of lane half h at
// k-step t reads k = 32h + 8t + j, i.e. x chunk 4h + t and code word t of the lane's 16 bytes.
// Q8_0 (the partial sum of a k-step is scaled by one block's d): k-step t = 2b + u reads
// k = 32b + 16h + 8u + j, i.e. x chunk 4b + 2h + u.
//
// One workgroup per (expert, 128 * ECT weight rows); wave w owns ECT column tiles of 32 weight
// rows and all the chunk's positions (MS m-subtiles of 32).  The gathered x rows go straight into
// ENS LDS stages, ENS - 1 k-tiles ahead; each lane's weight words go into a ring of ENS register
// buffers, ENS k-tiles ahead.  All loads share one in-order counter, so every load has until the
// wait ENS - 1 k-tiles after its issue; every lane issues the same loads every k-tile (clamped in
// range past the end), so that wait is exact.  The stages are distinct LDS arrays and the loop is
// unrolled by ENS, so the compiler sees which stage each read and each copy touch.
template <int FMT, int MS>
__device__ __forceinline__ void expert_chunk(const int32_t* __restrict__ sPos, int rows, uint8_t* const* stg,
                                             const uint8_t* __restrict__ sScl, int ssh, __amdgpu_buffer_rsrc_t rsX,
                                             __amdgpu_buffer_rsrc_t rsW, int64_t K, int64_t N, const int64_t* ncol,
                                             const int64_t* wrow, int64_t pos_per_row, void* __restrict__ y,
                                             int ydt) {
  constexpr int ECT = ex_ct<FMT>();
  constexpr int NW = WBuf<FMT>::LOADS * ECT;
  // loads allowed in flight at the top of k-tile kt: those issued after x(kt), i.e. the weights of
  // kt + 1 and the x and weights of the ENS - 2 steps in between
  constexpr int L = NW + (ENS - 2) * (MS + NW);
  static_assert(L < 64, "vmcnt range");
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int KT = (int)((K + EBK - 1) / EBK);
  const int kint = (int)K;

  // x copies: copy j (0..MS-1) of wave w covers chunk rows (4j + w)*8 .. +7; lane l -> row + l/8,
  // slot l%8.  Rows past the chunk copy the chunk's first position (never stored).
  uint32_t xoff[MS];
  int xc[MS];
#pragma unroll
  for (int j = 0; j < MS; ++j) {
    const int r = (4 * j + wave) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ex_xswz(r);
    const int32_t pos = sPos[r < rows ? r : 0];
    xoff[j] = (uint32_t)(((int64_t)(pos / pos_per_row) * K + 8 * c) * 2);
    xc[j] = c;
  }
  auto copy_x = [&](int kt, uint8_t* stage) __attribute__((always_inline)) {
    const int k0 = kt * EBK;
#pragma unroll
    for (int j = 0; j < MS; ++j) {
      const uint32_t v = k0 + 8 * xc[j] < kint ? xoff[j] : kExOOB;  // zeros past K
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsX, (lds_void*)(stage + (4 * j + wave_u) * 1024), 16, v,
                                               (uint32_t)(k0 * 2), 0, 0);
    }
  };
  // weight loads of this lane's rows (one per column tile)
  auto load_w = [&](int kt, WBuf<FMT>* wb) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < ECT; ++ct) {
      if constexpr (FMT == FMT_MXFP4) {
        const uint32_t vo = (uint32_t)(wrow[ct] * (K / 2) + 16 * h);
        wb[ct].c = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsW, vo, (uint32_t)(kt * 32), 0));
      } else {
        const int64_t rb = wrow[ct] * (K / 32) * 34 + (int64_t)kt * 68;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const int64_t o = rb + 34 * b + 2 + 16 * h;  // first code byte of this lane
          const uint32_t a = (uint32_t)(o & ~(int64_t)3);
          wb[ct].c[b] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rsW, a, 0, 0));
          wb[ct].c4[b] = __builtin_amdgcn_raw_buffer_load_b32(rsW, a + 16, 0, 0);
          wb[ct].d[b] = __builtin_amdgcn_raw_buffer_load_b16(rsW, (uint32_t)(rb + 34 * b), 0, 0);
        }
      }
    }
  };

  f32x16_t acc[ECT][MS];
#pragma unroll
  for (int ct = 0; ct < ECT; ++ct)
#pragma unroll
    for (int i = 0; i < MS; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[ct][i][r] = 0.0f;

  // Q8_0: byte shift of the lane's code bytes in its 4-byte aligned window, per block of a tile
  // (row bases are 2-byte aligned and a tile is 68 bytes, so the shift is the same for every tile)
  uint32_t qsh[ECT][2] = {};
  if constexpr (FMT == FMT_Q8_0) {
#pragma unroll
    for (int ct = 0; ct < ECT; ++ct)
#pragma unroll
      for (int b = 0; b < 2; ++b) qsh[ct][b] = (uint32_t)((wrow[ct] * (K / 32) * 34 + 34 * b + 2 + 16 * h) & 3);
  }

  auto compute = [&](int kt, const uint8_t* stage, const WBuf<FMT>* wb) __attribute__((always_inline)) {
    if constexpr (FMT == FMT_MXFP4) {
      // the scale of this lane half's block: 2^(s-127) as fp32 (s = 0: the subnormal 2^-127),
      // NaN for s = 255, and 0 past K
      const bool kin = kt * EBK + 32 * h < kint;
      float scl[ECT];
#pragma unroll
      for (int ct = 0; ct < ECT; ++ct) {
        const uint32_t sb = sScl[ssh + (32 * (wave * ECT + ct) + l32) * (K / 32) + 2 * kt + h];
        scl[ct] = !kin ? 0.0f
                       : __uint_as_float(sb == 255u ? 0x7fc00000u : (sb == 0u ? 0x00400000u : sb << 23));
      }
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        u32x4_t af[MS];
#pragma unroll
        for (int rt = 0; rt < MS; ++rt) {
          const int r = rt * 32 + l32;
          af[rt] = *(const u32x4_t*)(stage + (r * 8 + ((4 * h + t) ^ ex_xswz(r))) * 16);
        }
#pragma unroll
        for (int ct = 0; ct < ECT; ++ct) {
          const u32x4_t bf = decode_mxfp4(wb[ct].c[t], scl[ct]);
#pragma unroll
          for (int rt = 0; rt < MS; ++rt) acc[ct][rt] = mfma_bf16(af[rt], bf, acc[ct][rt]);
        }
      }
    } else {
      const f32x16_t zero16 = {0.0f};
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const bool live = kt * EBK + 32 * b < kint;
        f32x16_t p[ECT][MS];
        u32x4_t bf[ECT][2];
        float d[ECT];
#pragma unroll
        for (int ct = 0; ct < ECT; ++ct) {
          // the lane's 16 code bytes from the aligned window (shift 0 or 2 bytes)
          const u32x4_t cw = wb[ct].c[b];
          uint32_t q[4];
          q[0] = __builtin_amdgcn_alignbyte(cw[1], cw[0], qsh[ct][b]);
          q[1] = __builtin_amdgcn_alignbyte(cw[2], cw[1], qsh[ct][b]);
          q[2] = __builtin_amdgcn_alignbyte(cw[3], cw[2], qsh[ct][b]);
          q[3] = __builtin_amdgcn_alignbyte(wb[ct].c4[b], cw[3], qsh[ct][b]);
          d[ct] = live ? f16_bits_to_f32(wb[ct].d[b] & 0xffffu) : 0.0f;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            bf[ct][u][0] = pack2_bf16_i8(q[2 * u], q[2 * u] >> 8);
            bf[ct][u][1] = pack2_bf16_i8(q[2 * u] >> 16, q[2 * u] >> 24);
            bf[ct][u][2] = pack2_bf16_i8(q[2 * u + 1], q[2 * u + 1] >> 8);
            bf[ct][u][3] = pack2_bf16_i8(q[2 * u + 1] >> 16, q[2 * u + 1] >> 24);
          }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
          for (int rt = 0; rt < MS; ++rt) {
            const int r = rt * 32 + l32;
            const int c = 4 * b + 2 * h + u;
            const u32x4_t af = *(const u32x4_t*)(stage + (r * 8 + (c ^ ex_xswz(r))) * 16);
#pragma unroll
            for (int ct = 0; ct < ECT; ++ct) p[ct][rt] = mfma_bf16(af, bf[ct][u], u == 0 ? zero16 : p[ct][rt]);
          }
        }
#pragma unroll
        for (int ct = 0; ct < ECT; ++ct)
#pragma unroll
          for (int rt = 0; rt < MS; ++rt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[ct][rt][r] = __builtin_fmaf(d[ct], p[ct][rt][r], acc[ct][rt][r]);
      }
    }
  };

  WBuf<FMT> wbr[ENS][ECT];
  // One k-tile: wait for its x copies and weights, barrier (every wave is done with the stage the
  // copies below refill), copy x of kt + ENS - 1, compute, load the weights of kt + ENS into the
  // ring slot just consumed.  Steps past the last tile (completing a round) load clamped tiles and
  // compute nothing.
  auto step = [&](int kt, const uint8_t* cur, uint8_t* refill, WBuf<FMT>* wb) __attribute__((always_inline)) {
    ex_wait_vmcnt<L>();
    __builtin_amdgcn_s_barrier();
    copy_x(kt + ENS - 1 < KT ? kt + ENS - 1 : KT - 1, refill);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    if (kt < KT) compute(kt, cur, wb);
    __builtin_amdgcn_sched_barrier(0);
    load_w(kt + ENS < KT ? kt + ENS : KT - 1, wb);
    asm volatile("" ::: "memory");
  };

  // prologue: x and weights of tiles 0 .. ENS-2, then the weights of ENS-1 (same order of loads in
  // flight as at the top of every later step)
#pragma unroll
  for (int t = 0; t < ENS - 1; ++t) {
    copy_x(t < KT ? t : KT - 1, stg[t]);
    asm volatile("" ::: "memory");
    load_w(t < KT ? t : KT - 1, wbr[t]);
    asm volatile("" ::: "memory");
  }
  load_w(ENS - 1 < KT ? ENS - 1 : KT - 1, wbr[ENS - 1]);
  asm volatile("" ::: "memory");
  // the first round is peeled so that the loop is entered with the loads in flight in the same
  // order as at its back edge
#pragma unroll
  for (int j = 0; j < ENS; ++j) step(j, stg[j], stg[(j + ENS - 1) % ENS], wbr[j]);
  for (int kt = ENS; kt < KT; kt += ENS) {
#pragma unroll
    for (int j = 0; j < ENS; ++j) step(kt + j, stg[j], stg[(j + ENS - 1) % ENS], wbr[j]);
  }
  ex_wait_vmcnt<0>();  // no copy may still be writing LDS
  __syncthreads();     // every wave is done with the stages before the next chunk refills them

  // store: lane holds weight row ncol[ct] for positions 8*(r/4) + 4h + r%4 of each m-subtile
#pragma unroll
  for (int ct = 0; ct < ECT; ++ct) {
    if (ncol[ct] >= N) continue;
#pragma unroll
    for (int rt = 0; rt < MS; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rr = rt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        if (rr < rows) store_out(y, (int64_t)sPos[rr] * N + ncol[ct], acc[ct][rt][r], ydt);
      }
  }
}

template <int FMT>
__global__ __launch_bounds__(256, 2) void experts_kernel(const uint8_t* __restrict__ w0, const uint8_t* __restrict__ w1,
                                                         int64_t e, int64_t N, int64_t K,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ perm_pos,
                                                         const uint16_t* __restrict__ x, int64_t x_rows,
                                                         int64_t pos_per_row, void* __restrict__ y, int ydt) {
  static_assert(ENS == 5, "the stage arrays below");
  __shared__ __attribute__((aligned(16))) uint8_t st0[EMC * EBK * 2];
  __shared__ __attribute__((aligned(16))) uint8_t st1[EMC * EBK * 2];
  __shared__ __attribute__((aligned(16))) uint8_t st2[EMC * EBK * 2];
  __shared__ __attribute__((aligned(16))) uint8_t st3[EMC * EBK * 2];
  __shared__ __attribute__((aligned(16))) uint8_t st4[EMC * EBK * 2];
  __shared__ int32_t sPos[EMC];
  uint8_t* const stg[ENS] = {st0, st1, st2, st3, st4};

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31;
  constexpr int ECT = ex_ct<FMT>(), EBN = ex_bn<FMT>();
  const int64_t n_tiles = (N + EBN - 1) / EBN;
  const int64_t ex = blockIdx.x / n_tiles;
  const int64_t nt = blockIdx.x - ex * n_tiles;
  const int32_t off = offsets[ex];
  const int32_t cnt = offsets[ex + 1] - off;
  if (cnt <= 0) return;


  int64_t ncol[ECT], wrow[ECT];  // this lane's weight rows of the expert (one per column tile)
#pragma unroll
  for (int ct = 0; ct < ECT; ++ct) {
    ncol[ct] = nt * EBN + wave * (32 * ECT) + 32 * ct + l32;
    wrow[ct] = ex * N + (ncol[ct] < N ? ncol[ct] : N - 1);
  }
  const __amdgpu_buffer_rsrc_t rsX = ex_rsrc(x, x_rows * K * 2);
  const __amdgpu_buffer_rsrc_t rsW =
      ex_rsrc(w0, FMT == FMT_MXFP4 ? e * N * (K / 2) : e * N * (K / 32) * 34);
  // MXFP4: the scale bytes of the workgroup's weight rows for the whole k range (one contiguous
  // byte range), loaded once as aligned words; byte j of it sits at sScl[ssh + j]
  extern __shared__ uint32_t sScl32[];
  const uint8_t* sScl = (const uint8_t*)sScl32;
  int ssh = 0;
  if constexpr (FMT == FMT_MXFP4) {
    const __amdgpu_buffer_rsrc_t rsS = ex_rsrc(w1, e * N * (K / 32));
    const int64_t base = (ex * N + nt * EBN) * (K / 32);
    ssh = (int)(base & 3);
    const uint32_t a0 = (uint32_t)(base - ssh);
    const int nd = (int)((ssh + EBN * (K / 32) + 3) / 4);
    for (int i = tid; i < nd; i += 256) sScl32[i] = __builtin_amdgcn_raw_buffer_load_b32(rsS, a0 + 4u * i, 0, 0);
  }
  for (int32_t mc = 0; mc < cnt; mc += EMC) {
    const int rows = min(EMC, cnt - mc);
    __syncthreads();  // previous chunk's readers of sPos are done
    if (tid < EMC) sPos[tid] = tid < rows ? perm_pos[off + mc + tid] : -1;
    __syncthreads();
    const int msub = (rows + 31) >> 5;
    if (msub == 1)
      expert_chunk<FMT, 1>(sPos, rows, stg, sScl, ssh, rsX, rsW, K, N, ncol, wrow, pos_per_row, y, ydt);
    else if (msub == 2)
      expert_chunk<FMT, 2>(sPos, rows, stg, sScl, ssh, rsX, rsW, K, N, ncol, wrow, pos_per_row, y, ydt);
    else
      expert_chunk<FMT, 3>(sPos, rows, stg, sScl, ssh, rsX, rsW, K, N, ncol, wrow, pos_per_row, y, ydt);
  }
}

}  // namespace

hipError_t launch_route(const int64_t* ids, int64_t n_pos, int64_t e, int32_t* offsets, int32_t* perm, hipStream_t s) {
  route_kernel<<<(unsigned)e, 1024, (size_t)e * 4, s>>>(ids, n_pos, e, offsets, perm, nullptr, nullptr, 0, 0,
                                                        nullptr, 0, 0, nullptr);
  return hipGetLastError();
}

hipError_t launch_apply_experts(int fmt, const void* w0, const void* w1, int64_t e, int64_t n, int64_t k,
                                const int64_t* ids, int64_t n_pos, const void* x, int xdt, int64_t pos_per_row,
                                void* y, int ydt, int32_t* offsets, int32_t* perm, int32_t* order, float* xfac,
                                hipStream_t s) {
  (void)xdt;
  hipError_t err;
  if (e == 0 || k == 0) {  // no expert, or empty products: every row is zero
    zero_rows_kernel<<<(unsigned)n_pos, 256, 0, s>>>(n, y, ydt);
    return hipGetLastError();
  }
  // routing, expert order, and zero rows for the positions routed nowhere
  const int64_t x_rows = n_pos / pos_per_row;
  route_kernel<<<(unsigned)e, 1024, (size_t)(e > 1024 ? e : 1024) * 4, s>>>(
      ids, n_pos, e, offsets, perm, order, y, n, ydt, (const uint16_t*)x, x_rows, k, fmt == FMT_Q8_0 ? xfac : nullptr);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (fmt == FMT_Q8_0)
    return launch_experts_q8((const uint8_t*)w0, e, n, k, offsets, perm, order, xfac, (const uint16_t*)x, x_rows,
                             pos_per_row, y, ydt, s);
  if (fmt == FMT_MXFP4) {
    return launch_experts_mx((const uint8_t*)w0, (const uint8_t*)w1, e, n, k, offsets, perm, order,
                             (const uint16_t*)x, x_rows, pos_per_row, y, ydt, s);
  }
  const int64_t bn = fmt == FMT_MXFP4 ? ex_bn<FMT_MXFP4>() : ex_bn<FMT_Q8_0>();
  const int64_t grid = e * ((n + bn - 1) / bn);
  if (fmt == FMT_MXFP4)
    experts_kernel<FMT_MXFP4><<<(unsigned)grid, 256, (size_t)((bn * (k / 32) + 8 + 3) / 4 * 4), s>>>((const uint8_t*)w0, (const uint8_t*)w1, e, n, k, offsets,
                                                            perm, (const uint16_t*)x, x_rows, pos_per_row, y, ydt);
  else
    experts_kernel<FMT_Q8_0><<<(unsigned)grid, 256, 0, s>>>((const uint8_t*)w0, nullptr, e, n, k, offsets, perm,
                                                           (const uint16_t*)x, x_rows, pos_per_row, y, ydt);
  return hipGetLastError();
}

}  // namespace ql
