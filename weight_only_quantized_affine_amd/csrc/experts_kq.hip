// Routed apply for Q4_K and Q6_K experts (Nx_quant API docs, Products: apply_experts; Nx_quant
// Weights: Q4_K and Q6_K): y[p, :] = x[p / pos_per_row, :] . W_{ids[p]}^T in fp32, read from the
// blocks where they lie.  The routing (offsets, permutation, expert order) comes from experts.hip.
//
// Both formats are affine per sub-block: a Q4_K sub-block of 32 values is (d*sc)*q - dmin*m, a
// Q6_K sub-block of 16 is (d*sc)*(q - 32), with d*sc and dmin*m exact in fp32.  So the matrix cores
// take the codes themselves, as the bf16 values 128 + q (exact), against bf16 x, one product per
// sub-block (v_mfma_f32_16x16x32_bf16 for Q4_K's 32 values, v_mfma_f32_16x16x16_bf16 for Q6_K's 16),
// and each sub-block's fp32 sum D is folded into the accumulator with the lane's row parameters
// (fp16 x takes the f16 products, the codes then entering as the fp16 values 128 + q, also exact):
//   acc += s * D + (b - off * s) * X,   X = that sub-block's sum of x (from LDS),
// with s = d*sc, b = -dmin*m (Q4_K) or 0 (Q6_K), off = 128 (Q4_K) or 160 = 128 + 32 (Q6_K).  Every
// weight value enters exactly; the result differs from a sum of the decoded fp32 values only by
// fp32 rounding.
//
// One workgroup of 8 waves per (expert, 256 weight rows), in decreasing order of the experts'
// position counts; wave w owns two column tiles of 16 rows and all of the chunk's positions (up to
// 64: MS m-subtiles of 16).  Per 256-value block of k: the chunk's x rows go HBM -> LDS by DMA into
// one of two buffers (16-byte chunk c of row r at slot c ^ (r % 16), so that the 16 rows of one
// operand read hit 16 distinct bank groups), the sub-block sums are formed from them, and each lane
// reads its rows' block bytes into registers.  The x copies and weight loads of block kb + 1 are
// issued before block kb's sums and products, so they are in flight while those run.
#include "experts_common.hpp"

namespace ql {
namespace {
using namespace ex_detail;

constexpr int KQ_MC = 64;                 // positions per chunk
constexpr int KQ_CT = 2;                  // column tiles of 16 rows per wave
constexpr int KQ_W = 8;                   // waves per workgroup
constexpr int KQ_BN = KQ_W * 16 * KQ_CT;  // weight rows per workgroup
typedef __attribute__((ext_vector_type(4))) short s16x4_t;

typedef __attribute__((ext_vector_type(4))) _Float16 f16x4_t;

template <typename XT> struct KqOp;
template <> struct KqOp<BF16> {
  __device__ static f32x4_t k32(const u32x4_t& a, const u32x4_t& b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
  }
  __device__ static f32x4_t k16(const u32x2_t& a, const u32x2_t& b) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a), __builtin_bit_cast(s16x4_t, b),
                                                     f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
  }
  // bytes n0..n3 (each < 128) -> the bf16 pairs (128 + n0, 128 + n1) and (128 + n2, 128 + n3)
  __device__ static uint32_t pair_lo(uint32_t n) { return perm(0x43434343u, n, 0x04010400u); }
  __device__ static uint32_t pair_hi(uint32_t n) { return perm(0x43434343u, n, 0x04030402u); }
  __device__ static float lo(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static float hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
};
template <> struct KqOp<F16> {
  __device__ static f32x4_t k32(const u32x4_t& a, const u32x4_t& b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                  f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
  }
  __device__ static f32x4_t k16(const u32x2_t& a, const u32x2_t& b) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a), __builtin_bit_cast(f16x4_t, b),
                                                 f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
  }
  // bytes n0..n3 (each < 128) -> the fp16 pairs (128 + n0, 128 + n1) and (128 + n2, 128 + n3): 128 is
  // 0x5800 and its fp16 step is 1/8, so 128 + n has the bits 0x5800 | (n << 3)
  __device__ static uint32_t pair_lo(uint32_t n) { return (perm(0u, n, 0x0c010c00u) << 3) | 0x58005800u; }
  __device__ static uint32_t pair_hi(uint32_t n) { return (perm(0u, n, 0x0c030c02u) << 3) | 0x58005800u; }
  __device__ static float lo(uint32_t w) { return f16_bits_to_f32(w & 0xffffu); }
  __device__ static float hi(uint32_t w) { return f16_bits_to_f32(w >> 16); }
};

// One lane's data of one block for one column tile.
struct Q4Lane {
  u32x4_t hdr;   // d, dmin, the 12 scale bytes
  u32x2_t qs[4]; // quant bytes 32 c + 8 q .. + 7 of each 32-byte group c (lane quadrant q)
};
struct Q6Lane {
  uint32_t ql[2][4];  // low-bit bytes 64 h + 16 i + 4 q .. + 3 (h = 0, 1; i = 0..3)
  uint32_t qh[2][2];  // high-bit bytes 128 + 32 h + 16 i + 4 q .. + 3 (i = 0, 1)
  uint32_t sc[4];     // the 16 scale bytes
  uint32_t d;         // fp16 d
};

template <int FMT> struct KQ;
template <> struct KQ<4> {  // Q4_K
  static constexpr int kBytes = 144, kSub = 8, kSubLen = 32;
  static constexpr float kOff = 128.0f;
  using Lane = Q4Lane;
  // blocks are 16-byte aligned (144 = 9 * 16; the host checks the base)
  __device__ static void load(__amdgpu_buffer_rsrc_t rw, uint32_t boff, int q, Lane& L) {
    L.hdr = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, boff, 0, 0));
#pragma unroll
    for (int c = 0; c < 4; ++c)
      L.qs[c] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rw, boff + 16u + 32u * c + 8u * q, 0, 0));
  }
  // s = d*sc and b = -dmin*m of sub-block j
  __device__ static void params(const Lane& L, int j, float& s, float& b) {
    auto sb = [&](int i) { return (L.hdr[1 + (i >> 2)] >> (8 * (i & 3))) & 0xffu; };
    uint32_t sc, mn;
    if (j < 4) {
      sc = sb(j) & 63u;
      mn = sb(j + 4) & 63u;
    } else {
      sc = (sb(j + 4) & 15u) | ((sb(j - 4) >> 6) << 4);
      mn = (sb(j + 4) >> 4) | ((sb(j) >> 6) << 4);
    }
    s = f16_bits_to_f32(L.hdr[0] & 0xffffu) * (float)sc;
    b = -(f16_bits_to_f32(L.hdr[0] >> 16) * (float)mn);
  }
  // operand of sub-block j (k-slots 8q .. 8q + 7: values 8q .. of the sub-block): group c = j / 2,
  // low nibbles for even j, high for odd
  template <typename XT> __device__ static u32x4_t codes(const Lane& L, int j) {
    const u32x2_t w = L.qs[j >> 1];
    const int sh = 4 * (j & 1);
    const uint32_t n0 = (w[0] >> sh) & 0x0f0f0f0fu, n1 = (w[1] >> sh) & 0x0f0f0f0fu;
    return u32x4_t{KqOp<XT>::pair_lo(n0), KqOp<XT>::pair_hi(n0), KqOp<XT>::pair_lo(n1), KqOp<XT>::pair_hi(n1)};
  }
};
template <> struct KQ<5> {  // Q6_K
  static constexpr int kBytes = 210, kSub = 16, kSubLen = 16;
  static constexpr float kOff = 160.0f;
  using Lane = Q6Lane;
  // blocks are only 2-byte aligned (210 bytes): every word is read as two half-words
  __device__ static uint32_t w32(__amdgpu_buffer_rsrc_t rw, uint32_t off) {
    const uint32_t lo = __builtin_amdgcn_raw_buffer_load_b16(rw, off, 0, 0);
    const uint32_t hi = __builtin_amdgcn_raw_buffer_load_b16(rw, off + 2u, 0, 0);
    return lo | (hi << 16);
  }
  __device__ static void load(__amdgpu_buffer_rsrc_t rw, uint32_t boff, int q, Lane& L) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int i = 0; i < 4; ++i) L.ql[h][i] = w32(rw, boff + 64u * h + 16u * i + 4u * q);
#pragma unroll
      for (int i = 0; i < 2; ++i) L.qh[h][i] = w32(rw, boff + 128u + 32u * h + 16u * i + 4u * q);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) L.sc[i] = w32(rw, boff + 192u + 4u * i);
    L.d = __builtin_amdgcn_raw_buffer_load_b16(rw, boff + 208u, 0, 0);
  }
  __device__ static void params(const Lane& L, int j, float& s, float& b) {
    const int8_t sc = (int8_t)((L.sc[j >> 2] >> (8 * (j & 3))) & 0xffu);
    s = f16_bits_to_f32(L.d) * (float)sc;
    b = 0.0f;
  }
  // operand of sub-block j (k-slots 4q .. 4q + 3: values 16 j + 4q .. + 3 of the block): with
  // h = j / 8, g = (j % 8) / 2, l = 16 (j % 2) + 4q, the low bits are the nibble g / 2 of low-bit
  // bytes 64 h + 32 (g % 2) + l, the high bits bits 2g of high-bit bytes 128 + 32 h + l
  template <typename XT> __device__ static u32x2_t codes(const Lane& L, int j) {
    const int h = j >> 3, g = (j & 7) >> 1, i = j & 1;
    const uint32_t lo = (L.ql[h][2 * (g & 1) + i] >> (4 * (g >> 1))) & 0x0f0f0f0fu;
    const uint32_t hi = (L.qh[h][i] >> (2 * g)) & 0x03030303u;
    const uint32_t n = lo | (hi << 4);
    return u32x2_t{KqOp<XT>::pair_lo(n), KqOp<XT>::pair_hi(n)};
  }
};

template <int FMT, typename XT, int MS>
__device__ __forceinline__ void kq_chunk(const int32_t* __restrict__ sPos, int rows, uint8_t* sx0, uint8_t* sx1,
                                         float* sxs0, float* sxs1, __amdgpu_buffer_rsrc_t rsX, __amdgpu_buffer_rsrc_t rsW,
                                         int64_t K, int64_t N, int64_t ncol0, const uint32_t* wrow_off,
                                         int64_t pos_per_row, void* __restrict__ y, int ydt) {
  using F = KQ<FMT>;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int j16 = lane & 15, q = lane >> 4;
  const int KB = (int)(K / 256);
  f32x4_t acc[KQ_CT][MS];
#pragma unroll
  for (int ct = 0; ct < KQ_CT; ++ct)
#pragma unroll
    for (int rt = 0; rt < MS; ++rt) acc[ct][rt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // x copies: 16 MS rows x 32 chunks, two rows per wave instruction (1 KB): instruction i of wave w
  // covers rows 2 (KQ_W i + w) and the next; lane l -> row + l / 32, slot l % 32 (chunk (l % 32) ^
  // (row % 16)).  Rows past the chunk read zeros.
  constexpr int CPW = (16 * MS / 2 + KQ_W - 1) / KQ_W;
  uint32_t xoff[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int r = 2 * (KQ_W * i + wave) + (lane >> 5);
    const int c = (lane & 31) ^ (r & 15);
    xoff[i] = r < rows ? (uint32_t)((((int64_t)sPos[r] / pos_per_row) * K + 8 * c) * 2) : kExOOB;
  }
  auto copy_x = [&](int kb, uint8_t* buf) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CPW; ++i)
      if (2 * (KQ_W * i + wave_u) < 16 * MS)  // uniform
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsX, (lds_void*)(buf + (KQ_W * i + wave_u) * 1024), 16,
                                                 xoff[i] == kExOOB ? kExOOB : xoff[i] + (uint32_t)(kb * 512), 0, 0,
                                                 0);
  };
  auto load_w = [&](int kb, typename F::Lane* L) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < KQ_CT; ++ct) F::load(rsW, wrow_off[ct] + (uint32_t)(kb * F::kBytes), q, L[ct]);
  };

  typename F::Lane Lc[KQ_CT], Ln[KQ_CT];
  // Sub-block sums of the rows this wave copied: each lane sums the 8 values of the chunk its own
  // copy wrote, and the lanes of a sub-block (an aligned group of KQ_SL slots: the slot order is
  // the chunk order xor row % 16) add theirs; the first of them writes the sum.  Only this wave's
  // copies are read, so its own wait for them suffices; the barrier that follows publishes the sums.
  constexpr int KQ_SL = F::kSubLen / 8;  // chunks (and lanes) per sub-block: 4 or 2
  auto own_sums = [&](const uint8_t* buf, float* sum) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      if (2 * (KQ_W * i + wave_u) < 16 * MS) {  // uniform
        const int r = 2 * (KQ_W * i + wave) + (lane >> 5), slot = lane & 31;
        const u32x4_t v = *(const u32x4_t*)(buf + (r * 32 + slot) * 16);
        float ps = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) ps += KqOp<XT>::lo(v[e]) + KqOp<XT>::hi(v[e]);
#pragma unroll
        for (int o = 1; o < KQ_SL; o <<= 1) ps += __shfl_xor(ps, o);
        if ((slot & (KQ_SL - 1)) == 0) sum[((slot ^ (r & 15)) / KQ_SL) * KQ_MC + r] = ps;
      }
    }
  };
  copy_x(0, sx0);
  load_w(0, Lc);
  for (int kb = 0; kb < KB; ++kb) {
    uint8_t* const cur = (kb & 1) ? sx1 : sx0;
    float* const sum = (kb & 1) ? sxs1 : sxs0;
    ex_wait_vmcnt<0>();  // this wave's copies of block kb's x and its weights have landed
    own_sums(cur, sum);
    __syncthreads();     // every wave's x and sums of block kb are in LDS, and every wave is done
                         // with block kb - 1's buffers
    if (kb + 1 < KB) {   // uniform
      copy_x(kb + 1, (kb & 1) ? sx0 : sx1);
      load_w(kb + 1, Ln);
    }
#pragma unroll
    for (int j = 0; j < F::kSub; ++j) {
      float s[KQ_CT], bb[KQ_CT];
#pragma unroll
      for (int ct = 0; ct < KQ_CT; ++ct) {
        float b;
        F::params(Lc[ct], j, s[ct], b);
        bb[ct] = b - F::kOff * s[ct];
      }
#pragma unroll
      for (int rt = 0; rt < MS; ++rt) {
        const int r = rt * 16 + j16;
        // this lane's accumulator rows 4q .. 4q + 3 of the m-subtile: their sub-block sums
        const f32x4_t X = *(const f32x4_t*)(sum + j * KQ_MC + rt * 16 + 4 * q);
        f32x4_t D[KQ_CT];
        if constexpr (FMT == 4) {
          const int c = 4 * j + q;  // values 32 j + 8 q .. + 7
          const u32x4_t a = *(const u32x4_t*)(cur + (r * 32 + (c ^ (r & 15))) * 16);
#pragma unroll
          for (int ct = 0; ct < KQ_CT; ++ct) D[ct] = KqOp<XT>::k32(a, F::template codes<XT>(Lc[ct], j));
        } else {
          const int c = 2 * j + (q >> 1);  // values 16 j + 4 q .. + 3: half (q & 1) of chunk c
          const u32x2_t a = *(const u32x2_t*)(cur + (r * 32 + (c ^ (r & 15))) * 16 + 8 * (q & 1));
#pragma unroll
          for (int ct = 0; ct < KQ_CT; ++ct) D[ct] = KqOp<XT>::k16(a, F::template codes<XT>(Lc[ct], j));
        }
#pragma unroll
        for (int ct = 0; ct < KQ_CT; ++ct)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[ct][rt][e] = __builtin_fmaf(s[ct], D[ct][e], __builtin_fmaf(bb[ct], X[e], acc[ct][rt][e]));
      }
    }
#pragma unroll
    for (int ct = 0; ct < KQ_CT; ++ct) Lc[ct] = Ln[ct];
  }
  // outputs: lane holds column ncol0 + 16 ct for positions rt * 16 + 4q + e
#pragma unroll
  for (int ct = 0; ct < KQ_CT; ++ct) {
    const int64_t ncol = ncol0 + 16 * ct;
    if (ncol >= N) continue;
#pragma unroll
    for (int rt = 0; rt < MS; ++rt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = rt * 16 + 4 * q + e;
        if (rr < rows) {
          const float v = acc[ct][rt][e];
          uint8_t* p = (uint8_t*)y;
          const int64_t el = (int64_t)sPos[rr] * N + ncol;
          if (ydt == DT_F32)
            *(float*)(p + el * 4) = v;
          else
            *(uint16_t*)(p + el * 2) = (uint16_t)(ydt == DT_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v));
        }
      }
  }
}

template <int FMT, typename XT>
__global__ __launch_bounds__(KQ_W * 64, 2) void experts_kq_kernel(const uint8_t* __restrict__ blocks, int64_t e,
                                                                  int64_t N, int64_t K,
                                                                  const int32_t* __restrict__ offsets,
                                                                  const int32_t* __restrict__ perm_pos,
                                                                  const int32_t* __restrict__ order,
                                                                  const uint16_t* __restrict__ x, int64_t x_rows,
                                                                  int64_t pos_per_row, void* __restrict__ y, int ydt) {
  // two x buffers and two tables of sub-block sums (blocks kb and kb + 1), [sub-block][row] so
  // that a lane's four accumulator rows are one 16-byte read
  __shared__ __attribute__((aligned(16))) uint8_t sx0[KQ_MC * 256 * 2];
  __shared__ __attribute__((aligned(16))) uint8_t sx1[KQ_MC * 256 * 2];
  __shared__ __attribute__((aligned(16))) float sxs0[KQ_MC * 16];
  __shared__ __attribute__((aligned(16))) float sxs1[KQ_MC * 16];
  __shared__ int32_t sPos[KQ_MC];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int64_t n_tiles = (N + KQ_BN - 1) / KQ_BN;
  const int64_t rank = blockIdx.x / n_tiles;
  const int64_t nt = blockIdx.x - rank * n_tiles;
  const int64_t ex = order[rank];
  const int32_t off = offsets[ex];
  const int32_t cnt = offsets[ex + 1] - off;
  if (cnt <= 0) return;

  using F = KQ<FMT>;
  const int64_t row_bytes = K / 256 * F::kBytes;
  const __amdgpu_buffer_rsrc_t rsX = ex_rsrc(x, x_rows * K * 2);
  const __amdgpu_buffer_rsrc_t rsW = ex_rsrc(blocks, e * N * row_bytes);
  // this lane's weight rows, one per column tile (past N the last row stands in; never stored)
  const int64_t ncol0 = nt * KQ_BN + wave * (16 * KQ_CT) + (lane & 15);
  uint32_t wrow_off[KQ_CT];
#pragma unroll
  for (int ct = 0; ct < KQ_CT; ++ct) wrow_off[ct] = (uint32_t)((ex * N + min(ncol0 + 16 * ct, N - 1)) * row_bytes);

  for (int32_t mc = 0; mc < cnt; mc += KQ_MC) {
    const int rows = min(KQ_MC, cnt - mc);
    __syncthreads();  // the previous chunk's readers of sPos and of the buffers are done
    if (tid < KQ_MC) sPos[tid] = tid < rows ? perm_pos[off + mc + tid] : 0;
    __syncthreads();
    switch ((rows + 15) >> 4) {
      case 1: kq_chunk<FMT, XT, 1>(sPos, rows, sx0, sx1, sxs0, sxs1, rsX, rsW, K, N, ncol0, wrow_off, pos_per_row, y, ydt); break;
      case 2: kq_chunk<FMT, XT, 2>(sPos, rows, sx0, sx1, sxs0, sxs1, rsX, rsW, K, N, ncol0, wrow_off, pos_per_row, y, ydt); break;
      case 3: kq_chunk<FMT, XT, 3>(sPos, rows, sx0, sx1, sxs0, sxs1, rsX, rsW, K, N, ncol0, wrow_off, pos_per_row, y, ydt); break;
      default: kq_chunk<FMT, XT, 4>(sPos, rows, sx0, sx1, sxs0, sxs1, rsX, rsW, K, N, ncol0, wrow_off, pos_per_row, y, ydt); break;
    }
  }
}

}  // namespace

hipError_t launch_experts_kq(int fmt, const uint8_t* blocks, int64_t e, int64_t n, int64_t k, const int32_t* offsets,
                             const int32_t* perm, const int32_t* order, const uint16_t* x, int xdt, int64_t x_rows,
                             int64_t pos_per_row, void* y, int ydt, hipStream_t s) {
  const unsigned grid = (unsigned)(e * ((n + KQ_BN - 1) / KQ_BN));
#define QL_KQ_LAUNCH(F, XT)                                                                                         \
  experts_kq_kernel<F, XT><<<grid, KQ_W * 64, 0, s>>>(blocks, e, n, k, offsets, perm, order, x, x_rows, pos_per_row, y, \
                                                       ydt)
  if (fmt == 4 && xdt == DT_F16)
    QL_KQ_LAUNCH(4, F16);
  else if (fmt == 4)
    QL_KQ_LAUNCH(4, BF16);
  else if (xdt == DT_F16)
    QL_KQ_LAUNCH(5, F16);
  else
    QL_KQ_LAUNCH(5, BF16);
#undef QL_KQ_LAUNCH
  return hipGetLastError();
}

}  // namespace ql
