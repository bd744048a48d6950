// Prefill GEMM on affine-quantized weights with the CDNA4 matrix cores (Nx_quant API docs,
// Products: apply; GPTQModel wiki "MLX Apple Silicon", Concepts):
//   y[m,n] = sum_k x[m,k] * w[n,k],   w = code * scale + bias,   fp32 accumulation.
// The codes are dequantized in registers to fp16 -- every weight rounded once,
// w16 = RNE_f16(q*s + b) -- and x enters as fp16 too, scaled per row by a power of two so that
// every bf16 value of the row converts exactly; v_mfma_f32_32x32x16_f16 then accumulates y
// directly, with no per-group partial sums to fold.  The rounding of w to fp16 (half an ulp,
// 2^-12 relative) is the only error beyond fp32 accumulation: about 1.5e-4 relative per output
// row for unstructured weights.  (A bf16 copy of w, 2^-9, would cost ~1.7e-3.)
//
// Three launches (the two pre-passes share one, prep16_kernel):
//   xprep16: per row of x, t = the exponent that brings max|x| into [2^14, 2^15); the copy
//            x * 2^-t in fp16, permuted per 8 values to the order the code unpacking yields,
//            zero-padded to a multiple of 64 values and stored k-tile-major ([k/64][m][64]: the
//            x tile of a workgroup is one contiguous 32 KiB block, spread over every L2
//            channel, where rows of a row-major copy would fall on a few); the factor 2^t.
//   wprep16: per weight row a power of two 2^v with every S = s 2^(24-v) and B = b 2^-v of the
//            row below 2^15 (the largest in [2^14, 2^15)), so that S and B are exact fp16 values;
//            per group the fp16 pair (S, B); the factor 2^v.
//   gemm16:  the product; y = acc * 2^t[m] * 2^v[n] + layer bias.
// Dequantization: the bits of a code pair, masked into the two halves of a word, are the fp16
// subnormals q 2^-24 (exact); one v_pk_fma_f16 per pair computes fp16(q 2^-24 S + B) =
// fp16((q*s + b) * 2^-v) with one rounding.
//
// Tiling: 256 threads (4 waves, 2 x 2), workgroup tile 256 (m) x 128 (n) x 64 (k), each wave a
// 128 x 64 block of 4 x 2 v_mfma_f32_32x32x16_f16 tiles: one dequantized code fragment feeds four
// products.  x, packed code and record tiles go straight from HBM into three LDS stages (up to
// three tiles ahead of the compute); codes stay packed in LDS; each wave reads the fragments of
// the next tile into registers while it dequantizes and multiplies the current one (one wave
// per SIMD: the overlap has to come from within the wave).  Workgroup w takes m-tile
// w % m_tiles: the workgroups of one m-tile share an XCD (dispatch is round-robin over the 8
// XCDs) and so its L2 copy of the x rows.
// MFMA operand layout (32x32x16): lane l supplies row/column l%32 and k-slots 8*(l/32)..+7; the
// result register r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
// k-slots: lane half h at k-step t (0..3) of a 64-wide k-tile takes the 8-value chunk 4h + t, so
// a lane's codes for the whole tile are 16 (4-bit) or 32 (8-bit) consecutive bytes of its row and
// lie in one group (g >= 32); its (S, B) pair is the record of that group.
#include "device_common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace ql {
namespace {

#ifndef GEMM_PP_INTERLEAVE
#define GEMM_PP_INTERLEAVE 4  // vector instructions scheduled after each product of the ping-pong kernel
#endif
#ifndef GEMM_PP_COPY_IN_COMPUTE
#define GEMM_PP_COPY_IN_COMPUTE 0  // issue the HBM->LDS copies among the products instead of in the mem phase
#endif
#ifndef GEMM_PP_FRAG_FIRST
#define GEMM_PP_FRAG_FIRST 1  // ping-pong mem phase: fragment reads before the copies
#endif
#ifndef GEMM_PP_PRIO
#define GEMM_PP_PRIO 0  // raise the wave priority during the ping-pong compute phase
#endif
#ifndef GEMM_PP_DEQ_MEM
#define GEMM_PP_DEQ_MEM 3  // 3: dequantize in the mem phase, copies among the products; 0: dequantize among the products
#endif
#ifndef GEMM_PP_DEQ16
#define GEMM_PP_DEQ16 1  // 4-bit codes: one shift per word, odd nibbles masked in place with scale/16
#endif
#ifndef GEMM_PP_BAND
#define GEMM_PP_BAND 4  // m-tiles per band of the ping-pong kernel's tile order
#endif
#ifndef GEMM_BM
#define GEMM_BM 256
#endif
#ifndef GEMM_BN
#define GEMM_BN 128
#endif
constexpr int BM = GEMM_BM, BN = GEMM_BN, BK = 64;
// four waves, each a 128 x 64 block: WGN of them along n, BM / 128 along m
constexpr int WGN = BN / 64;
static_assert(BM % 128 == 0 && BN % 64 == 0 && (BM / 128) * WGN == 4, "four waves of 128 x 64");

typedef __attribute__((address_space(3))) void lds_void;

// Copy `bytes` (4 or 16) per lane from a buffer straight into LDS: lane l reads at byte
// voff + soff of the buffer and its bytes land at dst + bytes * l (dst and soff are uniform).
template <int BYTES>
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, uint8_t* dst) {
  if constexpr (BYTES == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, voff, soff, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 4, voff, soff, 0, 0);
}
// Raw buffer resource over `bytes` bytes at `base` (bytes < 2^31, checked by the host); offsets
// at or past the end read zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kOOB = 0x7ffffff0u;  // a buffer offset past every resource

// s_waitcnt with only the vector-memory count: vmcnt(N), other counters at their maximum.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// vmcnt(N) and lgkmcnt(0) together.
template <int N> __device__ __forceinline__ void wait_vmcnt_lgkm0() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// LDS swizzles (16-byte slot position within a row, XOR-ed with a function of the row) that keep
// the fragment reads of consecutive lanes (rows) on distinct banks:
//   x rows (8 slots):      c ^ xswz(r),   xswz(r) = (r & 7) ^ ((r >> 3) & 1)
//   code rows, 2 slots:    c ^ (((n >> 2) ^ (n >> 3)) & 1)
//   code rows, 4 slots:    c ^ (((n >> 1) & 3) ^ ((n >> 3) & 1))
__device__ __forceinline__ int xswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
template <int CH> __device__ __forceinline__ int bswz(int n) {
  return CH == 2 ? (((n >> 2) ^ (n >> 3)) & 1) : (((n >> 1) & 3) ^ ((n >> 3) & 1));
}

// A 32-bit constant placed in a VGPR once (the VOP3 forms take no literal operand, so the
// shift-and-mask-and-or of the unpacking only folds into one v_and_or_b32 with registers).
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

// A code pair in the two halves of a word as fp16 subnormals (bits q: value q 2^-24, exact) ->
// fp16(q S 2^-24 + B) per half, one v_pk_fma_f16 and one rounding: with S = s 2^(24-v) and
// B = b 2^-v exact in fp16, the value is fp16((q s + b) 2^-v).
__device__ __forceinline__ uint32_t deq2p(uint32_t p, f16x2_t S2, f16x2_t B2) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(__builtin_bit_cast(f16x2_t, p), S2, B2));
}

template <int BITS> struct Deq;
// 4-bit word (codes 0..7) -> operand pairs (0,4), (1,5), (2,6), (3,7).
template <> struct Deq<4> {
  __device__ __forceinline__ static void runp(const uint32_t* w, uint32_t* r, f16x2_t S2, f16x2_t B2, uint32_t mk) {
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = deq2p((w[0] >> (4 * j)) & mk, S2, B2);
  }
  // The same pairs with one shift per word: the odd nibbles of each 16-bit half are masked in place
  // (16 q, still a subnormal pattern, so 16 q 2^-24 exactly) and take S/16 (S16), so that every
  // product is the same as above whenever S/16 is exact.  mk4 = mk << 4.
  __device__ __forceinline__ static void runp16(const uint32_t* w, uint32_t* r, f16x2_t S2, f16x2_t S16, f16x2_t B2,
                                                uint32_t mk, uint32_t mk4) {
    const uint32_t hi = w[0] >> 8;
    r[0] = deq2p(w[0] & mk, S2, B2);
    r[1] = deq2p(w[0] & mk4, S16, B2);
    r[2] = deq2p(hi & mk, S2, B2);
    r[3] = deq2p(hi & mk4, S16, B2);
  }
};
// Two 8-bit words (codes 0..7) -> operand pairs (0,2), (1,3), (4,6), (5,7).
template <> struct Deq<8> {
  __device__ __forceinline__ static void runp(const uint32_t* w, uint32_t* r, f16x2_t S2, f16x2_t B2, uint32_t mk) {
    r[0] = deq2p(w[0] & mk, S2, B2);
    r[1] = deq2p((w[0] >> 8) & mk, S2, B2);
    r[2] = deq2p(w[1] & mk, S2, B2);
    r[3] = deq2p((w[1] >> 8) & mk, S2, B2);
  }
};

__device__ __forceinline__ f32x16_t mfma16(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c, 0,
                                                0, 0);
}

// ---------------------------------------------------------------- pre-pass over x
// One workgroup per row: the row's largest magnitude, then the scaled, permuted fp16 copy.
template <typename XT, int BITS>
__device__ __forceinline__ void xprep16_row(int64_t m, const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                            int64_t Kp, uint16_t* __restrict__ x16, float* __restrict__ xsc) {
  __shared__ uint32_t s_max[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nc = (int)(K / 8), ncp = (int)(Kp / 8);
  typedef __attribute__((address_space(1))) const u32x4_t gu32x4;
  const gu32x4* row = (const gu32x4*)(x + m * K);
  int t = 0;
  if constexpr (std::is_same<XT, BF16>::value) {
    // |bf16| compares as its 15 low bits
    uint32_t mx = 0;
    for (int c = tid; c < nc; c += 256) {
      const u32x4_t v = row[c];
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = max(mx, max(v[e] & 0x7fffu, (v[e] >> 16) & 0x7fffu));
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
    if (lane == 0) s_max[wave] = mx;
    __syncthreads();
    mx = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
    // exponent of the largest magnitude (subnormals: their leading bit's position)
    const int ef = (int)(mx >> 7);
    if (mx != 0) {
      const int e = ef > 0 ? ef - 127 : (31 - __builtin_clz(mx)) - 133;
      t = min(max(e - 14, -100), 100);
    }
  }
  const float f = __builtin_ldexpf(1.0f, -t);
  // k-tile-major: the 64 values of row m in k-tile kt sit at x16[(kt * M + m) * 64]
  u32x4_t* out = (u32x4_t*)x16 + m * 8;
  for (int c = tid; c < ncp; c += 256) {
    u32x4_t o = {0u, 0u, 0u, 0u};
    if (c < nc) {
      const u32x4_t v = row[c];
      float a[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a[2 * e] = (std::is_same<XT, BF16>::value ? bf16_bits_to_f32(v[e] & 0xffffu) : f16_bits_to_f32(v[e] & 0xffffu)) * f;
        a[2 * e + 1] = (std::is_same<XT, BF16>::value ? bf16_bits_to_f32(v[e] >> 16) : f16_bits_to_f32(v[e] >> 16)) * f;
      }
      // operand order of the unpacking: 4-bit (0,4,1,5,2,6,3,7), 8-bit (0,2,1,3,4,6,5,7)
      constexpr int P4[8] = {0, 4, 1, 5, 2, 6, 3, 7}, P8[8] = {0, 2, 1, 3, 4, 6, 5, 7};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i0 = BITS == 4 ? P4[2 * e] : P8[2 * e], i1 = BITS == 4 ? P4[2 * e + 1] : P8[2 * e + 1];
        const f16x2_t hv = {(_Float16)a[i0], (_Float16)a[i1]};
        o[e] = __builtin_bit_cast(uint32_t, hv);
      }
    }
    out[(int64_t)(c >> 3) * M * 8 + (c & 7)] = o;
  }
  if (tid == 0) xsc[m] = __builtin_ldexpf(1.0f, t);
}

// ---------------------------------------------------------------- pre-pass over the weights
// One wave per weight row (four per workgroup): the largest scale and bias magnitudes, then the
// records.
template <typename PT>
__device__ __forceinline__ void wprep16_rows(int64_t blk, const uint16_t* __restrict__ scales,
                                             const uint16_t* __restrict__ biases, int64_t N, int groups,
                                             float2* __restrict__ rec, float* __restrict__ wsc) {
  const int lane = threadIdx.x & 63;
  const int64_t n = blk * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const uint16_t* sr = scales + n * groups;
  const uint16_t* br = biases + n * groups;
  // v: S = s 2^(24-v) and B = b 2^-v below 2^15 for every group of the row (the largest S, or
  // the largest B when the biases bind, in [2^14, 2^15)), so both are exact fp16 values (down to
  // 2^-24 below the row's largest; v is clamped to [-126, 127]); the record holds (S, B)
  float smax = 0.0f, bmax = 0.0f;
  for (int g = lane; g < groups; g += 64) {
    smax = fmaxf(smax, fabsf(param_to_f32<PT>(sr[g])));
    bmax = fmaxf(bmax, fabsf(param_to_f32<PT>(br[g])));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    smax = fmaxf(smax, __shfl_xor(smax, off));
    bmax = fmaxf(bmax, __shfl_xor(bmax, off));
  }
  int v = -126;
  if (smax > 0.0f) {
    int e;
    (void)__builtin_frexpf(smax, &e);  // smax < 2^e
    v = max(v, e + 9);
  }
  if (bmax > 0.0f) {
    int e;
    (void)__builtin_frexpf(bmax, &e);
    v = max(v, e - 15);
  }
  if (smax == 0.0f && bmax == 0.0f) v = 0;
  v = min(v, 127);
  for (int g = lane; g < groups; g += 64) {
    const float s = param_to_f32<PT>(sr[g]), b = param_to_f32<PT>(br[g]);
    const uint32_t S = __builtin_bit_cast(uint16_t, (_Float16)__builtin_ldexpf(s, 24 - v));
    const uint32_t B = __builtin_bit_cast(uint16_t, (_Float16)__builtin_ldexpf(b, -v));
    rec[n * groups + g] = make_float2(__uint_as_float(S | (B << 16)), 0.0f);
  }
  if (lane == 0) wsc[n] = __builtin_ldexpf(1.0f, v);
}

// Both pre-passes in one launch: workgroups 0 .. M-1 take the x rows, the rest four weight rows
// each.
template <typename XT, typename PT, int BITS>
__global__ __launch_bounds__(256) void prep16_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t Kp,
                                                     uint16_t* __restrict__ x16, float* __restrict__ xsc,
                                                     const uint16_t* __restrict__ scales,
                                                     const uint16_t* __restrict__ biases, int64_t N, int groups,
                                                     float2* __restrict__ rec, float* __restrict__ wsc) {
  const int64_t b = blockIdx.x;
  if (b < M)
    xprep16_row<XT, BITS>(b, x, M, K, Kp, x16, xsc);
  else
    wprep16_rows<PT>(b - M, scales, biases, N, groups, rec, wsc);
}

// ---------------------------------------------------------------- main kernel
// TWO: two workgroups per CU with two LDS stages (for launches of at least two workgroups per
// CU), else one workgroup per CU with three stages.  part != NULL: this launch is split over k in
// `splits` ranges of k-tiles (workgroup id / tiles = its range) and writes fp32 partial products
// (row and column factors applied, no layer bias) to part[split][m][n].
template <int BITS, bool G32, bool TWO>
__global__ __launch_bounds__(256, TWO ? 2 : 1) void gemm16_kernel(const uint16_t* __restrict__ x16,
                                                                  const float* __restrict__ xsc, int64_t M, int64_t Kp,
                                                                  int64_t K, const uint32_t* __restrict__ packed,
                                                                  const float2* __restrict__ rec,
                                                                  const float* __restrict__ wsc, int64_t N, int groups,
                                                                  int g, const uint16_t* __restrict__ layer_bias,
                                                                  int lb_bf16, void* __restrict__ y, int ydt,
                                                                  int splits, float* __restrict__ part) {
  // vector instructions scheduled after each product in the compute (measured best: 4 with one
  // workgroup per CU, 3 with two)
  constexpr int kInterleave = TWO ? 3 : 4;
  constexpr int B_ROW = BK * BITS / 8;             // bytes of codes per weight row and tile: 32 or 64
  constexpr int BCH = B_ROW / 16;                  // 16-byte chunks per row: 2 or 4
  constexpr int A_BYTES = BM * BK * 2;             // 32 KiB
  constexpr int B_BYTES = BN * B_ROW;              // 4 or 8 KiB
  constexpr int RD = G32 ? 4 : 2;                  // record words per weight row and tile
  constexpr int R_BYTES = BN * RD * 4;             // 2 or 1 KiB
  constexpr int STAGE = A_BYTES + B_BYTES + R_BYTES;
  constexpr int NA = A_BYTES / (256 * 16);         // x copies per thread and tile
  constexpr int NB = B_BYTES / (256 * 16);         // code copies per thread and tile
  constexpr int NR = BN * RD / 256;                // record copies per thread and tile
  constexpr int L = NA + NB + NR;                  // copies per thread and tile
  static_assert(NA * 256 * 16 == A_BYTES && NB * 256 * 16 == B_BYTES && NR * 256 == BN * RD, "copy shares");
  __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st2[TWO ? 16 : STAGE];
  __shared__ float sXs[BM];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WGN, wn = wave % WGN;
  const int l32 = lane & 31, h = lane >> 5;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  const int64_t m_tiles = (M + BM - 1) / BM;
  const int64_t tiles = m_tiles * ((N + BN - 1) / BN);
  const int64_t tile = blockIdx.x % tiles;
  const int split = (int)(blockIdx.x / tiles);
  const int64_t mt = tile % m_tiles;
  const int64_t nt = tile / m_tiles;
  const int64_t m0 = mt * BM, n0 = nt * BN;
  // this workgroup's k-tiles: kb .. kb + KT - 1
  const int KT_all = (int)(Kp / BK);
  const int per = (KT_all + splits - 1) / splits;
  const int kb = split * per;
  const int KT = max(0, min(per, KT_all - kb));
  const int64_t row_bytes = K * BITS / 8;

  const uint32_t mk = vconst(BITS == 4 ? 0x000F000Fu : 0x00FF00FFu);
  const int gshift = __builtin_ctz((unsigned)g);

  // ---- copies of one tile into a stage (every lane, every tile)
  // x: copy i (0..NA-1) of wave w covers rows (BM/4)w + 8i .. +7; lane l -> row + l/8, slot l%8.
  uint32_t a_off[NA];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int r = (BM / 4) * wave + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ xswz(r);
    a_off[i] = m0 + r < M ? (uint32_t)(((m0 + r) * BK + 8 * c) * 2) : kOOB;
  }
  // codes: copy i (0..NB-1) of wave w covers rows (BN/4)w + (64/BCH)i ..; lane l -> row + l/BCH,
  // slot l%BCH.
  uint32_t b_off[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int n = (BN / 4) * wave + (64 / BCH) * i + lane / BCH;
    const int c = (lane % BCH) ^ bswz<BCH>(n);
    b_off[i] = n0 + n < N ? (uint32_t)((n0 + n) * row_bytes + 16 * c) : kOOB;
  }
  // records: word q = 64 (w + 4i) + lane of the stage -> row q / RD, word q % RD (the two words
  // of group k/g, or of groups k/32 and k/32 + 1 when g == 32)
  int r_row[NR], r_word[NR];
#pragma unroll
  for (int i = 0; i < NR; ++i) {
    const int q = 64 * (wave + 4 * i) + lane;
    r_row[i] = q / RD;
    r_word[i] = q % RD;
  }
  const __amdgpu_buffer_rsrc_t rsA = gemm_rsrc(x16, M * Kp * 2);
  const __amdgpu_buffer_rsrc_t rsB = gemm_rsrc(packed, N * row_bytes);
  const __amdgpu_buffer_rsrc_t rsR = gemm_rsrc(rec, N * (int64_t)groups * 8);
  auto copy_tile = [&](int kt, uint8_t* stage) __attribute__((always_inline)) {
    const int k0 = (kb + kt) * BK;
#pragma unroll
    for (int i = 0; i < NA; ++i)
      copy_to_lds<16>(rsA, a_off[i], (uint32_t)(k0 * M * 2), stage + ((BM / 4) * wave_u + 8 * i) * 128);
#pragma unroll
    for (int i = 0; i < NB; ++i)
      copy_to_lds<16>(rsB, b_off[i], (uint32_t)(k0 * BITS / 8),
                      stage + A_BYTES + ((BN / 4) * wave_u + (64 / BCH) * i) * B_ROW);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int gi = G32 ? (k0 >> 5) + (r_word[i] >> 1) : k0 >> gshift;
      const bool ok = n0 + r_row[i] < N && gi < groups;
      const uint32_t off = ok ? (uint32_t)((((n0 + r_row[i]) * groups + gi) * 2 + (r_word[i] & 1)) * 4) : kOOB;
      copy_to_lds<4>(rsR, off, 0u, stage + A_BYTES + B_BYTES + 64 * (wave_u + 4 * i) * 4);
    }
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // ---- fragments of one tile: this lane's x chunks (4 row-tiles x 4 k-steps), code words and
  // (s, c) record of each col-tile, read from a stage into registers one tile ahead
  struct Frag {
    u32x4_t a[4][4];
    uint32_t cw[2][2 * BCH];
    uint32_t sb[2];  // the fp16 pair (S, B) of each col-tile's group
  };
  auto load_frag = [&](const uint8_t* stage, Frag& f) __attribute__((always_inline)) {
    const uint8_t* sA = stage;
    const uint8_t* sB = stage + A_BYTES;
    const float* sR = (const float*)(stage + A_BYTES + B_BYTES);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int n = wn * 64 + ct * 32 + l32;
      const uint8_t* row = sB + n * B_ROW;
      const int sw = bswz<BCH>(n);
#pragma unroll
      for (int q = 0; q < BCH / 2; ++q) {
        const u32x4_t v = *(const u32x4_t*)(row + (((BCH / 2) * h + q) ^ sw) * 16);
        f.cw[ct][4 * q + 0] = v[0];
        f.cw[ct][4 * q + 1] = v[1];
        f.cw[ct][4 * q + 2] = v[2];
        f.cw[ct][4 * q + 3] = v[3];
      }
      const u32x2_t rr = *(const u32x2_t*)(sR + n * RD + (G32 ? 2 * h : 0));
      f.sb[ct] = rr[0];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        const int r = wm * 128 + rt * 32 + l32;
        const int c = 4 * h + t;
        f.a[rt][t] = *(const u32x4_t*)(sA + (r * 8 + (c ^ xswz(r))) * 16);
      }
  };
  auto dequant = [&](const Frag& f, int t, u32x4_t* bf) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      uint32_t r[4];
      const f16x2_t sb = __builtin_bit_cast(f16x2_t, f.sb[ct]);
      Deq<BITS>::runp(&f.cw[ct][t * (BITS / 4)], r, f16x2_t{sb[0], sb[0]}, f16x2_t{sb[1], sb[1]}, mk);
      bf[ct] = u32x4_t{r[0], r[1], r[2], r[3]};
    }
  };
  // The dequantization of k-step t+1 runs between the 8 products of k-step t: one product,
  // then a few vector instructions, so that the matrix core of this SIMD (whose only wave this
  // is) is fed while the next operands are made.
  auto compute = [&](const Frag& f) __attribute__((always_inline)) {
    u32x4_t bcur[2], bnext[2];
    dequant(f, 0, bcur);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < 3) dequant(f, t + 1, bnext);
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[rt][ct] = mfma16(f.a[rt][t], bcur[ct], acc[rt][ct]);
      if (t < 3) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
          __builtin_amdgcn_sched_group_barrier(0x002, kInterleave, 0);  // vector ALU
        }
      }
      bcur[0] = bnext[0];
      bcur[1] = bnext[1];
    }
  };

  // One k-tile, with tile kt's fragments already in registers: wait for tile kt+1's copies (and
  // for the reads of tile kt's fragments: lgkmcnt(0)), barrier -- now no wave reads stage kt % 3
  // any more and tile kt+1 is visible -- start the copies of tile kt+3 into stage kt % 3
  // (clamped: past the end they copy the last tile again into a stage no wave reads), read tile
  // kt+1's fragments, then compute tile kt.  Steps past the last tile (completing a round of six)
  // wait, copy and read like the others, so that the wait counts are the same on every path, and
  // compute nothing.
  auto step = [&](int kt, uint8_t* free_stage, const uint8_t* next_stage, const Frag& cur, Frag& nxt)
                  __attribute__((always_inline)) {
    wait_vmcnt_lgkm0<L>();
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    copy_tile(kt + 3 < KT ? kt + 3 : KT - 1, free_stage);
    __builtin_amdgcn_sched_barrier(0);
    load_frag(next_stage, nxt);
    if (kt < KT) compute(cur);
  };

  // x row scales of the tile (read in the epilogue; the first barrier publishes them)
  for (int i = tid; i < BM; i += 256) sXs[i] = m0 + i < M ? xsc[m0 + i] : 0.0f;
  if constexpr (TWO) {
    // two stages: tile kt+1 is copied while tile kt is computed
    auto step2 = [&](int kt, const uint8_t* cur, uint8_t* other) __attribute__((always_inline)) {
      wait_vmcnt_lgkm0<0>();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      copy_tile(kt + 1 < KT ? kt + 1 : KT - 1, other);
      __builtin_amdgcn_sched_barrier(0);
      if (kt < KT) {
        Frag f;
        load_frag(cur, f);
        compute(f);
      }
    };
    if (KT > 0) {
      copy_tile(0, st0);
      for (int kt = 0; kt < KT; kt += 2) {
        step2(kt, st0, st1);
        step2(kt + 1, st1, st0);
      }
      wait_vmcnt<0>();
    }
  } else if (KT > 0) {
    Frag f0, f1;
    copy_tile(0, st0);
    copy_tile(KT > 1 ? 1 : 0, st1);
    copy_tile(KT > 2 ? 2 : 0, st2);
    wait_vmcnt_lgkm0<2 * L>();
    __builtin_amdgcn_s_barrier();
    load_frag(st0, f0);
    // tile t lives in stage t % 3 and its fragments in f(t % 2)
    for (int kt = 0; kt < KT; kt += 6) {
      step(kt, st0, st1, f0, f1);
      step(kt + 1, st1, st2, f1, f0);
      step(kt + 2, st2, st0, f0, f1);
      step(kt + 3, st0, st1, f1, f0);
      step(kt + 4, st1, st2, f0, f1);
      step(kt + 5, st2, st0, f1, f0);
    }
    wait_vmcnt<0>();  // no copy may still be writing LDS when the workgroup ends
  }
  __syncthreads();

  // Epilogue: lane holds column l32 of each 32x32 tile, rows 8*(r/4) + 4*h + (r%4).
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int64_t col = n0 + wn * 64 + ct * 32 + l32;
    if (col >= N) continue;
    const float cs = wsc[col];
    const float add = layer_bias ? (lb_bf16 ? bf16_bits_to_f32(layer_bias[col]) : f16_bits_to_f32(layer_bias[col]))
                                 : 0.0f;
#pragma unroll
    for (int rt = 0; rt < 4; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = wm * 128 + rt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int64_t row = m0 + lr;
        if (row >= M) continue;
        if (part)
          part[(split * M + row) * N + col] = acc[rt][ct][r] * (sXs[lr] * cs);
        else
          store_out(y, row * N + col, acc[rt][ct][r] * (sXs[lr] * cs) + add, ydt);
      }
  }
}

// ---------------------------------------------------------------- ping-pong kernel
// Output of one wave of the ping-pong kernel (x rows wrow0 .. + 32 RT of the tile, columns ncol0 ..
// + 63), for y rows of 16-byte multiples (N a multiple of 8, y 16-byte aligned): one 32-row block at
// a time, the scaled values (acc * x row scale * column scale + layer bias, rounded once to y's
// dtype) go into this wave's part of the LDS stages, row-major with a padded pitch (the two lane
// halves' rows 4 apart land on distinct banks), then each lane writes whole 16-byte pieces of rows.
// ESZ = bytes per output element.
template <int ESZ, int RT>
__device__ __forceinline__ void pp_store(const f32x16_t (&acc)[RT][2], const float* sXs, const float* __restrict__ wsc,
                                         const uint16_t* __restrict__ lbias, int lb_bf16, int64_t M, int64_t N,
                                         int64_t m0, int wrow0, int64_t ncol0, uint8_t* st0, uint8_t* st1,
                                         uint8_t* st2, int stage_bytes, void* __restrict__ y, int ydt) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5;
  constexpr int P = 64 * ESZ + 32;        // LDS pitch of a block row (bytes)
  constexpr int BLK = 32 * P;             // one 32-row block
  constexpr int CPR = 64 * ESZ / 16;      // 16-byte pieces per row
  const int per_stage = stage_bytes / BLK;
  uint8_t* wbuf = wave < per_stage ? st0 + wave * BLK
                                   : (wave < 2 * per_stage ? st1 + (wave - per_stage) * BLK
                                                           : st2 + (wave - 2 * per_stage) * BLK);
  float cs[2], add[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int64_t col = ncol0 + ct * 32 + l32;
    const bool ok = col < N;
    cs[ct] = ok ? wsc[col] : 0.0f;
    add[ct] = (ok && lbias) ? (lb_bf16 ? bf16_bits_to_f32(lbias[col]) : f16_bits_to_f32(lbias[col])) : 0.0f;
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float xs[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4_t v = *(const f32x4_t*)(sXs + wrow0 + rt * 32 + 8 * q + 4 * h);
      xs[4 * q + 0] = v[0];
      xs[4 * q + 1] = v[1];
      xs[4 * q + 2] = v[2];
      xs[4 * q + 3] = v[3];
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float v = acc[rt][ct][r] * (xs[r] * cs[ct]) + add[ct];
        uint8_t* dst = wbuf + (8 * (r >> 2) + 4 * h + (r & 3)) * P + (ct * 32 + l32) * ESZ;
        if constexpr (ESZ == 4)
          *(float*)dst = v;
        else
          *(uint16_t*)dst = (uint16_t)(ydt == DT_BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v));
      }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the block is in LDS for every lane
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < CPR / 2; ++j) {
      const int i = j * 64 + lane;
      const int row = i / CPR, c = i % CPR;
      const int64_t grow = m0 + wrow0 + rt * 32 + row;
      const int64_t gcol = ncol0 + c * (16 / ESZ);
      const u32x4_t v = *(const u32x4_t*)(wbuf + row * P + c * 16);
      if (grow < M && gcol < N) *(u32x4_t*)((uint8_t*)y + (grow * N + gcol) * ESZ) = v;
    }
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // the reads are done before the next block is written
    asm volatile("" ::: "memory");
  }
}

// Records of the ping-pong kernel: group-major, rec4[group * n + row] = S | B << 16 (the fp16 pair
// of the four-wave kernel's records), so that the records of one group for 32 consecutive rows are
// 128 contiguous bytes.
// One workgroup per 64 weight rows: each wave finds the power of two of 16 rows, then all threads
// write the records group by group (64 rows, 256 contiguous bytes, per group).
template <typename PT>
__device__ __forceinline__ void wprep_pp_block(int64_t blk, const uint16_t* __restrict__ scales,
                                               const uint16_t* __restrict__ biases, int64_t N, int groups,
                                               uint32_t* __restrict__ rec4, float* __restrict__ wsc) {
  // One workgroup per 32 weight rows: the rows' (scale, bias) bit pairs are read into LDS, eight
  // threads per row, while the row's power of two is found; then the records are written group by
  // group (32 rows, 128 contiguous bytes, per group).
  extern __shared__ uint32_t s_pair[];  // [32][groups + 1]
  __shared__ int s_v[32];
  const int tid = threadIdx.x;
  const int64_t n0 = blk * 32;
  const int pitch = groups + 1;
  {
    // eight threads per row; with 16-byte aligned rows (groups a multiple of 8, aligned arrays)
    // thread (r, part) reads the row's 8-group chunks part, part + 8, ... as 16-byte loads, four
    // passes' loads issued before any is used; otherwise the groups part, part + 8, ... one by one
    const int r = tid >> 3, part = tid & 7;
    const int64_t n = n0 + r;
    float smax = 0.0f, bmax = 0.0f;
    const bool wide = (groups & 7) == 0 && (((uintptr_t)scales | (uintptr_t)biases) & 15) == 0;
    if (n < N && !wide) {
      const uint16_t* sr = scales + n * groups;
      const uint16_t* br = biases + n * groups;
      for (int g = part; g < groups; g += 8) {
        const uint32_t sbits = sr[g], bbits = br[g];
        s_pair[r * pitch + g] = sbits | (bbits << 16);
        smax = fmaxf(smax, fabsf(param_to_f32<PT>(sbits)));
        bmax = fmaxf(bmax, fabsf(param_to_f32<PT>(bbits)));
      }
    }
    if (n < N && wide) {
      const uint16_t* sr = scales + n * groups;
      const uint16_t* br = biases + n * groups;
      const int chunks = groups / 8;
      for (int c0 = part; c0 < chunks; c0 += 8 * 4) {
        u32x4_t sv[4], bv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = c0 + 8 * u;
          if (c < chunks) {
            sv[u] = *(const u32x4_t*)(sr + 8 * c);
            bv[u] = *(const u32x4_t*)(br + 8 * c);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int c = c0 + 8 * u;
          if (c < chunks) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const uint32_t sbits = (sv[u][e >> 1] >> (16 * (e & 1))) & 0xffffu;
              const uint32_t bbits = (bv[u][e >> 1] >> (16 * (e & 1))) & 0xffffu;
              s_pair[r * pitch + 8 * c + e] = sbits | (bbits << 16);
              smax = fmaxf(smax, fabsf(param_to_f32<PT>(sbits)));
              bmax = fmaxf(bmax, fabsf(param_to_f32<PT>(bbits)));
            }
          }
        }
      }
    }
#pragma unroll
    for (int off = 4; off >= 1; off >>= 1) {
      smax = fmaxf(smax, __shfl_xor(smax, off));
      bmax = fmaxf(bmax, __shfl_xor(bmax, off));
    }
    // the same power of two as the four-wave kernel's records (S and B exact fp16 values)
    int v = -126;
    if (smax > 0.0f) {
      int e;
      (void)__builtin_frexpf(smax, &e);
      v = max(v, e + 9);
    }
    if (bmax > 0.0f) {
      int e;
      (void)__builtin_frexpf(bmax, &e);
      v = max(v, e - 15);
    }
    if (smax == 0.0f && bmax == 0.0f) v = 0;
    v = min(v, 127);
    if (part == 0 && n < N) {
      s_v[r] = v;
      wsc[n] = __builtin_ldexpf(1.0f, v);
    }
  }
  __syncthreads();
  const int r = tid & 31;
  const int64_t n = n0 + r;
  if (n >= N) return;
  const int v = s_v[r];
  for (int g = tid >> 5; g < groups; g += 8) {
    const uint32_t pr = s_pair[r * pitch + g];
    const float sv = param_to_f32<PT>(pr & 0xffffu), bv = param_to_f32<PT>(pr >> 16);
    const uint32_t S = __builtin_bit_cast(uint16_t, (_Float16)__builtin_ldexpf(sv, 24 - v));
    const uint32_t B = __builtin_bit_cast(uint16_t, (_Float16)__builtin_ldexpf(bv, -v));
    rec4[(int64_t)g * N + n] = S | (B << 16);
  }
}

// One or more weights that share x (up to four: the projections a layer feeds from one input),
// their 256-row n-tiles numbered one after another.
struct PPWeight {
  const uint32_t* packed;
  const uint32_t* rec4;
  const float* wsc;
  const uint16_t* layer_bias;
  void* y;
  int64_t n;
  int64_t tile0;  // first n-tile of this weight in the launch
};
struct PPArgs {
  const uint16_t* x16;
  const float* xsc;
  int64_t M, Kp, K;
  int groups, lb_bf16, ydt, nw;
  PPWeight w[4];
};
struct PPPrepW {
  const uint16_t* scales;
  const uint16_t* biases;
  uint32_t* rec4;
  float* wsc;
  int64_t n;
  int64_t blk0;  // first workgroup of this weight's records
};
struct PPPrep {
  const uint16_t* x;
  uint16_t* x16;
  float* xsc;
  int64_t M, K, Kp, wblocks;
  int groups, nw;
  PPPrepW w[4];
};
// The x pre-pass (workgroups 0 .. M-1) and the record pre-pass of every weight in one launch.
template <typename XT, typename PT, int BITS>
__global__ __launch_bounds__(256) void prep_pp_kernel(const PPPrep p) {
  // the weights' record blocks first (workgroups 0 .. wblocks-1), then one workgroup per x row
  const int64_t b = blockIdx.x;
  if (b >= p.wblocks) {
    xprep16_row<XT, BITS>(b - p.wblocks, p.x, p.M, p.K, p.Kp, p.x16, p.xsc);
    return;
  }
  int j = 0;
#pragma unroll
  for (int i = 1; i < 4; ++i)
    if (i < p.nw && b >= p.w[i].blk0) j = i;
  wprep_pp_block<PT>(b - p.w[j].blk0, p.w[j].scales, p.w[j].biases, p.w[j].n, p.groups, p.w[j].rec4, p.w[j].wsc);
}

// 512 threads: eight waves, two per SIMD.  Workgroup tile BMT (m) x 256 (n) x BK (k): BK = 128 at
// 4 bits and 64 at 8 bits, so that a weight row's codes of one k-tile are 64 contiguous bytes (one
// full request).  Waves 0-3 (group 0) own weight rows 0-127 of the tile, waves 4-7 (group 1) rows
// 128-255; inside a group, wave (wm, wn) = ((w % 4) / 2, w % 2) owns x rows [BMT/2 wm, +BMT/2) and
// weight rows [64 wn, +64) of its group's half: (BMT/64) x 2 products of 32x32 per k-step,
// accumulators private to the wave.
// The two groups alternate roles every phase (ping-pong): one issues the products of a k-tile with
// all operands already in registers, while the other issues its half of the HBM->LDS copies of the
// tile two ahead, reads its fragments of the current tile from LDS and dequantizes them; a barrier
// ends each phase.  Group 1 trails group 0 by one phase, so each SIMD's matrix core is fed by one of
// its two waves at a time.  Three LDS stages: tile t in stage t % 3, read in phases 2t (group 0) and
// 2t+1 (group 1); the copies of tile t+2 go to stage (t+2) % 3 during the mem phases of tile t and
// their issuing waves wait for them at the end of the mem phases of tile t+1.
// k-slots: lane half h at k-step t takes the 8-value chunk c = KS h + t (KS = BK / 16 steps), so a
// lane's codes of a tile are 32 consecutive bytes of its row; x is staged as BK / 64 halves of 64
// values ([half][row][8 slots]), chunk c in half c / 8, slot c % 8.
// Records: the stage holds RW words per weight row (the tile's groups, zero past the last one) in
// blocks of 32 rows ([row / 32][word][row % 32]), copied 4 bytes per lane from rec4.
template <int BITS, int G, int BMT>
__global__ __launch_bounds__(512) void gemm_pp_kernel(const PPArgs a) {
  constexpr int BK = BITS == 4 ? 128 : 64;
  constexpr int KS = BK / 16;                      // k-steps of 16 per tile
  constexpr int HALVES = BK / 64;                  // 64-value x blocks per tile
  constexpr int WM = BMT / 2;                      // x rows per wave
  constexpr int RT = WM / 32;                      // 32-row tiles per wave
  constexpr int B_ROW = BK * BITS / 8;             // 64 bytes of codes per weight row and tile
  constexpr int A_HALF = BMT * 128;
  constexpr int A_BYTES = HALVES * A_HALF;
  constexpr int B_BYTES = 256 * B_ROW;
  constexpr int GPK = BK / G > 0 ? BK / G : 1;     // groups a tile touches
  constexpr int RW = GPK <= 2 ? 2 : 4;             // record words per row in a stage
  constexpr int R_BYTES = 256 * RW * 4;
  constexpr int STAGE = A_BYTES + B_BYTES + R_BYTES;
  constexpr int NA = HALVES * (BMT / 64);          // x copies per thread and mem phase
  constexpr int NB = 2;                            // code copies
  constexpr int NR = RW / 2;                       // record copies
  constexpr int NC = NA + NB + NR;
  static_assert(B_ROW == 64, "64-byte code rows per tile");
  // distinct arrays per stage: the compiler then knows that fragment reads of one stage do not
  // alias the copies in flight into another, and does not wait for those copies before the reads
  __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st2[STAGE];
  __shared__ __attribute__((aligned(16))) float sXs[BMT];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int grp = wave >> 2, w4 = wave & 3;
  const int wm = w4 >> 1, wn = w4 & 1;
  const int l32 = lane & 31, h = lane >> 5;
  const int w4_u = __builtin_amdgcn_readfirstlane(w4);
  const int grp_u = __builtin_amdgcn_readfirstlane(grp);

  const int64_t M = a.M;
  const int64_t m_tiles = (M + BMT - 1) / BMT;
  // Tile order: workgroups are dealt round-robin to the 8 XCDs, so workgroup w runs on XCD w % 8.
  // Each XCD takes a contiguous range of virtual tile ids, and ids run m-fastest inside bands of
  // GEMM_PP_BAND m-tiles: the workgroups an XCD runs at once share a few x tiles and a few weight
  // tiles in its L2 instead of every weight tile.
  const int64_t T = (int64_t)gridDim.x;
  int64_t v = blockIdx.x;
  if (T % 8 == 0) v = (int64_t)(blockIdx.x % 8) * (T / 8) + blockIdx.x / 8;
  int64_t mt, nt;
  {
    const int64_t n_tiles = T / m_tiles;
    const int64_t band = m_tiles % GEMM_PP_BAND == 0 ? GEMM_PP_BAND : 1;
    const int64_t per_band = band * n_tiles;
    const int64_t b = v / per_band, r = v % per_band;
    mt = b * band + r % band;
    nt = r / band;
  }
  int wi = 0;
#pragma unroll
  for (int j = 1; j < 4; ++j)
    if (j < a.nw && nt >= a.w[j].tile0) wi = j;
  const PPWeight W = a.w[wi];
  const int64_t m0 = mt * BMT, n0 = (nt - W.tile0) * 256;
  const int64_t N = W.n;
  const int64_t KB = a.Kp / 64;                    // 64-value x blocks
  const int KT = (int)((KB + HALVES - 1) / HALVES);
  const int64_t row_bytes = a.K * BITS / 8;
  const int groups = a.groups;

  const uint32_t mk = vconst(BITS == 4 ? 0x000F000Fu : 0x00FF00FFu);

  // ---- this thread's copies (its group's half of every tile)
  uint32_t a_off[BMT / 64];
#pragma unroll
  for (int i = 0; i < BMT / 64; ++i) {
    const int r = grp * (BMT / 2) + w4 * (BMT / 8) + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ xswz(r);
    a_off[i] = m0 + r < M ? (uint32_t)(((m0 + r) * 64 + 8 * c) * 2) : kOOB;
  }
  uint32_t b_off[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int n = grp * 128 + w4 * 32 + 16 * i + (lane >> 2);
    const int c = (lane & 3) ^ bswz<4>(n);
    b_off[i] = n0 + n < N ? (uint32_t)((n0 + n) * row_bytes + 16 * c) : kOOB;
  }
  const int r_row = grp * 128 + 32 * w4 + l32;  // record copies: row, word 2i + h
  const bool r_ok = n0 + r_row < N;
  const __amdgpu_buffer_rsrc_t rsA = gemm_rsrc(a.x16, M * a.Kp * 2);
  const __amdgpu_buffer_rsrc_t rsB = gemm_rsrc(W.packed, N * row_bytes);
  const __amdgpu_buffer_rsrc_t rsR = gemm_rsrc(W.rec4, N * (int64_t)groups * 4);
  // copy number c (0 .. NC-1) of this thread's share of tile kt: x blocks, then codes, then records
  auto copy_one = [&](int kt, uint8_t* stage, int c) __attribute__((always_inline)) {
    if (c < NA) {
      const int j = c / (BMT / 64), i = c % (BMT / 64);
      const int64_t kb = (int64_t)kt * HALVES + j;
      copy_to_lds<16>(rsA, kb < KB ? a_off[i] : kOOB, (uint32_t)(kb < KB ? kb * M * 128 : 0),
                      stage + j * A_HALF + (grp_u * (BMT / 2) + w4_u * (BMT / 8) + 8 * i) * 128);
    } else if (c < NA + NB) {
      const int i = c - NA;
      copy_to_lds<16>(rsB, kt < KT ? b_off[i] : kOOB, (uint32_t)((int64_t)kt * BK * BITS / 8),
                      stage + A_BYTES + (grp_u * 128 + w4_u * 32 + 16 * i) * B_ROW);
    } else {
      const int i = c - NA - NB;
      const int gk0 = (int)((int64_t)kt * BK / G);
      const int w = 2 * i + h;
      const bool ok = r_ok && w < GPK && gk0 + w < groups;
      const uint32_t off = ok ? (uint32_t)((((int64_t)(gk0 + w)) * N + n0 + r_row) * 4) : kOOB;
      copy_to_lds<4>(rsR, off, 0u,
                     stage + A_BYTES + B_BYTES + (((grp_u * 128 + 32 * w4_u) / 32) * RW + 2 * i) * 128);
    }
  };
  auto copy_half = [&](int kt, uint8_t* stage) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < HALVES; ++j) {
      const int64_t kb = (int64_t)kt * HALVES + j;
#pragma unroll
      for (int i = 0; i < BMT / 64; ++i)
        copy_to_lds<16>(rsA, kb < KB ? a_off[i] : kOOB, (uint32_t)(kb < KB ? kb * M * 128 : 0),
                        stage + j * A_HALF + (grp_u * (BMT / 2) + w4_u * (BMT / 8) + 8 * i) * 128);
    }
    const int64_t k0 = (int64_t)kt * BK;
#pragma unroll
    for (int i = 0; i < NB; ++i)
      copy_to_lds<16>(rsB, b_off[i], (uint32_t)(k0 * BITS / 8),
                      stage + A_BYTES + (grp_u * 128 + w4_u * 32 + 16 * i) * B_ROW);
    const int gk0 = (int)(k0 / G);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const int w = 2 * i + h;
      const bool ok = r_ok && w < GPK && gk0 + w < groups;
      const uint32_t off = ok ? (uint32_t)((((int64_t)(gk0 + w)) * N + n0 + r_row) * 4) : kOOB;
      copy_to_lds<4>(rsR, off, 0u,
                     stage + A_BYTES + B_BYTES + (((grp_u * 128 + 32 * w4_u) / 32) * RW + 2 * i) * 128);
    }
  };

  f32x16_t acc[RT][2];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // ---- fragments of one k-tile, read during the mem phase: x chunks (RT row-tiles x KS k-steps),
  // the code words and the group records of the wave's 2 col-tiles.  The codes are dequantized
  // during the compute phase, one k-step ahead of the products that take them.
  u32x4_t fa[RT][KS];
  uint32_t cw[2][8];
  uint32_t sb[2][GPK > 2 ? 2 : 1];
  auto mem_frag = [&](const uint8_t* stage) __attribute__((always_inline)) {
    const uint8_t* sA = stage;
    const uint8_t* sB = stage + A_BYTES;
    const uint32_t* sR = (const uint32_t*)(stage + A_BYTES + B_BYTES);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int n = grp * 128 + wn * 64 + ct * 32 + l32;
      const uint8_t* row = sB + n * B_ROW;
      const int sw = bswz<4>(n);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const u32x4_t v = *(const u32x4_t*)(row + ((2 * h + q) ^ sw) * 16);
        cw[ct][4 * q + 0] = v[0];
        cw[ct][4 * q + 1] = v[1];
        cw[ct][4 * q + 2] = v[2];
        cw[ct][4 * q + 3] = v[3];
      }
      // the group word of the lane's chunks: value offset 8 (KS h + t) of the tile
      const uint32_t* rr = sR + ((n >> 5) * RW) * 32 + l32;
      if constexpr (GPK > 2) {  // 4-bit, groups of 32: two groups per lane half
        sb[ct][0] = rr[(2 * h) * 32];
        sb[ct][1] = rr[(2 * h + 1) * 32];
      } else if constexpr (GPK == 2) {
        sb[ct][0] = rr[(8 * KS * h / G) * 32];
      } else {
        sb[ct][0] = rr[0];
      }
    }
#pragma unroll
    for (int t = 0; t < KS; ++t)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        const int r = wm * WM + rt * 32 + l32;
        const int c = KS * h + t;
        const int slot = c & 7;
        const uint8_t* half = sA + (c >> 3) * A_HALF;
        fa[rt][t] = *(const u32x4_t*)(half + (r * 8 + (slot ^ xswz(r))) * 16);
      }
  };
  const uint32_t mk4 = vconst(0x00F000F0u);
  auto dequant = [&](int t, u32x4_t* bq) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const uint32_t word = GPK > 2 ? sb[ct][t >= KS / 2 ? 1 : 0] : sb[ct][0];
      const f16x2_t sbv = __builtin_bit_cast(f16x2_t, word);
      uint32_t r[4];
      if constexpr (BITS == 4 && GEMM_PP_DEQ16) {
        const _Float16 s16 = sbv[0] * (_Float16)0.0625f;
        Deq<4>::runp16(&cw[ct][t], r, f16x2_t{sbv[0], sbv[0]}, f16x2_t{s16, s16}, f16x2_t{sbv[1], sbv[1]}, mk, mk4);
      } else {
        Deq<BITS>::runp(&cw[ct][t * (BITS / 4)], r, f16x2_t{sbv[0], sbv[0]}, f16x2_t{sbv[1], sbv[1]}, mk);
      }
      bq[ct] = u32x4_t{r[0], r[1], r[2], r[3]};
    }
  };
  // The products of the k-tile; the codes of k-step t+1 are dequantized between the products of
  // step t (one product, then a few vector instructions).
  // With copy_kt >= 0 the copies of tile copy_kt into copy_stage are spread over the products, one
  // after each k-step's products, so that the copy stream is issued evenly over the whole k-tile.
  auto compute = [&](int copy_kt, uint8_t* copy_stage) __attribute__((always_inline)) {
    u32x4_t bcur[2], bnext[2];
    dequant(0, bcur);
#pragma unroll
    for (int t = 0; t < KS; ++t) {
      if (t + 1 < KS) dequant(t + 1, bnext);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) acc[rt][ct] = mfma16(fa[rt][t], bcur[ct], acc[rt][ct]);
      constexpr int per_step = (NC + KS - 1) / KS;
#pragma unroll
      for (int c = t * per_step; c < (t + 1) * per_step && c < NC; ++c)
        if (copy_kt >= 0) copy_one(copy_kt, copy_stage, c);
      if (t + 1 < KS) {
#pragma unroll
        for (int i = 0; i < 2 * RT; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one product
          __builtin_amdgcn_sched_group_barrier(0x002, GEMM_PP_INTERLEAVE, 0);  // vector ALU
        }
        if (copy_kt >= 0 && t * per_step < NC) __builtin_amdgcn_sched_group_barrier(0x020, per_step, 0);  // copies
      }
      bcur[0] = bnext[0];
      bcur[1] = bnext[1];
    }
  };
  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // The dequantized operands of the whole k-tile, made in the mem phase: the vector work then runs
  // while the other wave of the SIMD issues its products, and the compute phase is products only.
  u32x4_t bq[GEMM_PP_DEQ_MEM ? KS : 1][2];
  // One k-tile: mem phase (the copies of tile t+2 into the stage tile t-1 freed, then tile t's
  // fragments; at its end this wave's copies of tile t+1 must have landed), barrier, compute phase
  // (products only), barrier.
  auto step = [&](int t, const uint8_t* cur, uint8_t* free_stage) __attribute__((always_inline)) {
    if (GEMM_PP_COPY_IN_COMPUTE) {
      // mem phase: fragments only; this wave's copies (issued during its previous compute phase)
      // must have landed before the barrier.  Compute phase: the products, with the copies of tile
      // t+2 spread among them.
      mem_frag(cur);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt_lgkm0<0>();
      barrier();
      if (GEMM_PP_PRIO) __builtin_amdgcn_s_setprio(1);
      compute(t + 2 < KT ? t + 2 : -1, free_stage);
      if (GEMM_PP_PRIO) __builtin_amdgcn_s_setprio(0);
      barrier();
      return;
    }
    if (GEMM_PP_DEQ_MEM == 3) {
      // mem phase: fragments and the dequantized codes of tile t; this wave's copies of tile t+1,
      // issued during its previous compute phase, must have landed (vmcnt(0)) before the barrier
      // that precedes the first read of tile t+1.  Compute phase: the products, with this wave's
      // copies of tile t+2 issued among them (one after each k-step's products), so that the
      // copy stream drains over both phases; past the last tile they read nothing (out-of-range
      // offsets) into the free stage.
      mem_frag(cur);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ts = 0; ts < KS; ++ts) {
        dequant(ts, bq[ts]);
        // pin the results in this phase: otherwise they are sunk to their use among the products
        asm volatile("" : "+v"(bq[ts][0]), "+v"(bq[ts][1]));
      }
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt_lgkm0<0>();
      barrier();
      constexpr int per = (NC + KS - 1) / KS;
#pragma unroll
      for (int ts = 0; ts < KS; ++ts) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) acc[rt][ct] = mfma16(fa[rt][ts], bq[ts][ct], acc[rt][ct]);
#pragma unroll
        for (int c = ts * per; c < (ts + 1) * per && c < NC; ++c) copy_one(t + 2, free_stage, c);
        __builtin_amdgcn_sched_barrier(0);
      }
      barrier();
      return;
    }
    if (GEMM_PP_FRAG_FIRST) {
      mem_frag(cur);
      __builtin_amdgcn_sched_barrier(0);
      if (t + 2 < KT) copy_half(t + 2, free_stage);
    } else {
      if (t + 2 < KT) copy_half(t + 2, free_stage);
      __builtin_amdgcn_sched_barrier(0);
      mem_frag(cur);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (t + 2 < KT)
      wait_vmcnt_lgkm0<NC>();
    else
      wait_vmcnt_lgkm0<0>();
    barrier();
    if (GEMM_PP_PRIO) __builtin_amdgcn_s_setprio(1);
    compute(-1, free_stage);
    if (GEMM_PP_PRIO) __builtin_amdgcn_s_setprio(0);
    barrier();
  };

  for (int i = tid; i < BMT; i += 512) sXs[i] = m0 + i < M ? a.xsc[m0 + i] : 0.0f;
  copy_half(0, st0);
  if (KT > 1) copy_half(1, st1);
  wait_vmcnt<0>();
  barrier();                  // tiles 0 and 1 are in LDS
  if (grp_u == 1) barrier();  // group 1 trails group 0 by one phase
  // tile t lives in stage t % 3
  for (int t = 0; t < KT; t += 3) {
    step(t, st0, st2);
    if (t + 1 < KT) step(t + 1, st1, st0);
    if (t + 2 < KT) step(t + 2, st2, st1);
  }
  wait_vmcnt<0>();            // no copy may still be writing LDS when the workgroup ends
  if (grp_u == 0) barrier();  // the same number of barriers on every wave

  // Epilogue: lane holds column l32 of each 32x32 tile, rows 8*(r/4) + 4*h + (r%4).
  const int64_t ncol0 = n0 + grp * 128 + wn * 64;  // the wave's first column
  if (N % 8 == 0 && ((uintptr_t)W.y & 15) == 0) {
    // every copy has landed and no wave reads the stages any more: they take the output blocks
    barrier();
    if (a.ydt == DT_F32)
      pp_store<4, RT>(acc, sXs, W.wsc, W.layer_bias, a.lb_bf16, M, N, m0, wm * WM, ncol0, st0, st1, st2, STAGE, W.y,
                      DT_F32);
    else if (a.ydt == DT_BF16)
      pp_store<2, RT>(acc, sXs, W.wsc, W.layer_bias, a.lb_bf16, M, N, m0, wm * WM, ncol0, st0, st1, st2, STAGE, W.y,
                      DT_BF16);
    else
      pp_store<2, RT>(acc, sXs, W.wsc, W.layer_bias, a.lb_bf16, M, N, m0, wm * WM, ncol0, st0, st1, st2, STAGE, W.y,
                      DT_F16);
    return;
  }
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int64_t col = ncol0 + ct * 32 + l32;
    if (col >= N) continue;
    const float cs = W.wsc[col];
    const float add = W.layer_bias ? (a.lb_bf16 ? bf16_bits_to_f32(W.layer_bias[col]) : f16_bits_to_f32(W.layer_bias[col]))
                                   : 0.0f;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = wm * WM + rt * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
        const int64_t row = m0 + lr;
        if (row >= M) continue;
        store_out(W.y, row * N + col, acc[rt][ct][r] * (sXs[lr] * cs) + add, a.ydt);
      }
  }
}

// Sum of the k-split partial products, plus the layer bias, rounded once to y's dtype.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ part, int splits, int64_t MN,
                                                            int64_t N, const uint16_t* __restrict__ layer_bias,
                                                            int lb_bf16, void* __restrict__ y, int ydt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= MN) return;
  float v = 0.0f;
  for (int s = 0; s < splits; ++s) v += part[s * MN + i];
  if (layer_bias) {
    const uint32_t b = layer_bias[i % N];
    v += lb_bf16 ? bf16_bits_to_f32(b) : f16_bits_to_f32(b);
  }
  store_out(y, i, v, ydt);
}

// Workspace: the fp16 copy of x (m * kp values), its row factors (m floats), the weight records
// (n * k/g pairs of floats) and row factors (n floats), for a launch split over k the fp32
// partial products (splits * m * n), and at the bitstream widths the codes as bytes (n * k), each
// padded to 256 bytes.
inline size_t pad256(size_t b) { return (b + 255u) & ~(size_t)255u; }
inline int64_t kpad(int64_t k) { return (k + BK - 1) / BK * BK; }
constexpr int64_t kCUs = 256;  // compute units of the gfx950 parts this library is built for
// k-splits of a launch: when the output tiles fill less than half of the CUs, up to 4 ranges of at
// least 8 k-tiles each, so that the workgroups reach about one per CU.
inline int gemm_splits(int64_t m, int64_t n, int64_t k) {
  const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  if (tiles * 2 > kCUs) return 1;
  int64_t s = kCUs / tiles;
  s = std::min<int64_t>(s, 4);
  s = std::min<int64_t>(s, kpad(k) / BK / 8);
  return s < 2 ? 1 : (int)s;
}

template <int BITS, bool G32>
hipError_t launch_main(const uint16_t* x16, const float* xsc, int64_t m, int64_t kp, int64_t k,
                       const uint32_t* packed, const float2* rec, const float* wsc, int64_t n, int groups, int g,
                       const uint16_t* lb, int lb_bf16, void* y, int ydt, int splits, float* part, hipStream_t s) {
  const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  if (splits == 1 && tiles >= 2 * kCUs && BITS == 4)
    gemm16_kernel<BITS, G32, true><<<(unsigned)tiles, 256, 0, s>>>(x16, xsc, m, kp, k, packed, rec, wsc, n, groups,
                                                                   g, lb, lb_bf16, y, ydt, 1, nullptr);
  else
    gemm16_kernel<BITS, G32, false><<<(unsigned)(tiles * splits), 256, 0, s>>>(
        x16, xsc, m, kp, k, packed, rec, wsc, n, groups, g, lb, lb_bf16, y, ydt, splits, part);
  return hipGetLastError();
}

#ifndef GEMM_PP
#define GEMM_PP 1
#endif
#ifndef GEMM_PP_MIN_TILES
#define GEMM_PP_MIN_TILES 128  // ping-pong kernel when its 128 x 256 tiles are at least this many
#endif
// One weight of a launch over weights that share x.
struct GemmW {
  const uint32_t* packed;
  const void* scales;
  const void* biases;
  const void* layer_bias;
  void* y;
  int64_t n;
};
// Workspace of a launch over weights sharing x: the fp16 copy of x and its row factors, then per
// weight the records (n * k/g words; the four-wave kernel's pairs take twice that) and row factors.
size_t ws_x_bytes(int64_t m, int64_t k) { return pad256((size_t)(m * kpad(k)) * 2u) + pad256((size_t)m * 4u); }
size_t ws_w_bytes(int64_t n, int64_t k, int g) { return pad256((size_t)(n * (k / g)) * 8u) + pad256((size_t)n * 4u); }

inline int64_t pp_tiles(int64_t m, const GemmW* w, int nw) {
  int64_t nt = 0;
  for (int j = 0; j < nw; ++j) nt += (w[j].n + 255) / 256;
  return (m + 127) / 128 * nt;
}
// (the record pre-pass stages 32 rows of k/g parameter pairs in at most 64 KiB of LDS)
inline bool pp_eligible(int64_t m, int64_t k, int g, const GemmW* w, int nw) {
  return GEMM_PP && 32 * (k / g + 1) * 4 <= 65536 && pp_tiles(m, w, nw) >= GEMM_PP_MIN_TILES;
}

// The ping-pong path over nw <= 4 weights sharing x: one pre-pass launch (x and every weight's
// records), one product launch.
template <int BITS, typename XT, typename PT>
hipError_t launch_pp(const void* x, int64_t m, int64_t k, const GemmW* w, int nw, int g, int ydt, void* ws,
                     hipStream_t s) {
  const int64_t kp = kpad(k);
  const int groups = (int)(k / g);
  uint8_t* p = (uint8_t*)ws;
  uint16_t* x16 = (uint16_t*)p;
  float* xsc = (float*)(p + pad256((size_t)(m * kp) * 2u));
  p += ws_x_bytes(m, k);
  PPPrep pr{};
  pr.x = (const uint16_t*)x;
  pr.x16 = x16;
  pr.xsc = xsc;
  pr.M = m;
  pr.K = k;
  pr.Kp = kp;
  pr.groups = groups;
  pr.nw = nw;
  PPArgs pa{};
  pa.x16 = x16;
  pa.xsc = xsc;
  pa.M = m;
  pa.Kp = kp;
  pa.K = k;
  pa.groups = groups;
  pa.lb_bf16 = std::is_same<XT, BF16>::value ? 1 : 0;
  pa.ydt = ydt;
  pa.nw = nw;
  int64_t blk = 0, nt = 0;
  for (int j = 0; j < nw; ++j) {
    uint32_t* rec4 = (uint32_t*)p;
    float* wsc = (float*)(p + pad256((size_t)(w[j].n * groups) * 8u));
    p += ws_w_bytes(w[j].n, k, g);
    pr.w[j] = PPPrepW{(const uint16_t*)w[j].scales, (const uint16_t*)w[j].biases, rec4, wsc, w[j].n, blk};
    blk += (w[j].n + 31) / 32;
    pa.w[j] = PPWeight{w[j].packed, rec4, wsc, (const uint16_t*)w[j].layer_bias, w[j].y, w[j].n, nt};
    nt += (w[j].n + 255) / 256;
  }
  pr.wblocks = blk;
  prep_pp_kernel<XT, PT, BITS><<<(unsigned)(blk + m), 256, (size_t)32 * (groups + 1) * 4, s>>>(pr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)((m + 127) / 128 * nt);
  if (g == 32)
    gemm_pp_kernel<BITS, 32, 128><<<grid, 512, 0, s>>>(pa);
  else if (g == 64)
    gemm_pp_kernel<BITS, 64, 128><<<grid, 512, 0, s>>>(pa);
  else
    gemm_pp_kernel<BITS, 128, 128><<<grid, 512, 0, s>>>(pa);
  return hipGetLastError();
}

template <int BITS, typename XT, typename PT>
hipError_t launch_t(const void* x, int64_t m, int64_t k, const uint32_t* packed, const void* scales,
                    const void* biases, int64_t n, int g, const void* layer_bias, void* y, int ydt, void* ws,
                    hipStream_t s) {
  {
    const GemmW w1{packed, scales, biases, layer_bias, y, n};
    if (pp_eligible(m, k, g, &w1, 1)) return launch_pp<BITS, XT, PT>(x, m, k, &w1, 1, g, ydt, ws, s);
  }
  const int64_t kp = kpad(k);
  const int groups = (int)(k / g);
  const int splits = gemm_splits(m, n, k);
  uint8_t* p = (uint8_t*)ws;
  uint16_t* x16 = (uint16_t*)p;
  p += pad256((size_t)(m * kp) * 2u);
  float* xsc = (float*)p;
  p += pad256((size_t)m * 4u);
  float2* rec = (float2*)p;
  p += pad256((size_t)(n * groups) * 8u);
  float* wsc = (float*)p;
  p += pad256((size_t)n * 4u);
  float* part = splits > 1 ? (float*)p : nullptr;
  prep16_kernel<XT, PT, BITS><<<(unsigned)(m + (n + 3) / 4), 256, 0, s>>>(
      (const uint16_t*)x, m, k, kp, x16, xsc, (const uint16_t*)scales, (const uint16_t*)biases, n, groups, rec, wsc);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int lb_bf16 = std::is_same<XT, BF16>::value ? 1 : 0;
  const uint16_t* lb = (const uint16_t*)layer_bias;
  e = g == 32 ? launch_main<BITS, true>(x16, xsc, m, kp, k, packed, rec, wsc, n, groups, g, lb, lb_bf16, y, ydt, splits,
                                        part, s)
              : launch_main<BITS, false>(x16, xsc, m, kp, k, packed, rec, wsc, n, groups, g, lb, lb_bf16, y, ydt,
                                         splits, part, s);
  if (e != hipSuccess || splits == 1) return e;
  const int64_t mn = m * n;
  splitk_reduce_kernel<<<(unsigned)((mn + 255) / 256), 256, 0, s>>>(part, splits, mn, n, lb, lb_bf16, y, ydt);
  return hipGetLastError();
}

// Bitstream widths (2, 3, 5, 6 bits): each lane turns one 32-code chunk of a row (BITS words) into
// its 32 codes as bytes, so that the 8-bit kernel reads them (byte i of a row: code i, the 8-bit
// affine layout).
template <int BITS>
__global__ __launch_bounds__(256) void stream_to_bytes_kernel(const uint32_t* __restrict__ packed, int64_t n,
                                                              int64_t k, uint8_t* __restrict__ codes8) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= n * (k / 32)) return;
  const uint32_t* src = packed + t * BITS;  // chunks are consecutive: row r, chunk c at r * k/32 + c
  uint32_t w[BITS];
#pragma unroll
  for (int i = 0; i < BITS; ++i) w[i] = src[i];
  uint32_t o[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    o[j] = stream_code<BITS>(w, 4 * j) | (stream_code<BITS>(w, 4 * j + 1) << 8) |
           (stream_code<BITS>(w, 4 * j + 2) << 16) | (stream_code<BITS>(w, 4 * j + 3) << 24);
  u32x4_t* dst = (u32x4_t*)(codes8 + t * 32);
  dst[0] = u32x4_t{o[0], o[1], o[2], o[3]};
  dst[1] = u32x4_t{o[4], o[5], o[6], o[7]};
}

size_t gemm_base_bytes(int64_t m, int64_t n, int64_t k, int g) {
  const int splits = gemm_splits(m, n, k);
  return pad256((size_t)(m * kpad(k)) * 2u) + pad256((size_t)m * 4u) + pad256((size_t)(n * (k / g)) * 8u) +
         pad256((size_t)n * 4u) + (splits > 1 ? pad256((size_t)(splits * m * n) * 4u) : 0u);
}

}  // namespace

// The regions above, then (bitstream widths) the codes as bytes, n * k.
size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int bits, int g) {
  return gemm_base_bytes(m, n, k, g) + (is_stream_bits(bits) ? pad256((size_t)(n * k)) : 0u);
}

hipError_t launch_gemm(const void* x, int xdt, int64_t m, int64_t k, const uint32_t* packed, const void* scales,
                       const void* biases, int pdt, int64_t n, int bits, int g, const void* layer_bias, void* y,
                       int ydt, void* ws, hipStream_t s);

// Weights that share x: one pre-pass and one ping-pong launch over all of them when the shape
// suits that kernel (4- and 8-bit codes, enough tiles), else one qlinear_gemm launch sequence per
// weight.  Either way each weight's result is the one its own qlinear_gemm call gives when that
// call takes the ping-pong kernel (the tiles and their sums do not depend on the other weights).
bool gemm_grouped_pp(int64_t m, int64_t k, const GemmWeight* w, int count, int bits, int g) {
  if (bits != 4 && bits != 8 && !is_stream_bits(bits)) return false;
  GemmW ww[4];
  for (int j = 0; j < count; ++j) ww[j] = GemmW{w[j].packed, w[j].scales, w[j].biases, w[j].layer_bias, w[j].y, w[j].n};
  return pp_eligible(m, k, g, ww, count);
}

// With the ping-pong launch at the bitstream widths, every weight's codes as bytes follow (n * k
// bytes each, padded to 256).
size_t gemm_grouped_workspace_bytes(int64_t m, int64_t k, const GemmWeight* w, int count, int bits, int g) {
  size_t pp = ws_x_bytes(m, k), single = 0;
  for (int j = 0; j < count; ++j) {
    pp += ws_w_bytes(w[j].n, k, g) + (is_stream_bits(bits) ? pad256((size_t)(w[j].n * k)) : 0u);
    single = std::max(single, gemm_workspace_bytes(m, w[j].n, k, bits, g));
  }
  return gemm_grouped_pp(m, k, w, count, bits, g) ? pp : single;
}

// Bitstream rows (2, 3, 5, 6 bits) -> one byte per code (the 8-bit layout) at codes8.
hipError_t launch_stream_to_bytes(const uint32_t* packed, int64_t n, int64_t k, int bits, uint8_t* codes8,
                                  hipStream_t s) {
  const unsigned nb = (unsigned)((n * (k / 32) + 255) / 256);
  if (bits == 2)
    stream_to_bytes_kernel<2><<<nb, 256, 0, s>>>(packed, n, k, codes8);
  else if (bits == 3)
    stream_to_bytes_kernel<3><<<nb, 256, 0, s>>>(packed, n, k, codes8);
  else if (bits == 5)
    stream_to_bytes_kernel<5><<<nb, 256, 0, s>>>(packed, n, k, codes8);
  else
    stream_to_bytes_kernel<6><<<nb, 256, 0, s>>>(packed, n, k, codes8);
  return hipGetLastError();
}

hipError_t launch_gemm_grouped(const void* x, int xdt, int64_t m, int64_t k, const GemmWeight* w, int count, int pdt,
                               int bits, int g, int ydt, void* ws, hipStream_t s) {
  if (!gemm_grouped_pp(m, k, w, count, bits, g)) {
    for (int j = 0; j < count; ++j) {
      if (w[j].n == 0) continue;
      const hipError_t e = launch_gemm(x, xdt, m, k, w[j].packed, w[j].scales, w[j].biases, pdt, w[j].n, bits, g,
                                       w[j].layer_bias, w[j].y, ydt, ws, s);
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  GemmW ww[4];
  int nw = 0;
  // bitstream widths: every weight's codes become bytes after the ping-pong launch's own workspace,
  // and the launch takes them as 8-bit codes
  uint8_t* codes8 = (uint8_t*)ws + ws_x_bytes(m, k);
  for (int j = 0; j < count; ++j) codes8 += ws_w_bytes(w[j].n, k, g);
  for (int j = 0; j < count; ++j) {
    if (w[j].n == 0) continue;
    const uint32_t* packed = w[j].packed;
    if (is_stream_bits(bits)) {
      const hipError_t e = launch_stream_to_bytes(w[j].packed, w[j].n, k, bits, codes8, s);
      if (e != hipSuccess) return e;
      packed = (const uint32_t*)codes8;
      codes8 += pad256((size_t)(w[j].n * k));
    }
    ww[nw++] = GemmW{packed, w[j].scales, w[j].biases, w[j].layer_bias, w[j].y, w[j].n};
  }
  if (is_stream_bits(bits)) bits = 8;
  const bool xb = xdt == DT_BF16, pb = pdt == DT_BF16;
  if (bits == 4) {
    if (xb && pb) return launch_pp<4, BF16, BF16>(x, m, k, ww, nw, g, ydt, ws, s);
    if (xb) return launch_pp<4, BF16, F16>(x, m, k, ww, nw, g, ydt, ws, s);
    if (pb) return launch_pp<4, F16, BF16>(x, m, k, ww, nw, g, ydt, ws, s);
    return launch_pp<4, F16, F16>(x, m, k, ww, nw, g, ydt, ws, s);
  }
  if (xb && pb) return launch_pp<8, BF16, BF16>(x, m, k, ww, nw, g, ydt, ws, s);
  if (xb) return launch_pp<8, BF16, F16>(x, m, k, ww, nw, g, ydt, ws, s);
  if (pb) return launch_pp<8, F16, BF16>(x, m, k, ww, nw, g, ydt, ws, s);
  return launch_pp<8, F16, F16>(x, m, k, ww, nw, g, ydt, ws, s);
}

hipError_t launch_gemm(const void* x, int xdt, int64_t m, int64_t k, const uint32_t* packed, const void* scales,
                       const void* biases, int pdt, int64_t n, int bits, int g, const void* layer_bias, void* y,
                       int ydt, void* ws, hipStream_t s) {
  const bool xb = xdt == DT_BF16, pb = pdt == DT_BF16;
  if (is_stream_bits(bits)) {
    uint8_t* codes8 = (uint8_t*)ws + gemm_base_bytes(m, n, k, g);
    const hipError_t e = launch_stream_to_bytes(packed, n, k, bits, codes8, s);
    if (e != hipSuccess) return e;
    packed = (const uint32_t*)codes8;
    bits = 8;
  }
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
