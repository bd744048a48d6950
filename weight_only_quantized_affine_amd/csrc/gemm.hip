// Prefill GEMM on affine-quantized weights with the CDNA4 matrix cores:
//   y[m,n] = sum_g s[n,g] * sum_{k in g} x[m,k] q[n,k]  +  sum_g b[n,g] * X[m,g],
// where X[m,g] = sum_{k in g} x[m,k].  This is the block-scaled contraction of the Nx_quant API
// docs (Products: apply; a tensor-core product scales each block's partial sum): the codes enter
// the bf16/f16 MFMA as exact small values, each group's fp32 partial sum is multiplied by its
// fp32 scale, and the additive bias of the MLX affine storage (GPTQModel wiki "MLX Apple
// Silicon", Concepts) enters through X.  No weight value is ever rounded to 16 bits, so the
// result carries fp32 accumulation error only.
//
// Encodings of a code q as an MFMA operand (exact):
//   4 bits: 1 + q/16, i.e. bits 0x3F80 | q << 3 (bf16) or 0x3C00 | q << 6 (f16); then
//           sum x*(1 + q/16) = X + P/16, so  s*P = 16s*P' - 16s*X  and -16s joins the bias.
//   8 bits: q itself (v_cvt_f32_ubyte + pack).
// The X-terms X*(b - 16s) are one extra MFMA per two groups inside the k-loop: A = the bf16
// hi/lo split of X, B = the bf16 hi/lo split of b and of -16s.
//
// Three launches: xprep (group sums of x and, for 4-bit codes, x permuted to the unpacking
// order), wprep (a 16-byte record per row and group: fp32 fold scale and the bf16 hi/lo
// operands of b and -16s), then the main kernel.  Groups of 128 run as two sub-groups of 64
// with the same record.
//
// Main kernel tiling: 256 threads (4 waves, 2x2), workgroup tile 128 (m) x 128 (n) x 64 (k), each
// wave a 64x64 block of 2x2 v_mfma_f32_32x32x16 tiles.  x and packed code tiles go straight from
// HBM into three LDS stages (two tiles ahead of the compute); the codes stay packed in LDS and
// each wave unpacks its own fragments in registers.
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

// Split an fp32 value into bf16 hi + lo (hi = RNE(v), lo = RNE(v - hi)).
__device__ __forceinline__ void split_bf16(float v, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_bits(v);
  lo = f32_to_bf16_bits(v - bf16_bits_to_f32(hi));
}

// ---------------------------------------------------------------- pre-pass over x
// Per (row, group): X[m, g] = sum of the group's x values (fp32, stored as bf16 hi | lo << 16)
// and, for 4-bit codes, a copy of the group's x values permuted per 8 to the order the 4-bit
// unpacking yields (x0,x4,x1,x5,x2,x6,x3,x7), so the main loop can copy x straight into LDS.

// Permute 8 consecutive 16-bit x values to the order the 4-bit unpacking yields: x0,x4,x1,x5,x2,x6,x3,x7.
__device__ __forceinline__ u32x4_t perm8(const u32x4_t& u) {
  u32x4_t r;
  r[0] = perm(u[2], u[0], 0x05040100u);
  r[1] = perm(u[2], u[0], 0x07060302u);
  r[2] = perm(u[3], u[1], 0x05040100u);
  r[3] = perm(u[3], u[1], 0x07060302u);
  return r;
}

// One thread per 16-byte chunk of x (8 values); the g/8 threads of a group are consecutive lanes
// and reduce their partial sums with lane exchanges.
template <typename XT, bool PERM>
__global__ __launch_bounds__(256) void xprep_kernel(const uint16_t* __restrict__ x, int64_t m, int64_t k, int g,
                                                    uint32_t* __restrict__ xs, uint16_t* __restrict__ xp) {
  const int64_t chunks = m * k / 8;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int lpg = g / 8;  // lanes per group: 4, 8 or 16 (chunks per row are a multiple of it)
  const bool live = t < chunks;
  u32x4_t u = live ? load16(x + 8 * t) : u32x4_t{0, 0, 0, 0};
  float s = 0.0f;
  const uint32_t ones = std::is_same<XT, BF16>::value ? 0x3F803F80u : 0x3C003C00u;
#pragma unroll
  for (int e = 0; e < 4; ++e) s = dot2(XT{}, u[e], ones, s);
  for (int off = 1; off < lpg; off <<= 1) s += __shfl_xor(s, off);
  if (!live) return;
  if (PERM) *(u32x4_t*)(xp + 8 * t) = perm8(u);
  if ((t & (lpg - 1)) == 0) {
    const uint32_t hi = f32_to_bf16_bits(s);
    const uint32_t lo = f32_to_bf16_bits(s - bf16_bits_to_f32(hi));
    xs[t / lpg] = hi | (lo << 16);  // (row, group) in row-major order
  }
}

// One thread per (output row n, sub-group): the record of the main loop,
//   { kFold * scale (fp32 bits), bias as bf16 hi | lo << 16, c = -kFold * scale (0 for 8-bit
//     codes) as bf16 hi | lo << 16, 0 }.
// The main loop works on sub-groups of ge = min(g, 64) values; a group of 128 gives two
// sub-groups with the same scale and bias (record j of a row comes from group j / (g / ge)).
template <typename PT, int BITS>
__global__ __launch_bounds__(256) void wprep_kernel(const uint16_t* __restrict__ scales,
                                                    const uint16_t* __restrict__ biases, int64_t count, int rep,
                                                    u32x4_t* __restrict__ rec) {
  constexpr float kFold = BITS == 4 ? 16.0f : 1.0f;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= count) return;
  const int64_t src = t / rep;  // rows hold a whole number of groups, so this stays in the row
  const float sc = kFold * param_to_f32<PT>(scales[src]);
  const float bv = param_to_f32<PT>(biases[src]);
  uint32_t bh, bl, ch, cl;
  split_bf16(bv, bh, bl);
  split_bf16(BITS == 4 ? -sc : 0.0f, ch, cl);
  rec[t] = u32x4_t{__float_as_uint(sc), bh | (bl << 16), ch | (cl << 16), 0u};
}

// ---------------------------------------------------------------- code unpacking

// A 32-bit constant placed in a VGPR once.  The VOP3 encodings of this target take no literal
// operand, so shift-and-mask-and-or only folds into one v_and_or_b32 when the mask and the magic
// bits are registers.
__device__ __forceinline__ uint32_t vconst(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "i"(c));
  return r;
}

template <int BITS, typename XT> struct Codes;
// 4-bit: word j -> 4 operand registers holding codes (0,4),(1,5),(2,6),(3,7) as 1 + q/16
// (mk = mask, mg = magic bits, both in registers: see vconst).
template <> struct Codes<4, BF16> {
  static constexpr uint32_t kMask = 0x00780078u, kMagic = 0x3F803F80u;
  __device__ __forceinline__ static void unpack(uint32_t w, uint32_t* r, uint32_t mk, uint32_t mg) {
    r[0] = ((w << 3) & mk) | mg;
    r[1] = ((w >> 1) & mk) | mg;
    r[2] = ((w >> 5) & mk) | mg;
    r[3] = ((w >> 9) & mk) | mg;
  }
};
template <> struct Codes<4, F16> {
  static constexpr uint32_t kMask = 0x03C003C0u, kMagic = 0x3C003C00u;
  __device__ __forceinline__ static void unpack(uint32_t w, uint32_t* r, uint32_t mk, uint32_t mg) {
    r[0] = ((w << 6) & mk) | mg;
    r[1] = ((w << 2) & mk) | mg;
    r[2] = ((w >> 2) & mk) | mg;
    r[3] = ((w >> 6) & mk) | mg;
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



// Ring of the bias-term operands of the last 8 groups (slot g % 8), in LDS:
//   sX:  X[m, g] as bf16 hi | lo << 16 at row * XR_PITCH + g % 8
//   sBC: bias b[n, g] and c[n, g] = -kFold * s[n, g], each as bf16 hi | lo << 16, at
//        col * BC_PITCH + 2 * (g % 8) (+1 for c)
// The odd pitches keep the per-lane reads free of bank conflicts.
constexpr int XR_PITCH = 9;
constexpr int BC_PITCH = 18;

typedef __attribute__((address_space(3))) void lds_void;

// Copy 16 bytes per lane from a buffer straight into LDS: lane l reads at byte voff + soff of
// the buffer and its bytes land at dst + 16 * l (dst and soff are the same for the whole wave).
__device__ __forceinline__ void copy_to_lds(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, uint8_t* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)dst, 16, voff, soff, 0, 0);
}
// Raw buffer resource over `bytes` bytes at `base` (bytes < 2^31, checked by the host).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t gemm_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

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
// the fragment reads of 8 and of 16 consecutive lanes (rows) on distinct banks:
//   x rows (8 slots):     c ^ xswz(r),   xswz(r) = (r & 7) ^ ((r >> 3) & 1)
//   code rows, 2 slots:   c ^ (((n >> 2) ^ (n >> 3)) & 1)
//   code rows, 4 slots:   c ^ (((n >> 1) & 3) ^ ((n >> 3) & 1))
__device__ __forceinline__ int xswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
template <int CH> __device__ __forceinline__ int bswz(int n) {
  return CH == 2 ? (((n >> 2) ^ (n >> 3)) & 1) : (((n >> 1) & 3) ^ ((n >> 3) & 1));
}

// Main loop layout.
//
// k-slots: MFMA slot j (0..7) of lane half h at k-step t (0..3) of a 64-wide k-tile reads the
// 8-value chunk kc(t, h) of the tile: kc = 4h + t when g >= 64 (a k-step then spans two chunks
// of one group), kc = 2t + h when g == 32 (every k-step inside one group).
//
// Stages: three LDS stages, each holding the tile's x rows (BM x 64 values) and packed code rows
// (BN x 64 codes), filled by direct global->LDS copies two tiles ahead of the compute.  x chunk c
// of row r sits at 16-byte slot r*8 + (c ^ xswz(r)); code chunk c of row n at slot
// n*CH + (c ^ bswz(n)), CH = chunks per row (see the swizzles above).  The stages are three distinct LDS arrays and the loop is unrolled
// by three, so the compiler sees which stage each read and each copy touch and never waits for
// copies in flight to another stage.
//
// Per-tile scalars (scales, biases, group sums of x) are loaded into registers one tile ahead
// and written to LDS just before the tile's barrier.  Every thread issues the same loads every
// iteration (clamped in range when not needed), so one vmcnt wait per tile is exact.
//
// The bias terms sum_g X[m,g] * (b[n,g] - kFold*s[n,g]) run inside the k-loop: once two more
// groups are complete, one MFMA per 32x32 tile takes group 2p + h in lane half h with the slots
// Xhi*bhi, Xhi*blo, Xlo*bhi, Xlo*blo, Xhi*chi, Xhi*clo, Xlo*chi, Xlo*clo.
template <int BITS, int G, typename XT, typename PT>
__global__ __launch_bounds__(256, BITS == 4 ? 2 : 1) void gemm_kernel(const uint16_t* __restrict__ xa, int64_t M, int64_t K,
                                                      const uint32_t* __restrict__ packed, int64_t N,
                                                      const uint16_t* __restrict__ layer_bias, void* __restrict__ y,
                                                      int ydt, const uint32_t* __restrict__ xsum,
                                                      const u32x4_t* __restrict__ wrec) {
  static_assert(G == 32 || G == 64, "the main loop takes sub-groups of 32 or 64 values");
  constexpr bool SPLIT = G == 64;
  constexpr float kFold = BITS == 4 ? 16.0f : 1.0f;  // partial sums of 1 + q/16 carry q/16
  constexpr int SPG = G / 16;                         // 16-wide k-steps per group: 2 or 4
  constexpr int A_BYTES = BM * BK * 2;                // 16 KiB
  constexpr int CH = BK * BITS / 8 / 16;              // 16-byte code chunks per row: 2 or 4
  constexpr int B_BYTES = BN * CH * 16;
  constexpr int STAGE = A_BYTES + B_BYTES;
  constexpr int LB = CH / 2;                          // code copies per wave per tile: 1 or 2
  constexpr int L = 4 + LB;                           // copies per wave per tile
  __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st2[STAGE];
  __shared__ float sS[2][BN][2];  // kFold * scale of the groups of k-steps {0,1} and {2,3}
  __shared__ __attribute__((aligned(16))) uint32_t sX[BM * XR_PITCH];
  __shared__ __attribute__((aligned(16))) uint32_t sBC[BN * BC_PITCH];

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

  uint32_t mk = 0, mg = 0;
  if constexpr (BITS == 4) {
    mk = vconst(Codes<4, XT>::kMask);
    mg = vconst(Codes<4, XT>::kMagic);
  }

  // ---- copies of one tile into a stage (every lane, every tile)
  // x: copy i (0..3) of wave w covers rows 32w + 8i .. +7, lane l -> row + l/8, slot l%8.
  // Each lane keeps a 32-bit byte offset from the tile's first column; the tile base is uniform.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t a_off[4];
  int a_c[4];  // x chunk this lane copies
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 32 * wave + 8 * i + (lane >> 3);
    const int c = (lane & 7) ^ xswz(r);
    const int64_t gr = m0 + r < M ? m0 + r : M - 1;
    a_off[i] = (uint32_t)((gr * K + 8 * c) * 2);
    a_c[i] = c;
  }
  // codes: copy i (0..LB-1) of wave w covers rows 32w + (32/LB)i .. ; lane l -> row + l/CH, slot l%CH.
  uint32_t b_off[LB];
  int b_c[LB];
#pragma unroll
  for (int i = 0; i < LB; ++i) {
    const int n = 32 * wave + (32 / LB) * i + lane / CH;
    const int c = (lane % CH) ^ bswz<CH>(n);
    const int64_t gn = n0 + n < N ? n0 + n : N - 1;
    b_off[i] = (uint32_t)((gn * words_per_row + 4 * c) * 4);
    b_c[i] = c;
  }
  const __amdgpu_buffer_rsrc_t rsA = gemm_rsrc(xa, M * K * 2);
  const __amdgpu_buffer_rsrc_t rsB = gemm_rsrc(packed, N * words_per_row * 4);
  auto copy_tile = [&](int kt, uint8_t* stage) __attribute__((always_inline)) {
    const int64_t k0 = kt * BK;
    const uint32_t sa = (uint32_t)(k0 * 2), sbo = (uint32_t)(k0 * BITS / 8);
    uint32_t ashift[4], bshift[LB];
#pragma unroll
    for (int i = 0; i < 4; ++i) ashift[i] = 0;
#pragma unroll
    for (int i = 0; i < LB; ++i) bshift[i] = 0;
    if constexpr (!SPLIT) {
      // chunks past K (a last tile of 32 values) copy the chunk 32 values earlier instead: finite
      // values whose products land in a group with scale 0 and no bias term
#pragma unroll
      for (int i = 0; i < 4; ++i) ashift[i] = k0 + 8 * a_c[i] < K ? 0u : 64u;
#pragma unroll
      for (int i = 0; i < LB; ++i) bshift[i] = k0 + b_c[i] * (128 / BITS) < K ? 0u : 4u * BITS;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) copy_to_lds(rsA, a_off[i] - ashift[i], sa, stage + (32 * wave_u + 8 * i) * 128);
#pragma unroll
    for (int i = 0; i < LB; ++i)
      copy_to_lds(rsB, b_off[i] - bshift[i], sbo, stage + A_BYTES + (32 * wave_u + (32 / LB) * i) * CH * 16);
  };

  // ---- per-tile scalars, one tile ahead in registers
  // thread -> x row tid/2 and half tid&1 (group sum of x), code row tid&127 and half tid>>7
  // (record of the group of that half: fold scale, bias and c operands; see wprep_kernel).
  const int a_row = tid >> 1, a_half = tid & 1;
  const int64_t a_grow = m0 + a_row < M ? m0 + a_row : M - 1;
  const int s_col = tid & (BN - 1), s_half = tid >> 7;
  const int64_t s_grow = n0 + s_col < N ? n0 + s_col : N - 1;
  const uint32_t* xs_row = xsum + a_grow * groups;
  const u32x4_t* wr_row = wrec + s_grow * groups;
  const int gshift = G == 32 ? 5 : 6;
  const int ngroups = (int)groups;
  uint32_t rx = 0;
  u32x4_t rw = {0, 0, 0, 0};
  auto load_scalars = [&](int kt) __attribute__((always_inline)) {
    const int ga = min((kt * BK + 32 * a_half) >> gshift, ngroups - 1);
    const int gs = min((kt * BK + 32 * s_half) >> gshift, ngroups - 1);
    rx = xs_row[ga];
    rw = wr_row[gs];
  };
  const int kint = (int)K;
  auto store_scalars = [&](int kt) __attribute__((always_inline)) {
    const int ka = kt * BK + 32 * a_half, ks = kt * BK + 32 * s_half;
    if (ka < kint && (ka & (G - 1)) == 0) sX[a_row * XR_PITCH + ((ka >> gshift) & 7)] = rx;
    sS[kt & 1][s_col][s_half] = ks < kint ? __uint_as_float(rw[0]) : 0.0f;
    if (ks < kint && (ks & (G - 1)) == 0)
      *(u32x2_t*)&sBC[s_col * BC_PITCH + 2 * ((ks >> gshift) & 7)] = u32x2_t{rw[1], rw[2]};
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

  // Bias terms of the group pair p (groups 2p, 2p+1): see the comment above the kernel.
  auto bias_pair = [&](int p) __attribute__((always_inline)) {
    const int gi = 2 * p + h;
    const bool live = gi < (int)groups;
    const int slot = gi & 7;
    u32x4_t ab[2], bb[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const uint32_t v = live ? sX[(wm * 64 + rt * 32 + l32) * XR_PITCH + slot] : 0u;
      const uint32_t hh = perm(v, v, 0x01000100u), ll = perm(v, v, 0x03020302u);
      ab[rt] = u32x4_t{hh, ll, hh, ll};
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      u32x2_t bc = live ? *(const u32x2_t*)&sBC[(wn * 64 + ct * 32 + l32) * BC_PITCH + 2 * slot] : u32x2_t{0, 0};
      bb[ct] = u32x4_t{bc[0], bc[0], bc[1], bc[1]};
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) acc[rt][ct] = mfma(BF16{}, ab[rt], bb[ct], acc[rt][ct]);
  };

  // ---- compute of one tile from a stage
  auto compute = [&](int kt, const uint8_t* stage) __attribute__((always_inline)) {
    // x fragments: 2 row-tiles x 4 k-steps
    u32x4_t af[2][4];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      const int r = wm * 64 + rt * 32 + l32;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int c = SPLIT ? 4 * h + t : 2 * t + h;
        af[rt][t] = *(const u32x4_t*)(stage + (r * 8 + (c ^ xswz(r))) * 16);
      }
    }
    // code words of this lane's column in each col-tile, for the 4 k-steps:
    //   4-bit: word t (SPLIT: of chunk h; else word 2t + h of the row)
    //   8-bit: words 2t, 2t+1 of the lane's 32 codes (SPLIT: chunks 2h, 2h+1; else chunk t, pair h)
    uint32_t cw[2][4][BITS / 4];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const int n = wn * 64 + ct * 32 + l32;
      const uint8_t* row = stage + A_BYTES + n * CH * 16;
      const int sw = bswz<CH>(n);
      if constexpr (CH == 2) {
        if constexpr (SPLIT) {
          const u32x4_t v = *(const u32x4_t*)(row + ((h ^ sw) * 16));
#pragma unroll
          for (int t = 0; t < 4; ++t) cw[ct][t][0] = v[t];
        } else {
          const u32x4_t v0 = *(const u32x4_t*)(row + (sw * 16));
          const u32x4_t v1 = *(const u32x4_t*)(row + ((1 ^ sw) * 16));
          cw[ct][0][0] = h ? v0[1] : v0[0];
          cw[ct][1][0] = h ? v0[3] : v0[2];
          cw[ct][2][0] = h ? v1[1] : v1[0];
          cw[ct][3][0] = h ? v1[3] : v1[2];
        }
      } else {
        if constexpr (SPLIT) {
          const u32x4_t v0 = *(const u32x4_t*)(row + (((2 * h) ^ sw) * 16));
          const u32x4_t v1 = *(const u32x4_t*)(row + (((2 * h + 1) ^ sw) * 16));
          cw[ct][0][0] = v0[0]; cw[ct][0][1] = v0[1];
          cw[ct][1][0] = v0[2]; cw[ct][1][1] = v0[3];
          cw[ct][2][0] = v1[0]; cw[ct][2][1] = v1[1];
          cw[ct][3][0] = v1[2]; cw[ct][3][1] = v1[3];
        } else {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const u32x4_t v = *(const u32x4_t*)(row + ((t ^ sw) * 16));
            cw[ct][t][0] = h ? v[2] : v[0];
            cw[ct][t][1] = h ? v[3] : v[1];
          }
        }
      }
    }

    const int sb = (int)(kt & 1);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const bool first = t % SPG == 0;
      const bool last = (t + 1) % SPG == 0;
      u32x4_t bf[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        uint32_t r[4];
        if constexpr (BITS == 4)
          Codes<4, XT>::unpack(cw[ct][t][0], r, mk, mg);
        else
          Codes<8, XT>::unpack2(cw[ct][t][0], cw[ct][t][BITS / 4 - 1], r);
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
          const float sc = sS[sb][wn * 64 + ct * 32 + l32][q];
#pragma unroll
          for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[rt][ct][r] = __builtin_fmaf(sc, P[rt][ct][r], acc[rt][ct][r]);
        }
      }
    }
  };

  int pairs_done = 0;
  // One k-tile: wait for its copies and scalars, publish the scalars, barrier, start the copies
  // of tile kt + 2 (clamped: past the end they refill the stage computed in the previous
  // iteration, which no wave reads again) and the scalars of tile kt + 1, then compute.
  const int KTi = (int)KT;
  auto step = [&](int kt, const uint8_t* cur, uint8_t* ahead2, auto first) __attribute__((always_inline)) {
    // steps past the last tile (to complete a round of three) wait, copy and load like the
    // others, so that the wait counts are the same on every path, and compute nothing
    const int kc = kt < KTi ? kt : KTi - 1;
    if constexpr (decltype(first)::value) wait_vmcnt<0>();  // after the prologue's copies
    else wait_vmcnt<L>();
    store_scalars(kc);
    wait_vmcnt_lgkm0<L>();
    __builtin_amdgcn_s_barrier();
    // the scalar loads go out before the copies (the wait counts above rely on that order)
    load_scalars(kc + 1 < KTi ? kc + 1 : KTi - 1);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    copy_tile(kc + 2 < KTi ? kc + 2 : KTi - 1, ahead2);
    __builtin_amdgcn_sched_barrier(0);
    if (kt < KTi) {
      compute(kt, cur);
      // bias terms of every group pair completed by this tile (the last tile also takes a
      // final odd group, paired with nothing)
      const int gdone = (kt == KTi - 1) ? ngroups : (BK * (kt + 1)) >> gshift;
      const int ptarget = (kt == KTi - 1) ? (gdone + 1) / 2 : gdone / 2;
      for (; pairs_done < ptarget; ++pairs_done) bias_pair(pairs_done);
    }
  };

  if (KTi > 0) {
    copy_tile(0, st0);
    copy_tile(KTi > 1 ? 1 : 0, st1);
    load_scalars(0);
    // tile t lives in stage t % 3; the first step is peeled so that the loop is entered with
    // the same order of loads in flight as its back edge
    step(0, st0, st2, std::true_type{});
    for (int kt = 1; kt < KTi; kt += 3) {
      step(kt, st1, st0, std::false_type{});
      step(kt + 1, st2, st1, std::false_type{});
      step(kt + 2, st0, st2, std::false_type{});
    }
    wait_vmcnt<0>();  // no copy may still be writing LDS when the workgroup ends
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

// Workspace: group sums of x (m * k/g words), the group records of the weights (n * k/g x 16
// bytes), each padded to 256 bytes, then the permuted copy of x (m * k 16-bit values; 4-bit).
inline size_t pad256(size_t b) { return (b + 255u) & ~(size_t)255u; }
inline size_t xsum_bytes(int64_t m, int64_t k, int g) { return pad256((size_t)(m * (k / g)) * 4u); }
inline size_t wrec_bytes(int64_t n, int64_t k, int g) { return pad256((size_t)(n * (k / g)) * 16u); }

template <int BITS, typename XT, typename PT>
hipError_t launch_t(const void* x, int64_t m, int64_t k, const uint32_t* packed, const void* scales,
                    const void* biases, int64_t n, int g, const void* layer_bias, void* y, int ydt, void* ws,
                    hipStream_t s) {
  const int ge = g < 64 ? g : 64;  // sub-group width of the main loop
  const int64_t subgroups = k / ge;
  uint32_t* xs = (uint32_t*)ws;
  u32x4_t* wr = (u32x4_t*)((uint8_t*)ws + xsum_bytes(m, k, ge));
  uint16_t* xp = (uint16_t*)((uint8_t*)ws + xsum_bytes(m, k, ge) + wrec_bytes(n, k, ge));
  const int64_t chunks = m * k / 8;
  xprep_kernel<XT, BITS == 4><<<(unsigned)((chunks + 255) / 256), 256, 0, s>>>((const uint16_t*)x, m, k, ge, xs, xp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t recs = n * subgroups;
  wprep_kernel<PT, BITS><<<(unsigned)((recs + 255) / 256), 256, 0, s>>>((const uint16_t*)scales,
                                                                         (const uint16_t*)biases, recs, g / ge, wr);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t tiles = ((m + BM - 1) / BM) * ((n + BN - 1) / BN);
  const uint16_t* xa = BITS == 4 ? xp : (const uint16_t*)x;
  const uint16_t* lb = (const uint16_t*)layer_bias;
  if (ge == 32)
    gemm_kernel<BITS, 32, XT, PT><<<(unsigned)tiles, 256, 0, s>>>(xa, m, k, packed, n, lb, y, ydt, xs, wr);
  else
    gemm_kernel<BITS, 64, XT, PT><<<(unsigned)tiles, 256, 0, s>>>(xa, m, k, packed, n, lb, y, ydt, xs, wr);
  return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(int64_t m, int64_t n, int64_t k, int g) {
  const int ge = g < 64 ? g : 64;
  return xsum_bytes(m, k, ge) + wrec_bytes(n, k, ge) + (size_t)(m * k) * 2u;
}

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
