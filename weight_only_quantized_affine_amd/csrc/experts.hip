// Routing and routed apply (Nx_quant API docs, Products: apply_experts): each position's x row
// through the expert its id names, zeros for ids out of [0, e), a row's bits independent of the
// other positions' experts.  Weights in MXFP4 (codes + E8M0 scales apart) or Q8_0 blocks
// (Nx_quant Weights), decoded while summing (no stored decoded weight).
//
// route_kernel: workgroup j scans all ids twice: counts ids below j (its offset) then writes the
// positions with id j in increasing order (wave ballots + an LDS prefix over the 4 waves), so the
// permutation is a stable counting sort, identical on every run.
//
// experts_kernel: one workgroup per (expert, 128 output rows); its 4 waves own 32 output rows
// each and loop over the expert's positions in chunks of 128 (m-subtiles of 32) and over k in
// tiles of 64.  The gathered x rows of a chunk are staged in LDS (shared by the waves); each
// lane loads and decodes the packed weights of its output row straight from HBM.
//   MXFP4: every scale byte s has a bf16 table of the 8 magnitudes times 2^(s-127) (exact; NaN
//          for s == 255) built in LDS at start; a byte of codes becomes a bf16 pair with
//          v_perm_b32 lookups, so the block scale costs nothing per element.
//   Q8_0:  int8 codes become exact bf16; each 32-block's fp32 partial sum is scaled by its d.
#include "device_common.hpp"
#include "launch.hpp"

namespace ql {
namespace {

// ---------------------------------------------------------------- routing

__global__ __launch_bounds__(256) void route_kernel(const int64_t* __restrict__ ids, int64_t n_pos, int64_t e,
                                                    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_out) {
  __shared__ int32_t s_wave[4];
  __shared__ int32_t s_tot[2];
  const int64_t j = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t below = 0, mine = 0;
  for (int64_t p = tid; p < n_pos; p += 256) {
    const int64_t v = ids[p];
    below += (v >= 0 && v < j) ? 1 : 0;
    mine += (v == j) ? 1 : 0;
  }
  // block sums of `below` and `mine`
  for (int off = 32; off >= 1; off >>= 1) {
    below += __shfl_xor(below, off);
    mine += __shfl_xor(mine, off);
  }
  if (tid < 2) s_tot[tid] = 0;
  __syncthreads();
  if (lane == 0) {
    atomicAdd(&s_tot[0], below);
    atomicAdd(&s_tot[1], mine);
  }
  __syncthreads();
  const int32_t base = s_tot[0];
  if (tid == 0) {
    offsets[j] = base;
    if (j == e - 1) offsets[e] = base + s_tot[1];
  }
  int32_t running = 0;
  for (int64_t p0 = 0; p0 < n_pos; p0 += 256) {
    const int64_t p = p0 + tid;
    const bool hit = p < n_pos && ids[p] == j;
    const uint64_t bal = __ballot(hit);
    const int32_t in_wave = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) s_wave[wave] = __popcll(bal);
    __syncthreads();
    int32_t before = running;
    for (int w = 0; w < wave; ++w) before += s_wave[w];
    if (hit) perm_out[base + before + in_wave] = (int32_t)p;
    running += s_wave[0] + s_wave[1] + s_wave[2] + s_wave[3];
    __syncthreads();
  }
}

// Zero the output rows of positions whose id is out of [0, e).
__global__ __launch_bounds__(256) void zero_unrouted_kernel(const int64_t* __restrict__ ids, int64_t n_pos, int64_t e,
                                                            int64_t n, void* __restrict__ y, int ydt) {
  const int64_t p = blockIdx.x;
  const int64_t v = ids[p];
  if (v >= 0 && v < e) return;
  const int64_t esz = ydt == DT_F32 ? 4 : 2;
  uint8_t* row = (uint8_t*)y + p * n * esz;
  for (int64_t i = threadIdx.x; i < n * esz / 2; i += 256) ((uint16_t*)row)[i] = 0;
}

// ---------------------------------------------------------------- routed apply

constexpr int EBN = 128, EBK = 64, EMC = 128;  // output rows / k / positions per chunk
constexpr int EA_PITCH = EBK + 8;              // bf16 per LDS row of the x tile

enum : int { FMT_MXFP4 = 1, FMT_Q8_0 = 2 };

__device__ __forceinline__ f32x16_t mfma_bf16(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// Order of 8 consecutive k-values within an operand register quad.
//   MXFP4 decode yields values (0,2),(4,6),(1,3),(5,7) of a code word; Q8_0 yields them in order.
__device__ __forceinline__ u32x4_t perm_x_mxfp4(const u32x4_t& u) {
  // u = (x0,x1),(x2,x3),(x4,x5),(x6,x7) -> (x0,x2),(x4,x6),(x1,x3),(x5,x7)
  u32x4_t r;
  r[0] = perm(u[1], u[0], 0x05040100u);
  r[1] = perm(u[3], u[2], 0x05040100u);
  r[2] = perm(u[1], u[0], 0x07060302u);
  r[3] = perm(u[3], u[2], 0x07060302u);
  return r;
}

// 8 MXFP4 codes (one word: byte i holds values 2i, 2i+1 in its low/high nibble) -> bf16 operand
// registers (v0,v2),(v4,v6),(v1,v3),(v5,v7) using the scale's byte tables (lo bytes, hi bytes).
__device__ __forceinline__ u32x4_t decode_mxfp4(uint32_t w, const u32x4_t& tab) {
  const uint32_t il = w & 0x07070707u;
  const uint32_t ih = (w >> 4) & 0x07070707u;
  const uint32_t llo = perm(tab[1], tab[0], il);  // low bytes of the even values
  uint32_t hlo = perm(tab[3], tab[2], il);        // high bytes of the even values
  const uint32_t lhi = perm(tab[1], tab[0], ih);
  uint32_t hhi = perm(tab[3], tab[2], ih);
  hlo |= (w << 4) & 0x80808080u;  // sign of the even values
  hhi |= w & 0x80808080u;         // sign of the odd values
  u32x4_t r;
  r[0] = perm(hlo, llo, 0x05010400u);  // v0, v2
  r[1] = perm(hlo, llo, 0x07030602u);  // v4, v6
  r[2] = perm(hhi, lhi, 0x05010400u);  // v1, v3
  r[3] = perm(hhi, lhi, 0x07030602u);  // v5, v7
  return r;
}

__device__ __forceinline__ uint32_t pack2_bf16_i8(uint32_t b0, uint32_t b1) {
  bf16x2_t v = {(__bf16)(float)(int32_t)(int8_t)b0, (__bf16)(float)(int32_t)(int8_t)b1};
  return __builtin_bit_cast(uint32_t, v);
}

template <int FMT>
__global__ __launch_bounds__(256) void experts_kernel(const uint8_t* __restrict__ w0, const uint8_t* __restrict__ w1,
                                                      int64_t e, int64_t N, int64_t K,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ perm_pos,
                                                      const uint16_t* __restrict__ x, int64_t pos_per_row,
                                                      void* __restrict__ y, int ydt) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[EMC * EA_PITCH];
  __shared__ __attribute__((aligned(16))) u32x4_t sTab[FMT == FMT_MXFP4 ? 256 : 1];
  __shared__ int32_t sPos[EMC];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, h = lane >> 5;
  const int64_t n_tiles = (N + EBN - 1) / EBN;
  const int64_t ex = blockIdx.x / n_tiles;
  const int64_t nt = blockIdx.x - ex * n_tiles;
  const int32_t off = offsets[ex];
  const int32_t cnt = offsets[ex + 1] - off;
  if (cnt <= 0) return;

  if (FMT == FMT_MXFP4) {
    // bf16 bits of magnitude i * 2^(s-127), i = 0..7, split into low-byte and high-byte tables.
    const uint32_t twice_mag = 0xC8643210u;
    const int s = tid;  // 256 threads, one scale byte each
    float p2;
    if (s == 0)
      p2 = __uint_as_float(0x00400000u);
    else if (s == 255)
      p2 = __uint_as_float(0x7fc00000u);
    else
      p2 = __uint_as_float((uint32_t)s << 23);
    uint32_t lo[2] = {0, 0}, hi[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float v = (float)((twice_mag >> (4 * i)) & 15u) * (0.5f * p2);
      const uint32_t b = f32_to_bf16_bits(v);  // exact: at most 2 significant bits
      lo[i >> 2] |= (b & 0xffu) << (8 * (i & 3));
      hi[i >> 2] |= (b >> 8) << (8 * (i & 3));
    }
    sTab[s] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  }

  const int64_t col = nt * EBN + wave * 32 + l32;  // this lane's output row of the expert
  const int64_t colc = col < N ? col : N - 1;
  const int64_t KT = (K + EBK - 1) / EBK;

  for (int32_t mc = 0; mc < cnt; mc += EMC) {
    const int rows = min(EMC, cnt - mc);
    const int msub = (rows + 31) >> 5;
    __syncthreads();  // previous chunk's readers of sPos/sA are done; tables visible
    if (tid < EMC) sPos[tid] = tid < rows ? perm_pos[off + mc + tid] : -1;
    __syncthreads();

    f32x16_t acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;

    // staging thread for the x tile: row tid/2, 32 k-values at (tid&1)*32
    const int a_row = tid >> 1, a_half = tid & 1;
    const int32_t a_pos = sPos[a_row];
    const uint16_t* a_src = a_pos >= 0 ? x + (int64_t)(a_pos / pos_per_row) * K : nullptr;

    for (int64_t kt = 0; kt < KT; ++kt) {
      const int64_t k0 = kt * EBK;
      // -- stage x rows (zeros for rows past the chunk or k past K)
      {
        u32x4_t v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t kk = k0 + a_half * 32 + 8 * j;
          v[j] = (a_src && kk < K) ? load16(a_src + kk) : u32x4_t{0, 0, 0, 0};
          if (FMT == FMT_MXFP4) v[j] = perm_x_mxfp4(v[j]);
        }
        uint16_t* dst = &sA[a_row * EA_PITCH + a_half * 32];
#pragma unroll
        for (int j = 0; j < 4; ++j) *(u32x4_t*)(dst + 8 * j) = v[j];
      }
      // -- this lane's packed weights of the k-tile, decoded into 4 k-steps of operands
      u32x4_t bf[4];
      float dsc[2] = {0.0f, 0.0f};
      if (FMT == FMT_MXFP4) {
        // codes: 32 bytes per row per k-tile; k-step t of lane half h needs word 2t + h
        const uint8_t* cp = w0 + (ex * N + colc) * (K / 2) + k0 / 2;
        const bool full = k0 + EBK <= K;
        u32x4_t c0 = load16(cp);
        u32x4_t c1 = full ? load16(cp + 16) : u32x4_t{0, 0, 0, 0};
        const uint8_t* sp = w1 + (ex * N + colc) * (K / 32) + k0 / 32;
        const uint32_t s0 = sp[0];
        const uint32_t s1 = full ? sp[1] : 0u;
        const u32x4_t t0 = sTab[s0], t1 = sTab[s1];
        const uint32_t words[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
#pragma unroll
        for (int t = 0; t < 4; ++t) bf[t] = decode_mxfp4(words[2 * t + h], t < 2 ? t0 : t1);
      } else {
        // Q8_0: k-step t = 2b + u of lane half h covers k = 32b + 16h + 8u + j: bytes
        // 2 + 16h + 8u .. +7 of block b.  Blocks are 2-byte aligned: read half-words.
        const uint8_t* bp = w0 + (ex * N + colc) * (K / 32 * 34) + (k0 / 32) * 34;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          const bool live = k0 + 32 * b < K;
          const uint16_t* hp = (const uint16_t*)(bp + 34 * b);
          uint32_t hw[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) hw[i] = live ? hp[1 + 8 * h + i] : 0u;
          dsc[b] = live ? f16_bits_to_f32(hp[0]) : 0.0f;
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            u32x4_t r;
#pragma unroll
            for (int q = 0; q < 4; ++q) r[q] = pack2_bf16_i8(hw[4 * u + q] & 0xffu, hw[4 * u + q] >> 8);
            bf[2 * b + u] = r;
          }
        }
      }
      __syncthreads();  // x tile staged
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        if (ms >= msub) break;
        const uint16_t* arow = &sA[(ms * 32 + l32) * EA_PITCH];
        if (FMT == FMT_MXFP4) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const u32x4_t af = *(const u32x4_t*)(arow + 16 * t + 8 * h);
            acc[ms] = mfma_bf16(af, bf[t], acc[ms]);
          }
        } else {
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const u32x4_t a0 = *(const u32x4_t*)(arow + 32 * b + 16 * h);
            const u32x4_t a1 = *(const u32x4_t*)(arow + 32 * b + 16 * h + 8);
            const f32x16_t zero16 = {0.0f};
            f32x16_t p = mfma_bf16(a0, bf[2 * b], zero16);
            p = mfma_bf16(a1, bf[2 * b + 1], p);
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[ms][r] = __builtin_fmaf(dsc[b], p[r], acc[ms][r]);
          }
        }
      }
      __syncthreads();  // done reading the x tile
    }

    // store: lane holds output row `col` for positions 8*(r/4) + 4h + r%4 of each m-subtile
    if (col < N) {
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        if (ms >= msub) break;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rr = ms * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
          if (rr < rows) store_out(y, (int64_t)sPos[rr] * N + col, acc[ms][r], ydt);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_route(const int64_t* ids, int64_t n_pos, int64_t e, int32_t* offsets, int32_t* perm, hipStream_t s) {
  route_kernel<<<(unsigned)e, 256, 0, s>>>(ids, n_pos, e, offsets, perm);
  return hipGetLastError();
}

hipError_t launch_apply_experts(int fmt, const void* w0, const void* w1, int64_t e, int64_t n, int64_t k,
                                const int64_t* ids, int64_t n_pos, const void* x, int xdt, int64_t pos_per_row,
                                void* y, int ydt, int32_t* offsets, int32_t* perm, hipStream_t s) {
  (void)xdt;
  zero_unrouted_kernel<<<(unsigned)n_pos, 256, 0, s>>>(ids, n_pos, e, n, y, ydt);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || e == 0) return err;
  err = launch_route(ids, n_pos, e, offsets, perm, s);
  if (err != hipSuccess) return err;
  const int64_t grid = e * ((n + EBN - 1) / EBN);
  if (fmt == FMT_MXFP4)
    experts_kernel<FMT_MXFP4><<<(unsigned)grid, 256, 0, s>>>((const uint8_t*)w0, (const uint8_t*)w1, e, n, k, offsets,
                                                            perm, (const uint16_t*)x, pos_per_row, y, ydt);
  else
    experts_kernel<FMT_Q8_0><<<(unsigned)grid, 256, 0, s>>>((const uint8_t*)w0, nullptr, e, n, k, offsets, perm,
                                                           (const uint16_t*)x, pos_per_row, y, ydt);
  return hipGetLastError();
}

}  // namespace ql
