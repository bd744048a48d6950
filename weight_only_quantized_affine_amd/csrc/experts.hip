// Routing for the routed apply (Nx_quant API docs, Products: apply_experts): each position's x
// row goes through the expert its id names, zeros for ids out of [0, e), a row's bits independent
// of the other positions' experts.  Weights in MXFP4 (codes + E8M0 scales apart) or Q8_0 blocks
// (Nx_quant Weights), decoded while summing (no stored decoded weight).
//
// route_kernel: workgroup j counts all ids in LDS (its offset and the experts' order by count),
// then writes the positions with id j in increasing order: a stable counting sort, identical on
// every run.  The apply kernels are in experts_mx.hip (MXFP4) and experts_q8.hip (Q8_0).
#include "experts_common.hpp"

namespace ql {
namespace {
using namespace ex_detail;

enum : int { FMT_MXFP4 = 1, FMT_Q8_0 = 2, FMT_MXFP4_BLOCKS = 3, FMT_Q4_K = 4, FMT_Q6_K = 5 };  // ql_format values

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
  hipError_t err;
  if (e == 0 || k == 0) {  // no expert, or empty products: every row is zero
    zero_rows_kernel<<<(unsigned)n_pos, 256, 0, s>>>(n, y, ydt);
    return hipGetLastError();
  }
  // routing, expert order, and zero rows for the positions routed nowhere
  const int64_t x_rows = n_pos / pos_per_row;
  route_kernel<<<(unsigned)e, 1024, (size_t)(e > 1024 ? e : 1024) * 4, s>>>(
      ids, n_pos, e, offsets, perm, order, y, n, ydt, (const uint16_t*)x, x_rows, k,
      fmt == FMT_Q8_0 && xdt == DT_BF16 ? xfac : nullptr);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (fmt == FMT_Q8_0)
    return launch_experts_q8((const uint8_t*)w0, e, n, k, offsets, perm, order, xfac, (const uint16_t*)x, xdt, x_rows,
                             pos_per_row, y, ydt, s);
  if (fmt == FMT_Q4_K || fmt == FMT_Q6_K)
    return launch_experts_kq(fmt, (const uint8_t*)w0, e, n, k, offsets, perm, order, (const uint16_t*)x, xdt, x_rows,
                             pos_per_row, y, ydt, s);
  // MXFP4 with its scales apart (w1), or in GGUF blocks (w1 = NULL)
  return launch_experts_mx((const uint8_t*)w0, fmt == FMT_MXFP4_BLOCKS ? nullptr : (const uint8_t*)w1, e, n, k,
                           offsets, perm, order, (const uint16_t*)x, xdt, x_rows, pos_per_row, y, ydt, s);
}

}  // namespace ql
