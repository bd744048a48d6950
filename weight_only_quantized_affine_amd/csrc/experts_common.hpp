// Helpers shared by the routed-apply kernels (experts.hip, experts_mx.hip): buffer resources,
// wait counts and the MXFP4 decode.
#pragma once
#include "device_common.hpp"
#include "launch.hpp"

namespace ql {
namespace ex_detail {

typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer resource over `bytes` bytes at `base` (bytes < 2^31, checked by the host): loads
// past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ex_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kExOOB = 0x7ffffff0u;  // a buffer offset past every resource

template <int N> __device__ __forceinline__ void ex_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// 8 MXFP4 codes (one word: byte i holds values 2i, 2i+1 in its low/high nibble) -> bf16 operand
// registers (v0,v1),(v2,v3),(v4,v5),(v6,v7) with the CDNA4 scaled conversion
// (v_cvt_scalef32_pk_bf16_fp4: one byte = two E2M1 codes, low nibble into the low half, times an
// fp32 scale, rounded to bf16).  With scale = 2^(s-127) the products have at most two
// significant bits, so they are exact for every scale byte s <= 254 (s = 0 gives bf16
// subnormals), overflow to inf where the format does, and a NaN scale (s = 255) gives NaN.
__device__ __forceinline__ u32x4_t decode_mxfp4(uint32_t w, float scale) {
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return r;
}

}  // namespace ex_detail
}  // namespace ql
