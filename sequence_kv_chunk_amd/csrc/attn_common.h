// Device helpers shared by the attention kernels: element loads/stores in
// either output dtype and the log-sum-exp merge of a chunk's partial into a
// running (O, lse).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sqkv_internal.h"

namespace sqkv {

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// Round-to-nearest-even float -> bf16 bits (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Load four consecutive elements (16-byte aligned for f32, 8-byte for bf16).
__device__ __forceinline__ void load4(const void* base, int64_t off, int dtype, float out[4]) {
  if (dtype == kF32) {
    float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
  } else {
    uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(base) + off);
    out[0] = bf16_bits_to_f32(v.x & 0xffffu);
    out[1] = bf16_bits_to_f32(v.x >> 16);
    out[2] = bf16_bits_to_f32(v.y & 0xffffu);
    out[3] = bf16_bits_to_f32(v.y >> 16);
  }
}

__device__ __forceinline__ void store4(void* base, int64_t off, int dtype, const float in[4]) {
  if (dtype == kF32) {
    *reinterpret_cast<float4*>(static_cast<float*>(base) + off) = make_float4(in[0], in[1], in[2], in[3]);
  } else {
    uint2 v;
    v.x = f32_to_bf16_bits(in[0]) | (f32_to_bf16_bits(in[1]) << 16);
    v.y = f32_to_bf16_bits(in[2]) | (f32_to_bf16_bits(in[3]) << 16);
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + off) = v;
  }
}

// Weights of the log-sum-exp merge of partial A (lse_a) and partial B
// (lse_b), both natural-log.  Returns the merged lse; wa, wb are the factors
// multiplying the normalised partial outputs.  An empty partial (-inf) gets
// weight 0; two empty partials give (0, 0, -inf).
__device__ __forceinline__ float lse_merge_weights(float lse_a, float lse_b, float& wa, float& wb) {
  float M = fmaxf(lse_a, lse_b);
  if (M == kNegInf) {
    wa = 0.f;
    wb = 0.f;
    return kNegInf;
  }
  float ea = (lse_a == kNegInf) ? 0.f : exp2f((lse_a - M) * kLog2e);
  float eb = (lse_b == kNegInf) ? 0.f : exp2f((lse_b - M) * kLog2e);
  float tot = ea + eb;
  float inv = 1.f / tot;
  wa = ea * inv;
  wb = eb * inv;
  return M + log2f(tot) * kLn2;
}

}  // namespace sqkv
