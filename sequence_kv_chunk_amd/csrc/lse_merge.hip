// Log-sum-exp merge of two partial attentions over disjoint key sets.
//
// Ring-attention Q&A (aivaro.ru answer 425), section 5: each new chunk's
// partial is folded into the running output by rescaling both with the
// exponent of their distance to the new running maximum.  In log-sum-exp form
// (one fp32 lse per row, normalised outputs):
//     lse = log(exp(lse_a) + exp(lse_b))
//     o   = exp(lse_a - lse) * o_a + exp(lse_b - lse) * o_b
// An empty partial (lse = -inf) contributes nothing.
//
// HBM-bound elementwise kernel: each thread owns four consecutive elements of
// one row (16-byte fp32 / 8-byte bf16 accesses); the D/4 threads of a row sit
// in the same wavefront, so in-place updates of lse (lse_out == lse_a) read
// before they write within one wave.  The partials are read once and the
// result written once, so the O accesses carry non-temporal hints.
#include "attn_common.h"

namespace sqkv {
namespace {

constexpr int kThreads = 256;

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// Four consecutive elements, non-temporal (16-byte fp32 / 8-byte bf16).
__device__ __forceinline__ void load4_nt(const void* base, int64_t off, int dtype, float out[4]) {
  if (dtype == kF32) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(static_cast<const float*>(base) + off));
    out[0] = v[0]; out[1] = v[1]; out[2] = v[2]; out[3] = v[3];
  } else {
    const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(static_cast<const uint16_t*>(base) + off));
    out[0] = bf16_bits_to_f32(v[0] & 0xffffu);
    out[1] = bf16_bits_to_f32(v[0] >> 16);
    out[2] = bf16_bits_to_f32(v[1] & 0xffffu);
    out[3] = bf16_bits_to_f32(v[1] >> 16);
  }
}

__device__ __forceinline__ void store4_nt(void* base, int64_t off, int dtype, const float in[4]) {
  if (dtype == kF32) {
    const f32x4_t v = {in[0], in[1], in[2], in[3]};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(static_cast<float*>(base) + off));
  } else {
    const u32x2_t v = {f32_to_bf16_bits(in[0]) | (f32_to_bf16_bits(in[1]) << 16),
                       f32_to_bf16_bits(in[2]) | (f32_to_bf16_bits(in[3]) << 16)};
    __builtin_nontemporal_store(v, reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(base) + off));
  }
}

template <int D>
__global__ void __launch_bounds__(kThreads) lse_merge_kernel(MergeParams p) {
  constexpr int TPR = D / 4;  // threads per row
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t gid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t t = gid / TPR;
  const int c = (int)(gid % TPR) * 4;
  if (t >= p.n) return;
  const int64_t row = ((int64_t)b * p.H + h) * p.n + t;
  float la = p.lse_a[row];
  float lb = p.lse_b[row];
  float wa, wb;
  float lse = lse_merge_weights(la, lb, wa, wb);
  float xa[4], xb[4], y[4];
  load4_nt(p.oa, b * p.a_sb + h * p.a_sh + t * p.a_sn + c, p.a_dtype, xa);
  load4_nt(p.ob, b * p.b_sb + h * p.b_sh + t * p.b_sn + c, p.b_dtype, xb);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // terms with zero weight are skipped so that an empty partial's payload
    // (whatever it holds) cannot leak in as NaN * 0
    float acc = 0.f;
    if (wa != 0.f) acc = wa * xa[i];
    if (wb != 0.f) acc = fmaf(wb, xb[i], acc);
    y[i] = acc;
  }
  store4_nt(p.oo, b * p.o_sb + h * p.o_sh + t * p.o_sn + c, p.o_dtype, y);
  if (c == 0) p.lse_o[row] = lse;
}

}  // namespace

hipError_t launch_lse_merge(const MergeParams& p, int d, hipStream_t s) {
  if (p.n == 0 || p.B == 0 || p.H == 0) return hipSuccess;
  int64_t threads = (int64_t)p.n * (d / 4);
  dim3 grid((unsigned)((threads + kThreads - 1) / kThreads), (unsigned)p.H, (unsigned)p.B);
  if (d == 128)
    hipLaunchKernelGGL(lse_merge_kernel<128>, grid, dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(lse_merge_kernel<64>, grid, dim3(kThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace sqkv
