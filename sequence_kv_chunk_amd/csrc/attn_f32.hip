// Chunk attention with fp32 inputs and fp32 arithmetic throughout.
//
// Ring-attention Q&A (aivaro.ru answer 425), section 5: for one query chunk
// and one key/value chunk, scores q.k, the row maximum, exponentials, the row
// sum (normaliser) and the weighted sum of values; the chunk's partial is
// then merged into the running output (online softmax).
//
// This is the exact-precision variant (no reduced-precision products): one
// lane owns one query row, keeps q and its output accumulator in registers
// and runs the online softmax over 32-key tiles of K and V staged in LDS
// (every lane reads the same K/V element at a time: an LDS broadcast).  The
// key/value chunks of a ring visit are met in ring order within one launch.  It is
// meant for correctness-critical fp32 use; the bf16 MFMA kernel is the
// throughput path.
#include "attn_common.h"

namespace sqkv {
namespace {

constexpr int kRows = 64;   // query rows per workgroup (one wavefront)
constexpr int kTile = 32;   // keys per LDS tile

template <int D>
__global__ void __launch_bounds__(kRows) attn_f32_kernel(AttnParams p) {
  __shared__ float ks[kTile][D];
  __shared__ float vs[kTile][D];
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int hk = h / p.group;
  const int t = blockIdx.x * kRows + threadIdx.x;
  const bool row_ok = t < p.n_q;
  const float* qrow = static_cast<const float*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)(row_ok ? t : 0) * p.q_sn;
  const float* kb0 = static_cast<const float*>(p.k) + b * p.k_sb + hk * p.k_sh;
  const float* vb0 = static_cast<const float*>(p.v) + b * p.v_sb + hk * p.v_sh;

  float q[D];
  float o[D];
#pragma unroll
  for (int e = 0; e < D; e += 4) {
    float4 x = row_ok ? *reinterpret_cast<const float4*>(qrow + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    q[e] = x.x; q[e + 1] = x.y; q[e + 2] = x.z; q[e + 3] = x.w;
    o[e] = o[e + 1] = o[e + 2] = o[e + 3] = 0.f;
  }
  const float c = p.scale_log2;
  const int64_t qpos = p.q_pos0 + t;
  const int64_t tmax = min((int64_t)blockIdx.x * kRows + kRows - 1, (int64_t)p.n_q - 1);
  float m = kNegInf;  // running max of logits, base-2 units
  float l = 0.f;      // running normaliser
  // chunks in ring order: visit s reads chunk j = (rank - s) mod P
  for (int s = 0; s < p.nseg; ++s) {
    const int j = (p.rank - s + p.P) % p.P;
    const float* kb = kb0 + (int64_t)j * p.k_cs;
    const float* vb = vb0 + (int64_t)j * p.v_cs;
    const int64_t kpos0 = p.k_pos0 + (int64_t)j * p.k_posstride;
    // causal: keys u with kpos0 + u <= max query position of this block
    int64_t n_keys = p.n_k;
    if (p.causal) n_keys = max((int64_t)0, min(n_keys, p.q_pos0 + tmax - kpos0 + 1));
    for (int64_t k0 = 0; k0 < n_keys; k0 += kTile) {
      __syncthreads();
      for (int i = threadIdx.x; i < kTile * D / 4; i += kRows) {
        int r = i / (D / 4), e = (i % (D / 4)) * 4;
        int64_t u = k0 + r;
        float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
        if (u < n_keys) {
          kx = *reinterpret_cast<const float4*>(kb + u * p.k_sn + e);
          vx = *reinterpret_cast<const float4*>(vb + u * p.v_sn + e);
        }
        *reinterpret_cast<float4*>(&ks[r][e]) = kx;
        *reinterpret_cast<float4*>(&vs[r][e]) = vx;
      }
      __syncthreads();
      float sc[kTile];
      float tmx = kNegInf;
#pragma unroll
      for (int jj = 0; jj < kTile; ++jj) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) acc = fmaf(q[e], ks[jj][e], acc);
        int64_t u = k0 + jj;
        bool vis = u < n_keys && (!p.causal || kpos0 + u <= qpos);
        sc[jj] = vis ? acc * c : kNegInf;
        tmx = fmaxf(tmx, sc[jj]);
      }
      float mn = fmaxf(m, tmx);
      if (mn != kNegInf) {
        float alpha = (m == mn) ? 1.f : exp2f(m - mn);
        l *= alpha;
#pragma unroll
        for (int e = 0; e < D; ++e) o[e] *= alpha;
        m = mn;
#pragma unroll
        for (int jj = 0; jj < kTile; ++jj) {
          float pj = exp2f(sc[jj] - m);
          l += pj;
#pragma unroll
          for (int e = 0; e < D; ++e) o[e] = fmaf(pj, vs[jj][e], o[e]);
        }
      }
    }
  }
  if (!row_ok) return;
  // chunk partial: normalised output and natural-log lse
  float lse_j = (l > 0.f) ? (m + log2f(l)) * kLn2 : kNegInf;
  float inv = (l > 0.f) ? 1.f / l : 0.f;
  const int64_t bh_row = (int64_t)b * p.Hq + h;
  float wi = 0.f, wj = 1.f, lse = lse_j;
  if (p.o_in != nullptr) lse = lse_merge_weights(p.lse_in[bh_row * p.lse_in_hs + t], lse_j, wi, wj);
  const int64_t ooff = b * p.oo_sb + h * p.oo_sh + (int64_t)t * p.oo_sn;
  const int64_t ioff = b * p.oi_sb + h * p.oi_sh + (int64_t)t * p.oi_sn;
#pragma unroll
  for (int e = 0; e < D; e += 4) {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) y[i] = (wj != 0.f) ? wj * (o[e + i] * inv) : 0.f;
    if (p.o_in != nullptr && wi != 0.f) {
      float x[4];
      load4(p.o_in, ioff + e, p.acc_dtype, x);
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = fmaf(wi, x[i], y[i]);
    }
    store4(p.o_out, ooff + e, p.out_dtype, y);
  }
  p.lse_out[bh_row * p.lse_out_hs + t] = lse;
}

}  // namespace

hipError_t launch_attn_f32(const AttnParams& p, int d, hipStream_t s) {
  if (p.n_q == 0) return hipSuccess;
  dim3 grid((unsigned)((p.n_q + kRows - 1) / kRows), (unsigned)p.Hq, (unsigned)p.B);
  if (d == 128)
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(kRows), 0, s, p);
  else
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(kRows), 0, s, p);
  return hipGetLastError();
}

}  // namespace sqkv
