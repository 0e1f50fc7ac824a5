// Chunk attention with fp32 inputs and fp32 arithmetic throughout.
//
// Ring-attention Q&A (aivaro.ru answer 425), section 5: for one query chunk
// and one key/value chunk, scores q.k, the row maximum, exponentials, the row
// sum (normaliser) and the weighted sum of values; the chunk's partial is
// then merged into the running output (online softmax).
//
// This is the exact-precision variant (no reduced-precision products): one
// lane owns one query row and keeps q and its output accumulator in
// registers; the four wavefronts of a workgroup share its 64 rows and split
// the visit's 32-key tiles between them (tile g goes to wave g mod 4), each
// running its own online softmax over its tiles, staged in its own LDS
// region (every lane reads the same K/V element at a time: an LDS
// broadcast).  At the end the waves' partial states of a row are merged in
// LDS (log-sum-exp weights), each wave finishing its share of the columns.
// The key/value chunks of a ring visit are met in ring order within one
// launch.  It is meant for correctness-critical fp32 use; the bf16 MFMA
// kernel is the throughput path.
#include "attn_common.h"

namespace sqkv {
namespace {

constexpr int kRows = 64;    // query rows per workgroup (one per lane)
constexpr int kTile = 32;    // keys per LDS tile

template <int D>
struct F32Cfg {
  static constexpr int SPLIT = 4;                              // wavefronts, each with every SPLIT-th tile
  // per wave: its K and V tile; reused at the end for the partial states
  static constexpr int TILES = SPLIT * 2 * kTile * D;         // floats
  static constexpr int STATE = kRows * (D + 2) * SPLIT;       // (o[D], m, l) per row and wave
  static constexpr int FLOATS = TILES > STATE ? TILES : STATE;
  static_assert(FLOATS * 4 <= 160 * 1024, "LDS");
  static_assert(D % (4 * SPLIT) == 0, "whole float4 column groups per wave");
};

template <int D>
__global__ void __launch_bounds__(kRows * F32Cfg<D>::SPLIT) attn_f32_kernel(AttnParams p) {
  constexpr int kSplit = F32Cfg<D>::SPLIT;
  extern __shared__ float lds_f[];
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kRows);
  const int lane = threadIdx.x % kRows;
  float* ks = lds_f + wave * 2 * kTile * D;    // [kTile][D]
  float* vs = ks + kTile * D;                  // [kTile][D]
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int hk = h / p.group;
  const int t = blockIdx.x * kRows + lane;
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
  int g = 0;          // tile number within the visit
  // chunks in ring order: visit s reads chunk j = (rank - s) mod P
  for (int s = 0; s < p.nseg; ++s) {
    const int j = (p.rank - s + p.P) % p.P;
    const float* kb = kb0 + (int64_t)j * p.k_cs;
    const float* vb = vb0 + (int64_t)j * p.v_cs;
    const int64_t kpos0 = p.k_pos0 + (int64_t)j * p.k_posstride;
    // causal: keys u with kpos0 + u <= max query position of this block
    int64_t n_keys = p.n_k;
    if (p.causal) n_keys = max((int64_t)0, min(n_keys, p.q_pos0 + tmax - kpos0 + 1));
    for (int64_t k0 = 0; k0 < n_keys; k0 += kTile, ++g) {
      if (g % kSplit != wave) continue;
      // this wave's region only: the wave's own LDS accesses complete in
      // order, so no workgroup barrier is needed (and the waves may make
      // different numbers of tiles)
      for (int i = lane; i < kTile * D / 4; i += kRows) {
        int r = i / (D / 4), e = (i % (D / 4)) * 4;
        int64_t u = k0 + r;
        float4 kx = make_float4(0.f, 0.f, 0.f, 0.f), vx = kx;
        if (u < n_keys) {
          kx = *reinterpret_cast<const float4*>(kb + u * p.k_sn + e);
          vx = *reinterpret_cast<const float4*>(vb + u * p.v_sn + e);
        }
        *reinterpret_cast<float4*>(ks + r * D + e) = kx;
        *reinterpret_cast<float4*>(vs + r * D + e) = vx;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      float sc[kTile];
      float tmx = kNegInf;
#pragma unroll
      for (int jj = 0; jj < kTile; ++jj) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < D; ++e) acc = fmaf(q[e], ks[jj * D + e], acc);
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
          for (int e = 0; e < D; ++e) o[e] = fmaf(pj, vs[jj * D + e], o[e]);
        }
      }
      // every lane's reads of this tile are done before the next one is staged
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  // Merge the waves' partial states of each row: state (o, m, l) of wave w
  // for row `lane` sits at st + (w * kRows + lane) * (D + 2).
  __syncthreads();   // every wave is done with its tiles
  float* st = lds_f;
  {
    float* mine = st + (wave * kRows + lane) * (D + 2);
#pragma unroll
    for (int e = 0; e < D; ++e) mine[e] = o[e];
    mine[D] = m;
    mine[D + 1] = l;
  }
  __syncthreads();
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < kSplit; ++w) M = fmaxf(M, st[(w * kRows + lane) * (D + 2) + D]);
  float a[kSplit];
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kSplit; ++w) {
    const float mw = st[(w * kRows + lane) * (D + 2) + D];
    a[w] = (mw == kNegInf) ? 0.f : exp2f(mw - M);
    L += a[w] * st[(w * kRows + lane) * (D + 2) + D + 1];
  }
  if (!row_ok) return;
  // chunk partial: normalised output and natural-log lse; this wave writes
  // columns [wave * D / kSplit, (wave + 1) * D / kSplit) of the row
  float lse_j = (L > 0.f) ? (M + log2f(L)) * kLn2 : kNegInf;
  float inv = (L > 0.f) ? 1.f / L : 0.f;
  const int64_t bh_row = (int64_t)b * p.Hq + h;
  float wi = 0.f, wj = 1.f, lse = lse_j;
  if (p.o_in != nullptr) lse = lse_merge_weights(p.lse_in[bh_row * p.lse_in_hs + t], lse_j, wi, wj);
  const int64_t ooff = b * p.oo_sb + h * p.oo_sh + (int64_t)t * p.oo_sn;
  const int64_t ioff = b * p.oi_sb + h * p.oi_sh + (int64_t)t * p.oi_sn;
  constexpr int kCols = D / kSplit;
  const int e0 = wave * kCols;
#pragma unroll
  for (int e = 0; e < kCols; e += 4) {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < kSplit; ++w) acc = fmaf(a[w], st[(w * kRows + lane) * (D + 2) + e0 + e + i], acc);
      y[i] = (wj != 0.f) ? wj * (acc * inv) : 0.f;
    }
    if (p.o_in != nullptr && wi != 0.f) {
      float x[4];
      load4(p.o_in, ioff + e0 + e, p.acc_dtype, x);
#pragma unroll
      for (int i = 0; i < 4; ++i) y[i] = fmaf(wi, x[i], y[i]);
    }
    store4(p.o_out, ooff + e0 + e, p.out_dtype, y);
  }
  if (wave == 0) p.lse_out[bh_row * p.lse_out_hs + t] = lse;
}

}  // namespace

hipError_t launch_attn_f32(const AttnParams& p, int d, hipStream_t s) {
  if (p.n_q == 0) return hipSuccess;
  dim3 grid((unsigned)((p.n_q + kRows - 1) / kRows), (unsigned)p.Hq, (unsigned)p.B);
  if (d == 128) {
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = allow_dyn_lds(reinterpret_cast<const void*>(&attn_f32_kernel<128>), F32Cfg<128>::FLOATS * 4, lds_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(kRows * F32Cfg<128>::SPLIT), F32Cfg<128>::FLOATS * 4, s, p);
  } else {
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = allow_dyn_lds(reinterpret_cast<const void*>(&attn_f32_kernel<64>), F32Cfg<64>::FLOATS * 4, lds_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(kRows * F32Cfg<64>::SPLIT), F32Cfg<64>::FLOATS * 4, s, p);
  }
  return hipGetLastError();
}

}  // namespace sqkv
