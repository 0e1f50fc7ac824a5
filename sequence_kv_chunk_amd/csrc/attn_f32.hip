// Chunk attention with fp32 inputs and fp32 arithmetic throughout.
//
// Ring-attention Q&A (aivaro.ru answer 425), section 5: for one query chunk
// and one key/value chunk, scores q.k, the row maximum, exponentials, the row
// sum (normaliser) and the weighted sum of values; the chunk's partial is
// then merged into the running output (online softmax).
//
// This is the exact-precision variant: the products run on the fp32 matrix
// cores (v_mfma_f32_32x32x2_f32: fp32 operands, fp32 accumulation, no
// reduced-precision rounding).  A workgroup takes 32 query rows; its four
// wavefronts split the visit's 32-key tiles between them (tile g goes to
// wave g mod 4), each running its own online softmax over its tiles, staged
// in its own LDS region.  Per tile a wave forms S^T = K Q^T (keys on the
// MFMA M axis, so a lane holds 16 keys of ONE query: the row maximum and sum
// are lane-local plus one exchange with the lane holding the query's other
// 16 keys) and O^T += V^T P^T, where P^T is the S^T registers themselves
// (the k index of a step pairs key 8g + x of one lane half with key
// 8g + 4 + x of the other).  Q^T stays in registers (lane half h holds
// d = h*D/2 .. h*D/2 + D/2 - 1 of its query).  At the end the waves' partial
// states of a row are merged in LDS (log-sum-exp weights).  The key/value
// chunks of a ring visit are met in ring order within one launch.  It is
// meant for correctness-critical fp32 use; the bf16 kernel is the
// throughput path.
#include "attn_common.h"

namespace sqkv {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kRows = 32;    // query rows per workgroup
constexpr int kTile = 32;    // keys per LDS tile
constexpr int kSplit = 4;    // wavefronts, each with every kSplit-th tile

template <int D>
struct F32Cfg {
  static constexpr int KROW = D + 4;                            // padded K row (floats): conflict-free b128 reads
  static constexpr int WAVE = kTile * KROW + kTile * D;         // one wave's K and V tile (floats)
  static constexpr int STATE = kSplit * kRows * (D + 2);        // (o[D], m, l) per wave and row
  static constexpr int FLOATS = kSplit * WAVE > STATE ? kSplit * WAVE : STATE;
  static_assert(FLOATS * 4 <= 160 * 1024, "LDS");
  static_assert(D % 32 == 0, "whole 32-row blocks of d");
};

__device__ __forceinline__ f32x16_t mfma_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D>
__global__ void __launch_bounds__(64 * kSplit) attn_f32_kernel(AttnParams p) {
  using C = F32Cfg<D>;
  constexpr int MB = D / 32;   // 32-row blocks of d in O^T
  extern __shared__ float lds_f[];
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / 64);
  const int lane = threadIdx.x % 64;
  const int l32 = lane & 31, hi = lane >> 5;
  float* ks = lds_f + wave * C::WAVE;          // [kTile][KROW]
  float* vs = ks + kTile * C::KROW;            // [kTile][D]
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int hk = h / p.group;
  const int q0 = blockIdx.x * kRows;
  const int t = q0 + l32;                      // this lane's query row
  const bool row_ok = t < p.n_q;
  const float* qrow = static_cast<const float*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)(row_ok ? t : 0) * p.q_sn;
  const float* kb0 = static_cast<const float*>(p.k) + b * p.k_sb + hk * p.k_sh;
  const float* vb0 = static_cast<const float*>(p.v) + b * p.v_sb + hk * p.v_sh;

  // Q^T operand: d = hi * D/2 + s of the lane's query (zeros past n_q)
  float q[D / 2];
#pragma unroll
  for (int e = 0; e < D / 2; e += 4) {
    const float4 x = row_ok ? *reinterpret_cast<const float4*>(qrow + hi * (D / 2) + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    q[e] = x.x; q[e + 1] = x.y; q[e + 2] = x.z; q[e + 3] = x.w;
  }
  // O^T: element j of block mb holds d = 32 mb + 8 (j/4) + 4 hi + j%4 of the query
  f32x16_t o[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) o[mb] = (f32x16_t){};
  const float c = p.scale_log2;
  const int64_t qpos = p.q_pos0 + t;
  const int64_t tmax = min((int64_t)q0 + kRows - 1, (int64_t)p.n_q - 1);
  float m = kNegInf;  // running max of logits, base-2 units (same in both lane halves)
  float l = 0.f;      // this lane's part of the running normaliser (its 16 keys of each tile)
  // The wave's tiles in the visit's order: tile g (counting the 32-key tiles
  // of every chunk, chunks in ring order: visit s reads chunk
  // j = (rank - s) mod P) goes to wave g mod kSplit.  A cursor (s, k0) names
  // a tile; the wave holds its next tile's rows in registers while it works
  // on the current one.
  auto chunk = [&](int s, const float*& kb, const float*& vb, int64_t& kpos0) -> int64_t {
    const int j = (p.rank - s + p.P) % p.P;
    kb = kb0 + (int64_t)j * p.k_cs;
    vb = vb0 + (int64_t)j * p.v_cs;
    kpos0 = p.k_pos0 + (int64_t)j * p.k_posstride;
    // causal: keys u with kpos0 + u <= max query position of this block
    int64_t n_keys = p.n_k;
    if (p.causal) n_keys = max((int64_t)0, min(n_keys, p.q_pos0 + tmax - kpos0 + 1));
    return n_keys;
  };
  // moves (s, k0) on by `steps` tiles; s = nseg past the last tile
  auto advance = [&](int& s, int64_t& k0, int steps) {
    k0 += (int64_t)steps * kTile;
    while (s < p.nseg) {
      const float* kb;
      const float* vb;
      int64_t kpos0;
      const int64_t span = (chunk(s, kb, vb, kpos0) + kTile - 1) / kTile * kTile;
      if (k0 < span) break;
      k0 -= span;
      ++s;
    }
  };
  // row r0 + kRpi * it of a tile, columns e .. e+3 (kRpi rows per pass)
  constexpr int kRpi = 256 / D;
  constexpr int kPass = kTile / kRpi;
  const int r0 = lane / (D / 4), e4 = (lane % (D / 4)) * 4;
  float4 pk[kPass], pv[kPass];
  auto fetch = [&](int s, int64_t k0) {
    if (s >= p.nseg) return;
    const float* kb;
    const float* vb;
    int64_t kpos0;
    const int64_t n_keys = chunk(s, kb, vb, kpos0);
    const int nv = (int)min(n_keys - k0, (int64_t)kTile);   // valid rows of the tile
    const float* kr = kb + (k0 + r0) * p.k_sn + e4;
    const float* vr = vb + (k0 + r0) * p.v_sn + e4;
    if (nv == kTile) {   // a whole tile (a uniform branch)
#pragma unroll
      for (int it = 0; it < kPass; ++it) {
        pk[it] = *reinterpret_cast<const float4*>(kr + (int64_t)(kRpi * it) * p.k_sn);
        pv[it] = *reinterpret_cast<const float4*>(vr + (int64_t)(kRpi * it) * p.v_sn);
      }
    } else {             // the chunk's last keys: rows past them are zeros
#pragma unroll
      for (int it = 0; it < kPass; ++it) {
        pk[it] = pv[it] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r0 + kRpi * it < nv) {
          pk[it] = *reinterpret_cast<const float4*>(kr + (int64_t)(kRpi * it) * p.k_sn);
          pv[it] = *reinterpret_cast<const float4*>(vr + (int64_t)(kRpi * it) * p.v_sn);
        }
      }
    }
  };
  int cs = 0;
  int64_t ck0 = 0;
  advance(cs, ck0, wave);
  fetch(cs, ck0);
  while (cs < p.nseg) {
    // this wave's LDS region only: the wave's own LDS accesses complete in
    // order, so no workgroup barrier is needed (and the waves may make
    // different numbers of tiles)
#pragma unroll
    for (int it = 0; it < kPass; ++it) {
      const int r = r0 + kRpi * it;
      *reinterpret_cast<float4*>(ks + r * C::KROW + e4) = pk[it];
      *reinterpret_cast<float4*>(vs + r * D + e4) = pv[it];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int ns = cs;
    int64_t nk0 = ck0;
    advance(ns, nk0, kSplit);
    fetch(ns, nk0);   // the wave's next tile, in flight while this one is used
    const float* kb;
    const float* vb;
    int64_t kpos0;
    const int64_t n_keys = chunk(cs, kb, vb, kpos0);
    const int64_t k0 = ck0;
    // S^T = K Q^T: step e pairs d = e (lane half 0) with d = D/2 + e (half 1)
    f32x16_t st = (f32x16_t){};
    const float* krow = ks + l32 * C::KROW + hi * (D / 2);
#pragma unroll
    for (int e = 0; e < D / 2; e += 4) {
      const float4 kx = *reinterpret_cast<const float4*>(krow + e);
      st = mfma_f32(kx.x, q[e], st);
      st = mfma_f32(kx.y, q[e + 1], st);
      st = mfma_f32(kx.z, q[e + 2], st);
      st = mfma_f32(kx.w, q[e + 3], st);
    }
    // element jj: key 8 (jj/4) + 4 hi + jj%4 of the tile, masked past the
    // chunk's visible keys and (causal) after the query: the lane sees the
    // tile's keys up to `lim`
    int64_t lim64 = n_keys - 1 - k0;
    if (p.causal) lim64 = min(lim64, qpos - kpos0 - k0);
    const int lim = (int)max(min(lim64, (int64_t)kTile), (int64_t)-1) - 4 * hi;
    float tmx = kNegInf;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      st[jj] = (8 * (jj / 4) + (jj % 4) <= lim) ? st[jj] * c : kNegInf;
      tmx = fmaxf(tmx, st[jj]);
    }
    tmx = fmaxf(tmx, __shfl_xor(tmx, 32));   // the query's other 16 keys
    // The row's reference m moves (and o, l are rescaled) only when the
    // tile's maximum exceeds it by more than kSlack (base-2 units): weights
    // then stay below 2^kSlack, which fp32 carries without loss, and the
    // rescale is rare after the first tiles.  No branch on the row's state
    // around the matrix products: they run for the whole wave whatever the
    // lane mask, so a row that has seen no key yet keeps alpha = 1 and gets
    // weights 0.
    constexpr float kSlack = 8.f;
    const bool bump = tmx != kNegInf && (m == kNegInf || tmx > m + kSlack);
    if (__any(bump)) {   // a wave-uniform branch: no MFMA inside
      const float mn = bump ? tmx : m;
      const float alpha = (m == kNegInf || !bump) ? 1.f : exp2f(m - mn);
      l *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) o[mb][jj] *= alpha;
      m = mn;
    }
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      // v_exp_f32: within an ulp for normal results; a weight below 2^-126
      // (flushed to 0) is far below the fp32 bar next to the row's largest (>= 1)
      st[jj] = (st[jj] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(st[jj] - m);
      l += st[jj];
    }
    // O^T += V^T P^T: step (gg, x) pairs key 8gg + x (half 0) with key
    // 8gg + 4 + x (half 1), i.e. element 4gg + x of each lane
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) {
        const float vx = vs[(8 * (jj / 4) + 4 * hi + (jj % 4)) * D + 32 * mb + l32];
        o[mb] = mfma_f32(vx, st[jj], o[mb]);
      }
    // every lane's reads of this tile are done before the next one is written
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    cs = ns;
    ck0 = nk0;
  }
  // Merge the waves' partial states of each row: state (o[D], m, l) of wave
  // w for row n sits at stt + (w * kRows + n) * (D + 2).
  __syncthreads();   // every wave is done with its tiles
  float* stt = lds_f;
  {
    float* mine = stt + (wave * kRows + l32) * (D + 2);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int gg = 0; gg < 4; ++gg)
#pragma unroll
        for (int x = 0; x < 4; ++x) mine[32 * mb + 8 * gg + 4 * hi + x] = o[mb][4 * gg + x];
    const float lsum = l + __shfl_xor(l, 32);
    if (hi == 0) {
      mine[D] = m;
      mine[D + 1] = lsum;
    }
  }
  __syncthreads();
  // thread -> (row n, column slice): 8 threads per row, D/8 columns each
  const int n = threadIdx.x / 8;
  const int t_out = q0 + n;
  if (t_out >= p.n_q) return;
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < kSplit; ++w) M = fmaxf(M, stt[(w * kRows + n) * (D + 2) + D]);
  float a[kSplit];
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kSplit; ++w) {
    const float mw = stt[(w * kRows + n) * (D + 2) + D];
    a[w] = (mw == kNegInf) ? 0.f : exp2f(mw - M);
    L += a[w] * stt[(w * kRows + n) * (D + 2) + D + 1];
  }
  // chunk partial: normalised output and natural-log lse, merged with the
  // running state when there is one
  const float lse_j = (L > 0.f) ? (M + log2f(L)) * kLn2 : kNegInf;
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
  const int64_t bh_row = (int64_t)b * p.Hq + h;
  float wi = 0.f, wj = 1.f, lse = lse_j;
  if (p.o_in != nullptr) lse = lse_merge_weights(p.lse_in[bh_row * p.lse_in_hs + t_out], lse_j, wi, wj);
  const int64_t ooff = b * p.oo_sb + h * p.oo_sh + (int64_t)t_out * p.oo_sn;
  const int64_t ioff = b * p.oi_sb + h * p.oi_sh + (int64_t)t_out * p.oi_sn;
  constexpr int kCols = D / 8;
  const int e0 = (threadIdx.x % 8) * kCols;
#pragma unroll
  for (int e = 0; e < kCols; e += 4) {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < kSplit; ++w) acc = fmaf(a[w], stt[(w * kRows + n) * (D + 2) + e0 + e + i], acc);
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
  if (threadIdx.x % 8 == 0) p.lse_out[bh_row * p.lse_out_hs + t_out] = lse;
}

}  // namespace

hipError_t launch_attn_f32(const AttnParams& p, int d, hipStream_t s) {
  if (p.n_q == 0) return hipSuccess;
  dim3 grid((unsigned)((p.n_q + kRows - 1) / kRows), (unsigned)p.Hq, (unsigned)p.B);
  if (d == 128) {
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = allow_dyn_lds(reinterpret_cast<const void*>(&attn_f32_kernel<128>), F32Cfg<128>::FLOATS * 4, lds_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(64 * kSplit), F32Cfg<128>::FLOATS * 4, s, p);
  } else {
    static std::atomic<uint64_t> lds_set{0};
    hipError_t e = allow_dyn_lds(reinterpret_cast<const void*>(&attn_f32_kernel<64>), F32Cfg<64>::FLOATS * 4, lds_set);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(64 * kSplit), F32Cfg<64>::FLOATS * 4, s, p);
  }
  return hipGetLastError();
}

}  // namespace sqkv
