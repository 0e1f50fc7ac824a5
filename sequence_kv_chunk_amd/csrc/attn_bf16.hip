// Chunk attention with bf16 inputs on gfx950 matrix cores.
//
// Ring-attention Q&A (aivaro.ru answer 425), section 5: for a query chunk and
// one resident key/value chunk compute the scores Q K^T, the row maximum, the
// exponentials, the row sum and P V; merge the chunk's partial into the
// running output with an online-softmax rescale.
//
// Design (gfx950, wave64, v_mfma_f32_32x32x16_bf16):
// * A workgroup of 4 wavefronts owns 256 query rows of one (batch, head); each
//   wavefront owns 64 rows (two 32-column MFMA blocks) and keeps its Q
//   fragments in registers for the whole key loop.
// * The scores are computed transposed, S^T = K Q^T (keys on the MFMA M axis,
//   queries on N).  In the 32x32 accumulator layout a lane then holds 16 keys
//   of ONE query column, so the row max and row sum are in-lane reductions plus
//   one exchange with the lane 32 apart -- no cross-lane reduction trees.
// * The same accumulator registers, rounded to bf16, are directly the B
//   operand of O^T = V^T P^T: the key order inside each 16-key contraction
//   step is taken from the accumulator layout, and V^T is read from LDS in
//   that same order.
// * K tiles (64 keys x d) sit in LDS row-major with a 16-byte row pad; V tiles
//   are transposed into LDS (V^T, d rows of 64 keys) with an XOR swizzle of
//   8-byte key groups so that both the transposing writes and the fragment
//   reads avoid bank conflicts.  Both are double-buffered: the global loads of
//   tile t+1 are in flight while tile t is computed.
// * Softmax runs in base 2 with scale*log2(e) folded into one FMA.  The
//   running maximum is only moved (and the accumulator rescaled) when a tile
//   raises it by more than kRescaleLog2; in between, weights are taken against
//   the slightly stale maximum, which leaves the normalised result unchanged
//   and bounds weights by 2^kRescaleLog2.
// * Causal masking is applied only on tiles that straddle the diagonal or the
//   ragged end of the chunk; tiles entirely above the diagonal are skipped.
#include "attn_common.h"

namespace sqkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQW = 64;              // query rows per wavefront
constexpr int kBM = kQW * kWaves;    // query rows per workgroup
constexpr int kBN = 64;              // keys per tile
constexpr float kRescaleLog2 = 8.0f;

template <int D>
struct Cfg {
  static constexpr int KC = D / 16;           // 16-wide contraction steps over d
  static constexpr int MD = D / 32;           // 32-row blocks of d in O^T
  static constexpr int KPITCH = D + 8;        // bf16 per K row in LDS
  static constexpr int K_STAGE = kBN * KPITCH;
  static constexpr int VT_STAGE = D * kBN;
  static constexpr int VPR = D / 8;           // 16-byte vectors per row
  static constexpr int KPT = D / 32;          // rows (keys) loaded per thread
  static constexpr int LDS_BYTES = 2 * (K_STAGE + VT_STAGE) * 2;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

// V^T tile: row d holds 64 keys as 16 groups of 4; group g of row d is stored
// at group position g ^ (d & 15) ^ ((d >> 4) & 7).
__device__ __forceinline__ int vt_index(int d, int key) {
  int g = (key >> 2) ^ (d & 15) ^ ((d >> 4) & 7);
  return d * kBN + g * 4 + (key & 3);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

template <int D>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(1, 1)))
attn_bf16_kernel(AttnParams p, int n_qtiles) {
  using C = Cfg<D>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
  uint16_t* k_lds = smem;                       // 2 stages
  uint16_t* vt_lds = smem + 2 * C::K_STAGE;     // 2 stages

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // Workgroup -> (b, h, q-tile).  Heads vary fastest so that consecutive
  // workgroups (spread round-robin over the XCDs) cover all heads; with a
  // causal mask the q-tiles are issued heaviest (last) first.
  const int BH = p.B * p.Hq;
  const int qt_rank = blockIdx.x / BH;
  const int bh = blockIdx.x - qt_rank * BH;
  const int qt = p.causal ? (n_qtiles - 1 - qt_rank) : qt_rank;
  const int b = bh / p.Hq;
  const int h = bh - b * p.Hq;
  const int hk = h / p.group;

  const int q0 = qt * kBM;                 // first row of the workgroup
  const int qw0 = q0 + wave * kQW;         // first row of this wavefront

  const uint16_t* qg = static_cast<const uint16_t*>(p.q) + b * p.q_sb + h * p.q_sh;
  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + b * p.k_sb + hk * p.k_sh;
  const uint16_t* vg = static_cast<const uint16_t*>(p.v) + b * p.v_sb + hk * p.v_sh;

  // ---- Q fragments (B operand of S^T = K Q^T) -------------------------------
  // lane holds Q[row = qw0 + 32*nb + l32][16*kc + 8*hi .. +7]
  u32x4_t qf[2][C::KC];
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    int row = qw0 + 32 * nb + l32;
    bool ok = row < p.n_q;
    const uint16_t* src = qg + (int64_t)(ok ? row : 0) * p.q_sn + 8 * hi;
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      u32x4_t z = {0u, 0u, 0u, 0u};
      qf[nb][kc] = ok ? *reinterpret_cast<const u32x4_t*>(src + 16 * kc) : z;
    }
  }

  // ---- key range -------------------------------------------------------------
  int64_t n_keys = p.n_k;
  const int q_last_wg = min(q0 + kBM, p.n_q) - 1;
  if (p.causal) {
    int64_t lim = p.q_pos0 + q_last_wg - p.k_pos0 + 1;
    n_keys = max((int64_t)0, min(n_keys, lim));
  }
  const int ntiles = (int)((n_keys + kBN - 1) / kBN);
  const int q_last_w = min(qw0 + kQW, p.n_q) - 1;   // last valid row of the wave
  const bool wave_active = qw0 < p.n_q;

  // ---- global -> register -> LDS staging -------------------------------------
  // thread owns rows kq*KPT .. kq*KPT+KPT-1 and the 8 columns 8*dg .. 8*dg+7
  const int dg = tid % C::VPR;
  const int kq = tid / C::VPR;
  u32x4_t kreg[C::KPT], vreg[C::KPT];

  auto load_tile = [&](int t) {
#pragma unroll
    for (int r = 0; r < C::KPT; ++r) {
      int64_t u = (int64_t)t * kBN + kq * C::KPT + r;
      u32x4_t z = {0u, 0u, 0u, 0u};
      bool ok = u < n_keys;
      int64_t uu = ok ? u : 0;
      kreg[r] = ok ? *reinterpret_cast<const u32x4_t*>(kg + uu * p.k_sn + 8 * dg) : z;
      vreg[r] = ok ? *reinterpret_cast<const u32x4_t*>(vg + uu * p.v_sn + 8 * dg) : z;
    }
  };
  auto store_tile = [&](int stage) {
    uint16_t* kd = k_lds + stage * C::K_STAGE;
    uint16_t* vd = vt_lds + stage * C::VT_STAGE;
#pragma unroll
    for (int r = 0; r < C::KPT; ++r)
      *reinterpret_cast<u32x4_t*>(kd + (kq * C::KPT + r) * C::KPITCH + 8 * dg) = kreg[r];
    // transpose: word w of a 16-byte row vector holds columns 8*dg+2w (low
    // half) and 8*dg+2w+1 (high half); gather the KPT keys of one column into
    // one 4- or 8-byte LDS chunk
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int d = 8 * dg + 2 * w + half;
        uint16_t* dst = vd + vt_index(d, kq * C::KPT);
        auto pick = [&](int r) -> uint32_t {
          return half ? (vreg[r][w] >> 16) : (vreg[r][w] & 0xffffu);
        };
        if constexpr (C::KPT == 4) {
          u32x2_t pk;
          pk[0] = pick(0) | (pick(1) << 16);
          pk[1] = pick(2) | (pick(3) << 16);
          *reinterpret_cast<u32x2_t*>(dst) = pk;
        } else {
          *reinterpret_cast<uint32_t*>(dst) = pick(0) | (pick(1) << 16);
        }
      }
    }
  };

  // ---- accumulators -------------------------------------------------------------
  f32x16_t oacc[C::MD][2];
#pragma unroll
  for (int md = 0; md < C::MD; ++md)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j) oacc[md][nb][j] = 0.f;
  float m_run[2] = {kNegInf, kNegInf};  // running max, base-2 units
  float l_run[2] = {0.f, 0.f};          // this lane's half of the row sum
  const float c = p.scale_log2;

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int stage = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);

    const int64_t key0 = (int64_t)t * kBN;        // first key of the tile
    // wave-level classification of this tile
    const bool skip = !wave_active || (p.causal && p.k_pos0 + key0 > p.q_pos0 + q_last_w);
    if (!skip) {
      const bool need_mask = (key0 + kBN > n_keys) ||
                             (p.causal && p.k_pos0 + key0 + kBN - 1 > p.q_pos0 + qw0);
      const uint16_t* kd = k_lds + stage * C::K_STAGE;
      const uint16_t* vd = vt_lds + stage * C::VT_STAGE;

      // S^T[key][query] for 64 keys (2 M-blocks) x 64 queries (2 N-blocks)
      f32x16_t s[2][2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
          for (int j = 0; j < 16; ++j) s[mb][nb][j] = 0.f;
#pragma unroll
      for (int kc = 0; kc < C::KC; ++kc) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          u32x4_t kf = *reinterpret_cast<const u32x4_t*>(kd + (32 * mb + l32) * C::KPITCH + 16 * kc + 8 * hi);
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            s[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[nb][kc]),
                                                                  s[mb][nb], 0, 0, 0);
        }
      }

      // accumulator element j of block mb holds key 32*mb + 8*(j/4) + 4*hi + j%4
      if (need_mask) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const int64_t qpos = p.q_pos0 + qw0 + 32 * nb + l32;
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
              int64_t u = key0 + 32 * mb + 8 * (j >> 2) + 4 * hi + (j & 3);
              bool vis = u < n_keys && (!p.causal || p.k_pos0 + u <= qpos);
              if (!vis) s[mb][nb][j] = kNegInf;
            }
        }
      }

      u32x4_t pf[2][4];   // bf16 weights: B operand of O^T = V^T P^T
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        float mx = kNegInf;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[mb][nb][j]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mxs = mx * c;
        if (__any(mxs > m_run[nb] + kRescaleLog2)) {
          const float mn = fmaxf(m_run[nb], mxs);
          const float alpha = (mn == m_run[nb]) ? 1.f : exp2f(m_run[nb] - mn);
          l_run[nb] *= alpha;
#pragma unroll
          for (int md = 0; md < C::MD; ++md)
#pragma unroll
            for (int j = 0; j < 16; ++j) oacc[md][nb][j] *= alpha;
          m_run[nb] = mn;
        }
        const float mneg = (m_run[nb] == kNegInf) ? 0.f : -m_run[nb];
        float ls = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            float e = __builtin_amdgcn_exp2f(fmaf(s[mb][nb][j], c, mneg));
            s[mb][nb][j] = e;
            ls += e;
          }
        l_run[nb] += ls;
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
          const int mb = cc >> 1, j0 = 8 * (cc & 1);
#pragma unroll
          for (int w = 0; w < 4; ++w)
            pf[nb][cc][w] = pack_bf16x2(s[mb][nb][j0 + 2 * w], s[mb][nb][j0 + 2 * w + 1]);
        }
      }

      // O^T[d][query] += V^T[d][key] P^T[key][query]; contraction step cc covers
      // keys 16*cc + {4*hi .. 4*hi+3} and 16*cc + 8 + {4*hi .. 4*hi+3}
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
        for (int md = 0; md < C::MD; ++md) {
          const int d = 32 * md + l32;
          u32x2_t a0 = *reinterpret_cast<const u32x2_t*>(vd + vt_index(d, 16 * cc + 4 * hi));
          u32x2_t a1 = *reinterpret_cast<const u32x2_t*>(vd + vt_index(d, 16 * cc + 8 + 4 * hi));
          u32x4_t vf = {a0[0], a0[1], a1[0], a1[1]};
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            oacc[md][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(vf), as_bf16x8(pf[nb][cc]),
                                                                     oacc[md][nb], 0, 0, 0);
        }
      }
    }

    if (t + 1 < ntiles) store_tile(stage ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, merge into the running (O, lse), store ------------
  if (!wave_active) return;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int row = qw0 + 32 * nb + l32;
    const float lt = l_run[nb] + __shfl_xor(l_run[nb], 32);
    if (row >= p.n_q) continue;
    const float lse_j = (lt > 0.f) ? (m_run[nb] + log2f(lt)) * kLn2 : kNegInf;
    const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
    const int64_t srow = ((int64_t)b * p.Hq + h) * p.n_q + row;
    float wi = 0.f, wj = 1.f, lse = lse_j;
    if (p.o_in != nullptr) lse = lse_merge_weights(p.lse_in[srow], lse_j, wi, wj);
    const float f = wj * inv;
    const int64_t ooff = b * p.oo_sb + h * p.oo_sh + (int64_t)row * p.oo_sn;
    const int64_t ioff = b * p.oi_sb + h * p.oi_sh + (int64_t)row * p.oi_sn;
#pragma unroll
    for (int md = 0; md < C::MD; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * md + 8 * g + 4 * hi;
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) y[r] = oacc[md][nb][4 * g + r] * f;
        if (p.o_in != nullptr && wi != 0.f) {
          float x[4];
          load4(p.o_in, ioff + d0, p.acc_dtype, x);
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = fmaf(wi, x[r], y[r]);
        }
        store4(p.o_out, ooff + d0, p.out_dtype, y);
      }
    if (hi == 0) p.lse_out[srow] = lse;
  }
}

template <int D>
hipError_t launch_d(const AttnParams& p, hipStream_t s) {
  using C = Cfg<D>;
  const int n_qtiles = (p.n_q + kBM - 1) / kBM;
  const int64_t blocks = (int64_t)n_qtiles * p.B * p.Hq;
  if (blocks == 0) return hipSuccess;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bf16_kernel<D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS_BYTES);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(attn_bf16_kernel<D>, dim3((unsigned)blocks), dim3(kThreads), C::LDS_BYTES, s, p,
                     n_qtiles);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnParams& p, int d, hipStream_t s) {
  if (d == 128) return launch_d<128>(p, s);
  return launch_d<64>(p, s);
}

}  // namespace sqkv
