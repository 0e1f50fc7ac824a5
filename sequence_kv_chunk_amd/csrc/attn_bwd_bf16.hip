// Backward of chunk attention with bf16 inputs on gfx950 matrix cores.
//
// Ring-attention Q&A (aivaro.ru answer 425), "pet project" steps 5-7: the
// ring forward is followed by a loss and a backward pass.  The gradients of
// O = softmax(S) V, S = scale * Q K^T, are (row by row):
//     P = exp(S - lse),  dV = P^T dO,  dP = dO V^T,
//     dS = P * (dP - D) with D = rowsum(dO * O),
//     dQ = scale * dS K,  dK = scale * dS^T Q.
// With the rows' log-sum-exp over ALL keys (what the forward returns), P for
// one (query chunk, key chunk) pair is the full softmax restricted to that
// pair, so a ring backward is a sum of per-pair contributions.  One launch of
// each kernel below adds one pair's share into fp32 dq, dk, dv.
//
// Two kernels, as in the usual split of the attention backward:
// * attn_bwd_dq: parallel over query rows (8 waves x 32 rows per workgroup,
//   two waves per SIMD).  Per 64-key tile it forms S^T = K Q^T and
//   dP^T = V dO^T (keys on the MFMA M axis: a lane holds 16 keys of ONE
//   query, so lse and D are one scalar per lane), the weights and dS^T in
//   registers, and dQ^T += K^T dS^T with the K^T operand read from LDS with
//   ds_read_b64_tr_b16 and dS^T rounded to bf16 as the B operand.  The two
//   32-key blocks of a tile are staggered so that one block's VALU work runs
//   between the other block's MFMAs.
// * attn_bwd_dkdv: parallel over keys (4 waves x 32 keys per workgroup, one
//   wave per SIMD: K and -V rows of the wave's keys in registers, dK^T and
//   dV^T accumulators alongside).  Per 32-query block it forms S = Q K^T and
//   D - dP (queries on M: a lane holds 16 queries of ONE key), P and dS, and
//   dV^T += dO^T P, dK^T += Q^T dS with transposed reads of the dO and Q
//   tiles, three blocks in flight at once.  The query heads of a GQA group
//   are walked inside the workgroup so that a key/value head's gradients sum
//   over them without atomics.
// Tiles (64 rows) are copied global -> LDS by buffer_load ... lds, two
// (dQ) or three (dK/dV) stages deep.  Every tile is read both as rows
// (ds_read_b128) and transposed (ds_read_b64_tr_b16); the 16-byte chunk
// swizzle below keeps both conflict-free.
#include <type_traits>
#include <utility>

#include "attn_common.h"

namespace sqkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
#define SQKV_LDS __attribute__((address_space(3)))

constexpr int kTR = 64;   // rows per LDS tile (keys in the dq kernel, queries in the dk/dv kernel)

template <int D, int NWAVES>
struct BCfg {
  static constexpr int KC = D / 16;            // 16-wide contraction steps over d
  static constexpr int MD = D / 32;            // 32-row blocks of d
  static constexpr int NCH = D / 8;            // 16-byte chunks per row
  static constexpr int ROWB = D * 2;           // bytes per row
  static constexpr int TILE = kTR * ROWB;      // bytes per tile
  static constexpr int RPW = 1024 / ROWB;      // rows per wave-wide 1 KiB load
  static constexpr int NL = TILE / 1024 / NWAVES;   // loads per wave per tile
  static_assert(NL >= 1 && (TILE / 1024) % NWAVES == 0, "tile loads must spread evenly over the waves");
};

// Position of 16-byte chunk c of tile row r: c ^ swz(r).  The low part (by
// r % 4) sends the transpose reads of four consecutive rows to distinct bank
// groups; the high part (by (r / 4) % 4, one coset of the first pattern
// each) makes the 16 rows of a row read distinct as well.
template <int D>
__device__ __forceinline__ int swz(int r) {
  const int f = (r & 3) == 0 ? 0 : (r & 3) == 1 ? 6 : (r & 3) == 2 ? 12 : 10;
  return (f ^ ((r >> 2) & 3)) & (D / 8 - 1);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ u32x4_t lds_b128(uint32_t addr) {
  return *reinterpret_cast<SQKV_LDS const u32x4_t*>((size_t)addr);
}

__device__ __forceinline__ i16x4_t lds_tr16(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<SQKV_LDS i16x4_t*>((size_t)addr));
}

__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = (int)(uint32_t)b;
  r[1] = (int)(uint32_t)(b >> 32);
  r[2] = (int)bytes;                 // num_records: bytes past this read as 0
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from the buffer at `voff` into LDS at m0 + 16 * lane.
__device__ __forceinline__ void dma16(uint32_t voff, i32x4_t rsrc, uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" :: "v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}

// 4 bytes per lane from the buffer at `voff` into LDS at m0 + 4 * lane.
__device__ __forceinline__ void dma4(uint32_t voff, i32x4_t rsrc, uint32_t lds) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" :: "v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}

// s_waitcnt immediate (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8).
constexpr unsigned waitcnt_imm(int vm, int lgkm) {
  return (unsigned)((vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8));
}

// Wait for every DMA and LDS read of this wave, then meet the other waves.
__device__ __forceinline__ void drain_and_sync() {
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
  asm volatile("s_barrier" ::: "memory");
}

// Copies rows [row0, row0 + kTR) of a [n, d] bf16 view (valid rows < n) into
// an LDS tile at `lds`; wave-wide load i of the tile fills rows
// (i * NWAVES + wave) * RPW ..; rows past n arrive as zeros.
template <int D, int NWAVES>
struct TileDma {
  using C = BCfg<D, NWAVES>;
  uint32_t voff[C::NL];
  uint32_t m0_wave;

  __device__ void init(int lane, int wave, int snb) {
#pragma unroll
    for (int i = 0; i < C::NL; ++i) {
      const int r = (i * NWAVES + wave) * C::RPW + lane / C::NCH;
      voff[i] = (uint32_t)(r * snb) + (((lane % C::NCH) ^ swz<D>(r)) * 16);
    }
    m0_wave = (uint32_t)(wave * C::RPW * C::ROWB);
  }
  __device__ void issue(const unsigned char* base, int snb, int row0, int n, uint32_t lds) const {
    const int nv = __builtin_amdgcn_readfirstlane(min(max(n - row0, 0), kTR));
    const i32x4_t rs = buffer_rsrc(base + (int64_t)row0 * snb, (uint32_t)nv * (uint32_t)snb);
#pragma unroll
    for (int i = 0; i < C::NL; ++i) dma16(voff[i], rs, lds + m0_wave + i * NWAVES * C::RPW * C::ROWB);
  }
};

// Row read (A operand, 32 rows x 16 d): lane holds row rb + l32, d columns
// 16 * kc + 8 * hi .. +7.  Returns the lane's LDS byte offset for kc = 0
// relative to the tile; kc adds nothing fixed (the swizzle differs per kc),
// so the offsets are kept per kc.
template <int D>
__device__ __forceinline__ uint32_t row_ofs(int row, int kc, int hi) {
  return (uint32_t)(row * (D * 2) + (((2 * kc + hi) ^ swz<D>(row)) * 16));
}

// Transposed read (A operand, 32 d rows x 16 tile rows): the 16-lane group
// g = lane / 16 reads tile rows 16 * cc + 4 * hi + {0..3} (part 0) and the
// same + 8 (part 1) at d columns 32 * md + 16 * (g & 1) + {0..15}; group lane
// a16 supplies row a16 / 4, columns 4 * (a16 % 4) .. +3.  Offset for cc = 0
// relative to the tile; cc adds 16 rows (the swizzle repeats every 16 rows,
// but differs between the two parts).
template <int D>
__device__ __forceinline__ uint32_t tr_ofs(int lane, int md, int part) {
  const int hi = lane >> 5, a16 = lane & 15;
  const int r = 4 * hi + (a16 >> 2) + 8 * part;
  const int c = 4 * md + 2 * ((lane >> 4) & 1) + ((a16 & 3) >> 1);
  return (uint32_t)(r * (D * 2) + ((c ^ swz<D>(r)) * 16) + (a16 & 1) * 8);
}

__device__ __forceinline__ bf16x8_t tr_frag(uint32_t a0, uint32_t a1) {
  const i16x4_t lo = lds_tr16(a0);
  const i16x4_t up = lds_tr16(a1);
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Global row loads of one lane's 8 d-values (16 bytes) of a bf16 row, zero
// when the row is invalid.
__device__ __forceinline__ u32x4_t load_row8(const uint16_t* rowp, bool ok, int e0) {
  const u32x4_t z = {0u, 0u, 0u, 0u};
  return ok ? *reinterpret_cast<const u32x4_t*>(rowp + e0) : z;
}

template <int R>
using Step = std::integral_constant<int, R>;

// f(Step<0>{}), ..., f(Step<N-1>{}) as straight-line code.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(Step<I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Keeps a value in registers at this point of the program (the compiler may
// not sink its computation past it or recompute it later).
template <typename T>
__device__ __forceinline__ void pin(T& x) { asm volatile("" : "+v"(x)); }

// ============================================================================
// dQ: query rows in registers, K/V tiles streamed
// ============================================================================
constexpr int kDqWaves = 8;
constexpr int kDqRows = 32 * kDqWaves;

template <int D>
__global__ void __launch_bounds__(64 * kDqWaves)
__attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dq_kernel(BwdParams p, int n_qtiles) {
  using C = BCfg<D, kDqWaves>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const uint32_t lds0 = (uint32_t)(size_t)(SQKV_LDS unsigned char*)smem;
  const uint32_t K_LDS = lds0, V_LDS = lds0 + 2 * C::TILE;   // two stages each

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  const int BH = p.B * p.Hq;
  const int qt_rank = blockIdx.x / BH;
  const int bh = blockIdx.x - qt_rank * BH;
  const int qt = p.causal ? (n_qtiles - 1 - qt_rank) : qt_rank;
  const int b = bh / p.Hq, h = bh - (bh / p.Hq) * p.Hq;
  const int hk = h / p.group;
  const int q0 = qt * kDqRows, qw0 = q0 + wave * 32;
  const int row = qw0 + l32;
  const bool row_ok = row < p.n_q;

  // Q and dO rows of the lane's query (B operands of S^T and dP^T)
  const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)(row_ok ? row : 0) * p.q_sn;
  const uint16_t* drow = static_cast<const uint16_t*>(p.dout) + b * p.do_sb + h * p.do_sh +
                         (int64_t)(row_ok ? row : 0) * p.do_sn;
  u32x4_t qf[C::KC], dof[C::KC];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) {
    qf[kc] = load_row8(qrow, row_ok, 16 * kc + 8 * hi);
    dof[kc] = load_row8(drow, row_ok, 16 * kc + 8 * hi);
  }
  const int64_t srow = ((int64_t)b * p.Hq + h) * p.n_q + (row_ok ? row : 0);
  const float lse = row_ok ? p.lse[srow] : kNegInf;
  // P = exp2(c * s - lse2); a row that sees no key anywhere has P = 0
  const float lse2 = (lse == kNegInf) ? __builtin_huge_valf() : lse * kLog2e;
  const float Dq = row_ok ? p.D[srow] : 0.f;
  const float c = p.scale_log2;

  // visible keys of the block: causal keys up to the last query's position
  int n_vis = p.n_k;
  if (p.causal) {
    const int64_t qpos_last = p.q_pos0 + min(q0 + kDqRows, p.n_q) - 1;
    n_vis = (int)max((int64_t)0, min((int64_t)p.n_k, qpos_last - p.k_pos0 + 1));
  }
  const int T = (n_vis + kTR - 1) / kTR;
  const int64_t qpos = p.q_pos0 + row;   // this lane's query position

  const unsigned char* kg = reinterpret_cast<const unsigned char*>(
      static_cast<const uint16_t*>(p.k) + b * p.k_sb + hk * p.k_sh);
  const unsigned char* vg = reinterpret_cast<const unsigned char*>(
      static_cast<const uint16_t*>(p.v) + b * p.v_sb + hk * p.v_sh);
  const int k_snb = (int)(p.k_sn * 2), v_snb = (int)(p.v_sn * 2);
  TileDma<D, kDqWaves> dk_dma, dv_dma;
  dk_dma.init(lane, wave, k_snb);
  dv_dma.init(lane, wave, v_snb);

  // Lane addresses of the row fragments (K rows for S^T; the V rows for
  // dP^T sit two tiles further) and of the transposed K fragments, in the
  // stage of the current tile; the other stage is one tile away.
  uint32_t ra[C::KC], ta[C::MD][2];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) ra[kc] = K_LDS + row_ofs<D>(l32, kc, hi);
#pragma unroll
  for (int md = 0; md < C::MD; ++md) {
    ta[md][0] = K_LDS + tr_ofs<D>(lane, md, 0);
    ta[md][1] = K_LDS + tr_ofs<D>(lane, md, 1);
  }
  auto move_addr = [&](uint32_t delta) {
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      ra[kc] += delta;
      pin(ra[kc]);
    }
#pragma unroll
    for (int md = 0; md < C::MD; ++md) {
      ta[md][0] += delta;
      ta[md][1] += delta;
      pin(ta[md][0]);
      pin(ta[md][1]);
    }
  };

  f32x16_t acc[C::MD];
#pragma unroll
  for (int md = 0; md < C::MD; ++md) acc[md] = (f32x16_t){};

  // A tile is two blocks of 32 keys.  Block nb: S^T and dP^T (2 KC MFMAs,
  // the two chains alternating), then P, dS^T (VALU), then dQ^T += K^T dS^T
  // (2 MD MFMAs, transposed K fragments of the block's 32 keys).  Element j
  // of block nb holds key t*64 + 32*nb + 8*(j/4) + 4*hi + j%4 of query `row`.
  f32x16_t s[2], dp[2];
  u32x4_t dsf[4];
  float w[2][16];
  auto sd_read = [&](auto NB, auto M) -> u32x4_t {
    constexpr int nb = decltype(NB)::value, m = decltype(M)::value;
    return lds_b128(ra[m / 2] + (uint32_t)(nb * 32 * C::ROWB + (m & 1) * 2 * C::TILE));
  };
  auto sd_mfma = [&](auto NB, auto M, const u32x4_t& fr) {
    constexpr int nb = decltype(NB)::value, m = decltype(M)::value, kc = m / 2;
    if constexpr ((m & 1) == 0) s[nb] = mfma(as_bf16x8(fr), as_bf16x8(qf[kc]), kc == 0 ? (f32x16_t){} : s[nb]);
    else dp[nb] = mfma(as_bf16x8(fr), as_bf16x8(dof[kc]), kc == 0 ? (f32x16_t){} : dp[nb]);
  };
  auto dq_read = [&](auto NB, auto M) -> bf16x8_t {
    constexpr int nb = decltype(NB)::value, m = decltype(M)::value;
    constexpr int cc = 2 * nb + m / C::MD, md = m % C::MD;
    return tr_frag(ta[md][0] + (uint32_t)(16 * cc * C::ROWB), ta[md][1] + (uint32_t)(16 * cc * C::ROWB));
  };
  auto dq_mfma = [&](auto NB, auto M, const bf16x8_t& fr) {
    constexpr int nb = decltype(NB)::value, m = decltype(M)::value;
    constexpr int cc = 2 * nb + m / C::MD, md = m % C::MD;
    acc[md] = mfma(fr, as_bf16x8(dsf[cc]), acc[md]);
  };
  // Item k of block nb's 20 (5 per group g of 4 keys): the group's four
  // elements, then the mask (only for a block that reaches past a query's
  // last visible key) and the bf16 packs.
  bool msk[2];
  int lk = 0;
  auto sm_item = [&](auto NB, auto K) {
    constexpr int nb = decltype(NB)::value, k = decltype(K)::value, g = k / 5, r = k % 5;
    if constexpr (r < 4) {
      constexpr int j = 4 * g + r;
      const float pr = __builtin_amdgcn_exp2f(fmaf(s[nb][j], c, -lse2));
      w[nb][j] = pr * (dp[nb][j] - Dq);
    } else {
      if (msk[nb]) {
#pragma unroll
        for (int x = 0; x < 4; ++x) w[nb][4 * g + x] = (32 * nb + 8 * g + x <= lk) ? w[nb][4 * g + x] : 0.f;
      }
      constexpr int half = g / 2, xx = 2 * (g & 1);
      dsf[2 * nb + half][xx] = pack_bf16x2(w[nb][4 * g], w[nb][4 * g + 1]);
      dsf[2 * nb + half][xx + 1] = pack_bf16x2(w[nb][4 * g + 2], w[nb][4 * g + 3]);
      pin(dsf[2 * nb + half]);
    }
  };

  // Slot schedule of one tile (one MFMA per slot):
  //   A  slots  0..15  S^T, dP^T of block 0
  //   B  slots 16..31  S^T, dP^T of block 1    + P, dS^T of block 0
  //   C  slots 32..39  dQ^T of block 0         + P, dS^T of block 1, keys 0..15
  //   D  slots 40..47  dQ^T of block 1         + P, dS^T of block 1, keys 16..31
  // (dQ^T of block 1 reads the keys 0..15 packs in its first four slots and
  // the keys 16..31 packs, made in slots 40..43, in its last four).
  constexpr int NSD = 2 * C::KC, NDQ = 2 * C::MD;
  constexpr int kSlots = 2 * NSD + 2 * NDQ;
  constexpr int kLead = 3;
  constexpr auto kSlotB = [](int k) { return NSD + (k * NSD) / 20; };
  constexpr auto kSlotC = [](int k) {
    return k < 10 ? 2 * NSD + (k * NDQ) / 10 : 2 * NSD + NDQ + ((k - 10) * (NDQ / 2)) / 10;
  };
  auto read_frag = [&](auto I, u32x4_t (&sdfr)[2 * NSD], bf16x8_t (&dqfr)[2 * NDQ]) {
    constexpr int i = decltype(I)::value;
    if constexpr (i < NSD) sdfr[i] = sd_read(Step<0>{}, Step<i>{});
    else if constexpr (i < 2 * NSD) sdfr[i] = sd_read(Step<1>{}, Step<i - NSD>{});
    else if constexpr (i < 2 * NSD + NDQ) dqfr[i - 2 * NSD] = dq_read(Step<0>{}, Step<i - 2 * NSD>{});
    else dqfr[i - 2 * NSD] = dq_read(Step<1>{}, Step<i - 2 * NSD - NDQ>{});
  };

  if (T > 0) {
    dk_dma.issue(kg, k_snb, 0, n_vis, K_LDS);
    dv_dma.issue(vg, v_snb, 0, n_vis, V_LDS);
  }
  for (int t = 0; t < T; ++t) {
    drain_and_sync();                       // tile t landed; the other stage is free
    if (t + 1 < T) {
      const uint32_t other = (uint32_t)((t + 1) & 1) * C::TILE;
      dk_dma.issue(kg, k_snb, (t + 1) * kTR, n_vis, K_LDS + other);
      dv_dma.issue(vg, v_snb, (t + 1) * kTR, n_vis, V_LDS + other);
    }
    if (t > 0) move_addr((t & 1) ? (uint32_t)C::TILE : (uint32_t)(-(int)C::TILE));
    // keys past the visible range or after the query get weight 0
    const int kbase = t * kTR;
    int64_t lastk = p.causal ? (qpos - p.k_pos0 - kbase) : (int64_t)kTR;   // last visible key of the tile
    lastk = min(lastk, (int64_t)(n_vis - kbase - 1));
    lk = (int)max((int64_t)-1, min(lastk, (int64_t)kTR)) - 4 * hi;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
      msk[nb] = (kbase + 32 * nb + 32 > n_vis) ||
                (p.causal && p.k_pos0 + kbase + 32 * nb + 31 > p.q_pos0 + qw0);

    u32x4_t sdfr[2 * NSD];
    bf16x8_t dqfr[2 * NDQ];
    static_for<kLead>([&](auto I) { read_frag(I, sdfr, dqfr); });
    static_for<kSlots>([&](auto I) {
      constexpr int i = decltype(I)::value;
      if constexpr (i + kLead < kSlots) read_frag(Step<i + kLead>{}, sdfr, dqfr);
      if constexpr (i < NSD) sd_mfma(Step<0>{}, Step<i>{}, sdfr[i]);
      else if constexpr (i < 2 * NSD) sd_mfma(Step<1>{}, Step<i - NSD>{}, sdfr[i]);
      else if constexpr (i < 2 * NSD + NDQ) dq_mfma(Step<0>{}, Step<i - 2 * NSD>{}, dqfr[i - 2 * NSD]);
      else dq_mfma(Step<1>{}, Step<i - 2 * NSD - NDQ>{}, dqfr[i - 2 * NSD]);
      static_for<20>([&](auto K) {
        constexpr int k = decltype(K)::value;
        if constexpr (kSlotB(k) == i) sm_item(Step<0>{}, K);
        if constexpr (kSlotC(k) == i) sm_item(Step<1>{}, K);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  }
  __builtin_amdgcn_s_waitcnt(0);   // no DMA may outlive the workgroup's LDS

  if (row_ok) {
    float* dqr = p.dq + b * p.dq_sb + h * p.dq_sh + (int64_t)row * p.dq_sn;
#pragma unroll
    for (int md = 0; md < C::MD; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * md + 8 * g + 4 * hi;
        float4 x = *reinterpret_cast<float4*>(dqr + d0);
        x.x = fmaf(p.scale, acc[md][4 * g + 0], x.x);
        x.y = fmaf(p.scale, acc[md][4 * g + 1], x.y);
        x.z = fmaf(p.scale, acc[md][4 * g + 2], x.z);
        x.w = fmaf(p.scale, acc[md][4 * g + 3], x.w);
        *reinterpret_cast<float4*>(dqr + d0) = x;
      }
  }
}

// ============================================================================
// dK, dV: key rows in registers, Q/dO tiles streamed
// ============================================================================
constexpr int kKvWaves = 4;
constexpr int kKvRows = 32 * kKvWaves;
constexpr int kKvStages = 3;   // LDS stages of (Q tile, dO tile, lse, D)


// S and dP of one 32-query block for the wave's 32 keys: element j holds
// query 8*(j/4) + 4*hi + j%4 of the block, key `key` (lane % 32).
struct SdBlock {
  f32x16_t s, dp;
};

// The weights P and dS of one block rounded to bf16, as B operands of the
// dV and dK products: half h covers queries 16*h .. 16*h + 15 of the block.
struct PdsBlock {
  u32x4_t pf[2], df[2];
};

// Walks 32-query blocks u = 0, 1, ... over the (query head of the GQA group,
// 64-query tile) sequence, two blocks per tile.  Step u is a software
// pipeline of three blocks: the S and dP products of block u+2, the
// softmax-gradient VALU work of block u+1 and the dV, dK products of block u
// share one slot schedule (one MFMA per slot, S/dP and dV/dK alternating,
// the VALU work spread over the slots), so the VALU work of one block runs
// under the MFMAs of the others.  Tiles sit in three LDS stages: at the top
// of tile tau (blocks 2tau, 2tau+1) tiles tau and tau+1 have landed, and the
// copy of tile tau+2 goes into the stage of tile tau-1, which every wave has
// finished reading.
template <int D>
__global__ void __launch_bounds__(64 * kKvWaves)
__attribute__((amdgpu_waves_per_eu(1, 1)))
attn_bwd_dkdv_kernel(BwdParams p) {
  using C = BCfg<D, kKvWaves>;
  constexpr int NSD = 2 * C::KC;      // S and dP MFMAs per block
  constexpr int NKV = 4 * C::MD;      // dV and dK MFMAs per block
  static_assert(NSD == NKV, "one S/dP MFMA per dV/dK MFMA");
  constexpr int kSlots = NSD + NKV;
  constexpr int kLead = 4;            // fragments are read this many slots ahead
  constexpr int kItems = 24;          // softmax-gradient work items per block (6 per 4 queries)
  constexpr uint32_t kStage = 2 * C::TILE;                 // Q tile, then dO tile
  constexpr uint32_t kStats = kKvStages * kStage;          // per stage: lse (256 B), D (256 B)
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const uint32_t lds0 = (uint32_t)(size_t)(SQKV_LDS unsigned char*)smem;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  const int BH = p.B * p.Hkv;
  const int kt = blockIdx.x / BH;
  const int bh = blockIdx.x - kt * BH;
  const int b = bh / p.Hkv, hk = bh - (bh / p.Hkv) * p.Hkv;
  const int k0 = kt * kKvRows, kw0 = k0 + wave * 32;
  const int key = kw0 + l32;
  const bool key_ok = key < p.n_k;

  // the first query that can see the workgroup's first key
  int qstart = 0;
  if (p.causal) qstart = (int)min((int64_t)p.n_q, max((int64_t)0, p.k_pos0 + k0 - p.q_pos0));
  const int t0 = qstart / kTR;
  const int T = (p.n_q + kTR - 1) / kTR;
  const int Tq = T - t0;                      // tiles per query head
  const int NT = p.group * Tq;                // tiles of the whole walk
  if (NT <= 0) return;                        // no query sees these keys: nothing to add

  // K and V rows of the lane's key (B operands of S and dP); a key past the
  // chunk end reads zeros and only ever touches its own (unstored) column
  const uint16_t* krow = static_cast<const uint16_t*>(p.k) + b * p.k_sb + hk * p.k_sh + (int64_t)(key_ok ? key : 0) * p.k_sn;
  const uint16_t* vrow = static_cast<const uint16_t*>(p.v) + b * p.v_sb + hk * p.v_sh + (int64_t)(key_ok ? key : 0) * p.v_sn;
  u32x4_t kf[C::KC], vf[C::KC];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) {
    kf[kc] = load_row8(krow, key_ok, 16 * kc + 8 * hi);
    vf[kc] = load_row8(vrow, key_ok, 16 * kc + 8 * hi);
  }
  // -V: the dP product of a block starts from the rows' D and ends at
  // D - dO V^T = -(dP - D)
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) vf[kc] ^= (u32x4_t){0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  const int64_t kpos = p.k_pos0 + key;
  const int64_t kpos_wave_last = p.k_pos0 + kw0 + 31;
  const float c = p.scale_log2;

  const int q_snb = (int)(p.q_sn * 2), o_snb = (int)(p.do_sn * 2);
  TileDma<D, kKvWaves> q_dma, o_dma;
  q_dma.init(lane, wave, q_snb);
  o_dma.init(lane, wave, o_snb);

  f32x16_t dka[C::MD], dva[C::MD];
#pragma unroll
  for (int md = 0; md < C::MD; ++md) {
    dka[md] = (f32x16_t){};
    dva[md] = (f32x16_t){};
  }

  // Q, dO rows [t*64, t*64 + 64) of query head hk*group + gi, and their lse
  // and D (wave 0: one 64-lane dword load each), into LDS stage `stage`;
  // rows past the chunk end arrive as zeros.
  auto issue_tile = [&](int gi, int t, int stage) {
    const int h = hk * p.group + gi;
    const unsigned char* qg = reinterpret_cast<const unsigned char*>(
        static_cast<const uint16_t*>(p.q) + b * p.q_sb + h * p.q_sh);
    const unsigned char* og = reinterpret_cast<const unsigned char*>(
        static_cast<const uint16_t*>(p.dout) + b * p.do_sb + h * p.do_sh);
    const uint32_t base = lds0 + (uint32_t)stage * kStage;
    q_dma.issue(qg, q_snb, t * kTR, p.n_q, base);
    o_dma.issue(og, o_snb, t * kTR, p.n_q, base + C::TILE);
    if (wave == 0) {
      const int nv = __builtin_amdgcn_readfirstlane(min(max(p.n_q - t * kTR, 0), kTR));
      const int64_t row = ((int64_t)b * p.Hq + h) * p.n_q + (int64_t)t * kTR;
      const uint32_t sl = lds0 + kStats + (uint32_t)stage * 512u;
      dma4((uint32_t)(lane * 4), buffer_rsrc(p.lse + row, (uint32_t)nv * 4u), sl);
      dma4((uint32_t)(lane * 4), buffer_rsrc(p.D + row, (uint32_t)nv * 4u), sl + 256u);
    }
  };

  // ---- one block's pieces -------------------------------------------------
  // S/dP MFMA m: m < KC, S from the Q tile (kc = m); m >= KC, D - dP from the
  // dO tile (kc = m - KC), starting from the block's D values `dinit`.  Each
  // reads a row fragment at ra[kc] + qb*32 rows.
  auto sd_read = [&](auto M, const uint32_t (&ra)[C::KC], auto QB) -> u32x4_t {
    constexpr int m = decltype(M)::value, qb = decltype(QB)::value;
    constexpr int kc = m % C::KC;
    return lds_b128(ra[kc] + (uint32_t)(qb * 32 * C::ROWB + (m / C::KC) * C::TILE));
  };
  auto sd_mfma = [&](auto M, SdBlock& o, const u32x4_t& fr, const f32x16_t& dinit) {
    constexpr int m = decltype(M)::value, kc = m % C::KC;
    if constexpr (m < C::KC)
      o.s = mfma(as_bf16x8(fr), as_bf16x8(kf[kc]), kc == 0 ? (f32x16_t){} : o.s);
    else
      o.dp = mfma(as_bf16x8(fr), as_bf16x8(vf[kc]), kc == 0 ? dinit : o.dp);
  };
  // D of the 32 queries of half QB of a tile (stats at `sa`), laid out as
  // the dP accumulator: element j holds query 8*(j/4) + 4*hi + j%4.
  auto d_init = [&](uint32_t sa, auto QB) -> f32x16_t {
    constexpr int qb = decltype(QB)::value;
    f32x16_t r;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const u32x4_t v = lds_b128(sa + 256u + (uint32_t)((32 * qb + 8 * g) * 4));
#pragma unroll
      for (int x = 0; x < 4; ++x) r[4 * g + x] = __uint_as_float(v[x]);
    }
    return r;
  };
  // dV/dK MFMA m: half = m / (2 MD), md = (m / 2) % MD; even: dV^T += dO^T P
  // (transposed dO fragment), odd: dK^T += Q^T dS (transposed Q fragment).
  auto kv_read = [&](auto M, const uint32_t (&ta)[C::MD][2], auto QB) -> bf16x8_t {
    constexpr int m = decltype(M)::value, qb = decltype(QB)::value;
    constexpr int half = m / (2 * C::MD), md = (m / 2) % C::MD;
    constexpr uint32_t o = (uint32_t)((32 * qb + 16 * half) * C::ROWB + ((m & 1) ? 0 : C::TILE));
    return tr_frag(ta[md][0] + o, ta[md][1] + o);
  };
  auto kv_mfma = [&](auto M, const PdsBlock& w, const bf16x8_t& fr) {
    constexpr int m = decltype(M)::value;
    constexpr int half = m / (2 * C::MD), md = (m / 2) % C::MD;
    if constexpr ((m & 1) == 0) dva[md] = mfma(fr, as_bf16x8(w.pf[half]), dva[md]);
    else dka[md] = mfma(fr, as_bf16x8(w.df[half]), dka[md]);
  };

  // Softmax-gradient work of a block: P = exp2(c*s - lse*log2e) and
  // dS = P (dP - D) = -P (D - dP), masked causally, rounded to bf16.  Item k
  // of the 24: for each 4-query group g = k / 6: the group's lse, its four
  // elements, then the mask and the bf16 packs.  The group's lse is read
  // from LDS a few slots before its first item.
  struct SmState {
    u32x4_t lr[4];
    float nl[4];
    float pw[16], dsw[16];
    int lo;
    bool msk;
  };
  auto sm_read = [&](SmState& st, uint32_t sa, auto QB, auto G) {
    constexpr int qb = decltype(QB)::value, g = decltype(G)::value;
    st.lr[g] = lds_b128(sa + (uint32_t)((32 * qb + 8 * g) * 4));
  };
  auto sm_setup = [&](SmState& st, int t, auto QB) {
    constexpr int qb = decltype(QB)::value;
    const int qb0 = t * kTR + 32 * qb;
    const int64_t q0pos = p.q_pos0 + qb0;
    st.msk = p.causal && kpos_wave_last > q0pos;
    const int64_t lo = kpos - q0pos - 4 * hi;
    st.lo = (int)min(max(lo, (int64_t)-1), (int64_t)33);
  };
  auto sm_item = [&](auto K, SmState& st, const SdBlock& sd, PdsBlock& w) {
    constexpr int k = decltype(K)::value, g = k / 6, r = k % 6;
    if constexpr (r == 0) {
      // lse = -inf only for a row that sees no key anywhere, so none of
      // this pair: the causal mask below (a select) zeroes its elements
#pragma unroll
      for (int x = 0; x < 4; ++x) st.nl[x] = -__uint_as_float(st.lr[g][x]) * kLog2e;
    } else if constexpr (r <= 4) {
      constexpr int x = r - 1, j = 4 * g + x;
      const float pr = __builtin_amdgcn_exp2f(fmaf(sd.s[j], c, st.nl[x]));
      st.pw[j] = pr;
      st.dsw[j] = -(pr * sd.dp[j]);
    } else {
      if (st.msk) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const bool vis = 8 * g + x >= st.lo;
          st.pw[4 * g + x] = vis ? st.pw[4 * g + x] : 0.f;
          st.dsw[4 * g + x] = vis ? st.dsw[4 * g + x] : 0.f;
        }
      }
      constexpr int half = g / 2, xx = 2 * (g & 1);
      w.pf[half][xx] = pack_bf16x2(st.pw[4 * g], st.pw[4 * g + 1]);
      w.pf[half][xx + 1] = pack_bf16x2(st.pw[4 * g + 2], st.pw[4 * g + 3]);
      w.df[half][xx] = pack_bf16x2(st.dsw[4 * g], st.dsw[4 * g + 1]);
      w.df[half][xx + 1] = pack_bf16x2(st.dsw[4 * g + 2], st.dsw[4 * g + 3]);
      pin(w.pf[half]);
      pin(w.df[half]);
    }
  };
  constexpr auto kSlotOfItem = [](int k) { return 1 + (k * (kSlots - 2)) / kItems; };

  // Per-tile addresses: row fragments of tile tau+1 (ra), transposed
  // fragments of tile tau (ta), statistics of tiles tau and tau+1.  Moving
  // to the next tile adds the distance between the stages' bases.
  uint32_t ra[C::KC], ta[C::MD][2], sa_cur, sa_nxt;
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) ra[kc] = lds0 + row_ofs<D>(l32, kc, hi);                       // stage 0
#pragma unroll
  for (int md = 0; md < C::MD; ++md) {
    ta[md][0] = lds0 + (uint32_t)(kKvStages - 1) * kStage + tr_ofs<D>(lane, md, 0);   // stage S-1
    ta[md][1] = lds0 + (uint32_t)(kKvStages - 1) * kStage + tr_ofs<D>(lane, md, 1);
  }
  auto move_addr = [&](int s_cur, int s_nxt, uint32_t d_cur, uint32_t d_nxt) {
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      ra[kc] += d_nxt;
      pin(ra[kc]);
    }
#pragma unroll
    for (int md = 0; md < C::MD; ++md) {
      ta[md][0] += d_cur;
      ta[md][1] += d_cur;
      pin(ta[md][0]);
      pin(ta[md][1]);
    }
    sa_cur = lds0 + kStats + (uint32_t)s_cur * 512u + (uint32_t)(16 * hi);
    sa_nxt = lds0 + kStats + (uint32_t)s_nxt * 512u + (uint32_t)(16 * hi);
  };

  // One pipeline step: dV/dK of the block in `kvw` (tile tau, half QB of
  // the tile), the softmax gradient of `smi` into `smo` (statistics at
  // sa_sm, query tile t_sm, half 1 - QB) and S/dP of the block after it into
  // `sdo` (tile tau+1, half QB, statistics at sa_sd).
  auto step = [&](auto QB, const PdsBlock& kvw, const SdBlock& smi, PdsBlock& smo, SdBlock& sdo,
                  uint32_t sa_sm, int t_sm, uint32_t sa_sd) {
    constexpr int qb = decltype(QB)::value;
    using SQB = Step<1 - qb>;
    SmState st;
    sm_read(st, sa_sm, SQB{}, Step<0>{});
    const f32x16_t dinit = d_init(sa_sd, QB);
    sm_setup(st, t_sm, SQB{});
    bf16x8_t kvfr[NKV];
    u32x4_t sdfr[NSD];
    static_for<kLead>([&](auto I) {
      constexpr int i = decltype(I)::value;
      if constexpr ((i & 1) == 0) kvfr[i / 2] = kv_read(Step<i / 2>{}, ta, QB);
      else sdfr[i / 2] = sd_read(Step<i / 2>{}, ra, QB);
    });
    static_for<kSlots>([&](auto I) {
      constexpr int i = decltype(I)::value, ia = i + kLead;
      if constexpr (ia < kSlots) {
        if constexpr ((ia & 1) == 0) kvfr[ia / 2] = kv_read(Step<ia / 2>{}, ta, QB);
        else sdfr[ia / 2] = sd_read(Step<ia / 2>{}, ra, QB);
      }
      static_for<3>([&](auto G) {
        constexpr int g = decltype(G)::value + 1;
        if constexpr (kSlotOfItem(6 * g) - 3 == i) sm_read(st, sa_sm, SQB{}, Step<g>{});
      });
      if constexpr ((i & 1) == 0) kv_mfma(Step<i / 2>{}, kvw, kvfr[i / 2]);
      else sd_mfma(Step<i / 2>{}, sdo, sdfr[i / 2], dinit);
      static_for<kItems>([&](auto K) {
        if constexpr (kSlotOfItem(decltype(K)::value) == i) sm_item(K, st, smi, smo);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  // ---- prologue: tiles 0 and 1 in flight, S/dP of blocks 0 and 1, P/dS of block 0
  int gi_d = 0, t_d = t0;                     // next tile to copy
  auto advance = [&](int& gi, int& t) {
    if (++t == T) {
      t = t0;
      ++gi;
    }
  };
  issue_tile(gi_d, t_d, 0);
  advance(gi_d, t_d);
  if (NT > 1) {
    issue_tile(gi_d, t_d, 1);
    advance(gi_d, t_d);
  }
  drain_and_sync();

  SdBlock sA, sB;
  PdsBlock wA, wB;
  sa_nxt = lds0 + kStats + (uint32_t)(16 * hi);   // statistics of tile 0 (stage 0)
  {
    const f32x16_t d0 = d_init(sa_nxt, Step<0>{}), d1 = d_init(sa_nxt, Step<1>{});
    static_for<NSD>([&](auto M) { sd_mfma(M, sA, sd_read(M, ra, Step<0>{}), d0); });
    static_for<NSD>([&](auto M) { sd_mfma(M, sB, sd_read(M, ra, Step<1>{}), d1); });
    SmState st;
    static_for<4>([&](auto G) { sm_read(st, sa_nxt, Step<0>{}, G); });
    sm_setup(st, t0, Step<0>{});
    static_for<kItems>([&](auto K) { sm_item(K, st, sA, wA); });
  }

  int s_cur = 0;                              // stage of tile tau
  int t_cur = t0, gi_cur = 0;                 // query tile of tau
  for (int tau = 0; tau < NT; ++tau) {
    if (tau > 0) drain_and_sync();            // tile tau+1 landed; tile tau-1 no longer read
    const int s_nxt = s_cur == kKvStages - 1 ? 0 : s_cur + 1;
    if (tau + 2 < NT) {
      const int s_dma = s_nxt == kKvStages - 1 ? 0 : s_nxt + 1;   // the stage of tile tau-1
      issue_tile(gi_d, t_d, s_dma);
      advance(gi_d, t_d);
    }
    int gi_n = gi_cur, t_nxt = t_cur;
    advance(gi_n, t_nxt);
    // ra moves from tile tau's stage to tile tau+1's, ta from tau-1's to tau's
    const uint32_t back = (uint32_t)(-(int)((kKvStages - 1) * kStage));
    move_addr(s_cur, s_nxt, s_cur == 0 ? back : kStage, tau == 0 ? kStage : (s_nxt == 0 ? back : kStage));
    step(Step<0>{}, wA, sB, wB, sA, sa_cur, t_cur, sa_nxt);   // dV/dK(2tau), P/dS(2tau+1), S/dP(2tau+2)
    step(Step<1>{}, wB, sA, wA, sB, sa_nxt, t_nxt, sa_nxt);   // dV/dK(2tau+1), P/dS(2tau+2), S/dP(2tau+3)
    s_cur = s_nxt;
    t_cur = t_nxt;
    gi_cur = gi_n;
  }
  __builtin_amdgcn_s_waitcnt(0);   // no DMA may outlive the workgroup's LDS

  if (key_ok) {

    float* dkr = p.dk + b * p.dk_sb + hk * p.dk_sh + (int64_t)key * p.dk_sn;
    float* dvr = p.dv + b * p.dv_sb + hk * p.dv_sh + (int64_t)key * p.dv_sn;
#pragma unroll
    for (int md = 0; md < C::MD; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * md + 8 * g + 4 * hi;
        float4 x = *reinterpret_cast<float4*>(dkr + d0);
        x.x = fmaf(p.scale, dka[md][4 * g + 0], x.x);
        x.y = fmaf(p.scale, dka[md][4 * g + 1], x.y);
        x.z = fmaf(p.scale, dka[md][4 * g + 2], x.z);
        x.w = fmaf(p.scale, dka[md][4 * g + 3], x.w);
        *reinterpret_cast<float4*>(dkr + d0) = x;
        float4 y = *reinterpret_cast<float4*>(dvr + d0);
        y.x += dva[md][4 * g + 0];
        y.y += dva[md][4 * g + 1];
        y.z += dva[md][4 * g + 2];
        y.w += dva[md][4 * g + 3];
        *reinterpret_cast<float4*>(dvr + d0) = y;
      }
  }
}

// ============================================================================
// D = rowsum(dO * O)
// ============================================================================
template <int D>
__global__ void __launch_bounds__(256) bwd_rowdot_kernel(RowDotParams p) {
  // one row per 16 lanes: each lane takes D/16 consecutive elements
  constexpr int E = D / 16;
  const int64_t rows = (int64_t)p.B * p.H * p.n;
  const int64_t r = ((int64_t)blockIdx.x * 256 + threadIdx.x) / 16;
  const int sub = threadIdx.x & 15;
  float acc = 0.f;
  if (r < rows) {
    const int64_t t = r % p.n, bh = r / p.n;
    const int64_t hh = bh % p.H, bb = bh / p.H;
    const int64_t oo = bb * p.o_sb + hh * p.o_sh + t * p.o_sn + sub * E;
    const int64_t od = bb * p.do_sb + hh * p.do_sh + t * p.do_sn + sub * E;
#pragma unroll
    for (int e = 0; e < E; e += 4) {
      float a[4], g[4];
      load4(p.o, oo + e, p.dtype, a);
      load4(p.dout, od + e, p.dtype, g);
      acc = fmaf(a[0], g[0], acc);
      acc = fmaf(a[1], g[1], acc);
      acc = fmaf(a[2], g[2], acc);
      acc = fmaf(a[3], g[3], acc);
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (r < rows && sub == 0) p.D[r] = acc;
}

// LDS of the dK/dV kernel: three stages of (Q tile, dO tile) and of the
// tiles' lse and D.
template <int D>
constexpr int kKvLds = kKvStages * (2 * BCfg<D, kKvWaves>::TILE + 512);

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t s) {
  using Cq = BCfg<D, kDqWaves>;
  using Ck = BCfg<D, kKvWaves>;
  static std::atomic<uint64_t> dq_set{0}, kv_set{0};
  hipError_t e = allow_dyn_lds(reinterpret_cast<const void*>(&attn_bwd_dq_kernel<D>), 4 * Cq::TILE, dq_set);
  if (e != hipSuccess) return e;
  e = allow_dyn_lds(reinterpret_cast<const void*>(&attn_bwd_dkdv_kernel<D>), kKvLds<D>, kv_set);
  if (e != hipSuccess) return e;
  const int n_qtiles = (p.n_q + kDqRows - 1) / kDqRows;
  const int64_t bq = (int64_t)n_qtiles * p.B * p.Hq;
  if (bq > 0)
    hipLaunchKernelGGL(attn_bwd_dq_kernel<D>, dim3((unsigned)bq), dim3(64 * kDqWaves), 4 * Cq::TILE, s, p, n_qtiles);
  const int n_ktiles = (p.n_k + kKvRows - 1) / kKvRows;
  const int64_t bk = (int64_t)n_ktiles * p.B * p.Hkv;
  if (bk > 0)
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<D>, dim3((unsigned)bk), dim3(64 * kKvWaves), kKvLds<D>, s, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd_bf16(const BwdParams& p, int d, hipStream_t s) {
  if (p.n_q == 0 || p.n_k == 0) return hipSuccess;
  return d == 128 ? launch_bwd_d<128>(p, s) : launch_bwd_d<64>(p, s);
}

hipError_t launch_bwd_rowdot(const RowDotParams& p, int d, hipStream_t s) {
  const int64_t rows = (int64_t)p.B * p.H * p.n;
  if (rows == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((rows * 16 + 255) / 256);
  if (d == 128)
    hipLaunchKernelGGL(bwd_rowdot_kernel<128>, dim3(blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(bwd_rowdot_kernel<64>, dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace sqkv
