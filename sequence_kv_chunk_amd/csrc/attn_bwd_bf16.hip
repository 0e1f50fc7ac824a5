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
// * attn_bwd_dkdv: parallel over keys (128 keys per workgroup, 8 waves, two
//   per SIMD).  The two waves of a SIMD share 32 keys: one holds their K
//   rows and forms S = Q K^T and P, the other holds -V and forms D - dP and
//   dS (queries on M: a lane holds 16 queries of ONE key); P and dS cross
//   between them through LDS, and each accumulates dV^T += dO^T P and
//   dK^T += Q^T dS (transposed reads of the dO and Q tiles) for its half of
//   d.  The query heads of a GQA group are walked inside the workgroup so
//   that a key/value head's gradients sum over them without atomics.
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
constexpr int kKvRows = 128;    // keys per workgroup
constexpr int kKvStages = 3;    // LDS stages of (Q tile, dO tile, lse, D)

// Two waves per SIMD, a pair of waves per 32 keys.  Waves w and w + 4 (one
// SIMD) take the same 32 keys.  Wave w (role 0) holds the K rows of the keys
// and forms S = Q K^T and P; wave w + 4 (role 1) holds the -V rows and forms
// D - dP and dS = P (dP - D).  Each accumulates dV^T and dK^T for its own
// half of d, so a wave holds half the accumulators a single wave over the
// same keys would, and the pair issues the MFMAs of one such wave.  P goes
// from role 0 to role 1, and dS back, through LDS (bf16, lane to lane in the
// B-operand layout), with one barrier per 32-query block.
// Step u (blocks u = 0, 1, ... of the walk; the step after the last block
// only finishes dK):
//   role 0: S of block u+1 and its P (written out), dV^T += dO^T P of block
//           u, dK^T += Q^T dS of block u-1 (dS written by role 1 in step u-1);
//   role 1: D - dP of block u+1, dS of block u (P written by role 0 in step
//           u-1, D - dP from its own step u-1, written out), dV^T of block u,
//           dK^T of block u-1.
// A step issues its LDS reads ahead of its MFMAs (those of dK after the S or
// D - dP products are under way; the row fragments of an even step before
// the barrier ahead of it), so that the two waves of a SIMD see the read
// latency about once per step.  Tiles sit in three LDS stages (the three Q
// tiles, then the three dO tiles, then their lse and D); the copy of tile
// tau+2 is issued after the barrier that ends block 2tau, the last one to
// read tile tau-1, and waited for at the barrier that ends block 2tau+2.
// The loop runs three tiles (six steps) per iteration so that every stage
// index and every register of the two-block rotation is a constant.
constexpr int kKvWaves = 8;
constexpr uint32_t kXchg = 2 * 1024;   // one block's P or dS: two 1 KiB halves of 64 lanes x 16 bytes

template <int D>
constexpr uint32_t kKvMainLds = kKvStages * (2 * BCfg<D, kKvWaves>::TILE + 512);
// LDS: Q tiles of the three stages, dO tiles, (lse, D) of the three stages,
// then per pair two P and two dS buffers.
template <int D>
constexpr int kKvLds = (int)(kKvMainLds<D> + 4 * 4 * kXchg);

template <int D>
__global__ void __launch_bounds__(64 * kKvWaves)
__attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bwd_dkdv_kernel(BwdParams p) {
  using C = BCfg<D, kKvWaves>;
  constexpr int MH = C::MD / 2;                     // 32-row blocks of d per half
  constexpr uint32_t kQ0 = 0, kO0 = kKvStages * C::TILE;   // first Q tile, first dO tile
  constexpr uint32_t kStats = 2 * kKvStages * C::TILE;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const uint32_t lds0 = (uint32_t)(size_t)(SQKV_LDS unsigned char*)smem;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l32 = lane & 31, hi = lane >> 5;
  const int pr = wave & 3, role = wave >> 2;

  const int BH = p.B * p.Hkv;
  const int kt = blockIdx.x / BH;
  const int bh = blockIdx.x - kt * BH;
  const int b = bh / p.Hkv, hk = bh - (bh / p.Hkv) * p.Hkv;
  const int k0 = kt * kKvRows, kw0 = k0 + pr * 32;
  const int key = kw0 + l32;
  const bool key_ok = key < p.n_k;

  // the first query that can see the workgroup's first key
  int qstart = 0;
  if (p.causal) qstart = (int)min((int64_t)p.n_q, max((int64_t)0, p.k_pos0 + k0 - p.q_pos0));
  const int t0 = qstart / kTR;
  const int T = (p.n_q + kTR - 1) / kTR;
  const int NT = p.group * (T - t0);          // tiles of the whole walk
  if (NT <= 0) return;                        // no query sees these keys: nothing to add
  const int NB = 2 * NT;                      // 32-query blocks

  // K (role 0) or -V (role 1) rows of the lane's key: B operands of S and of
  // D - dP; a key past the chunk end reads zeros and only ever touches its
  // own (unstored) column
  const uint16_t* brow =
      role == 0 ? static_cast<const uint16_t*>(p.k) + b * p.k_sb + hk * p.k_sh + (int64_t)(key_ok ? key : 0) * p.k_sn
                : static_cast<const uint16_t*>(p.v) + b * p.v_sb + hk * p.v_sh + (int64_t)(key_ok ? key : 0) * p.v_sn;
  const uint32_t sgn = role == 0 ? 0u : 0x80008000u;
  u32x4_t bfr[C::KC];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) bfr[kc] = load_row8(brow, key_ok, 16 * kc + 8 * hi) ^ (u32x4_t){sgn, sgn, sgn, sgn};
  const int64_t kpos = p.k_pos0 + key;
  const int64_t kpos_wave_last = p.k_pos0 + kw0 + 31;
  const float c = p.scale_log2;

  const int q_snb = (int)(p.q_sn * 2), o_snb = (int)(p.do_sn * 2);
  TileDma<D, kKvWaves> q_dma, o_dma;
  q_dma.init(lane, wave, q_snb);
  o_dma.init(lane, wave, o_snb);
  auto issue_tile = [&](int gi, int t, int stage) {
    const int h = hk * p.group + gi;
    const unsigned char* qg = reinterpret_cast<const unsigned char*>(
        static_cast<const uint16_t*>(p.q) + b * p.q_sb + h * p.q_sh);
    const unsigned char* og = reinterpret_cast<const unsigned char*>(
        static_cast<const uint16_t*>(p.dout) + b * p.do_sb + h * p.do_sh);
    q_dma.issue(qg, q_snb, t * kTR, p.n_q, lds0 + kQ0 + (uint32_t)stage * C::TILE);
    o_dma.issue(og, o_snb, t * kTR, p.n_q, lds0 + kO0 + (uint32_t)stage * C::TILE);
    if (wave == 0) {
      const int nv = __builtin_amdgcn_readfirstlane(min(max(p.n_q - t * kTR, 0), kTR));
      const int64_t row = ((int64_t)b * p.Hq + h) * p.n_q + (int64_t)t * kTR;
      const uint32_t sl = lds0 + kStats + (uint32_t)stage * 512u;
      dma4((uint32_t)(lane * 4), buffer_rsrc(p.lse + row, (uint32_t)nv * 4u), sl);
      dma4((uint32_t)(lane * 4), buffer_rsrc(p.D + row, (uint32_t)nv * 4u), sl + 256u);
    }
  };

  f32x16_t dka[MH], dva[MH];
#pragma unroll
  for (int mh = 0; mh < MH; ++mh) {
    dka[mh] = (f32x16_t){};
    dva[mh] = (f32x16_t){};
  }

  // Lane addresses in stage 0: row fragments of the Q (role 0) or dO (role
  // 1) tile, row l32 of the first half; transposed fragments of the Q tile
  // for the wave's half of d (the dO tiles are kO0 further); the lse (role
  // 0) or D (role 1) of the lane's first four queries; the pair's exchange
  // buffers at the lane's 16-byte slot of each half.
  uint32_t ra[C::KC], ta[MH][2];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc) ra[kc] = lds0 + (role == 0 ? kQ0 : kO0) + row_ofs<D>(l32, kc, hi);
#pragma unroll
  for (int mh = 0; mh < MH; ++mh) {
    ta[mh][0] = lds0 + tr_ofs<D>(lane, role * MH + mh, 0);
    ta[mh][1] = lds0 + tr_ofs<D>(lane, role * MH + mh, 1);
  }
  const uint32_t sa = lds0 + kStats + (uint32_t)(16 * hi + 256 * role);
  const uint32_t xa = lds0 + kKvMainLds<D> + (uint32_t)pr * 4 * kXchg + (uint32_t)lane * 16;

  // ---- pieces of a block (tile stage S, half QB of the tile) ---------------
  // Row fragments of S (role 0) or D - dP (role 1) of a block.
  auto sd_frags = [&](auto S, auto QB, u32x4_t (&fr)[C::KC]) {
    constexpr uint32_t so = (uint32_t)(decltype(S)::value * C::TILE + decltype(QB)::value * 32 * C::ROWB);
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) fr[kc] = lds_b128(ra[kc] + so);
  };
  // The block's lse (role 0) or D (role 1) as the accumulator layout:
  // element j holds query 8*(j/4) + 4*hi + j%4 of the block.
  auto stats = [&](auto S, auto QB, u32x4_t (&st)[4]) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
      st[g] = lds_b128(sa + (uint32_t)(decltype(S)::value * 512 + (32 * decltype(QB)::value + 8 * g) * 4));
  };
  // S = Q K^T (role 0, from 0) or D - dP = D - dO V^T (role 1, from D).
  auto sd_mfma = [&](auto R, const u32x4_t (&fr)[C::KC], const u32x4_t (&st)[4]) -> f32x16_t {
    f32x16_t acc;
    if constexpr (decltype(R)::value == 0) {
      acc = (f32x16_t){};
    } else {
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int x = 0; x < 4; ++x) acc[4 * g + x] = __uint_as_float(st[g][x]);
    }
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) acc = mfma(as_bf16x8(fr[kc]), as_bf16x8(bfr[kc]), acc);
    return acc;
  };
  // P of a block from its S and lse, masked causally (query tile t, half
  // qb), rounded to bf16 in the B-operand layout: half h holds queries
  // 16h + {4hi..4hi+3, 8+4hi..8+4hi+3}.  lse = -inf only for a row that sees
  // no key anywhere, hence none of this pair: the mask (a select) zeroes its
  // elements.
  auto make_p = [&](const f32x16_t& s, const u32x4_t (&lr)[4], int t, int qb, u32x4_t (&pf)[2]) {
    float pw[16];
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int x = 0; x < 4; ++x)
        pw[4 * g + x] = __builtin_amdgcn_exp2f(fmaf(s[4 * g + x], c, -__uint_as_float(lr[g][x]) * kLog2e));
    const int64_t q0pos = p.q_pos0 + (int64_t)t * kTR + 32 * qb;
    if (p.causal && kpos_wave_last > q0pos) {
      const int lo = (int)min(max(kpos - q0pos - 4 * hi, (int64_t)-1), (int64_t)33);
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int x = 0; x < 4; ++x) pw[4 * g + x] = (8 * g + x >= lo) ? pw[4 * g + x] : 0.f;
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int half = g / 2, xx = 2 * (g & 1);
      pf[half][xx] = pack_bf16x2(pw[4 * g], pw[4 * g + 1]);
      pf[half][xx + 1] = pack_bf16x2(pw[4 * g + 2], pw[4 * g + 3]);
    }
  };
  // dS = P (dP - D) = -P (D - dP) of a block (role 1), from its bf16 P.
  auto make_ds = [&](const u32x4_t (&pf)[2], const f32x16_t& dm, u32x4_t (&df)[2]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int half = g / 2, xx = 2 * (g & 1);
      float d4[4];
#pragma unroll
      for (int y = 0; y < 2; ++y) {
        const uint32_t w = pf[half][xx + y];
        d4[2 * y] = -(__uint_as_float(w << 16) * dm[4 * g + 2 * y]);
        d4[2 * y + 1] = -(__uint_as_float(w & 0xffff0000u) * dm[4 * g + 2 * y + 1]);
      }
      df[half][xx] = pack_bf16x2(d4[0], d4[1]);
      df[half][xx + 1] = pack_bf16x2(d4[2], d4[3]);
    }
  };
  // Transposed fragments of a block for dV^T += dO^T P (DK = false, dO
  // tile) or dK^T += Q^T dS (DK = true, Q tile), the wave's half of d;
  // fragment 2*mh + hf covers 32-row block mh of the half, queries 16 hf ..
  // of the block.
  auto kv_frags = [&](auto S, auto QB, auto DK, bf16x8_t (&fr)[2 * MH]) {
    constexpr uint32_t so = (uint32_t)(decltype(S)::value * C::TILE + (decltype(DK)::value ? kQ0 : kO0));
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const uint32_t o = so + (uint32_t)((32 * decltype(QB)::value + 16 * hf) * C::ROWB);
#pragma unroll
      for (int mh = 0; mh < MH; ++mh) fr[2 * mh + hf] = tr_frag(ta[mh][0] + o, ta[mh][1] + o);
    }
  };
  auto kv_mfma = [&](auto DK, const bf16x8_t (&fr)[2 * MH], const u32x4_t (&w)[2]) {
#pragma unroll
    for (int mh = 0; mh < MH; ++mh)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        if constexpr (decltype(DK)::value) dka[mh] = mfma(fr[2 * mh + hf], as_bf16x8(w[hf]), dka[mh]);
        else dva[mh] = mfma(fr[2 * mh + hf], as_bf16x8(w[hf]), dva[mh]);
      }
  };
  auto x_write = [&](uint32_t buf, const u32x4_t (&v)[2]) {
    *reinterpret_cast<SQKV_LDS u32x4_t*>((size_t)(xa + buf)) = v[0];
    *reinterpret_cast<SQKV_LDS u32x4_t*>((size_t)(xa + buf + 1024)) = v[1];
  };
  auto x_read = [&](uint32_t buf, u32x4_t (&v)[2]) {
    v[0] = lds_b128(xa + buf);
    v[1] = lds_b128(xa + buf + 1024);
  };

  // ---- the walk (one copy of the loop per role) ------------------------------
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

  auto walk = [&](auto R) {
    constexpr int r = decltype(R)::value;
    // w[u & 1]: P of block u (role 0) or dS of block u (role 1); dm: role 1's
    // D - dP of the block whose dS comes next.
    u32x4_t w[2][2];
    f32x16_t dm;
    // The row fragments of an even step (and role 1's D of its block u+1)
    // come from a tile landed before the barrier ahead of it, so they are
    // read before that barrier.
    u32x4_t pre_fr[C::KC], pre_st[4];
    auto prefetch = [&](auto SU1) {
      sd_frags(SU1, Step<1>{}, pre_fr);
      if constexpr (r == 1) stats(SU1, Step<1>{}, pre_st);
    };
    {
      u32x4_t fr[C::KC], st[4];
      sd_frags(Step<0>{}, Step<0>{}, fr);
      stats(Step<0>{}, Step<0>{}, st);
      if constexpr (r == 0) {
        make_p(sd_mfma(R, fr, st), st, t0, 0, w[0]);
        x_write(0u, w[0]);
      } else {
        dm = sd_mfma(R, fr, st);
      }
    }
    prefetch(Step<0>{});
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    asm volatile("s_barrier" ::: "memory");

    int t_cur = t0, t_nxt = t0, gi_n = 0;     // query tiles of tau and tau+1
    advance(gi_n, t_nxt);

    // One step: block u = 2 tau + QB; SP, SC, SN are the stages of tiles
    // tau-1, tau, tau+1.
    auto step = [&](auto SP, auto SC, auto SN, auto QB, int tau) {
      constexpr int qb = decltype(QB)::value;
      using SU1 = std::conditional_t<qb == 0, decltype(SC), decltype(SN)>;   // stage of block u+1
      using SM1 = std::conditional_t<qb == 0, decltype(SP), decltype(SC)>;  // stage of block u-1
      using QO = Step<1 - qb>;                                               // half of blocks u+1, u-1
      const int u = 2 * tau + qb;
      const bool nxt = u + 1 < NB, cur = u < NB, prv = u >= 1 && u <= NB;
      u32x4_t fr[C::KC], st[4], xw[2];
      bf16x8_t fv[2 * MH], fk[2 * MH];
      if constexpr (qb == 0) {
#pragma unroll
        for (int kc = 0; kc < C::KC; ++kc) fr[kc] = pre_fr[kc];
        if constexpr (r == 0) kv_frags(SC, QB, Step<0>{}, fv);
        if constexpr (r == 1) {
#pragma unroll
          for (int g = 0; g < 4; ++g) st[g] = pre_st[g];
        }
      } else {
        sd_frags(SU1{}, QO{}, fr);
        if constexpr (r == 1) stats(SU1{}, QO{}, st);   // D of block u+1
        if constexpr (r == 0) kv_frags(SC, QB, Step<0>{}, fv);
      }
      if constexpr (r == 1) x_read((uint32_t)qb * kXchg, xw);   // P of block u
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (r == 0) {
        const f32x16_t a = sd_mfma(R, fr, st);   // S of block u+1 (st unused: from 0)
        // read while those run: the dK fragments, dS of block u-1, lse of block u+1
        kv_frags(SM1{}, QO{}, Step<1>{}, fk);
        x_read((uint32_t)(2 + ((u + 1) & 1)) * kXchg, xw);
        stats(SU1{}, QO{}, st);
        if (cur) kv_mfma(Step<0>{}, fv, w[qb]);
        if (prv) kv_mfma(Step<1>{}, fk, xw);
        if (nxt) {
          make_p(a, st, qb == 0 ? t_cur : t_nxt, 1 - qb, w[1 - qb]);
          x_write((uint32_t)(1 - qb) * kXchg, w[1 - qb]);
        }
      } else {
        // dS of block u first (VALU while the partner wave's S products
        // run), then D - dP of block u+1 into the same registers
        if (cur) {
          make_ds(xw, dm, w[qb]);
          x_write((uint32_t)(2 + qb) * kXchg, w[qb]);
        }
        dm = sd_mfma(R, fr, st);
        kv_frags(SC, QB, Step<0>{}, fv);
        kv_frags(SM1{}, QO{}, Step<1>{}, fk);
        if (cur) kv_mfma(Step<0>{}, fv, xw);
        if (prv) kv_mfma(Step<1>{}, fk, w[1 - qb]);
      }
      if constexpr (qb == 0) {
        // the next step reads tile tau+1
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        asm volatile("s_barrier" ::: "memory");
        if (tau + 2 < NT) {
          issue_tile(gi_d, t_d, decltype(SP)::value);   // tile tau+2 takes the stage of tile tau-1
          advance(gi_d, t_d);
        }
      } else {
        prefetch(SN);   // block u+2: tile tau+1, half 1
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
        asm volatile("s_barrier" ::: "memory");
        t_cur = t_nxt;
        advance(gi_n, t_nxt);
      }
    };
    for (int tau = 0; 2 * tau <= NB; tau += 3) {
      step(Step<2>{}, Step<0>{}, Step<1>{}, Step<0>{}, tau);
      step(Step<2>{}, Step<0>{}, Step<1>{}, Step<1>{}, tau);
      step(Step<0>{}, Step<1>{}, Step<2>{}, Step<0>{}, tau + 1);
      step(Step<0>{}, Step<1>{}, Step<2>{}, Step<1>{}, tau + 1);
      step(Step<1>{}, Step<2>{}, Step<0>{}, Step<0>{}, tau + 2);
      step(Step<1>{}, Step<2>{}, Step<0>{}, Step<1>{}, tau + 2);
    }
  };
  if (role == 0) walk(Step<0>{});
  else walk(Step<1>{});
  __builtin_amdgcn_s_waitcnt(0);   // no DMA may outlive the workgroup's LDS

  if (key_ok) {
    float* dkr = p.dk + b * p.dk_sb + hk * p.dk_sh + (int64_t)key * p.dk_sn;
    float* dvr = p.dv + b * p.dv_sb + hk * p.dv_sh + (int64_t)key * p.dv_sn;
#pragma unroll
    for (int mh = 0; mh < MH; ++mh)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * (role * MH + mh) + 8 * g + 4 * hi;
        float4 x = *reinterpret_cast<float4*>(dkr + d0);
        x.x = fmaf(p.scale, dka[mh][4 * g + 0], x.x);
        x.y = fmaf(p.scale, dka[mh][4 * g + 1], x.y);
        x.z = fmaf(p.scale, dka[mh][4 * g + 2], x.z);
        x.w = fmaf(p.scale, dka[mh][4 * g + 3], x.w);
        *reinterpret_cast<float4*>(dkr + d0) = x;
        float4 y = *reinterpret_cast<float4*>(dvr + d0);
        y.x += dva[mh][4 * g + 0];
        y.y += dva[mh][4 * g + 1];
        y.z += dva[mh][4 * g + 2];
        y.w += dva[mh][4 * g + 3];
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

template <int D>
hipError_t launch_bwd_d(const BwdParams& p, hipStream_t s) {
  using Cq = BCfg<D, kDqWaves>;
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
