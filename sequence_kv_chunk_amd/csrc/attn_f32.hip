// Chunk attention with fp32 inputs and fp32 arithmetic throughout.
//
// Ring-attention Q&A (aivaro.ru answer 425), section 5: for one query chunk
// and one key/value chunk, scores q.k, the row maximum, exponentials, the row
// sum (normaliser) and the weighted sum of values; the chunk's partial is
// then merged into the running output (online softmax).
//
// This is the exact-precision variant: the products run on the fp32 matrix
// cores (v_mfma_f32_32x32x2_f32: fp32 operands, fp32 accumulation, no
// reduced-precision rounding).  Per 32-key tile a wave forms S^T = K Q^T
// (keys on the MFMA M axis, so a lane holds 16 keys of ONE query: the row
// maximum and sum are lane-local plus one exchange with the lane holding the
// query's other 16 keys) and O^T += V^T P^T, where P^T is the S^T registers
// themselves (the k index of a step pairs key 8g + x of one lane half with
// key 8g + 4 + x of the other).  Q^T stays in registers (lane half h holds
// d = h*D/2 .. h*D/2 + D/2 - 1 of its query).  The visit's tiles (every
// chunk's, chunks in ring order: visit s reads chunk j = (rank - s) mod P)
// are dealt to several key splits, each with its own online softmax, and the
// splits' states of a row are merged at the end (log-sum-exp weights).
//
// Two kernels, chosen by the size of the launch:
// * attn_f32_shared (launches that fill the device): 8 wavefronts, two per
//   SIMD, take 128 query rows; wave w owns rows 32 (w % 4) .. + 31 and key
//   split w / 4.  The four waves of a split share each of its tiles, copied
//   global -> LDS by buffer_load ... lds (no register staging; rows past the
//   visible keys arrive as zeros) two stages deep.  K rows are copied as
//   they are, 16 bytes per lane, their 16-byte chunks XOR-swizzled by the row
//   index so that the 32 rows read at one column fall in distinct banks.  V
//   is copied transposed, 4 bytes per lane (a copy gathers one column of the
//   tile's 32 keys into an LDS row), so that one 16-byte read returns the
//   four keys that four consecutive P V MFMAs of a lane take; its 16-byte
//   chunks are XOR-swizzled by (row / 2) % 8, which spreads the 16 rows one
//   read touches over distinct banks.
// * attn_f32_split (small launches, e.g. one short chunk per rank): four
//   wavefronts take 32 query rows and split the keys four ways, each wave
//   with its own LDS tile filled from registers, holding its next tile's
//   rows in registers while it works on the current one: four times the
//   workgroups of the shared kernel for the same rows.
// It is meant for correctness-critical fp32 use; the bf16 kernel is the
// throughput path.
#include <type_traits>
#include <utility>

#include "attn_common.h"

namespace sqkv {
namespace {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
#define SQKV_LDS __attribute__((address_space(3)))

constexpr int kTile = 32;   // keys per tile

__device__ __forceinline__ f32x16_t mfma_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Max / sum with the lane 32 apart (the lane holding the query's other 16
// keys): v_permlane32_swap of x with itself gives both values in every lane.
__device__ __forceinline__ float max_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int I>
using Int = std::integral_constant<int, I>;

// f(Int<0>{}), ..., f(Int<N-1>{}) as straight-line code.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(Int<I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for_n(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---- pieces shared by both kernels ------------------------------------------

// The visit of a block of query rows whose last row is tmax: chunk s of the
// visit with its base pointers, the position of its key 0 and the keys the
// block can see (causal: up to the block's last query position).  A cursor
// (s, k0) names a tile: key k0 of the chunk of visit s; the Cursor struct
// also carries its chunk's values.
struct Visit {
  const AttnParams& p;
  const float* kb0;
  const float* vb0;
  int64_t tmax;

  __device__ int64_t chunk(int s, const float*& kb, const float*& vb, int64_t& kpos0) const {
    int j = p.rank - s;   // visit s reads chunk (rank - s) mod P (0 <= s < P)
    if (j < 0) j += p.P;
    kb = kb0 + (int64_t)j * p.k_cs;
    vb = vb0 + (int64_t)j * p.v_cs;
    kpos0 = p.k_pos0 + (int64_t)j * p.k_posstride;
    int64_t n_keys = p.n_k;
    if (p.causal) n_keys = max((int64_t)0, min(n_keys, p.q_pos0 + tmax - kpos0 + 1));
    return n_keys;
  }
  // moves (s, k0) on by `steps` tiles; s = nseg past the last tile
  __device__ void advance(int& s, int64_t& k0, int steps) const {
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
  }
  // A cursor that keeps its chunk's values: they are recomputed only when it
  // crosses into the next chunk.
  struct Cursor {
    int s;
    int64_t k0, span, n_keys, kpos0;
    const float* kb;
    const float* vb;
  };
  __device__ void load(Cursor& c) const {
    if (c.s < p.nseg) {
      c.n_keys = chunk(c.s, c.kb, c.vb, c.kpos0);
      c.span = (c.n_keys + kTile - 1) / kTile * kTile;
    }
  }
  __device__ Cursor start(int steps) const {
    Cursor c;
    c.s = 0;
    c.k0 = 0;
    load(c);
    move(c, steps);
    return c;
  }
  __device__ void move(Cursor& c, int steps) const {
    c.k0 += (int64_t)steps * kTile;
    while (c.s < p.nseg && c.k0 >= c.span) {
      c.k0 -= c.span;
      ++c.s;
      load(c);
    }
  }
  // tiles of the whole visit
  __device__ int tiles() const {
    int T = 0;
    for (int s = 0; s < p.nseg; ++s) {
      const float* kb;
      const float* vb;
      int64_t kpos0;
      T += (int)((chunk(s, kb, vb, kpos0) + kTile - 1) / kTile);
    }
    return T;
  }
};

// One tile after S^T (scores already in base-2 units: Q carries
// scale * log2(e)): the mask when the tile needs one (element jj is key
// 8 (jj/4) + 4 hi + jj%4 of the tile; the lane sees keys up to lim + 4 hi),
// the online-softmax update and O^T += V^T P^T, with vread4(mb, gg) the V^T
// elements the lane feeds to steps (gg, 0..3) of d-block mb: column
// 32 mb + l32 of key rows 8 gg + 4 hi + 0..3.
template <int D, typename VRead4>
__device__ __forceinline__ void softmax_pv(f32x16_t& st, f32x16_t (&o)[D / 32], float& m, float& l, bool masked,
                                           int lim, VRead4 vread4) {
  if (masked) {   // a wave-uniform branch: no MFMA inside
#pragma unroll
    for (int jj = 0; jj < 16; ++jj)
      if (8 * (jj / 4) + (jj % 4) > lim) st[jj] = kNegInf;
  }
  float tmx = st[0];
#pragma unroll
  for (int jj = 1; jj < 16; ++jj) tmx = fmaxf(tmx, st[jj]);
  tmx = max_half(tmx);   // with the query's other 16 keys
  // The row's reference m moves (and o, l are rescaled) only when the tile's
  // maximum exceeds it by more than kSlack (base-2 units): weights then stay
  // below 2^kSlack, which fp32 carries without loss, and the rescale is rare
  // after the first tiles.  No branch on the row's state around the matrix
  // products: they run for the whole wave whatever the lane mask, so a row
  // that has seen no key yet keeps alpha = 1 and gets weights 0.
  constexpr float kSlack = 8.f;
  const bool bump = tmx != kNegInf && (m == kNegInf || tmx > m + kSlack);
  if (__any(bump)) {   // a wave-uniform branch: no MFMA inside
    const float mn = bump ? tmx : m;
    const float alpha = (m == kNegInf || !bump) ? 1.f : exp2f(m - mn);
    l *= alpha;
#pragma unroll
    for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) o[mb][jj] *= alpha;
    m = mn;
  }
  // v_exp_f32: within an ulp for normal results, 0 at -inf; a weight below
  // 2^-126 (flushed to 0) is far below the fp32 bar next to the row's
  // largest (>= 1).  A row that has seen no key yet (m = -inf) has only -inf
  // scores: subtracting 0 keeps their weights 0.
  const float mref = (m == kNegInf) ? 0.f : m;
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    st[jj] = __builtin_amdgcn_exp2f(st[jj] - mref);
    l += st[jj];
  }
  // step (gg, x) pairs key 8gg + x (half 0) with key 8gg + 4 + x (half 1),
  // i.e. element 4gg + x of each lane.  Each group of four MFMAs takes the
  // operands read one group earlier (the fence keeps the next read ahead of
  // the MFMAs, so its latency runs under them).
  constexpr int NG = D / 32 * 4;
  f32x4_t vb[2];
  vb[0] = vread4(0, 0);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if (g + 1 < NG) vb[(g + 1) & 1] = vread4((g + 1) / 4, (g + 1) % 4);
    __builtin_amdgcn_sched_barrier(0);
    const int mb = g / 4, gg = g % 4;
#pragma unroll
    for (int x = 0; x < 4; ++x) o[mb] = mfma_f32(vb[g & 1][x], st[4 * gg + x], o[mb]);
  }
}

// A wave's partial state of its 32 rows into LDS: row n's (o[D], m, l) at
// state + n * (D + 4) floats.
template <int D>
__device__ __forceinline__ void write_state(float* state, int l32, int hi, const f32x16_t (&o)[D / 32], float m,
                                            float l) {
  float* mine = state + l32 * (D + 4);
#pragma unroll
  for (int mb = 0; mb < D / 32; ++mb)
#pragma unroll
    for (int gg = 0; gg < 4; ++gg)
      *reinterpret_cast<float4*>(mine + 32 * mb + 8 * gg + 4 * hi) =
          make_float4(o[mb][4 * gg], o[mb][4 * gg + 1], o[mb][4 * gg + 2], o[mb][4 * gg + 3]);
  const float lsum = sum_half(l);
  if (hi == 0) {
    mine[D] = m;
    mine[D + 1] = lsum;
  }
}

// Merges the NS partial states of each of the block's ROWS rows (split w of
// row n at stt + (w * ROWS + n) * (D + 4)), normalises, merges with the
// running state when there is one and stores: THREADS / ROWS threads per
// row, each with D / (THREADS / ROWS) columns.
template <int D, int NS, int ROWS, int THREADS>
__device__ __forceinline__ void merge_store(const AttnParams& p, const float* stt, int b, int h, int q0) {
  constexpr int PITCH = D + 4;
  constexpr int TPR = THREADS / ROWS;
  static_assert(TPR * ROWS == THREADS && D % (4 * TPR) == 0, "whole rows per thread group");
  const int n = threadIdx.x / TPR;
  const int t_out = q0 + n;
  if (t_out >= p.n_q) return;
  float M = kNegInf;
#pragma unroll
  for (int w = 0; w < NS; ++w) M = fmaxf(M, stt[(w * ROWS + n) * PITCH + D]);
  float a[NS];
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < NS; ++w) {
    const float mw = stt[(w * ROWS + n) * PITCH + D];
    a[w] = (mw == kNegInf) ? 0.f : exp2f(mw - M);
    L += a[w] * stt[(w * ROWS + n) * PITCH + D + 1];
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
  constexpr int kCols = D / TPR;
  const int e0 = (threadIdx.x % TPR) * kCols;
#pragma unroll
  for (int e = 0; e < kCols; e += 4) {
    float y[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < NS; ++w) acc = fmaf(a[w], stt[(w * ROWS + n) * PITCH + e0 + e + i], acc);
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
  if (threadIdx.x % TPR == 0) p.lse_out[bh_row * p.lse_out_hs + t_out] = lse;
}

// Q^T operand of the lane's query row t (zeros past n_q): d = hi * D/2 + s,
// times c = scale * log2(e), so that S^T = K Q^T holds the logits in base-2
// units (one fp32 rounding per element of Q instead of one per score).
template <int D>
__device__ __forceinline__ void load_qt(const AttnParams& p, int b, int h, int t, int hi, float (&q)[D / 2]) {
  const bool row_ok = t < p.n_q;
  const float* qrow = static_cast<const float*>(p.q) + b * p.q_sb + h * p.q_sh + (int64_t)(row_ok ? t : 0) * p.q_sn;
  const float c = p.scale_log2;
#pragma unroll
  for (int e = 0; e < D / 2; e += 4) {
    const float4 x = row_ok ? *reinterpret_cast<const float4*>(qrow + hi * (D / 2) + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    q[e] = x.x * c; q[e + 1] = x.y * c; q[e + 2] = x.z * c; q[e + 3] = x.w * c;
  }
}

// ---- attn_f32_shared: 128 rows, two key splits sharing LDS tiles -------------

constexpr int kRowWaves = 4;                  // 32-row groups per workgroup
constexpr int kSplits = 2;                    // key splits: tile g goes to split g % 2
constexpr int kShWaves = kRowWaves * kSplits; // wave w: rows 32 (w % 4) .., split w / 4
constexpr int kShRows = 32 * kRowWaves;       // query rows per workgroup
constexpr int kStages = 2;                    // LDS stages per split

template <int D>
struct ShCfg {
  static constexpr int ROWB = D * 4;                     // bytes per row
  static constexpr int TILE = kTile * ROWB;              // bytes per K or V tile
  static constexpr int NCH = D / 4;                      // 16-byte chunks per row
  static constexpr int RPW = 1024 / ROWB;                // rows per wave-wide 1 KiB copy
  static constexpr int NL = TILE / 1024 / kRowWaves;     // K copies per wave and tile (16 bytes per lane)
  static constexpr int NVT = D / 2 / kRowWaves;          // V^T copies per wave and tile (two rows of 32 keys each)
  static constexpr int STAGE = 2 * TILE;                 // a stage: K tile, then V tile
  static constexpr int SPLIT = kStages * STAGE;          // one split's stages
  static constexpr int TILES = kSplits * SPLIT;
  static constexpr int STATES = kSplits * kShRows * (D + 4) * 4;
  static constexpr int LDS = TILES > STATES ? TILES : STATES;
  static_assert(NL >= 1 && (TILE / 1024) % kRowWaves == 0, "tile copies must spread evenly over a split's waves");
  static_assert(D % 32 == 0, "whole 32-row blocks of d");
  static_assert(LDS <= 160 * 1024, "LDS");
};

// 16-byte chunk c of K row r sits at chunk c ^ swz_k(r); chunk c (keys
// 4c .. 4c+3) of V^T row r (column r of V) at c ^ swz_vt(r).
__device__ __forceinline__ int swz_k(int r) { return r & 15; }
__device__ __forceinline__ int swz_vt(int r) { return (r >> 1) & 7; }

// Buffer resource over `bytes` bytes from `base`: reads past them return 0.
__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = (int)(uint32_t)b;
  r[1] = (int)(uint32_t)(b >> 32);   // stride 0: a raw byte range
  r[2] = (int)bytes;
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from the buffer at `voff` into LDS at m0 + 16 * lane.
__device__ __forceinline__ void dma16(uint32_t voff, i32x4_t rsrc, uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" :: "v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}

// 4 bytes per lane from the buffer at `voff` into LDS at m0 + 4 * lane.  (An
// immediate offset would move the LDS destination as well as the source.)
__device__ __forceinline__ void dma4(uint32_t voff, i32x4_t rsrc, uint32_t lds) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds" :: "v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}

// Wait for every copy and LDS access of this wave, then meet the other waves.
__device__ __forceinline__ void drain_and_sync() {
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("s_barrier" ::: "memory");
}

template <int D>
__global__ void __launch_bounds__(64 * kShWaves) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_f32_shared(AttnParams p) {
  using C = ShCfg<D>;
  constexpr int MB = D / 32;   // 32-row blocks of d in O^T
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const uint32_t lds0 = (uint32_t)(size_t)(SQKV_LDS unsigned char*)smem;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x / 64);
  const int lane = threadIdx.x % 64;
  const int l32 = lane & 31, hi = lane >> 5;
  const int rg = wave % kRowWaves, ks = wave / kRowWaves;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int hk = h / p.group;
  const int q0 = blockIdx.x * kShRows;
  const int t = q0 + 32 * rg + l32;            // this lane's query row
  float q[D / 2];
  load_qt<D>(p, b, h, t, hi, q);
  // O^T: element j of block mb holds d = 32 mb + 8 (j/4) + 4 hi + j%4 of the query
  f32x16_t o[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) o[mb] = (f32x16_t){};
  const int64_t qpos = p.q_pos0 + t;
  const int64_t qpos_w0 = p.q_pos0 + q0 + 32 * rg;   // the wave's first query
  float m = kNegInf;  // running max of logits, base-2 units (same in both lane halves)
  float l = 0.f;      // this lane's part of the running normaliser (its 16 keys of each tile)
  const Visit vis{p, static_cast<const float*>(p.k) + b * p.k_sb + hk * p.k_sh,
                  static_cast<const float*>(p.v) + b * p.v_sb + hk * p.v_sh,
                  min((int64_t)q0 + kShRows - 1, (int64_t)p.n_q - 1)};
  const int T = vis.tiles();

  // K copies: wave-wide copy i of a split's tile fills rows
  // (i * kRowWaves + rg) * RPW ..; the lane fills row r0 + lane / NCH at
  // chunk position lane % NCH, so it reads source chunk (lane % NCH) ^ swz(row).
  const int k_snb = (int)(p.k_sn * 4), v_snb = (int)(p.v_sn * 4);
  uint32_t dko[C::NL];
#pragma unroll
  for (int i = 0; i < C::NL; ++i) {
    const int r = (i * kRowWaves + rg) * C::RPW + lane / C::NCH;
    dko[i] = (uint32_t)(r * k_snb) + (uint32_t)(((lane % C::NCH) ^ swz_k(r)) * 16);
  }
  // V^T copies: copy i fills V^T rows (columns of V) 2 (4 i + rg) and the
  // next, one per lane half; lane slot s = lane % 32 of row r takes key
  // 4 ((s / 4) ^ swz_vt(r)) + s % 4.  swz_vt(r) = (4 i + rg) % 8 takes two
  // values (i even, odd): one source offset each, plus 32 i bytes (the column).
  uint32_t dvt[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) {
    const int slot = lane % 32;
    const int key = 4 * ((slot / 4) ^ ((4 * par + rg) & 7)) + slot % 4;
    dvt[par] = (uint32_t)(key * v_snb) + (uint32_t)(8 * rg + 4 * (lane / 32));
  }
  const uint32_t split0 = lds0 + (uint32_t)(ks * C::SPLIT);
  const uint32_t m0_wave = (uint32_t)(rg * C::RPW * C::ROWB);
  auto issue = [&](const Visit::Cursor& c, int stage) {
    const int64_t k0 = c.k0;
    const int nv = (int)min(c.n_keys - k0, (int64_t)kTile);   // valid rows of the tile (>= 1)
    // the byte range of rows 0 .. nv-1 exactly (row strides may be below a row)
    const i32x4_t rk = buffer_rsrc(c.kb + k0 * p.k_sn, (uint32_t)((nv - 1) * k_snb + C::ROWB));
    const i32x4_t rv = buffer_rsrc(c.vb + k0 * p.v_sn, (uint32_t)((nv - 1) * v_snb + C::ROWB));
    const uint32_t st = split0 + (uint32_t)(stage * C::STAGE);
#pragma unroll
    for (int i = 0; i < C::NL; ++i) dma16(dko[i], rk, st + m0_wave + (uint32_t)(i * kRowWaves * C::RPW * C::ROWB));
    static_for_n<C::NVT>([&](auto I) {
      constexpr int i = decltype(I)::value;
      dma4(dvt[i & 1] + 32 * i, rv, st + (uint32_t)(C::TILE + 256 * (4 * i + rg)));
    });
  };

  // lane addresses in stage 0 of the split: K row l32 (chunks of the lane's
  // half of d); V^T row l32 of d-block 0, its chunk holding keys 8 gg + 4 hi ..
  const SQKV_LDS unsigned char* sbase = (const SQKV_LDS unsigned char*)smem + ks * C::SPLIT;
  // chunk g of the lane's half of d in stage 0, each a whole address held in
  // a register (opaque to the compiler, which would otherwise split it into
  // a shared base plus an offset and add them again for every read), so that
  // a read adds only the stage offset as an immediate
  uint32_t kaddr[D / 8];
#pragma unroll
  for (int g = 0; g < D / 8; ++g) {
    kaddr[g] = (uint32_t)(size_t)(sbase + l32 * C::ROWB + (((hi * (C::NCH / 2) + g) ^ swz_k(l32)) * 16));
    asm volatile("" : "+v"(kaddr[g]));
  }
  int vto[4];
#pragma unroll
  for (int gg = 0; gg < 4; ++gg) vto[gg] = C::TILE + l32 * 128 + (((2 * gg + hi) ^ swz_vt(l32)) * 16);

  Visit::Cursor cc = vis.start(ks);          // this wave's tile: step i is tile 2 i + ks
  Visit::Cursor dc = cc;                      // the next tile to copy
  const int nsteps = (T + kSplits - 1) / kSplits;
  if (ks < T) issue(dc, 0);
  // step i: its tiles sit in stage i % 2 (a constant in each half of the
  // unrolled loop, so that every LDS offset is an immediate)
  auto step = [&](auto STG, int i) {
    constexpr int stage = decltype(STG)::value;
    drain_and_sync();                         // step i's tiles landed; the other stage is free
    vis.move(dc, kSplits);
    if (kSplits * (i + 1) + ks < T) issue(dc, 1 - stage);
    if (kSplits * i + ks < T) {
      const int64_t n_keys = cc.n_keys, kpos0 = cc.kpos0, ck0 = cc.k0;
      // S^T = K Q^T: step e pairs d = e (lane half 0) with d = D/2 + e (half
      // 1); each group of four MFMAs takes the K operands read one group earlier
      auto kread = [&](int g) {
        return *reinterpret_cast<const SQKV_LDS f32x4_t*>((size_t)(kaddr[g] + stage * C::STAGE));
      };
      f32x16_t st = (f32x16_t){};
      f32x4_t kb2[2];
      kb2[0] = kread(0);
#pragma unroll
      for (int g = 0; g < D / 8; ++g) {
        if (g + 1 < D / 8) kb2[(g + 1) & 1] = kread(g + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int x = 0; x < 4; ++x) st = mfma_f32(kb2[g & 1][x], q[4 * g + x], st);
      }
      // visible keys of the tile: the chunk's, and (causal) up to the query;
      // no mask when every key is visible to every row of the wave
      const bool masked = n_keys - ck0 < kTile || (p.causal && kpos0 + ck0 + kTile - 1 > qpos_w0);
      int64_t lim64 = n_keys - 1 - ck0;
      if (p.causal) lim64 = min(lim64, qpos - kpos0 - ck0);
      const int lim = (int)max(min(lim64, (int64_t)kTile), (int64_t)-1) - 4 * hi;
      // V^T row 32 mb + l32 (its swizzle is that of row l32: 32 mb / 2 is a
      // multiple of 8)
      const SQKV_LDS unsigned char* vt = sbase + stage * C::STAGE;
      softmax_pv<D>(st, o, m, l, masked, lim, [&](int mb, int gg) {
        return *reinterpret_cast<const SQKV_LDS f32x4_t*>(vt + vto[gg] + mb * 32 * 128);
      });
      vis.move(cc, kSplits);
    }
  };
  for (int i = 0; i < nsteps; i += 2) {
    step(Int<0>{}, i);
    if (i + 1 < nsteps) step(Int<1>{}, i + 1);
  }
  drain_and_sync();   // every wave is done with the tiles: the LDS takes the states
  float* stt = reinterpret_cast<float*>(smem);
  write_state<D>(stt + (ks * kShRows + 32 * rg) * (D + 4), l32, hi, o, m, l);
  __syncthreads();
  merge_store<D, kSplits, kShRows, 64 * kShWaves>(p, stt, b, h, q0);
}

// ---- attn_f32_split: 32 rows, four key splits, one wave each ----------------

constexpr int kSpRows = 32;   // query rows per workgroup
constexpr int kSpWaves = 4;   // wavefronts, each with every kSpWaves-th tile

template <int D>
struct SpCfg {
  static constexpr int KROW = D + 4;                            // padded K row (floats): conflict-free b128 reads
  static constexpr int WAVE = kTile * KROW + kTile * D;         // one wave's K and V tile (floats)
  static constexpr int STATES = kSpWaves * kSpRows * (D + 4);   // (o[D], m, l) per wave and row
  static constexpr int FLOATS = kSpWaves * WAVE > STATES ? kSpWaves * WAVE : STATES;
  static_assert(FLOATS * 4 <= 160 * 1024, "LDS");
  static_assert(D % 32 == 0, "whole 32-row blocks of d");
};

template <int D>
__global__ void __launch_bounds__(64 * kSpWaves) attn_f32_split(AttnParams p) {
  using C = SpCfg<D>;
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
  const int q0 = blockIdx.x * kSpRows;
  const int t = q0 + l32;                      // this lane's query row
  float q[D / 2];
  load_qt<D>(p, b, h, t, hi, q);
  f32x16_t o[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) o[mb] = (f32x16_t){};
  const int64_t qpos = p.q_pos0 + t;
  float m = kNegInf;
  float l = 0.f;
  const Visit vis{p, static_cast<const float*>(p.k) + b * p.k_sb + hk * p.k_sh,
                  static_cast<const float*>(p.v) + b * p.v_sb + hk * p.v_sh,
                  min((int64_t)q0 + kSpRows - 1, (int64_t)p.n_q - 1)};
  // The wave's tiles: tile g of the visit goes to wave g mod kSpWaves; the
  // wave holds its next tile's rows in registers while it works on the
  // current one.  Row r0 + kRpi * it of a tile, columns e4 .. e4+3.
  constexpr int kRpi = 256 / D;
  constexpr int kPass = kTile / kRpi;
  const int r0 = lane / (D / 4), e4 = (lane % (D / 4)) * 4;
  float4 pk[kPass], pv[kPass];
  auto fetch = [&](int s, int64_t k0) {
    if (s >= p.nseg) return;
    const float* kb;
    const float* vb;
    int64_t kpos0;
    const int64_t n_keys = vis.chunk(s, kb, vb, kpos0);
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
  vis.advance(cs, ck0, wave);
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
    vis.advance(ns, nk0, kSpWaves);
    fetch(ns, nk0);   // the wave's next tile, in flight while this one is used
    const float* kb;
    const float* vb;
    int64_t kpos0;
    const int64_t n_keys = vis.chunk(cs, kb, vb, kpos0);
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
    const bool masked = n_keys - ck0 < kTile || (p.causal && kpos0 + ck0 + kTile - 1 > p.q_pos0 + q0);
    int64_t lim64 = n_keys - 1 - ck0;
    if (p.causal) lim64 = min(lim64, qpos - kpos0 - ck0);
    const int lim = (int)max(min(lim64, (int64_t)kTile), (int64_t)-1) - 4 * hi;
    softmax_pv<D>(st, o, m, l, masked, lim, [&](int mb, int gg) {
      const float* col = vs + (8 * gg + 4 * hi) * D + 32 * mb + l32;
      return (f32x4_t){col[0], col[D], col[2 * D], col[3 * D]};
    });
    // every lane's reads of this tile are done before the next one is written
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    cs = ns;
    ck0 = nk0;
  }
  __syncthreads();   // every wave is done with its tiles: the LDS takes the states
  write_state<D>(lds_f + wave * kSpRows * (D + 4), l32, hi, o, m, l);
  __syncthreads();
  merge_store<D, kSpWaves, kSpRows, 64 * kSpWaves>(p, lds_f, b, h, q0);
}

template <int D>
hipError_t launch_d(const AttnParams& p, hipStream_t s) {
  // The shared-tile kernel once its workgroups cover every compute unit;
  // below that the split kernel, with four times as many workgroups.
  int ncu = 0;
  hipError_t e = device_cu_count(&ncu);
  if (e != hipSuccess) return e;
  const int64_t sh_groups = (int64_t)((p.n_q + kShRows - 1) / kShRows) * p.Hq * p.B;
  if (sh_groups >= ncu) {
    static std::atomic<uint64_t> lds_set{0};
    e = allow_dyn_lds(reinterpret_cast<const void*>(&attn_f32_shared<D>), ShCfg<D>::LDS, lds_set);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((p.n_q + kShRows - 1) / kShRows), (unsigned)p.Hq, (unsigned)p.B);
    hipLaunchKernelGGL(attn_f32_shared<D>, grid, dim3(64 * kShWaves), ShCfg<D>::LDS, s, p);
  } else {
    static std::atomic<uint64_t> lds_set{0};
    e = allow_dyn_lds(reinterpret_cast<const void*>(&attn_f32_split<D>), SpCfg<D>::FLOATS * 4, lds_set);
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((p.n_q + kSpRows - 1) / kSpRows), (unsigned)p.Hq, (unsigned)p.B);
    hipLaunchKernelGGL(attn_f32_split<D>, grid, dim3(64 * kSpWaves), SpCfg<D>::FLOATS * 4, s, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_f32(const AttnParams& p, int d, hipStream_t s) {
  if (p.n_q == 0) return hipSuccess;
  return d == 128 ? launch_d<128>(p, s) : launch_d<64>(p, s);
}

}  // namespace sqkv
