// Chunk attention with bf16 inputs on gfx950 matrix cores.
//
// Ring-attention Q&A (aivaro.ru answer 425), section 5: for a query chunk and
// each resident key/value chunk compute the scores Q K^T, the row maximum, the
// exponentials, the row sum and P V, and fold every chunk into the running
// output with the online-softmax rescale.  Sections 2-3: the chunks are met in
// ring order, the rank's own chunk first.  One launch walks all the chunks a
// query block has to see (one chunk for a single ring step), so the running
// (max, sum, output) state stays in registers across chunk boundaries.
//
// Design (gfx950, wave64, v_mfma_f32_32x32x16_bf16):
// * A workgroup of 8 wavefronts (two per SIMD) owns 256 query rows of one
//   (batch, head); each wavefront owns 32 rows and keeps their Q fragments in
//   registers.  Two waves per SIMD let the hardware overlap one wave's LDS
//   reads and softmax arithmetic with the other wave's MFMAs; a wave fits in
//   256 registers.
// * Keys are processed in tiles of 64 (two 32-key MFMA blocks).  Scores are
//   computed transposed, S^T = K Q^T (keys on the MFMA M axis, queries on N):
//   in the 32x32 accumulator layout a lane holds 16 keys of ONE query per
//   block, so the row max and row sum are in-lane reductions plus one
//   v_permlane32_swap with the lane 32 apart.
// * Those accumulators, rounded to bf16, are directly the B operand of
//   O^T = V^T P^T; the key order inside a 16-key contraction step follows the
//   accumulator layout and the V^T operand is read in that order with
//   ds_read_b64_tr_b16 (a 4x16 block of V rows transposed across 16 lanes),
//   so V is stored in LDS exactly as it sits in memory.
// * K and V tiles (64 keys x d) are copied global -> LDS by buffer_load ...
//   lds (16 bytes per lane, no register staging); rows past the end of a
//   chunk fall outside the buffer's range and arrive as zeros.  16-byte chunks
//   of a row are XOR-swizzled so that the K fragment reads (ds_read_b128) and
//   the V transpose reads hit distinct banks.
// * Software pipeline, per wavefront and iteration t:
//       S(t+2) = K(t+2) Q^T      (MFMA)
//       O     += V(t)^T P(t)^T   (MFMA)
//       softmax of S(t+1)        (VALU / transcendental)
//   Score and P V MFMAs alternate one at a time with small groups of softmax
//   work between them, fenced with sched_barrier so the compiler keeps that
//   order; LDS fragments are read a few MFMAs ahead.  K and V tiles go
//   through four LDS stages each and are fetched three iterations before use;
//   the loop is unrolled by four so that every stage address is an
//   instruction immediate.  The DMA loads are inline assembly, their
//   completion counted with explicit s_waitcnt vmcnt, because the compiler
//   would otherwise wait for every in-flight LDS DMA before each LDS read.
//   The loop runs 4k iterations for a visit of T <= 4k+1 tiles: the tiles
//   past T are empty (fully masked, zero-filled) and contribute nothing, and
//   the P V of tile 4k after the loop runs only when T = 4k+1.
// * Softmax runs in base 2, in up to two passes over the visit.  Both take
//   the fp32 score of the bf16 Q and K and multiply it by scale*log2(e) in
//   fp32 right before the exponential, so the exponent carries only fp32
//   rounding (Q itself is never rescaled and re-rounded).  The fast pass
//   takes 2^(score*c) as the weight with no maximum: a multiply and an
//   exponential per score and nothing else.  A workgroup keeps its result
//   when every row sum lies in a range that rules out overflow and harmful
//   underflow; otherwise it runs the exact pass: the running maximum folded
//   into the same FMA, moved (and O rescaled) only when a tile raises it by
//   more than kRescaleLog2; weights are taken against the slightly stale
//   maximum in between, which leaves the normalised result unchanged and
//   bounds weights by 2^kRescaleLog2.  The row sum is taken over the weights
//   as they enter the P V product (rounded to bf16).
// * Masks (causal diagonal, ragged chunk end) are applied only to tiles that
//   need them; tiles entirely in the future of the whole block are never
//   fetched.
#include <type_traits>
#include <utility>

#include "attn_common.h"

namespace sqkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
#define SQKV_LDS __attribute__((address_space(3)))

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kQW = 32;              // query rows per wavefront
constexpr int kBM = kQW * kWaves;    // query rows per workgroup
constexpr int kBN = 64;              // keys per tile
constexpr int kNB = kBN / 32;        // 32-key blocks of the score tile
constexpr int kNCC = kBN / 16;       // 16-key contraction steps of P V per tile
constexpr int kStages = 4;           // LDS stages per tensor (= loop unroll)
constexpr float kRescaleLog2 = 8.0f;

template <int D>
struct Cfg {
  static constexpr int KC = D / 16;                      // 16-wide contraction steps over d
  static constexpr int MD = D / 32;                      // 32-row blocks of d in O^T
  static constexpr int NCH = D / 8;                      // 16-byte chunks per row
  static constexpr int ROWB = D * 2;                     // bytes per row
  static constexpr int TILE = kBN * ROWB;                // bytes per K or V tile
  static constexpr int RPW = 1024 / ROWB;                // rows per wave-wide 1 KiB load
  static constexpr int NLT = TILE / 1024;                // wave-wide loads per tile
  static constexpr int NL = NLT / kWaves;                // loads per wave per tile
  static constexpr int K_LDS = 0;                        // kStages K tiles
  static constexpr int V_LDS = kStages * TILE;           // kStages V tiles
  static constexpr int LDS_BYTES = 2 * kStages * TILE;
  // epilogue staging, one region per wave: its 32 output rows as fp32 at a
  // padded pitch (rows 16 bytes apart in bank terms), then the rows' merge
  // weights; it reuses the K/V stages once the visit's last LDS read is done
  static constexpr int STAGE_PITCH = D * 4 + 16;
  static constexpr int STAGE_WAVE = kQW * STAGE_PITCH + kQW * 4;
  static constexpr int STAGE_BYTES = kWaves * STAGE_WAVE;
  static constexpr int FLAG_OFS = LDS_BYTES > STAGE_BYTES ? LDS_BYTES : STAGE_BYTES;
  static constexpr int LDS_ALLOC = FLAG_OFS + 16;       // + the workgroup's redo flag
  // every wave issues the same number of loads per tile, so that its vmcnt
  // bookkeeping is uniform
  static_assert(NL >= 1 && NLT % kWaves == 0, "tile loads must spread evenly over the waves");
  static_assert(LDS_ALLOC <= 160 * 1024, "LDS");
};

// Position of 16-byte chunk c of tile row r: c ^ swizzle(r).
template <int D>
__device__ __forceinline__ int swz_k(int r) { return r & (Cfg<D>::NCH - 1); }
template <int D>
__device__ __forceinline__ int swz_v(int r) {
  // rows r..r+3 of a transpose read touch chunk pairs {c, c+1}: these four
  // masks send the 8 (or 16, for four consecutive chunks) reads to distinct
  // bank groups
  const int f = (r & 3) == 0 ? 0 : (r & 3) == 1 ? 6 : (r & 3) == 2 ? 12 : 10;
  return f & (Cfg<D>::NCH - 1);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

// Max / sum with the lane 32 apart (the other half of a query's keys):
// v_permlane32_swap of x with itself yields both halves in every lane.
__device__ __forceinline__ float max_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float sum_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Keeps a value's computation where it is written: the compiler may not sink
// it past this point (e.g. into the next loop iteration), which would undo
// the hand interleaving of VALU work with the MFMAs.
template <typename T>
__device__ __forceinline__ void pin(T& x) { asm volatile("" : "+v"(x)); }

// LDS reads take pointers derived from the LDS array by in-bounds offsets, so
// that a constant part of the offset folds into the instruction's immediate.
typedef SQKV_LDS unsigned char* lds_ptr;

__device__ __forceinline__ u32x4_t lds_b128(lds_ptr p) {
  return *reinterpret_cast<SQKV_LDS const u32x4_t*>(p);
}

__device__ __forceinline__ i16x4_t lds_tr16(lds_ptr p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<SQKV_LDS i16x4_t*>(p));
}

__device__ __forceinline__ i32x4_t buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  i32x4_t r;
  r[0] = (int)(uint32_t)b;
  r[1] = (int)(uint32_t)(b >> 32);   // stride 0: a raw byte range
  r[2] = (int)bytes;                 // num_records: bytes past this read as 0
  r[3] = 0x00020000;
  return r;
}

// 16 bytes per lane from the buffer at `voff` into LDS at m0 + 16 * lane.
__device__ __forceinline__ void dma16(uint32_t voff, i32x4_t rsrc, uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" :: "v"(voff), "s"(rsrc), "{m0}"(lds) : "memory");
}

// s_waitcnt immediate (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8).
constexpr unsigned waitcnt_imm(int vm, int lgkm) {
  return (unsigned)((vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8));
}
constexpr unsigned kWaitVm0 = waitcnt_imm(0, 15);
constexpr unsigned kWaitLgkm0 = waitcnt_imm(63, 0);

// Meet the other wavefronts once every LDS read of this wave has returned:
// after it, LDS that all waves have finished reading may be overwritten.
__device__ __forceinline__ void lds_reads_done_sync() {
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  asm volatile("s_barrier" ::: "memory");
}

// As above, and first wait until at most N of this wave's vector-memory
// operations are in flight: every DMA issued before the last N has landed,
// so after the barrier it is visible in LDS to the whole workgroup.  The
// last L LDS reads of the wave (reads of stages nobody overwrites next) may
// still be in flight.
template <int N, int L = 0>
__device__ __forceinline__ void wait_dma_and_sync() {
  static_assert(N >= 0 && N < 64 && L >= 0 && L < 16, "waitcnt immediate");
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(N, L));
  asm volatile("s_barrier" ::: "memory");
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

// PACKED: the sequence packs several samples (p.seg holds their sorted start
// positions); a query sees only the keys of its own sample.
template <int D, bool PACKED>
__global__ void __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(2, 2)))
attn_bf16_kernel(AttnParams params, int n_qtiles, int n_items) {
  using C = Cfg<D>;
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  // LDS offset of the dynamic allocation (no static LDS in this kernel)
  const uint32_t lds0 = (uint32_t)(size_t)(SQKV_LDS unsigned char*)smem;

  // The grid holds one workgroup per CU and each workgroup walks its items
  // (one (b, h, q-tile) visit each) in turn: workgroup g takes items g,
  // 2G-1-g, 2G+g, 4G-1-g, ... of the G-wide rounds, so that in a list issued
  // heaviest first a heavy item pairs with a light one.  A visit's output
  // stores then drain while the next visit sets up and loads its Q and
  // first tiles, and the launch pays for one workgroup start per CU rather
  // than one per item.
  const int G = gridDim.x;
  for (int round = 0;; ++round) {
  const int item = round * G + ((round & 1) ? G - 1 - (int)blockIdx.x : (int)blockIdx.x);
  if (item >= n_items) break;
  // The parameters are read from the kernel argument segment through a
  // pointer the compiler cannot see through, once per visit: otherwise it
  // keeps every one of them in registers across all visits and spills.
  typedef const __attribute__((address_space(4))) AttnParams KernArgParams;   // scalar-loadable
  KernArgParams* pk_visit = (KernArgParams*)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(pk_visit));
  KernArgParams& p = *pk_visit;
  // (likewise the lane's constants, recomputed per visit rather than held)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int a16 = lane & 15;

  // Item -> (b, h, q-tile).  Item i runs on XCD i % 8 in even rounds and on
  // XCD 7 - i % 8 in odd ones (workgroups are dealt round-robin to the 8
  // XCDs, each with its own L2); the grouping below only needs the items of
  // one round that share i % 8 to share an XCD.  When every workgroup has about the same work
  // (no mask, or a causal visit of several chunks, where the diagonal chunk
  // is a small part) the linear id is remapped so that each XCD walks a
  // contiguous range of (b, h, q-tile) with the q-tiles of one head adjacent,
  // and the workgroups streaming one head's K/V run together on one XCD and
  // share its L2 (causal: heaviest q-tile of the head first).  A causal visit
  // of one chunk grows with the q-tile: heads vary fastest (every XCD gets a
  // mix) and the q-tiles are issued heaviest first.  Packed samples keep that
  // order too (measured: the remap is ~20% slower with 2k-token samples).  In
  // that order the `group` query heads that share a key/value head (GQA) are
  // dealt to one XCD at consecutive slots, so that they stream the same key /
  // value tiles through its L2 together: ids are permuted inside every run of
  // 8*group (a tail shorter than that keeps its order).
  const int BH = p.B * p.Hq;
  int bh, qt;
  if (p.causal && (p.nseg < 2 || PACKED)) {
    const int span = 8 * p.group;
    int lid = item;
    if (lid < (n_items / span) * span) {
      const int unit = (lid / span) * 8 + (lid & 7);   // (q-tile, key/value head), on XCD lid % 8
      lid = unit * p.group + (lid >> 3) % p.group;
    }
    const int qt_rank = lid / BH;
    bh = lid - qt_rank * BH;
    qt = n_qtiles - 1 - qt_rank;
  } else {
    constexpr int kXcds = 8;
    const int per = n_items / kXcds, rem = n_items % kXcds;
    const int xcd = item % kXcds;
    const int logical = xcd * per + min(xcd, rem) + item / kXcds;
    bh = logical / n_qtiles;
    qt = logical - bh * n_qtiles;
    if (p.causal) qt = n_qtiles - 1 - qt;
  }
  const int b = bh / p.Hq;
  const int h = bh - b * p.Hq;
  const int hk = h / p.group;

  const int q0 = qt * kBM;                 // first row of the workgroup
  const int qw0 = q0 + wave * kQW;         // first row of this wavefront

  const uint16_t* qg = static_cast<const uint16_t*>(p.q) + b * p.q_sb + h * p.q_sh;
  const unsigned char* kg = reinterpret_cast<const unsigned char*>(
      static_cast<const uint16_t*>(p.k) + b * p.k_sb + hk * p.k_sh);
  const unsigned char* vg = reinterpret_cast<const unsigned char*>(
      static_cast<const uint16_t*>(p.v) + b * p.v_sb + hk * p.v_sh);
  const int k_snb = (int)(p.k_sn * 2), v_snb = (int)(p.v_sn * 2);   // row strides in bytes
  const int64_t k_csb = p.k_cs * 2, v_csb = p.v_cs * 2;             // chunk strides in bytes

  // ---- Q fragments (B operand of S^T = K Q^T) -------------------------------
  // lane holds Q[row = qw0 + l32][16*kc + 8*hi .. +7]
  u32x4_t qf[C::KC];
  auto load_q = [&]() {
    const int row = qw0 + l32;
    const bool ok = row < p.n_q;
    const uint16_t* src = qg + (int64_t)(ok ? row : 0) * p.q_sn + 8 * hi;
#pragma unroll
    for (int kc = 0; kc < C::KC; ++kc) {
      const u32x4_t z = {0u, 0u, 0u, 0u};
      qf[kc] = ok ? *reinterpret_cast<const u32x4_t*>(src + 16 * kc) : z;
    }
    // No wait here: the Q loads are older than the visit's first K/V DMA,
    // so the first DMA wait (vector memory completes in order) also covers
    // them, and the two latencies overlap (measured: ~2 us per visit).
  };
  load_q();

  // ---- per-lane LDS offsets ---------------------------------------------------
  // K fragment (A operand of S^T): row l32, 16-byte chunk 2*kc + hi
  const lds_ptr lds = (lds_ptr)smem;
  lds_ptr kofs[C::KC];
#pragma unroll
  for (int kc = 0; kc < C::KC; ++kc)
    kofs[kc] = lds + C::K_LDS + l32 * C::ROWB + (((2 * kc + hi) ^ swz_k<D>(l32)) * 16);
  // V^T fragment via transpose reads: the 16-lane group g = lane/16 reads key
  // rows 16*cc + 4*hi + {0..3} (and +8) at d columns 32*md + 16*(g&1) + {0..15};
  // group lane a16 supplies row a16/4, columns 4*(a16%4) .. +3
  lds_ptr vofs[C::MD];
#pragma unroll
  for (int md = 0; md < C::MD; ++md) {
    const int r = 4 * hi + (a16 >> 2);
    const int c = 4 * md + 2 * ((lane >> 4) & 1) + ((a16 & 3) >> 1);
    vofs[md] = lds + C::V_LDS + r * C::ROWB + ((c ^ swz_v<D>(r)) * 16) + (a16 & 1) * 8;
  }
  // DMA: wave-wide load i of a tile fills rows r0 = (i*kWaves + wave)*RPW ..
  // r0 + RPW - 1; the lane fills row r0 + lane/NCH at chunk position lane%NCH,
  // so it reads source chunk (lane%NCH) ^ swizzle(row).  dko/dvo are the
  // lanes' byte offsets inside a tile.
  uint32_t dko[C::NL], dvo[C::NL];
#pragma unroll
  for (int i = 0; i < C::NL; ++i) {
    const int r = (i * kWaves + wave) * C::RPW + lane / C::NCH;
    dko[i] = (uint32_t)(r * k_snb) + (((lane % C::NCH) ^ swz_k<D>(r)) * 16);
    dvo[i] = (uint32_t)(r * v_snb) + (((lane % C::NCH) ^ swz_v<D>(r)) * 16);
  }

  // ---- scores and masks --------------------------------------------------------
  // S^T tile: 64 keys (M, two 32-key blocks nb) x the wave's 32 queries (N);
  // element j of block nb holds key 32*nb + 8*(j/4) + 4*hi + j%4 of query
  // qw0 + l32.  Score MFMA m covers block nb = m % 2, contraction step
  // kc = m / 2 (the two blocks' accumulation chains alternate).
  struct STile {
    f32x16_t b[kNB];
  };
  auto kfrag = [&](int m, auto stage) {
    return lds_b128(kofs[m / kNB] + decltype(stage)::value * C::TILE + (m % kNB) * 32 * C::ROWB);
  };
  auto mfma_s = [&](STile& s, u32x4_t kf, int m) {
    const f32x16_t z = {};
    const int nb = m % kNB, kc = m / kNB;
    s.b[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kf), as_bf16x8(qf[kc]), kc == 0 ? z : s.b[nb], 0, 0, 0);
  };
  auto scores = [&](STile& s, auto stage) {
#pragma unroll
    for (int m = 0; m < kNB * C::KC; ++m) mfma_s(s, kfrag(m, stage), m);
  };

  // Causal masks only touch tiles of the first chunk of the visit (the rank's
  // own): those at or after tile tt_mask can hold a key after this wave's
  // first query.
  // qrel: position of this wave's first query relative to the own chunk's
  // first key (clamped: beyond +-2^30 no own tile is on the diagonal)
  const int64_t kpos_own = p.k_pos0 + (int64_t)p.rank * p.k_posstride;
  const int qrel = (int)min((int64_t)(1 << 30), max((int64_t)-(1 << 30), p.q_pos0 + qw0 - kpos_own));
  const int tt_mask = max(0, (qrel + 1) / kBN);

  // Packed samples: the sample of a query starts at the largest sample start
  // <= its position; lo_row for this lane's row, lo_blk for the block's first
  // row (the earliest key any row of the block can see), lo_wmax for the
  // wave's last row (tiles starting before it need the sample mask).
  int64_t lo_row = 0, lo_blk = 0, lo_wmax = 0;
  if constexpr (PACKED) {
    auto sample_start = [&](int64_t pos) {
      int a = 0, e = p.n_seg;
      while (e - a > 1) {
        const int m = (a + e) >> 1;
        if (p.seg[m] <= pos) a = m;
        else e = m;
      }
      return p.seg[a];
    };
    lo_row = sample_start(p.q_pos0 + min(qw0 + l32, p.n_q - 1));
    lo_blk = sample_start(p.q_pos0 + q0);
    const uint64_t u = (uint64_t)lo_row;
    lo_wmax = (int64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(u >> 32), 31) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 31));
  }

  // The visit: chunks in ring order, and in each chunk the tiles holding keys
  // visible to at least one of the block's query rows.  Only the first chunk
  // (the rank's own, or the single chunk of one ring step) can be cut short
  // by the causal mask; every later chunk of a ring lies entirely in the past
  // of the rank's queries and is visited whole.  Tile g < ntl0 is tile g of
  // the own chunk.
  int64_t lim0 = p.n_k;   // visible keys of the own chunk for this block
  if (p.causal) {
    const int64_t qpos_last = p.q_pos0 + min(q0 + kBM, p.n_q) - 1;
    lim0 = max((int64_t)0, min(lim0, qpos_last - kpos_own + 1));
  }
  const int ntl0 = (int)((lim0 + kBN - 1) / kBN);
  const int ntl_full = (p.n_k + kBN - 1) / kBN;
  // Packed samples narrow the visit to keys from lo_blk on: own-chunk tiles
  // from t0_own, chunks down to the one holding lo_blk (nseg_v of them), and
  // in that last chunk the tiles from t_lo.
  int t0_own = 0, nseg_v = p.nseg, t_lo = 0;
  if constexpr (PACKED) {
    if (lo_blk >= kpos_own || p.k_posstride == 0) {
      t0_own = (int)min((int64_t)ntl0, max((int64_t)0, (lo_blk - kpos_own) / kBN));
      nseg_v = 1;
    } else {
      const int64_t jl = max((int64_t)0, (lo_blk - p.k_pos0) / p.k_posstride);
      nseg_v = min(p.nseg, p.rank - (int)jl + 1);
      t_lo = (int)min((int64_t)ntl_full, max((int64_t)0, (lo_blk - p.k_pos0 - jl * p.k_posstride) / kBN));
    }
  }
  const int T = ntl0 - t0_own <= 0 ? 0 : (ntl0 - t0_own) + (nseg_v >= 2 ? (nseg_v - 1) * ntl_full - t_lo : 0);

  // Tile g of the visit with nv valid keys starting at key position kp:
  // own-chunk tiles from tt_mask on are masked on the causal diagonal, short
  // tiles past their last key; with packed samples, tiles reaching past the
  // wave's first query or starting before its last row's sample are masked
  // key by key against each row's [sample start, position].
  const int64_t qpos_w0 = p.q_pos0 + qw0;
  auto mask = [&](STile& s, int g, int nv, int64_t kp) {
    if constexpr (PACKED) {
      if (!(nv < kBN || kp + kBN - 1 > qpos_w0 || kp < lo_wmax)) return;
      const int64_t last = min(p.q_pos0 + qw0 + l32 - kp, (int64_t)nv - 1);   // last visible key
      const int64_t first = lo_row - kp;                                       // first visible key
      const int lk = (int)max((int64_t)-1, min(last, (int64_t)kBN)) - 4 * hi;
      const int fk = (int)max((int64_t)0, min(first, (int64_t)kBN + 1)) - 4 * hi;
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int u = 32 * nb + 8 * (j >> 2) + (j & 3);
          if (u > lk || u < fk) s.b[nb][j] = kNegInf;
        }
      return;
    }
    const bool diag = p.causal && g >= tt_mask && g < ntl0;
    if (!(nv < kBN || diag)) return;
    int64_t rel = (int64_t)qrel + l32 - (int64_t)g * kBN;   // last visible key of the tile
    if (!diag || rel > kBN) rel = kBN;
    // key u = (32*nb + 8*(j/4) + j%4) + 4*hi is masked when u > lastk; the
    // lane term moves to the right so that the left side is an immediate
    const int lk = (int)min(rel, (int64_t)nv - 1) - 4 * hi;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (32 * nb + 8 * (j >> 2) + (j & 3) > lk) s.b[nb][j] = kNegInf;
  };

  // ---- online softmax state --------------------------------------------------
  f32x16_t oacc[C::MD];
#pragma unroll
  for (int md = 0; md < C::MD; ++md) oacc[md] = (f32x16_t){};
  float m_run = kNegInf;   // running max, base-2 units
  float l_run = 0.f;       // this lane's half of the row sum: l_run + l_run2
  float l_run2 = 0.f;
  float alpha = 1.f;
  float mpart[4], pmax = kNegInf, mxs = kNegInf, mneg = 0.f;
  bool upd = false, resc = false;
  const float c = p.scale_log2;

  // ---- the softmax of one tile in small work groups ------------------------------
  // A lane holds 32 scores of its query: x(e) = block e / 16, element e % 16.
  // P columns cc (16 keys of the P V contraction step cc) are x(8*cc) ..
  // x(8*cc + 7).  The groups are spread over the MFMAs of the next tiles;
  // none is a long dependency chain (the wave issues in order).
  // The fast pass (FAST) takes 2^(score * c) with no maximum and no
  // subtraction; only the exponential groups remain.
  // Fast pass: score e of the lane's 32 gets its multiply and exponential on
  // its own, so that they spread one per MFMA slot (measured: 1.5% faster
  // than groups of four).
  constexpr int kFastGroups = kNB * 16;
  auto sm_fast = [&](STile& v, int e) {
    v.b[e >> 4][e & 15] = __builtin_amdgcn_exp2f(v.b[e >> 4][e & 15] * c);
  };
  auto sm_group = [&](STile& v, int g) {
    auto x = [&](int e) { return v.b[e >> 4][e & 15]; };
    if (g == 0) {                      // partial maxima over x(0..11)
#pragma unroll
      for (int k = 0; k < 4; ++k) mpart[k] = __builtin_fmaxf(__builtin_fmaxf(x(3 * k), x(3 * k + 1)), x(3 * k + 2));
    } else if (g == 1 || g == 2) {     // x(12..19), x(20..27)
      const int e0 = 12 + 8 * (g - 1);
#pragma unroll
      for (int k = 0; k < 4; ++k)
        mpart[k] = __builtin_fmaxf(__builtin_fmaxf(x(e0 + 2 * k), x(e0 + 2 * k + 1)), mpart[k]);
    } else if (g == 3) {               // x(28..31) and the tree's root
      mpart[0] = __builtin_fmaxf(__builtin_fmaxf(x(28), x(29)), mpart[0]);
      mpart[1] = __builtin_fmaxf(__builtin_fmaxf(x(30), x(31)), mpart[1]);
      pmax = __builtin_fmaxf(__builtin_fmaxf(mpart[0], mpart[1]), __builtin_fmaxf(mpart[2], mpart[3]));
    } else if (g == 4) {               // the other half of the keys; compare
      mxs = max_half(pmax) * c;
      upd = mxs > m_run + kRescaleLog2;
    } else if (g == 5) {               // move the running max if any lane needs it
      const bool u = __any(upd);
      const float mn = u ? __builtin_fmaxf(m_run, mxs) : m_run;
      alpha = (mn == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - mn);
      l_run *= alpha;                  // the packs add this tile's weights
      l_run2 *= alpha;
      resc = resc || u;
      m_run = mn;
      mneg = (mn == kNegInf) ? 0.f : -mn;
    } else {                           // 4 exponentials
      const int e0 = 4 * (g - 6);
#pragma unroll
      for (int e = e0; e < e0 + 4; ++e) v.b[e >> 4][e & 15] = __builtin_amdgcn_exp2f(fmaf(x(e), c, mneg));
    }
  };
  constexpr int kGroups = 6 + 8;

  // bf16 weights (B operand of O^T = V^T P^T) of one tile: the P V MFMAs of
  // iteration t read tile t's columns while tile t+1's are packed behind them.
  // The row sum is accumulated over the packed weights, two per
  // v_dot2_f32_bf16 against (1, 1), alternately into l_run and l_run2 (two
  // chains of half the length: measured ~0.5% faster).  (`ones` sits in a
  // register so that the VOP3 form takes the accumulator directly.)
  u32x4_t pf[kNCC];
  bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  asm volatile("" : "+v"(ones));
  auto pack = [&](const STile& v, int cc) {
    const int j0 = 8 * (cc & 1);
    const f32x16_t& vb = v.b[cc >> 1];
    u32x4_t& w4 = pf[cc];
#pragma unroll
    for (int w = 0; w < 4; ++w) w4[w] = pack_bf16x2(vb[j0 + 2 * w], vb[j0 + 2 * w + 1]);
    pin(w4);
    // (pairs taken with shufflevector: bit-casting single 32-bit elements of
    // w4 to bf16x2 was miscompiled into reads of element 0 only)
    const bf16x8_t p8 = as_bf16x8(w4);
    l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 0, 1), ones, l_run, false);
    l_run2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 2, 3), ones, l_run2, false);
    l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 4, 5), ones, l_run, false);
    l_run2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p8, p8, 6, 7), ones, l_run2, false);
  };
  // O *= alpha when the running max moved (rare).
  auto rescale = [&]() {
#pragma unroll
    for (int md = 0; md < C::MD; ++md) oacc[md] *= alpha;
  };

  // O^T[d][query] += V^T[d][key] P^T[key][query]; contraction step cc covers
  // keys 16*cc + {4*hi .. 4*hi+3} and 16*cc + 8 + {4*hi .. 4*hi+3}
  auto vfrag = [&](int cc, int md, auto stage) {
    const lds_ptr a = vofs[md] + decltype(stage)::value * C::TILE + (16 * cc) * C::ROWB;
    const i16x4_t lo = lds_tr16(a);
    const i16x4_t up = lds_tr16(a + 8 * C::ROWB);
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  auto mfma_pv = [&](bf16x8_t vf, int cc, int md) {
    oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, as_bf16x8(pf[cc]), oacc[md], 0, 0, 0);
  };
  auto pv = [&](auto stage) {
#pragma unroll
    for (int cc = 0; cc < kNCC; ++cc)
#pragma unroll
      for (int md = 0; md < C::MD; ++md) mfma_pv(vfrag(cc, md, stage), cc, md);
  };

  // ---- K/V tile DMA -----------------------------------------------------------
  // One walker per tensor, in scalar registers, steps through the tiles of the
  // visit; crossing into the next chunk (rare) reloads the chunk base, and
  // past the last chunk the tiles are empty.  Chunk j of the pool starts
  // j*csb bytes after chunk 0; visit s reads chunk (rank - s) mod P.
  struct DmaWalk {
    const unsigned char* ptr;   // first row of the current tile
    int rows;                   // rows of the current chunk from this tile on
    int tl;                     // tiles of the current chunk from this tile on
    int j;                      // current chunk
    int left;                   // chunks of the visit after the current one
    int64_t kp;                 // key position of the current tile (packed samples only)
  };
  auto walk_start = [&](const unsigned char* hbase, int64_t csb, int snb) {
    return DmaWalk{hbase + (int64_t)p.rank * csb + (int64_t)t0_own * kBN * snb, (int)lim0 - t0_own * kBN,
                   ntl0 - t0_own, p.rank, nseg_v - 1, kpos_own + (int64_t)t0_own * kBN};
  };
  auto walk_step = [&](DmaWalk& w, const unsigned char* hbase, int64_t csb, int snb) {
    w.ptr += kBN * snb;
    w.rows -= kBN;
    if constexpr (PACKED) w.kp += kBN;
    if (--w.tl == 0) {
      if (w.left > 0) {
        w.left -= 1;
        w.j = (w.j == 0 ? p.P : w.j) - 1;
        w.ptr = hbase + (int64_t)w.j * csb;
        w.rows = p.n_k;
        w.tl = ntl_full;
        if constexpr (PACKED) {
          w.kp = p.k_pos0 + (int64_t)w.j * p.k_posstride;
          if (w.left == 0) {               // the last chunk starts at tile t_lo
            w.ptr += (int64_t)t_lo * kBN * snb;
            w.rows -= t_lo * kBN;
            w.tl -= t_lo;
            w.kp += (int64_t)t_lo * kBN;
          }
        }
      } else {
        w.rows = -(1 << 30);   // the visit is over
      }
    }
  };
  // One buffer resource spans the tile's valid rows: rows past the end of the
  // chunk (and every row of an empty tile) read as zeros.  Returns the tile's
  // valid rows.
  const uint32_t m0_wave = (uint32_t)(wave * C::RPW * C::ROWB);   // this wave's rows of a tile
  auto issue = [&](const DmaWalk& w, int snb, uint32_t stage, const uint32_t* voff) {
    // (readfirstlane: the value is uniform; it keeps the clamp on the scalar
    // unit, where the buffer resource has to live)
    const int nv = __builtin_amdgcn_readfirstlane(min(max(w.rows, 0), kBN));
    const i32x4_t rs = buffer_rsrc(w.ptr, (uint32_t)nv * (uint32_t)snb);
    // (the laundering keeps the compiler from precomputing every stage's
    // destination and holding them all in scalar registers)
    uint32_t mw = m0_wave;
    asm volatile("" : "+s"(mw));
#pragma unroll
    for (int i = 0; i < C::NL; ++i) dma16(voff[i], rs, stage + mw + i * kWaves * C::RPW * C::ROWB);
    return nv;
  };
  DmaWalk wk, wv;
  int64_t kp_issued = 0;   // key position of the last V tile issued (packed samples)
  auto issue_k = [&](int stage) {
    issue(wk, k_snb, lds0 + C::K_LDS + stage * C::TILE, dko);
    walk_step(wk, kg, k_csb, k_snb);
  };
  auto issue_v = [&](int stage) {
    const int nv = issue(wv, v_snb, lds0 + C::V_LDS + stage * C::TILE, dvo);
    if constexpr (PACKED) kp_issued = wv.kp;
    walk_step(wv, vg, v_csb, v_snb);
    return nv;
  };

  // ---- main loop -----------------------------------------------------------------

  // One loop iteration issues 2*NB*KC MFMAs in slots: even slot 2m is score
  // MFMA m, odd slot 2m+1 is P V MFMA m (columns cc = m / MD, d-block
  // md = m % MD).  K fragment m is first needed at slot 2m, V fragment m at
  // slot 2m + 1; both are read kLead slots earlier (the first ones in the last
  // slots of the previous iteration).
  constexpr int kMF = kNB * C::KC;        // MFMAs of each kind per tile
  static_assert(kMF == kNCC * C::MD, "score and P V MFMA counts");
  constexpr int kSlots = 2 * kMF;
  constexpr int kLead = 4;
  constexpr int kPre = kLead / 2;         // fragments of each kind read ahead
  static_assert(kLead % 2 == 0, "reads alternate K, V: an even lead keeps both kinds kPre ahead");
  constexpr int kPreLds = 3 * kPre;       // their LDS instructions (K: 1, V: 2)
  // The iteration's K and V DMA go out a few slots into it rather than all
  // right after the barrier, where the eight waves would issue them at once
  // (measured: ~1% faster).  Any slot is safe: the stages they overwrite were
  // last read in the previous iteration, before its barrier.
  constexpr int kDmaSlotK = kSlots / 8, kDmaSlotV = kSlots / 4 + 2;
  // softmax group g at slot kSlotOfGroup(g).  Pack cc overwrites the weights
  // of columns cc, so it comes after the exponentials of those columns (groups
  // 6 + 2*cc, 7 + 2*cc) and after the last P V MFMA of this iteration that
  // reads them (slot 2*MD*(cc+1) - 1); a pack that falls past the last slot
  // runs after the slot loop.  The fast pass has only the exponentials: one
  // score per slot, in order.
  constexpr auto kSlotOfGroup = [](int g) { return (g * kSlots) / (kGroups + kNCC); };
  constexpr auto kSlotOfFast = [](int e) { return (e * kSlots) / kFastGroups; };
  static_assert(kSlotOfFast(kFastGroups - 1) < kSlots && kSlotOfGroup(kGroups - 1) < kSlots,
                "every softmax group must fall inside the slot loop");
  constexpr auto kSlotOfPack = [=](int cc, bool fast) {
    const int after_exp = fast ? kSlotOfFast(8 * cc + 7) + 1 : kSlotOfGroup(7 + 2 * cc) + 1;
    const int after_pv = 2 * C::MD * (cc + 1);
    return after_exp > after_pv ? after_exp : after_pv;
  };
  // One pass over the visit.  The state starts afresh: the fast pass with the
  // reference exponent fixed at 0, the exact pass with the running maximum.
  auto run_pass = [&](auto fast) {
    constexpr bool FAST = decltype(fast)::value;
#pragma unroll
    for (int md = 0; md < C::MD; ++md) oacc[md] = (f32x16_t){};
    m_run = FAST ? 0.f : kNegInf;
    l_run = 0.f;
    l_run2 = 0.f;
    alpha = 1.f;
    mneg = 0.f;
    resc = false;
    wk = walk_start(kg, k_csb, k_snb);
    wv = walk_start(vg, v_csb, v_snb);
    kp_issued = 0;
    STile sa, sb;
    issue_k(0);                          // K(0) .. K(3) into stages 0..3
    issue_k(1);
    issue_k(2);
    const int nv0 = issue_v(0);          // V(0), V(1)
    const int64_t kp0 = kp_issued;
    issue_k(3);
    const int nv1 = issue_v(1);
    const int64_t kp1 = kp_issued;
    wait_dma_and_sync<4 * C::NL>();      // K(0), K(1) landed
    scores(sa, Step<0>{});
    scores(sb, Step<1>{});
    mask(sa, 0, nv0, kp0);
    mask(sb, 1, nv1, kp1);
    if constexpr (FAST) {
#pragma unroll
      for (int j = 0; j < kFastGroups; ++j) sm_fast(sa, j);
    } else {
#pragma unroll
      for (int g = 0; g < kGroups; ++g) sm_group(sa, g);     // O is still zero: no rescale
    }
#pragma unroll
    for (int cc = 0; cc < kNCC; ++cc) pack(sa, cc);
    pin(l_run);
    pin(l_run2);
    lds_reads_done_sync();               // K stage 0 is free
    issue_k(0);                          // K(4)
    int nv_next = issue_v(2);            // V(2); valid keys of the tile masked next
    int64_t kp_next = kp_issued;
    int g = 2;                           // tile masked at the end of the current iteration

    u32x4_t kfr[kMF];
    bf16x8_t vfr[kMF];
    auto read_k = [&](int f, auto stage) { kfr[f] = kfrag(f, stage); };
    auto read_v = [&](int v, auto stage) { vfr[v] = vfrag(v / C::MD, v % C::MD, stage); };
    // first fragments of iteration 0 (K(2) in stage 2, V(0) in stage 0); K(3)
    // and V(1), which iteration 0 reads ahead, have landed as well
    wait_dma_and_sync<2 * C::NL>();
#pragma unroll
    for (int f = 0; f < kPre; ++f) {
      read_k(f, Step<2>{});
      read_v(f, Step<0>{});
    }

    // Iteration t = 4k + R: K(t+5) and V(t+3) are fetched; S(t+2) computed
    // into `nx`; O += V(t) P(t); S(t+1) in `cu` goes through the softmax into
    // P(t+1).  Its last slots read the first fragments of K(t+3) and V(t+1)
    // (made visible by the previous iteration's barrier); it ends by waiting
    // for K(t+4), V(t+2), which iteration t+1 reads ahead.
    auto body = [&](auto R, STile& nx, STile& cu) {
      constexpr int r = decltype(R)::value;
      constexpr int ks = (r + 2) % kStages, vs = r;
      const int nv_mask = nv_next;         // tile t+2
      const int64_t kp_mask = kp_next;
      resc = false;
      static_for<kSlots>([&](auto I) {
        constexpr int i = decltype(I)::value;
        if constexpr (i == kDmaSlotK) issue_k((r + 5) % kStages);          // K(t+5)
        if constexpr (i == kDmaSlotV) {
          nv_next = issue_v((r + 3) % kStages);   // V(t+3)
          kp_next = kp_issued;
        }
        constexpr int ahead = i + kLead, fa = ahead >> 1;   // fragment needed kLead slots from now
        if constexpr ((ahead & 1) == 0) {
          if constexpr (fa >= kMF) read_k(fa - kMF, Step<(r + 3) % kStages>{});
          else if constexpr (fa >= kPre) read_k(fa, Step<ks>{});
        } else {
          if constexpr (fa >= kMF) read_v(fa - kMF, Step<(r + 1) % kStages>{});
          else if constexpr (fa >= kPre) read_v(fa, Step<vs>{});
        }
        constexpr int m = i >> 1;
        if constexpr ((i & 1) == 0) mfma_s(nx, kfr[m], m);
        else mfma_pv(vfr[m], m / C::MD, m % C::MD);
        if constexpr (FAST) {
          static_for<kFastGroups>([&](auto J) {
            if constexpr (kSlotOfFast(decltype(J)::value) == i) sm_fast(cu, decltype(J)::value);
          });
        } else {
          static_for<kGroups>([&](auto G) {
            if constexpr (kSlotOfGroup(decltype(G)::value) == i) sm_group(cu, decltype(G)::value);
          });
        }
        static_for<kNCC>([&](auto Q) {
          if constexpr (kSlotOfPack(decltype(Q)::value, FAST) == i) pack(cu, decltype(Q)::value);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
      static_for<kNCC>([&](auto Q) {
        if constexpr (kSlotOfPack(decltype(Q)::value, FAST) >= kSlots) pack(cu, decltype(Q)::value);
      });
      pin(l_run);
      pin(l_run2);
      if constexpr (!FAST)
        if (resc) rescale();
      mask(nx, g, nv_mask, kp_mask);
      g += 1;
      wait_dma_and_sync<2 * C::NL, kPreLds>();   // K(t+4), V(t+2) landed
    };
    // T - 1 iterations, padded to a multiple of 4 with empty tiles; iteration
    // t adds tile t's P V, so the last tile's P V after the loop is needed
    // only when no padding was added (otherwise it adds zeros)
    const int iters = (T - 1 + 3) & ~3;
    for (int t = 0; t < iters; t += 4) {
      body(Step<0>{}, sa, sb);
      body(Step<1>{}, sb, sa);
      body(Step<2>{}, sa, sb);
      body(Step<3>{}, sb, sa);
    }
    if (iters == T - 1) pv(Step<0>{});   // V of the last tile landed above
    };

  // The fast pass (weights 2^(score * c) with no maximum subtracted) is kept
  // when every row's sum lies in [2^-24, 2^40] and every accumulator is
  // finite: then no weight overflowed (each is at most the sum) and the ones
  // that underflowed (below 2^-126) are under 2^-100 of the sum.  Its weights
  // are then the exact pass's up to the fp32 rounding of the exponent and a
  // factor 2^m common to a row, which the normalisation cancels.  Otherwise the whole workgroup (its waves
  // share the LDS pipeline) runs the exact pass with the running maximum.
  volatile int* redo_flag = reinterpret_cast<volatile int*>(smem + C::FLAG_OFS);
  if (threadIdx.x == 0) *redo_flag = 0;
  if (T > 0) {
    run_pass(std::true_type{});
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    const float lt = sum_half(l_run + l_run2);
    bool ok = (qw0 + l32 >= p.n_q) || (lt >= 0x1p-24f && lt <= 0x1p40f);
#pragma unroll
    for (int md = 0; md < C::MD; ++md)
#pragma unroll
      for (int j = 0; j < 16; ++j) ok &= __builtin_isfinite(oacc[md][j]);
    if (__any(!ok) && lane == 0) *redo_flag = 1;
    lds_reads_done_sync();   // (the first barrier of the pass ordered the clearing before this)
    if (*redo_flag != 0) {
      run_pass(std::false_type{});
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      lds_reads_done_sync();
    }
  }
  // No DMA is in flight and no wave reads the K/V stages any more: the
  // epilogue may stage its rows there.
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  // ---- epilogue: normalise, merge into the running (O, lse), store ------------
  // The output parameters are read from the kernel argument segment here,
  // through a pointer the compiler cannot see through: otherwise it loads
  // them early and keeps ~20 scalar registers live across the loop.
  // A lane holds 64 of its row's d values in groups of four, so storing from
  // the accumulators writes 8 or 16 bytes at a time scattered over 32 rows
  // (measured: ~1 us per visit slower than the staging below).  Instead
  // each wave writes its rows, normalised, as fp32 into its own LDS region,
  // reads them back in row order and stores whole rows: D/4 lanes per row,
  // 4 values each, merged there with the running (o_in) rows when present.
  {
    // (in the constant address space: a generic pointer would let every
    // output store alias the parameters, and the compiler then waits for each
    // store to complete before reading them again)
    KernArgParams* pk = (KernArgParams*)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(pk));
    KernArgParams& pe = *pk;
    const int row = qw0 + l32;
    const float lt = sum_half(l_run + l_run2);
    const int64_t bh_row = (int64_t)b * pe.Hq + h;
    float wi = 0.f, f = 0.f;
    if (row < pe.n_q) {
      const float lse_j = (lt > 0.f) ? (m_run + log2f(lt)) * kLn2 : kNegInf;
      const float inv = (lt > 0.f) ? 1.f / lt : 0.f;
      float wj = 1.f, lse = lse_j;
      if (pe.o_in != nullptr) lse = lse_merge_weights(pe.lse_in[bh_row * pe.lse_in_hs + row], lse_j, wi, wj);
      f = wj * inv;
      if (hi == 0) pe.lse_out[bh_row * pe.lse_out_hs + row] = lse;
    }
    const lds_ptr stage = lds + wave * C::STAGE_WAVE;
#pragma unroll
    for (int md = 0; md < C::MD; ++md)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * md + 8 * g + 4 * hi;
        const f32x4_t y = {oacc[md][4 * g] * f, oacc[md][4 * g + 1] * f, oacc[md][4 * g + 2] * f,
                           oacc[md][4 * g + 3] * f};
        *reinterpret_cast<SQKV_LDS f32x4_t*>(stage + l32 * C::STAGE_PITCH + d0 * 4) = y;
      }
    if (hi == 0) *reinterpret_cast<SQKV_LDS float*>(stage + kQW * C::STAGE_PITCH + l32 * 4) = wi;
    // the wave's own LDS writes, complete before its lanes read each other's
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // D/4 lanes per row, 256/D rows per pass
    constexpr int kLanesPerRow = D / 4, kRowsPerPass = 64 / kLanesPerRow;
    static_assert(kQW % kRowsPerPass == 0, "whole passes over the wave's rows");
    const int c = 4 * (lane % kLanesPerRow);    // this lane's 4 values of a row
    const int r0 = lane / kLanesPerRow;
    // element offsets of (row qw0 + r0, column c) and the step to the next pass
    const int64_t obase = b * pe.oo_sb + h * pe.oo_sh + (int64_t)(qw0 + r0) * pe.oo_sn + c;
    const int64_t ibase = b * pe.oi_sb + h * pe.oi_sh + (int64_t)(qw0 + r0) * pe.oi_sn + c;
    const int64_t ostep = kRowsPerPass * pe.oo_sn, istep = kRowsPerPass * pe.oi_sn;
    const bool bf16_out = pe.out_dtype == kBF16;
    const int n_q = pe.n_q, acc_dtype = pe.acc_dtype;
    const void* const o_in = pe.o_in;
    void* const o_out = pe.o_out;
#pragma unroll 4
    for (int it = 0; it < kQW / kRowsPerPass; ++it) {
      const int r = kRowsPerPass * it + r0;     // row of the wave
      if (qw0 + r < n_q) {
        f32x4_t y = *reinterpret_cast<SQKV_LDS const f32x4_t*>(stage + r * C::STAGE_PITCH + c * 4);
        if (o_in != nullptr) {
          const float w = *reinterpret_cast<SQKV_LDS const float*>(stage + kQW * C::STAGE_PITCH + r * 4);
          if (w != 0.f) {
            float x[4];
            load4(o_in, ibase + it * istep, acc_dtype, x);
#pragma unroll
            for (int k = 0; k < 4; ++k) y[k] = fmaf(w, x[k], y[k]);
          }
        }
        const int64_t off = obase + it * ostep;
        if (bf16_out) {   // round to nearest even in hardware, two values per instruction
          const uint2 v = {pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3])};
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(o_out) + off) = v;
        } else {
          *reinterpret_cast<f32x4_t*>(static_cast<float*>(o_out) + off) = y;
        }
      }
    }
  }
  // every wave is done with this visit's LDS (fragments, flag) before the
  // next one's DMA and flag clearing
  lds_reads_done_sync();
  }
}

// Compute units of the current device (one persistent workgroup each).
hipError_t cu_count(int* n) {
  constexpr int kMaxDev = 64;
  static std::atomic<int> cache[kMaxDev] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < kMaxDev;
  if (cached && (*n = cache[dev].load(std::memory_order_relaxed)) > 0) return hipSuccess;
  e = hipDeviceGetAttribute(n, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (*n < 1) *n = 1;
  if (cached) cache[dev].store(*n, std::memory_order_relaxed);
  return hipSuccess;
}

template <int D, bool PACKED>
hipError_t launch_d(const AttnParams& p, hipStream_t s) {
  using C = Cfg<D>;
  const int n_qtiles = (p.n_q + kBM - 1) / kBM;
  const int64_t blocks = (int64_t)n_qtiles * p.B * p.Hq;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;   // the host validation keeps items below 2^31
  int ncu = 0;
  hipError_t ec = cu_count(&ncu);
  if (ec != hipSuccess) return ec;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = allow_dyn_lds(reinterpret_cast<const void*>(&attn_bf16_kernel<D, PACKED>), C::LDS_ALLOC, lds_set);
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)(blocks < ncu ? blocks : ncu);
  hipLaunchKernelGGL((attn_bf16_kernel<D, PACKED>), dim3(grid), dim3(kThreads), C::LDS_ALLOC, s, p, n_qtiles,
                     (int)blocks);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bf16(const AttnParams& p, int d, hipStream_t s) {
  if (p.seg != nullptr) return d == 128 ? launch_d<128, true>(p, s) : launch_d<64, true>(p, s);
  return d == 128 ? launch_d<128, false>(p, s) : launch_d<64, false>(p, s);
}

}  // namespace sqkv
