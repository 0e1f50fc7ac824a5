// Ulysses sequence<->head all-to-all on one HBM pool.
//
// "Метод контекстного параллелизма Ulysses" (stuffynlp post 213): each of the
// P ranks holds its sequence part for all heads; the all_to_all hands rank r
// the whole sequence for its head group (and the inverse after attention);
// with GQA the key/value heads are copied up to the group size.
//
// With all P shards resident in one pool the exchange is a pure permutation
// of contiguous runs.  For seq->head without replication, viewing the source
// as [L][P][run] (run = H/P * d elements: rank r's head group of one token),
// the destination is [P][L][run]: a transpose of the two outer axes with the
// run kept contiguous.  At the 128k Llama-like shape a run is 4 heads * 128 *
// 2 B = 1 KiB, i.e. exactly one 64-lane x 16-byte wavefront access, so every
// read and every write is already a full, aligned, coalesced transaction; an
// LDS transpose would add traffic without improving coalescing.  The kernel is
// therefore a streaming copy with non-temporal hints (the data is touched
// once).  Each thread moves kItems vectors (16 bytes where the run allows).
// Measured at the 128k shape: one vector per thread in 256-thread workgroups
// reaches ~6.4 TB/s, as fast as a plain linear copy of the same bytes in the
// same launch shape, while four vectors per thread (more loads in flight, 4x
// fewer workgroups) reach ~6.0 TB/s and plain (temporal) loads and stores
// ~5.2 TB/s.
#include "sqkv_internal.h"

namespace sqkv {
namespace {

// Division of 32-bit unsigned numerators by a runtime divisor via a
// multiply-high and shift (Granlund & Montgomery, "Division by invariant
// integers using multiplication", 1994, round-up variant).
struct FastDiv {
  uint32_t d, m, l;
};

FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  f.l = 0;
  while ((1ull << f.l) < d) ++f.l;
  f.m = (uint32_t)((((1ull << 32) * ((1ull << f.l) - d)) / d) + 1);
  return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  uint64_t t = __umulhi(n, f.m);
  return (uint32_t)((t + n) >> f.l);
}

template <int V> struct VecOf;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
template <> struct VecOf<16> { typedef u32x4_t T; };
template <> struct VecOf<8> { typedef u32x2_t T; };
template <> struct VecOf<4> { typedef uint32_t T; };
template <> struct VecOf<2> { typedef uint16_t T; };
template <> struct VecOf<1> { typedef uint8_t T; };

constexpr int kThreads = 256;
constexpr int kItems = 1;

enum Mode { kSeqToHead = 0, kSeqToHeadRep = 1, kHeadToSeq = 2 };  // kSeqToHeadRep: replicate_kernel

struct KParams {
  PermuteParams p;
  uint32_t total_vec;   // vectors to move (to read, with replication)
  int64_t run_bytes;    // contiguous bytes per unit
  FastDiv f_vpr;        // vectors per run
  FastDiv f_P;
  FastDiv f_Hl;
  FastDiv f_Hsrc;
};

template <int V, int MODE>
__global__ void __launch_bounds__(kThreads) permute_kernel(KParams kp) {
  typedef typename VecOf<V>::T vec_t;
  const PermuteParams& p = kp.p;
  const uint32_t base = (uint32_t)blockIdx.x * (kThreads * kItems) + threadIdx.x;
  vec_t buf[kItems];
  int64_t dst_off[kItems];
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    uint32_t g = base + i * kThreads;
    dst_off[i] = -1;
    if (g < kp.total_vec) {
      uint32_t unit = fdiv(g, kp.f_vpr);
      int64_t kb = (int64_t)(g - unit * kp.f_vpr.d) * V;
      // unit = s * P + r ; one head group (run) of one token per unit
      uint32_t s = fdiv(unit, kp.f_P);
      uint32_t r = unit - s * kp.f_P.d;
      int64_t lin = (int64_t)unit * kp.run_bytes;
      int64_t other = ((int64_t)r * p.L + s) * kp.run_bytes;
      int64_t so = (MODE == kSeqToHead) ? lin : other;
      int64_t dof = (MODE == kSeqToHead) ? other : lin;
      buf[i] = __builtin_nontemporal_load(reinterpret_cast<const vec_t*>(p.src + so + kb));
      dst_off[i] = dof + kb;
    }
  }
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    if (dst_off[i] >= 0)
      __builtin_nontemporal_store(buf[i], reinterpret_cast<vec_t*>(p.dst + dst_off[i]));
  }
}

// seq->head with key/value heads copied R = H_dst / H_src times.  Source
// unit = s * H_src + hs is head row hs of token s (s over the whole sequence,
// the shards one after the other); it goes to destination heads j = hs*R ..
// hs*R + R-1, i.e. rank j / Hl, slot j % Hl.  Each source vector is read once
// and stored R times from its register; a thread first loads kRepItems
// vectors (one per 256-thread stride), then issues their stores copy by copy.
// Measured at 128k tokens, d = 128, R = 8: one vector per thread 4.3 TB/s,
// four 5.1 TB/s, sixteen 5.2 TB/s; every destination row is a separate
// 32 MiB rank region, and a store-only fill with that eight-region pattern
// runs at ~5.3 TB/s against ~6.2 TB/s for one linear fill of the same bytes.
constexpr int kRepItems = 4;

template <int V>
__global__ void __launch_bounds__(kThreads) replicate_kernel(KParams kp) {
  typedef typename VecOf<V>::T vec_t;
  const PermuteParams& p = kp.p;
  const uint32_t g0 = (uint32_t)blockIdx.x * (kThreads * kRepItems) + threadIdx.x;
  vec_t v[kRepItems];
  uint32_t s[kRepItems], hs[kRepItems];
  int64_t kb[kRepItems];
  bool ok[kRepItems];
#pragma unroll
  for (int i = 0; i < kRepItems; ++i) {
    const uint32_t g = g0 + i * kThreads;
    ok[i] = g < kp.total_vec;
    if (ok[i]) {
      const uint32_t unit = fdiv(g, kp.f_vpr);
      kb[i] = (int64_t)(g - unit * kp.f_vpr.d) * V;
      s[i] = fdiv(unit, kp.f_Hsrc);
      hs[i] = unit - s[i] * kp.f_Hsrc.d;
      v[i] = __builtin_nontemporal_load(reinterpret_cast<const vec_t*>(p.src + (int64_t)unit * p.row_bytes + kb[i]));
    }
  }
  for (int k = 0; k < p.R; ++k) {
#pragma unroll
    for (int i = 0; i < kRepItems; ++i) {
      if (!ok[i]) continue;
      const uint32_t j = hs[i] * (uint32_t)p.R + k;
      const uint32_t r = fdiv(j, kp.f_Hl);
      const uint32_t hl = j - r * kp.f_Hl.d;
      __builtin_nontemporal_store(
          v[i], reinterpret_cast<vec_t*>(p.dst + (((int64_t)r * p.L + s[i]) * p.Hl + hl) * p.row_bytes + kb[i]));
    }
  }
}

int pick_vec(int64_t run_bytes, const void* a, const void* b) {
  uintptr_t al = (uintptr_t)a | (uintptr_t)b;
  for (int v = 16; v > 1; v >>= 1)
    if (run_bytes % v == 0 && (al % v) == 0) return v;
  return 1;
}

template <int MODE>
hipError_t launch_mode(const PermuteParams& p, int64_t run_bytes, int64_t units, hipStream_t s) {
  int V = pick_vec(run_bytes, p.src, p.dst);
  KParams kp;
  kp.p = p;
  int64_t vpr = run_bytes / V;
  int64_t total = units * vpr;
  if (total == 0) return hipSuccess;
  kp.total_vec = (uint32_t)total;
  kp.run_bytes = run_bytes;
  kp.f_vpr = make_fastdiv((uint32_t)vpr);
  kp.f_P = make_fastdiv((uint32_t)p.P);
  kp.f_Hl = make_fastdiv((uint32_t)p.Hl);
  kp.f_Hsrc = make_fastdiv((uint32_t)p.H_src);
  if constexpr (MODE == kSeqToHeadRep) {
    dim3 grid((unsigned)((total + kThreads * kRepItems - 1) / (kThreads * kRepItems)));
    switch (V) {
      case 16: hipLaunchKernelGGL((replicate_kernel<16>), grid, dim3(kThreads), 0, s, kp); break;
      case 8: hipLaunchKernelGGL((replicate_kernel<8>), grid, dim3(kThreads), 0, s, kp); break;
      case 4: hipLaunchKernelGGL((replicate_kernel<4>), grid, dim3(kThreads), 0, s, kp); break;
      case 2: hipLaunchKernelGGL((replicate_kernel<2>), grid, dim3(kThreads), 0, s, kp); break;
      default: hipLaunchKernelGGL((replicate_kernel<1>), grid, dim3(kThreads), 0, s, kp); break;
    }
  } else {
    dim3 grid((unsigned)((total + kThreads * kItems - 1) / (kThreads * kItems)));
    switch (V) {
      case 16: hipLaunchKernelGGL((permute_kernel<16, MODE>), grid, dim3(kThreads), 0, s, kp); break;
      case 8: hipLaunchKernelGGL((permute_kernel<8, MODE>), grid, dim3(kThreads), 0, s, kp); break;
      case 4: hipLaunchKernelGGL((permute_kernel<4, MODE>), grid, dim3(kThreads), 0, s, kp); break;
      case 2: hipLaunchKernelGGL((permute_kernel<2, MODE>), grid, dim3(kThreads), 0, s, kp); break;
      default: hipLaunchKernelGGL((permute_kernel<1, MODE>), grid, dim3(kThreads), 0, s, kp); break;
    }
  }
  return hipGetLastError();
}

}  // namespace


hipError_t launch_seq_to_head(const PermuteParams& p, hipStream_t s) {
  if (p.R == 1) {
    int64_t run = (int64_t)p.Hl * p.row_bytes;
    return launch_mode<kSeqToHead>(p, run, (int64_t)p.L * p.P, s);
  }
  return launch_mode<kSeqToHeadRep>(p, p.row_bytes, (int64_t)p.L * p.H_src, s);
}

hipError_t launch_head_to_seq(const PermuteParams& p, hipStream_t s) {
  int64_t run = (int64_t)p.Hl * p.row_bytes;
  return launch_mode<kHeadToSeq>(p, run, (int64_t)p.L * p.P, s);
}

}  // namespace sqkv
