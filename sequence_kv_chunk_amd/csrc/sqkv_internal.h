// Internal declarations shared by the host layer (api.cpp) and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace sqkv {

// Raises `kernel`'s dynamic LDS limit to `bytes` on the current device, once
// per device (each device holds its own copy of the kernel and its
// attributes); `done` records the devices already set, one bit each.
inline hipError_t allow_dyn_lds(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
  if (bit != 0 && (done.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit != 0) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// Compute units of the current device, cached per device.
inline hipError_t device_cu_count(int* n) {
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

enum DType : int { kF32 = 0, kBF16 = 1 };

// One attention launch: a query chunk against `nseg` key/value chunks visited
// in ring order.  Views are [B, H, n, d] with element strides.  Visit s reads
// chunk j = (rank - s) mod P, which starts j*k_cs (j*v_cs) elements after k
// (v; the chunk strides may be negative) and whose key 0 sits at global
// position k_pos0 + j*k_posstride.  With a causal mask only the first chunk
// visited (the rank's own) may hold keys after a query; later ones must lie
// entirely in its past.  A single chunk is nseg = P = 1, rank = 0.
struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t k_cs, v_cs;         // chunk strides of the key / value pools
  int64_t k_posstride;        // positions between consecutive chunks
  int nseg, P, rank;
  const void* o_in;  // nullptr: no running state
  int64_t oi_sb, oi_sh, oi_sn;
  const float* lse_in;
  void* o_out;
  int64_t oo_sb, oo_sh, oo_sn;
  float* lse_out;
  // lse of query row t of (b, h) is lse_*[(b*Hq + h)*lse_*_hs + t]
  int64_t lse_in_hs, lse_out_hs;
  int B, Hq, Hkv, n_q, n_k;
  int group;          // Hq / Hkv
  int acc_dtype;      // dtype of o_in
  int out_dtype;      // dtype of o_out
  float scale_log2;   // scale * log2(e): logits are handled in base 2
  int causal;
  int64_t q_pos0, k_pos0;
  // packed samples (nullptr: one sample): sorted start positions, seg[0] = 0;
  // a query sees only keys of its own sample (with the causal mask)
  const int64_t* seg;
  int n_seg;
};

// One chunk pair of the attention backward: query chunk (q, dout, lse, D)
// against key/value chunk (k, v); adds the pair's share into dq (fp32
// [B, Hq, n_q, d]) and dk, dv (fp32 [B, Hkv, n_k, d]).  lse and D are dense
// [B, Hq, n_q] fp32: the rows' natural-log log-sum-exp over ALL keys and
// rowsum(dO * O).
struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  int64_t q_sb, q_sh, q_sn;
  int64_t k_sb, k_sh, k_sn;
  int64_t v_sb, v_sh, v_sn;
  int64_t do_sb, do_sh, do_sn;
  const float* lse;
  const float* D;
  float* dq;
  float* dk;
  float* dv;
  int64_t dq_sb, dq_sh, dq_sn;
  int64_t dk_sb, dk_sh, dk_sn;
  int64_t dv_sb, dv_sh, dv_sn;
  int B, Hq, Hkv, n_q, n_k;
  int group;          // Hq / Hkv
  float scale;        // logits are scale * (q . k)
  float scale_log2;   // scale * log2(e)
  int causal;
  int64_t q_pos0, k_pos0;
};

// D = rowsum(dO * O) per query row.
struct RowDotParams {
  const void* o;
  const void* dout;
  int64_t o_sb, o_sh, o_sn;
  int64_t do_sb, do_sh, do_sn;
  float* D;            // dense [B, H, n]
  int B, H, n;
  int dtype;           // of o and dout
};

struct MergeParams {
  const void* oa;
  int64_t a_sb, a_sh, a_sn;
  const float* lse_a;
  int a_dtype;
  const void* ob;
  int64_t b_sb, b_sh, b_sn;
  const float* lse_b;
  int b_dtype;
  void* oo;
  int64_t o_sb, o_sh, o_sn;
  float* lse_o;
  int o_dtype;
  int B, H, n;
};

// Ulysses run copy: `units` runs of `run_bytes` bytes each.
struct PermuteParams {
  const unsigned char* src;
  unsigned char* dst;
  int64_t L;       // full sequence length
  int64_t n;       // L / P
  int P;
  int H_src;       // heads in the seq-sharded layout
  int Hl;          // heads per rank in the head-sharded layout
  int R;           // replication factor (H_dst / H_src), 1 for head->seq
  int64_t row_bytes;  // d * elem_bytes
};

hipError_t launch_attn_bf16(const AttnParams& p, int d, hipStream_t s);
hipError_t launch_attn_f32(const AttnParams& p, int d, hipStream_t s);
hipError_t launch_lse_merge(const MergeParams& p, int d, hipStream_t s);
hipError_t launch_bwd_rowdot(const RowDotParams& p, int d, hipStream_t s);
hipError_t launch_attn_bwd_bf16(const BwdParams& p, int d, hipStream_t s);
hipError_t launch_seq_to_head(const PermuteParams& p, hipStream_t s);
hipError_t launch_head_to_seq(const PermuteParams& p, hipStream_t s);

}  // namespace sqkv
