// Host side of the C ABI declared in include/sqkv.h: argument validation
// (before any HIP call), kernel selection and the ring loop over resident
// chunks.  No allocation, no synchronisation; every launch goes on the
// caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <initializer_list>
#include <mutex>
#include <string>
#include <utility>

#include "../../include/sqkv.h"
#include "sqkv_internal.h"

#define SQKV_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local std::string g_last_error;

sqkv_status fail(sqkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

sqkv_status ok() {
  g_last_error.clear();
  return SQKV_OK;
}

sqkv_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SQKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int dtype_bytes(int dt) { return dt == SQKV_F32 ? 4 : 2; }
bool dtype_ok(int dt) { return dt == SQKV_F32 || dt == SQKV_BF16; }

// Byte range [lo, hi) touched by a [B, H, n, d] view (strides >= 0).
struct Range {
  uintptr_t lo = 0, hi = 0;
  bool empty() const { return hi <= lo; }
};

Range view_range(const sqkv_view& v, int B, int H, int64_t n, int d, int eb) {
  Range r;
  if (B <= 0 || H <= 0 || n <= 0 || d <= 0) return r;
  int64_t last = (int64_t)(B - 1) * v.sb + (int64_t)(H - 1) * v.sh + (n - 1) * v.sn + d;
  r.lo = (uintptr_t)v.ptr;
  r.hi = r.lo + (uintptr_t)(last * eb);
  return r;
}

Range dense_range(const void* p, int64_t elems, int eb) {
  Range r;
  if (elems <= 0) return r;
  r.lo = (uintptr_t)p;
  r.hi = r.lo + (uintptr_t)(elems * eb);
  return r;
}

bool overlap(const Range& a, const Range& b) {
  if (a.empty() || b.empty()) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool same_view(const sqkv_view& a, const sqkv_view& b) {
  return a.ptr == b.ptr && a.sb == b.sb && a.sh == b.sh && a.sn == b.sn;
}

// 16-byte alignment of the base pointer and of every stride (in bytes).
bool view_aligned(const sqkv_view& v, int eb) {
  if (((uintptr_t)v.ptr) % 16) return false;
  return (v.sb * eb) % 16 == 0 && (v.sh * eb) % 16 == 0 && (v.sn * eb) % 16 == 0;
}

bool strides_nonneg(const sqkv_view& v) { return v.sb >= 0 && v.sh >= 0 && v.sn >= 0; }

// No two rows (runs of d elements) of an output view share an element.  The
// dimensions (stride, count) are sorted by stride and each stride must reach
// past the span of those below it: sufficient, and exact for the nested
// layouts of dense tensors and their transposes.
bool rows_disjoint(int64_t d, std::initializer_list<std::pair<int64_t, int64_t>> dims) {
  std::pair<int64_t, int64_t> s[4];
  int n = 0;
  for (const auto& x : dims)
    if (x.second > 1 && n < 4) s[n++] = x;
  std::sort(s, s + n);
  int64_t span = d;
  for (int i = 0; i < n; ++i) {
    if (s[i].first < span) return false;
    span += s[i].first * (s[i].second - 1);
  }
  return true;
}

bool rows_disjoint(const sqkv_view& v, int B, int H, int64_t n, int d) {
  return rows_disjoint(d, {{v.sb, B}, {v.sh, H}, {v.sn, n}});
}

struct AttnCheck {
  sqkv_view q, k, v, o_in, o_out;
  const float* lse_in;
  float* lse_out;
  int B, Hq, Hkv;
  int64_t n_q, n_k, kv_extent_extra_bytes;  // extra bytes past chunk 0 (ring pools)
  int d, in_dt, acc_dt, out_dt;
  float scale;
};

// Validation shared by ra_chunk_attention and ra_ring_attention.
sqkv_status check_attention(const AttnCheck& a) {
  if (a.B < 1 || a.Hq < 1 || a.Hkv < 1 || a.n_q < 0 || a.n_k < 0)
    return fail(SQKV_EINVAL, "sizes must be positive (B=%d Hq=%d Hkv=%d n_q=%lld n_k=%lld)", a.B, a.Hq,
                a.Hkv, (long long)a.n_q, (long long)a.n_k);
  if (a.Hq % a.Hkv != 0)
    return fail(SQKV_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", a.Hq, a.Hkv);
  if (!(a.scale > 0.f) || !std::isfinite(a.scale))
    return fail(SQKV_EINVAL, "scale must be finite and > 0 (got %g)", (double)a.scale);
  if (a.d != 64 && a.d != 128) return fail(SQKV_EUNSUPPORTED, "head dim d=%d not in {64, 128}", a.d);
  if (!dtype_ok(a.in_dt) || !dtype_ok(a.acc_dt) || !dtype_ok(a.out_dt))
    return fail(SQKV_EUNSUPPORTED, "dtype must be SQKV_F32 or SQKV_BF16");
  if (a.B > 65535 || a.Hq > 65535) return fail(SQKV_EUNSUPPORTED, "B and Hq must be <= 65535");
  if (a.n_q > (1ll << 30) || a.n_k > (1ll << 30))
    return fail(SQKV_EUNSUPPORTED, "chunk lengths above 2^30 are not supported");
  // the bf16 kernel numbers its 256-row work items with 32-bit ints; the fp32
  // kernel's grid rows hold ceil(n_q/128) workgroups of 512 threads
  if ((a.n_q + 255) / 256 * a.B * a.Hq > 0x7fffffffll)
    return fail(SQKV_EUNSUPPORTED, "B*Hq*ceil(n_q/256) must be below 2^31");
  if (a.in_dt == SQKV_F32 && a.n_q > (1ll << 30) - 128)
    return fail(SQKV_EUNSUPPORTED, "fp32 query chunks must be below 2^30 - 128 rows");
  if (a.n_q == 0) return ok();
  if (!a.q.ptr || !a.o_out.ptr || !a.lse_out) return fail(SQKV_EINVAL, "null q, o_out or lse_out");
  if (a.n_k > 0 && (!a.k.ptr || !a.v.ptr)) return fail(SQKV_EINVAL, "null k or v");
  if ((a.o_in.ptr == nullptr) != (a.lse_in == nullptr))
    return fail(SQKV_EINVAL, "o_in and lse_in must both be given or both be NULL");
  for (const sqkv_view* v : {&a.q, &a.k, &a.v, &a.o_in, &a.o_out})
    if (!strides_nonneg(*v)) return fail(SQKV_EINVAL, "negative stride");
  const int ieb = dtype_bytes(a.in_dt);
  if (!view_aligned(a.q, ieb) || (a.n_k > 0 && (!view_aligned(a.k, ieb) || !view_aligned(a.v, ieb))))
    return fail(SQKV_EUNSUPPORTED, "q/k/v pointers and strides must be 16-byte aligned");
  if (!view_aligned(a.o_out, dtype_bytes(a.out_dt)) ||
      (a.o_in.ptr && !view_aligned(a.o_in, dtype_bytes(a.acc_dt))))
    return fail(SQKV_EUNSUPPORTED, "output pointers and strides must be 16-byte aligned");
  if (((uintptr_t)a.lse_out) % 4 || ((uintptr_t)a.lse_in) % 4)
    return fail(SQKV_EUNSUPPORTED, "lse must be 4-byte aligned");
  // the attention kernels address a key/value tile through a 32-bit byte
  // range; the bf16 kernel's range is rows x row stride, so its key/value
  // rows must not overlap
  if (a.k.sn * ieb >= (1ll << 24) || a.v.sn * ieb >= (1ll << 24))
    return fail(SQKV_EUNSUPPORTED, "key/value row strides must be below 16 MiB");
  if (a.in_dt == SQKV_BF16 && a.n_k > 0 && (a.k.sn < a.d || a.v.sn < a.d))
    return fail(SQKV_EUNSUPPORTED, "bf16 key/value row strides must be at least d (rows may not overlap)");
  if (!rows_disjoint(a.o_out, a.B, a.Hq, a.n_q, a.d)) return fail(SQKV_EINVAL, "rows of o_out overlap each other");
  // aliasing: outputs may only coincide exactly with the running state
  const int64_t rows = (int64_t)a.B * a.Hq * a.n_q;
  Range ro = view_range(a.o_out, a.B, a.Hq, a.n_q, a.d, dtype_bytes(a.out_dt));
  Range rl = dense_range(a.lse_out, rows, 4);
  Range rq = view_range(a.q, a.B, a.Hq, a.n_q, a.d, ieb);
  Range rk = view_range(a.k, a.B, a.Hkv, a.n_k, a.d, ieb);
  Range rv = view_range(a.v, a.B, a.Hkv, a.n_k, a.d, ieb);
  if (!rk.empty()) rk.hi += a.kv_extent_extra_bytes;
  if (!rv.empty()) rv.hi += a.kv_extent_extra_bytes;
  for (const Range* r : {&rq, &rk, &rv}) {
    if (overlap(ro, *r)) return fail(SQKV_EINVAL, "o_out overlaps q, k or v");
    if (overlap(rl, *r)) return fail(SQKV_EINVAL, "lse_out overlaps q, k or v");
  }
  if (overlap(ro, rl)) return fail(SQKV_EINVAL, "o_out overlaps lse_out");
  if (a.o_in.ptr) {
    Range ri = view_range(a.o_in, a.B, a.Hq, a.n_q, a.d, dtype_bytes(a.acc_dt));
    Range rli = dense_range(a.lse_in, rows, 4);
    bool o_alias = same_view(a.o_in, a.o_out) && a.acc_dt == a.out_dt;
    if (!o_alias && overlap(ri, ro)) return fail(SQKV_EINVAL, "o_out partially overlaps o_in");
    if (a.lse_in != a.lse_out && overlap(rli, rl)) return fail(SQKV_EINVAL, "lse_out partially overlaps lse_in");
    if (overlap(ri, rl) || overlap(rli, ro)) return fail(SQKV_EINVAL, "o and lse buffers overlap");
  }
  return ok();
}

sqkv::AttnParams make_params(const sqkv_view& q, const sqkv_view& k, const sqkv_view& v, const sqkv_view& o_in,
                             const float* lse_in, const sqkv_view& o_out, float* lse_out, int B, int Hq,
                             int Hkv, int n_q, int n_k, int acc_dt, int out_dt, float scale, int causal,
                             int64_t q_pos0, int64_t k_pos0) {
  sqkv::AttnParams p;
  p.q = q.ptr; p.q_sb = q.sb; p.q_sh = q.sh; p.q_sn = q.sn;
  p.k = k.ptr; p.k_sb = k.sb; p.k_sh = k.sh; p.k_sn = k.sn;
  p.v = v.ptr; p.v_sb = v.sb; p.v_sh = v.sh; p.v_sn = v.sn;
  p.o_in = o_in.ptr; p.oi_sb = o_in.sb; p.oi_sh = o_in.sh; p.oi_sn = o_in.sn;
  p.lse_in = o_in.ptr ? lse_in : nullptr;
  p.o_out = o_out.ptr; p.oo_sb = o_out.sb; p.oo_sh = o_out.sh; p.oo_sn = o_out.sn;
  p.lse_out = lse_out;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.n_q = n_q; p.n_k = n_k;
  p.group = Hq / Hkv;
  p.acc_dtype = acc_dt;
  p.out_dtype = out_dt;
  p.scale_log2 = scale * 1.44269504088896340736f;
  p.causal = causal ? 1 : 0;
  p.q_pos0 = q_pos0;
  p.k_pos0 = k_pos0;
  p.lse_in_hs = p.lse_out_hs = n_q;   // dense [B, Hq, n_q]
  p.seg = nullptr;
  p.n_seg = 0;
  // a single chunk; ra_ring_attention widens this to the ring visit
  p.k_cs = p.v_cs = 0;
  p.k_posstride = 0;
  p.nseg = 1;
  p.P = 1;
  p.rank = 0;
  return p;
}

hipError_t launch_attention(const sqkv::AttnParams& p, int d, int in_dt, hipStream_t s) {
  return in_dt == SQKV_BF16 ? sqkv::launch_attn_bf16(p, d, s) : sqkv::launch_attn_f32(p, d, s);
}

}  // namespace

SQKV_EXPORT const char* sqkv_last_error(void) { return g_last_error.c_str(); }

SQKV_EXPORT sqkv_status ra_chunk_attention(sqkv_view q, sqkv_view k, sqkv_view v, sqkv_view o_in,
                                           const float* lse_in, sqkv_view o_out, float* lse_out, int B,
                                           int Hq, int Hkv, int n_q, int n_k, int d, sqkv_dtype in_dtype,
                                           sqkv_dtype acc_dtype, sqkv_dtype out_dtype, float scale,
                                           int causal, int64_t q_pos0, int64_t k_pos0, void* stream) {
  AttnCheck a{q, k, v, o_in, o_out, lse_in, lse_out, B, Hq, Hkv, n_q, n_k, 0, d,
              in_dtype, acc_dtype, out_dtype, scale};
  sqkv_status st = check_attention(a);
  if (st != SQKV_OK || n_q == 0) return st;
  sqkv::AttnParams p = make_params(q, k, v, o_in, lse_in, o_out, lse_out, B, Hq, Hkv, n_q, n_k, acc_dtype,
                                   out_dtype, scale, causal, q_pos0, k_pos0);
  return hip_status(launch_attention(p, d, in_dtype, (hipStream_t)stream), "ra_chunk_attention launch");
}

SQKV_EXPORT sqkv_status ra_ring_attention(sqkv_view q, sqkv_view k, sqkv_view v, int64_t k_chunk_stride,
                                          int64_t v_chunk_stride, sqkv_view o, float* lse, int B, int Hq,
                                          int Hkv, int n, int d, int P, int rank, sqkv_dtype in_dtype,
                                          sqkv_dtype out_dtype, float scale, int causal, void* stream) {
  if (P < 1 || rank < 0 || rank >= P) return fail(SQKV_EINVAL, "need P >= 1 and 0 <= rank < P (P=%d rank=%d)", P, rank);
  if (k_chunk_stride < 0 || v_chunk_stride < 0) return fail(SQKV_EINVAL, "negative chunk stride");
  const int ieb = dtype_bytes(in_dtype);
  if ((k_chunk_stride * ieb) % 16 || (v_chunk_stride * ieb) % 16)
    return fail(SQKV_EUNSUPPORTED, "chunk strides must be multiples of 16 bytes");
  AttnCheck a{q, k, v, sqkv_view{nullptr, 0, 0, 0}, o, nullptr, lse, B, Hq, Hkv, n, n,
              (int64_t)(P - 1) * std::max(k_chunk_stride, v_chunk_stride) * ieb, d,
              in_dtype, SQKV_F32, out_dtype, scale};
  sqkv_status st = check_attention(a);
  if (st != SQKV_OK || n == 0) return st;
  // One launch visits the chunks in ring order, the rank's own first, then the
  // one arriving from the previous rank: j = (rank - s) mod P.  With a causal
  // mask the chunks after the rank's own (j > rank) are entirely in the future
  // of its queries, so the visit stops after chunk 0 (s = rank).
  sqkv::AttnParams p = make_params(q, k, v, sqkv_view{nullptr, 0, 0, 0}, nullptr, o, lse, B, Hq, Hkv, n, n,
                                   SQKV_F32, out_dtype, scale, causal, (int64_t)rank * n, 0);
  p.k_cs = k_chunk_stride;
  p.v_cs = v_chunk_stride;
  p.k_posstride = n;
  p.P = P;
  p.rank = rank;
  p.nseg = causal ? rank + 1 : P;
  return hip_status(launch_attention(p, d, in_dtype, (hipStream_t)stream), "ra_ring_attention launch");
}

SQKV_EXPORT sqkv_status ra_ring_attention_packed(sqkv_view q, sqkv_view k, sqkv_view v, int64_t k_chunk_stride,
                                                 int64_t v_chunk_stride, sqkv_view o, float* lse,
                                                 const int64_t* seg_starts, int n_seg, int B, int Hq, int Hkv, int n,
                                                 int d, int P, int rank, sqkv_dtype in_dtype, sqkv_dtype out_dtype,
                                                 float scale, void* stream) {
  if (n_seg < 1 || !seg_starts) return fail(SQKV_EINVAL, "need at least one sample start (n_seg=%d)", n_seg);
  if (((uintptr_t)seg_starts) % 8) return fail(SQKV_EUNSUPPORTED, "seg_starts must be 8-byte aligned");
  if (in_dtype != SQKV_BF16) return fail(SQKV_EUNSUPPORTED, "packed samples need bf16 inputs");
  if (P < 1 || rank < 0 || rank >= P) return fail(SQKV_EINVAL, "need P >= 1 and 0 <= rank < P (P=%d rank=%d)", P, rank);
  if (k_chunk_stride < 0 || v_chunk_stride < 0) return fail(SQKV_EINVAL, "negative chunk stride");
  if ((k_chunk_stride * 2) % 16 || (v_chunk_stride * 2) % 16)
    return fail(SQKV_EUNSUPPORTED, "chunk strides must be multiples of 16 bytes");
  AttnCheck a{q, k, v, sqkv_view{nullptr, 0, 0, 0}, o, nullptr, lse, B, Hq, Hkv, n, n,
              (int64_t)(P - 1) * std::max(k_chunk_stride, v_chunk_stride) * 2, d,
              in_dtype, SQKV_F32, out_dtype, scale};
  sqkv_status st = check_attention(a);
  if (st != SQKV_OK || n == 0) return st;
  if (overlap(dense_range(seg_starts, n_seg, 8), view_range(o, B, Hq, n, d, dtype_bytes(out_dtype))) ||
      overlap(dense_range(seg_starts, n_seg, 8), dense_range(lse, (int64_t)B * Hq * n, 4)))
    return fail(SQKV_EINVAL, "seg_starts overlaps an output");
  sqkv::AttnParams p = make_params(q, k, v, sqkv_view{nullptr, 0, 0, 0}, nullptr, o, lse, B, Hq, Hkv, n, n,
                                   SQKV_F32, out_dtype, scale, 1, (int64_t)rank * n, 0);
  p.k_cs = k_chunk_stride;
  p.v_cs = v_chunk_stride;
  p.k_posstride = n;
  p.P = P;
  p.rank = rank;
  p.nseg = rank + 1;
  p.seg = seg_starts;
  p.n_seg = n_seg;
  return hip_status(launch_attention(p, d, in_dtype, (hipStream_t)stream), "ra_ring_attention_packed launch");
}

namespace {

// Validation of a zigzag call.  The work buffers are checked only when
// `work_given` (the no-allocation variant brings its own).
sqkv_status check_zigzag(sqkv_view q, sqkv_view k, sqkv_view v, int64_t k_chunk_stride, int64_t v_chunk_stride,
                         sqkv_view o, float* lse, float* work_o, float* work_lse, bool work_given, int B, int Hq,
                         int Hkv, int n, int d, int P, int rank, sqkv_dtype in_dtype, sqkv_dtype out_dtype,
                         float scale) {
  if (P < 1 || rank < 0 || rank >= P) return fail(SQKV_EINVAL, "need P >= 1 and 0 <= rank < P (P=%d rank=%d)", P, rank);
  if (n % 2) return fail(SQKV_EINVAL, "the local shard length n=%d must be even (two pieces)", n);
  if (k_chunk_stride < 0 || v_chunk_stride < 0) return fail(SQKV_EINVAL, "negative chunk stride");
  const int ieb = dtype_bytes(in_dtype);
  if ((k_chunk_stride * ieb) % 16 || (v_chunk_stride * ieb) % 16)
    return fail(SQKV_EUNSUPPORTED, "chunk strides must be multiples of 16 bytes");
  AttnCheck a{q, k, v, sqkv_view{nullptr, 0, 0, 0}, o, nullptr, lse, B, Hq, Hkv, n, n,
              (int64_t)(P - 1) * std::max(k_chunk_stride, v_chunk_stride) * ieb, d,
              in_dtype, SQKV_F32, out_dtype, scale};
  sqkv_status st = check_attention(a);
  if (st != SQKV_OK || n == 0 || !work_given) return st;
  const int c = n / 2;
  if (!work_o || !work_lse) return fail(SQKV_EINVAL, "null work_o or work_lse");
  if (((uintptr_t)work_o) % 16 || ((uintptr_t)work_lse) % 4)
    return fail(SQKV_EUNSUPPORTED, "work_o must be 16-byte and work_lse 4-byte aligned");
  const int64_t rows = (int64_t)B * Hq * c;
  Range rw = dense_range(work_o, rows * d, 4), rwl = dense_range(work_lse, rows, 4);
  Range rq = view_range(q, B, Hq, n, d, ieb), ro = view_range(o, B, Hq, n, d, dtype_bytes(out_dtype));
  Range rl = dense_range(lse, (int64_t)B * Hq * n, 4);
  Range rk = view_range(k, B, Hkv, n, d, ieb), rv = view_range(v, B, Hkv, n, d, ieb);
  rk.hi += a.kv_extent_extra_bytes;
  rv.hi += a.kv_extent_extra_bytes;
  for (const Range* r : {&rq, &ro, &rl, &rk, &rv})
    if (overlap(rw, *r) || overlap(rwl, *r)) return fail(SQKV_EINVAL, "work buffers overlap q, k, v, o or lse");
  if (overlap(rw, rwl)) return fail(SQKV_EINVAL, "work_o overlaps work_lse");
  return ok();
}

// The three launches of a validated zigzag call (n > 0).
sqkv_status launch_zigzag(sqkv_view q, sqkv_view k, sqkv_view v, int64_t k_chunk_stride, int64_t v_chunk_stride,
                          sqkv_view o, float* lse, float* work_o, float* work_lse, int B, int Hq, int Hkv, int n,
                          int d, int P, int rank, sqkv_dtype in_dtype, sqkv_dtype out_dtype, float scale,
                          void* stream) {
  const int ieb = dtype_bytes(in_dtype);
  const int c = n / 2;
  auto rows_from = [](sqkv_view x, int64_t t0, int eb) {
    x.ptr = static_cast<char*>(x.ptr) + t0 * x.sn * eb;
    return x;
  };
  const int oeb = dtype_bytes(out_dtype);
  const sqkv_view q_early = q, q_late = rows_from(q, c, ieb);
  const sqkv_view o_early = o, o_late = rows_from(o, c, oeb);
  const sqkv_view w{work_o, (int64_t)Hq * c * d, (int64_t)c * d, d};
  const sqkv_view none{nullptr, 0, 0, 0};
  hipStream_t hs = (hipStream_t)stream;

  // 1. early piece (positions rank*c ..) against the early pieces of ranks
  //    rank, rank-1, .., 0: the own piece on its diagonal, the rest in the past
  sqkv::AttnParams p1 = make_params(q_early, k, v, none, nullptr, o_early, lse, B, Hq, Hkv, c, c, SQKV_F32,
                                    out_dtype, scale, 1, (int64_t)rank * c, 0);
  p1.k_cs = k_chunk_stride;
  p1.v_cs = v_chunk_stride;
  p1.k_posstride = c;
  p1.P = P;
  p1.rank = rank;
  p1.nseg = rank + 1;
  p1.lse_out_hs = n;
  hipError_t e = launch_attention(p1, d, in_dtype, hs);
  if (e != hipSuccess) return hip_status(e, "ra_zigzag_attention launch 1");

  // 2. late piece (positions (2P-1-rank)*c ..) against every early piece, all
  //    in its past: an unmasked ring visit, partial into the work buffers
  sqkv::AttnParams p2 = make_params(q_late, k, v, none, nullptr, w, work_lse, B, Hq, Hkv, c, c, SQKV_F32,
                                    SQKV_F32, scale, 0, 0, 0);
  p2.k_cs = k_chunk_stride;
  p2.v_cs = v_chunk_stride;
  p2.k_posstride = c;
  p2.P = P;
  p2.rank = rank;
  p2.nseg = P;
  e = launch_attention(p2, d, in_dtype, hs);
  if (e != hipSuccess) return hip_status(e, "ra_zigzag_attention launch 2");

  // 3. late piece against the late pieces of ranks rank, rank+1, .., P-1
  //    (positions (2P-1-j)*c: the own piece on its diagonal, the rest in the
  //    past), merged with the partial of step 2.  Numbered j' = P-1-j the late
  //    pieces sit at positions (P + j')*c and the visit is the causal ring of
  //    rank P-1-rank over a pool that starts at rank P-1's late piece and
  //    steps backwards through the shards.
  const sqkv_view k3 = rows_from(sqkv_view{static_cast<char*>(k.ptr) + (int64_t)(P - 1) * k_chunk_stride * ieb,
                                           k.sb, k.sh, k.sn}, c, ieb);
  const sqkv_view v3 = rows_from(sqkv_view{static_cast<char*>(v.ptr) + (int64_t)(P - 1) * v_chunk_stride * ieb,
                                           v.sb, v.sh, v.sn}, c, ieb);
  sqkv::AttnParams p3 = make_params(q_late, k3, v3, w, work_lse, o_late, lse + c, B, Hq, Hkv, c, c, SQKV_F32,
                                    out_dtype, scale, 1, (int64_t)(2 * P - 1 - rank) * c, (int64_t)P * c);
  p3.k_cs = -k_chunk_stride;
  p3.v_cs = -v_chunk_stride;
  p3.k_posstride = c;
  p3.P = P;
  p3.rank = P - 1 - rank;
  p3.nseg = P - rank;
  p3.lse_in_hs = c;
  p3.lse_out_hs = n;
  return hip_status(launch_attention(p3, d, in_dtype, hs), "ra_zigzag_attention launch 3");
}

}  // namespace

namespace {

// Scratch of the no-allocation zigzag entry point: the late piece's fp32
// partial (O, then lse).  A file-scope device array, so each GPU the library
// runs on holds its own copy from module load until the process ends, at the
// address hipGetSymbolAddress gives on that device.  In host code the array's
// name is a host-side stand-in, never a device address: only the per-device
// pointers below reach kernels.
constexpr size_t kZigzagScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kZigzagScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
unsigned char* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on the current device, looked up once per device.
sqkv_status scratch_on_current_device(unsigned char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SQKV_EUNSUPPORTED, "device index %d above %d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr) return fail(SQKV_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = static_cast<unsigned char*>(p);
  }
  *out = g_scratch_ptr[dev];
  return SQKV_OK;
}

}  // namespace

SQKV_EXPORT size_t ra_zigzag_attention_noalloc_max_bytes(void) { return kZigzagScratchBytes; }

SQKV_EXPORT sqkv_status ra_zigzag_attention_noalloc(sqkv_view q, sqkv_view k, sqkv_view v,
                                                    int64_t k_chunk_stride, int64_t v_chunk_stride, sqkv_view o,
                                                    float* lse, int B, int Hq, int Hkv, int n, int d, int P,
                                                    int rank, sqkv_dtype in_dtype, sqkv_dtype out_dtype,
                                                    float scale, void* stream) {
  sqkv_status st = check_zigzag(q, k, v, k_chunk_stride, v_chunk_stride, o, lse, nullptr, nullptr, false, B, Hq,
                                Hkv, n, d, P, rank, in_dtype, out_dtype, scale);
  if (st != SQKV_OK || n == 0) return st;
  // work_o [B, Hq, n/2, d] fp32, then work_lse [B, Hq, n/2] fp32 at the next
  // 256-byte boundary
  const uint64_t rows = (uint64_t)B * (uint64_t)Hq * (uint64_t)(n / 2);
  const uint64_t cap_rows = (kZigzagScratchBytes - 256) / (4 * (uint64_t)(d + 1));
  if (rows > cap_rows)
    return fail(SQKV_EUNSUPPORTED,
                "ra_zigzag_attention_noalloc: B*Hq*n/2 = %llu rows need %llu bytes of scratch, above its "
                "%llu-byte maximum; use ra_zigzag_attention with caller-owned work buffers",
                (unsigned long long)rows, (unsigned long long)(rows * 4 * (uint64_t)(d + 1)),
                (unsigned long long)kZigzagScratchBytes);
  const uint64_t o_bytes = (rows * 4 * (uint64_t)d + 255) & ~(uint64_t)255;
  unsigned char* base = nullptr;
  st = scratch_on_current_device(&base);
  if (st != SQKV_OK) return st;
  return launch_zigzag(q, k, v, k_chunk_stride, v_chunk_stride, o, lse, reinterpret_cast<float*>(base),
                       reinterpret_cast<float*>(base + o_bytes), B, Hq, Hkv, n, d, P, rank, in_dtype, out_dtype,
                       scale, stream);
}

SQKV_EXPORT sqkv_status ra_zigzag_attention(sqkv_view q, sqkv_view k, sqkv_view v, int64_t k_chunk_stride,
                                            int64_t v_chunk_stride, sqkv_view o, float* lse, float* work_o,
                                            float* work_lse, int B, int Hq, int Hkv, int n, int d, int P,
                                            int rank, sqkv_dtype in_dtype, sqkv_dtype out_dtype, float scale,
                                            void* stream) {
  sqkv_status st = check_zigzag(q, k, v, k_chunk_stride, v_chunk_stride, o, lse, work_o, work_lse, true, B, Hq,
                                Hkv, n, d, P, rank, in_dtype, out_dtype, scale);
  if (st != SQKV_OK || n == 0) return st;
  return launch_zigzag(q, k, v, k_chunk_stride, v_chunk_stride, o, lse, work_o, work_lse, B, Hq, Hkv, n, d, P,
                       rank, in_dtype, out_dtype, scale, stream);
}

namespace {

// Validation of one backward chunk pair (views as in the forward; dq, dk, dv
// fp32; lse and D dense fp32 [B, Hq, n_q]).
sqkv_status check_bwd(const sqkv_view& q, const sqkv_view& k, const sqkv_view& v, const sqkv_view& dout,
                      const float* lse, const float* D, const sqkv_view& dq, const sqkv_view& dk,
                      const sqkv_view& dv, int B, int Hq, int Hkv, int64_t n_q, int64_t n_k, int64_t kv_extra,
                      int64_t dkv_extra, int d, int in_dt, float scale) {
  if (B < 1 || Hq < 1 || Hkv < 1 || n_q < 0 || n_k < 0)
    return fail(SQKV_EINVAL, "sizes must be positive (B=%d Hq=%d Hkv=%d n_q=%lld n_k=%lld)", B, Hq, Hkv,
                (long long)n_q, (long long)n_k);
  if (Hq % Hkv != 0) return fail(SQKV_EINVAL, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(SQKV_EINVAL, "scale must be finite and > 0");
  if (d != 64 && d != 128) return fail(SQKV_EUNSUPPORTED, "head dim d=%d not in {64, 128}", d);
  if (in_dt != SQKV_BF16) return fail(SQKV_EUNSUPPORTED, "the backward takes bf16 q, k, v and dout");
  if (B > 65535 || Hq > 65535) return fail(SQKV_EUNSUPPORTED, "B and Hq must be <= 65535");
  if (n_q > (1ll << 30) || n_k > (1ll << 30)) return fail(SQKV_EUNSUPPORTED, "chunk lengths above 2^30");
  if (n_q == 0 || n_k == 0) return ok();
  // one-dimensional grids of 512-thread workgroups: at most 2^23 of each kind
  if ((n_q + 255) / 256 * B * Hq >= (1ll << 23) || (n_k + 127) / 128 * B * Hkv >= (1ll << 23))
    return fail(SQKV_EUNSUPPORTED, "B*Hq*ceil(n_q/256) and B*Hkv*ceil(n_k/128) must be below 2^23");
  if (!q.ptr || !k.ptr || !v.ptr || !dout.ptr || !lse || !D || !dq.ptr || !dk.ptr || !dv.ptr)
    return fail(SQKV_EINVAL, "null pointer");
  for (const sqkv_view* x : {&q, &k, &v, &dout, &dq, &dk, &dv})
    if (!strides_nonneg(*x)) return fail(SQKV_EINVAL, "negative stride");
  if (!view_aligned(q, 2) || !view_aligned(k, 2) || !view_aligned(v, 2) || !view_aligned(dout, 2) ||
      !view_aligned(dq, 4) || !view_aligned(dk, 4) || !view_aligned(dv, 4))
    return fail(SQKV_EUNSUPPORTED, "pointers and strides must be 16-byte aligned");
  if (((uintptr_t)lse | (uintptr_t)D) % 4) return fail(SQKV_EUNSUPPORTED, "lse and D must be 4-byte aligned");
  if (k.sn * 2 >= (1ll << 24) || v.sn * 2 >= (1ll << 24) || q.sn * 2 >= (1ll << 24) || dout.sn * 2 >= (1ll << 24))
    return fail(SQKV_EUNSUPPORTED, "row strides must be below 16 MiB");
  // tiles are copied as rows x row stride bytes: rows may not overlap
  if (k.sn < d || v.sn < d || q.sn < d || dout.sn < d)
    return fail(SQKV_EUNSUPPORTED, "row strides of q, k, v and dout must be at least d (rows may not overlap)");
  if (!rows_disjoint(dq, B, Hq, n_q, d) || !rows_disjoint(dk, B, Hkv, n_k, d) || !rows_disjoint(dv, B, Hkv, n_k, d))
    return fail(SQKV_EINVAL, "rows of dq, dk or dv overlap each other");
  const int64_t rows = (int64_t)B * Hq * n_q;
  Range rq = view_range(q, B, Hq, n_q, d, 2), ro = view_range(dout, B, Hq, n_q, d, 2);
  Range rk = view_range(k, B, Hkv, n_k, d, 2), rv = view_range(v, B, Hkv, n_k, d, 2);
  rk.hi += kv_extra;
  rv.hi += kv_extra;
  Range rl = dense_range(lse, rows, 4), rD = dense_range(D, rows, 4);
  Range gq = view_range(dq, B, Hq, n_q, d, 4);
  Range gk = view_range(dk, B, Hkv, n_k, d, 4), gv = view_range(dv, B, Hkv, n_k, d, 4);
  gk.hi += dkv_extra;
  gv.hi += dkv_extra;
  for (const Range* g : {&gq, &gk, &gv})
    for (const Range* r : {&rq, &ro, &rk, &rv, &rl, &rD})
      if (overlap(*g, *r)) return fail(SQKV_EINVAL, "a gradient buffer overlaps an input");
  if (overlap(gq, gk) || overlap(gq, gv) || overlap(gk, gv)) return fail(SQKV_EINVAL, "gradient buffers overlap");
  return ok();
}

sqkv::BwdParams make_bwd(const sqkv_view& q, const sqkv_view& k, const sqkv_view& v, const sqkv_view& dout,
                         const float* lse, const float* D, const sqkv_view& dq, const sqkv_view& dk,
                         const sqkv_view& dv, int B, int Hq, int Hkv, int n_q, int n_k, float scale, int causal,
                         int64_t q_pos0, int64_t k_pos0) {
  sqkv::BwdParams p;
  p.q = q.ptr; p.q_sb = q.sb; p.q_sh = q.sh; p.q_sn = q.sn;
  p.k = k.ptr; p.k_sb = k.sb; p.k_sh = k.sh; p.k_sn = k.sn;
  p.v = v.ptr; p.v_sb = v.sb; p.v_sh = v.sh; p.v_sn = v.sn;
  p.dout = dout.ptr; p.do_sb = dout.sb; p.do_sh = dout.sh; p.do_sn = dout.sn;
  p.lse = lse;
  p.D = D;
  p.dq = static_cast<float*>(dq.ptr); p.dq_sb = dq.sb; p.dq_sh = dq.sh; p.dq_sn = dq.sn;
  p.dk = static_cast<float*>(dk.ptr); p.dk_sb = dk.sb; p.dk_sh = dk.sh; p.dk_sn = dk.sn;
  p.dv = static_cast<float*>(dv.ptr); p.dv_sb = dv.sb; p.dv_sh = dv.sh; p.dv_sn = dv.sn;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.n_q = n_q; p.n_k = n_k;
  p.group = Hq / Hkv;
  p.scale = scale;
  p.scale_log2 = scale * 1.44269504088896340736f;
  p.causal = causal ? 1 : 0;
  p.q_pos0 = q_pos0;
  p.k_pos0 = k_pos0;
  return p;
}

sqkv_view offset_view(sqkv_view x, int64_t elems, int eb) {
  x.ptr = static_cast<char*>(x.ptr) + elems * eb;
  return x;
}

}  // namespace

SQKV_EXPORT sqkv_status ra_attention_bwd_preprocess(sqkv_view o, sqkv_view dout, float* D, int B, int H, int n,
                                                    int d, sqkv_dtype dtype, void* stream) {
  if (B < 1 || H < 1 || n < 0) return fail(SQKV_EINVAL, "sizes must be positive");
  if (d != 64 && d != 128) return fail(SQKV_EUNSUPPORTED, "head dim d=%d not in {64, 128}", d);
  if (!dtype_ok(dtype)) return fail(SQKV_EUNSUPPORTED, "dtype must be SQKV_F32 or SQKV_BF16");
  if (n == 0) return ok();
  // 16 threads per row in a one-dimensional grid
  if ((int64_t)B * H * n > (1ll << 28) - 16) return fail(SQKV_EUNSUPPORTED, "B*H*n must be below 2^28 - 16 rows");
  if (!o.ptr || !dout.ptr || !D) return fail(SQKV_EINVAL, "null pointer");
  if (!strides_nonneg(o) || !strides_nonneg(dout)) return fail(SQKV_EINVAL, "negative stride");
  const int eb = dtype_bytes(dtype);
  if (!view_aligned(o, eb) || !view_aligned(dout, eb) || ((uintptr_t)D) % 4)
    return fail(SQKV_EUNSUPPORTED, "pointers and strides must be 16-byte aligned (D 4-byte)");
  Range rD = dense_range(D, (int64_t)B * H * n, 4);
  if (overlap(rD, view_range(o, B, H, n, d, eb)) || overlap(rD, view_range(dout, B, H, n, d, eb)))
    return fail(SQKV_EINVAL, "D overlaps o or dout");
  sqkv::RowDotParams p;
  p.o = o.ptr; p.o_sb = o.sb; p.o_sh = o.sh; p.o_sn = o.sn;
  p.dout = dout.ptr; p.do_sb = dout.sb; p.do_sh = dout.sh; p.do_sn = dout.sn;
  p.D = D;
  p.B = B; p.H = H; p.n = n;
  p.dtype = dtype;
  return hip_status(sqkv::launch_bwd_rowdot(p, d, (hipStream_t)stream), "ra_attention_bwd_preprocess launch");
}

SQKV_EXPORT sqkv_status ra_chunk_attention_bwd(sqkv_view q, sqkv_view k, sqkv_view v, sqkv_view dout,
                                               const float* lse, const float* D, sqkv_view dq, sqkv_view dk,
                                               sqkv_view dv, int B, int Hq, int Hkv, int n_q, int n_k, int d,
                                               sqkv_dtype in_dtype, float scale, int causal, int64_t q_pos0,
                                               int64_t k_pos0, void* stream) {
  sqkv_status st = check_bwd(q, k, v, dout, lse, D, dq, dk, dv, B, Hq, Hkv, n_q, n_k, 0, 0, d, in_dtype, scale);
  if (st != SQKV_OK || n_q == 0 || n_k == 0) return st;
  sqkv::BwdParams p = make_bwd(q, k, v, dout, lse, D, dq, dk, dv, B, Hq, Hkv, n_q, n_k, scale, causal, q_pos0, k_pos0);
  return hip_status(sqkv::launch_attn_bwd_bf16(p, d, (hipStream_t)stream), "ra_chunk_attention_bwd launch");
}

SQKV_EXPORT sqkv_status ra_ring_attention_bwd(sqkv_view q, sqkv_view k, sqkv_view v, int64_t k_chunk_stride,
                                              int64_t v_chunk_stride, sqkv_view dout, const float* lse,
                                              const float* D, sqkv_view dq, sqkv_view dk, sqkv_view dv,
                                              int64_t dkv_chunk_stride, int B, int Hq, int Hkv, int n, int d,
                                              int P, int rank, sqkv_dtype in_dtype, float scale, int causal,
                                              void* stream) {
  if (P < 1 || rank < 0 || rank >= P) return fail(SQKV_EINVAL, "need P >= 1 and 0 <= rank < P (P=%d rank=%d)", P, rank);
  if (k_chunk_stride < 0 || v_chunk_stride < 0 || dkv_chunk_stride < 0) return fail(SQKV_EINVAL, "negative chunk stride");
  if ((k_chunk_stride * 2) % 16 || (v_chunk_stride * 2) % 16 || (dkv_chunk_stride * 4) % 16)
    return fail(SQKV_EUNSUPPORTED, "chunk strides must be multiples of 16 bytes");
  sqkv_status st = check_bwd(q, k, v, dout, lse, D, dq, dk, dv, B, Hq, Hkv, n, n,
                             (int64_t)(P - 1) * std::max(k_chunk_stride, v_chunk_stride) * 2,
                             (int64_t)(P - 1) * dkv_chunk_stride * 4, d, in_dtype, scale);
  if (st != SQKV_OK || n == 0) return st;
  if (!rows_disjoint(d, {{dk.sb, B}, {dk.sh, Hkv}, {dk.sn, n}, {dkv_chunk_stride, P}}) ||
      !rows_disjoint(d, {{dv.sb, B}, {dv.sh, Hkv}, {dv.sn, n}, {dkv_chunk_stride, P}}))
    return fail(SQKV_EINVAL, "the chunks of dk or dv overlap each other");
  // chunks in ring order, the rank's own first: j = (rank - s) mod P; with a
  // causal mask the chunks after the rank's own are entirely in the future
  const int nseg = causal ? rank + 1 : P;
  for (int s = 0; s < nseg; ++s) {
    const int j = (rank - s + P) % P;
    sqkv::BwdParams p = make_bwd(q, offset_view(k, j * k_chunk_stride, 2), offset_view(v, j * v_chunk_stride, 2),
                                 dout, lse, D, dq, offset_view(dk, j * dkv_chunk_stride, 4),
                                 offset_view(dv, j * dkv_chunk_stride, 4), B, Hq, Hkv, n, n, scale, causal,
                                 (int64_t)rank * n, (int64_t)j * n);
    hipError_t e = sqkv::launch_attn_bwd_bf16(p, d, (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e, "ra_ring_attention_bwd launch");
  }
  return ok();
}

SQKV_EXPORT sqkv_status ra_lse_merge(sqkv_view o_a, const float* lse_a, sqkv_dtype a_dtype, sqkv_view o_b,
                                     const float* lse_b, sqkv_dtype b_dtype, sqkv_view o_out, float* lse_out,
                                     sqkv_dtype out_dtype, int B, int H, int n, int d, void* stream) {
  if (B < 1 || H < 1 || n < 0) return fail(SQKV_EINVAL, "sizes must be positive");
  if (d != 64 && d != 128) return fail(SQKV_EUNSUPPORTED, "head dim d=%d not in {64, 128}", d);
  if (!dtype_ok(a_dtype) || !dtype_ok(b_dtype) || !dtype_ok(out_dtype))
    return fail(SQKV_EUNSUPPORTED, "dtype must be SQKV_F32 or SQKV_BF16");
  if (B > 65535 || H > 65535) return fail(SQKV_EUNSUPPORTED, "B and H must be <= 65535");
  // a grid row of four elements per thread per (b, h)
  if ((int64_t)n * (d / 4) > 0xffffff00ll) return fail(SQKV_EUNSUPPORTED, "n*d/4 must be below 2^32 - 256");
  if (n == 0) return ok();
  if (!o_a.ptr || !o_b.ptr || !o_out.ptr || !lse_a || !lse_b || !lse_out)
    return fail(SQKV_EINVAL, "null pointer");
  for (const sqkv_view* v : {&o_a, &o_b, &o_out})
    if (!strides_nonneg(*v)) return fail(SQKV_EINVAL, "negative stride");
  if (!view_aligned(o_a, dtype_bytes(a_dtype)) || !view_aligned(o_b, dtype_bytes(b_dtype)) ||
      !view_aligned(o_out, dtype_bytes(out_dtype)))
    return fail(SQKV_EUNSUPPORTED, "pointers and strides must be 16-byte aligned");
  if (((uintptr_t)lse_a | (uintptr_t)lse_b | (uintptr_t)lse_out) % 4)
    return fail(SQKV_EUNSUPPORTED, "lse must be 4-byte aligned");
  const int64_t rows = (int64_t)B * H * n;
  Range ro = view_range(o_out, B, H, n, d, dtype_bytes(out_dtype));
  Range rl = dense_range(lse_out, rows, 4);
  Range ra = view_range(o_a, B, H, n, d, dtype_bytes(a_dtype));
  Range rb = view_range(o_b, B, H, n, d, dtype_bytes(b_dtype));
  Range rla = dense_range(lse_a, rows, 4), rlb = dense_range(lse_b, rows, 4);
  bool alias_a = same_view(o_out, o_a) && out_dtype == a_dtype;
  bool alias_b = same_view(o_out, o_b) && out_dtype == b_dtype;
  if (!rows_disjoint(o_out, B, H, n, d)) return fail(SQKV_EINVAL, "rows of o_out overlap each other");
  if ((!alias_a && overlap(ro, ra)) || (!alias_b && overlap(ro, rb)))
    return fail(SQKV_EINVAL, "o_out partially overlaps an input");
  if ((lse_out != lse_a && overlap(rl, rla)) || (lse_out != lse_b && overlap(rl, rlb)))
    return fail(SQKV_EINVAL, "lse_out partially overlaps an input");
  if (overlap(ro, rl) || overlap(ro, rla) || overlap(ro, rlb) || overlap(rl, ra) || overlap(rl, rb))
    return fail(SQKV_EINVAL, "o and lse buffers overlap");
  sqkv::MergeParams p;
  p.oa = o_a.ptr; p.a_sb = o_a.sb; p.a_sh = o_a.sh; p.a_sn = o_a.sn; p.lse_a = lse_a; p.a_dtype = a_dtype;
  p.ob = o_b.ptr; p.b_sb = o_b.sb; p.b_sh = o_b.sh; p.b_sn = o_b.sn; p.lse_b = lse_b; p.b_dtype = b_dtype;
  p.oo = o_out.ptr; p.o_sb = o_out.sb; p.o_sh = o_out.sh; p.o_sn = o_out.sn; p.lse_o = lse_out;
  p.o_dtype = out_dtype;
  p.B = B; p.H = H; p.n = n;
  return hip_status(sqkv::launch_lse_merge(p, d, (hipStream_t)stream), "ra_lse_merge launch");
}

namespace {

sqkv_status check_permute(const void* src, void* dst, int P, int64_t L, int H_src, int H_dst, int d,
                          int elem_bytes, const char* who) {
  if (P < 1 || L < 0 || H_src < 1 || H_dst < 1 || d < 1)
    return fail(SQKV_EINVAL, "%s: sizes must be positive", who);
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8)
    return fail(SQKV_EINVAL, "%s: elem_bytes must be 1, 2, 4 or 8", who);
  if (L % P) return fail(SQKV_EINVAL, "%s: L=%lld not divisible by P=%d", who, (long long)L, P);
  if (H_dst % P) return fail(SQKV_EINVAL, "%s: heads (%d) not divisible by the group size P=%d", who, H_dst, P);
  if (H_dst % H_src) return fail(SQKV_EINVAL, "%s: H_dst=%d is not a multiple of H_src=%d", who, H_dst, H_src);
  const int64_t bytes_src = L * H_src * (int64_t)d * elem_bytes;
  const int64_t bytes_dst = L * H_dst * (int64_t)d * elem_bytes;
  if (bytes_dst == 0) return ok();
  if (!src || !dst) return fail(SQKV_EINVAL, "%s: null pointer", who);
  if (((uintptr_t)src | (uintptr_t)dst) % elem_bytes)
    return fail(SQKV_EUNSUPPORTED, "%s: pointers must be aligned to the element size", who);
  if (overlap(dense_range(src, bytes_src, 1), dense_range(dst, bytes_dst, 1)))
    return fail(SQKV_EINVAL, "%s: src and dst overlap", who);
  if (bytes_dst / elem_bytes >= (1ll << 32) - 4096)
    return fail(SQKV_EUNSUPPORTED, "%s: more than 2^32 elements per call", who);
  if (L >= (1ll << 31)) return fail(SQKV_EUNSUPPORTED, "%s: L must be < 2^31", who);
  return ok();
}

}  // namespace

SQKV_EXPORT sqkv_status ulysses_seq_to_head(const void* src, void* dst, int P, int64_t L, int H_src, int H_dst,
                                            int d, int elem_bytes, void* stream) {
  sqkv_status st = check_permute(src, dst, P, L, H_src, H_dst, d, elem_bytes, "ulysses_seq_to_head");
  if (st != SQKV_OK || L == 0) return st;
  sqkv::PermuteParams p;
  p.src = (const unsigned char*)src;
  p.dst = (unsigned char*)dst;
  p.L = L;
  p.n = L / P;
  p.P = P;
  p.H_src = H_src;
  p.Hl = H_dst / P;
  p.R = H_dst / H_src;
  p.row_bytes = (int64_t)d * elem_bytes;
  return hip_status(sqkv::launch_seq_to_head(p, (hipStream_t)stream), "ulysses_seq_to_head launch");
}

SQKV_EXPORT sqkv_status ulysses_head_to_seq(const void* src, void* dst, int P, int64_t L, int H, int d,
                                            int elem_bytes, void* stream) {
  sqkv_status st = check_permute(src, dst, P, L, H, H, d, elem_bytes, "ulysses_head_to_seq");
  if (st != SQKV_OK || L == 0) return st;
  sqkv::PermuteParams p;
  p.src = (const unsigned char*)src;
  p.dst = (unsigned char*)dst;
  p.L = L;
  p.n = L / P;
  p.P = P;
  p.H_src = H;
  p.Hl = H / P;
  p.R = 1;
  p.row_bytes = (int64_t)d * elem_bytes;
  return hip_status(sqkv::launch_head_to_seq(p, (hipStream_t)stream), "ulysses_head_to_seq launch");
}

SQKV_EXPORT sqkv_status usp_attention(const void* q, const void* k, const void* v, void* o, void* work_q,
                                      void* work_k, void* work_v, void* work_o, float* lse, int P_u, int P_r,
                                      int64_t L, int H, int H_kv, int d, float scale, int causal, void* stream) {
  if (P_u < 1 || P_r < 1) return fail(SQKV_EINVAL, "need P_u >= 1 and P_r >= 1 (P_u=%d P_r=%d)", P_u, P_r);
  const int P = P_u * P_r;
  if (L < 0 || L % P) return fail(SQKV_EINVAL, "L=%lld must be a multiple of P_u*P_r=%d", (long long)L, P);
  if (H < 1 || H_kv < 1 || H % H_kv) return fail(SQKV_EINVAL, "H (%d) must be a multiple of H_kv (%d)", H, H_kv);
  if (H % P_u) return fail(SQKV_EINVAL, "H (%d) must be a multiple of P_u (%d)", H, P_u);
  if (P_u % H_kv && H_kv % P_u)
    return fail(SQKV_EINVAL, "key/value heads (%d) and P_u (%d): one must divide the other", H_kv, P_u);
  // what the attention phase would reject is rejected here, before the first
  // phase is enqueued
  if (d != 64 && d != 128) return fail(SQKV_EUNSUPPORTED, "head dim d=%d not in {64, 128}", d);
  if (L / P_r > (1ll << 30)) return fail(SQKV_EUNSUPPORTED, "ring chunks of L/P_r=%lld tokens are above 2^30", (long long)(L / P_r));
  if (H / P_u > 65535) return fail(SQKV_EUNSUPPORTED, "H/P_u must be <= 65535");
  if (L == 0) return ok();
  if (!q || !k || !v || !o || !work_q || !work_k || !work_v || !work_o || !lse)
    return fail(SQKV_EINVAL, "null pointer");
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)work_q | (uintptr_t)work_k |
       (uintptr_t)work_v | (uintptr_t)work_o) % 16 || ((uintptr_t)lse) % 4)
    return fail(SQKV_EUNSUPPORTED, "q, k, v, o and the work buffers must be 16-byte aligned, lse 4-byte");
  const int64_t n = L / P, S = L / P_r;          // tokens per shard, per ring chunk (= P_u * n)
  const int Hl = H / P_u, Hkd = std::max(H_kv, P_u), Hkl = Hkd / P_u;
  const int64_t qe = (int64_t)P * n * H * d, ke = (int64_t)P * n * H_kv * d, we = (int64_t)P_r * P_u * S * Hkl * d;
  {
    Range rq = dense_range(q, qe, 2), rk = dense_range(k, ke, 2), rv = dense_range(v, ke, 2), ro = dense_range(o, qe, 2);
    Range wq = dense_range(work_q, qe, 2), wk = dense_range(work_k, we, 2), wv = dense_range(work_v, we, 2),
          wo = dense_range(work_o, qe, 2), rl = dense_range(lse, (int64_t)P_r * P_u * Hl * S, 4);
    const Range* all[] = {&rq, &rk, &rv, &ro, &wq, &wk, &wv, &wo, &rl};
    for (int i = 0; i < 9; ++i)
      for (int j = i + 1; j < 9; ++j)
        if ((i >= 3 || j >= 3) && overlap(*all[i], *all[j]))
          return fail(SQKV_EINVAL, "usp_attention buffers overlap (%d, %d)", i, j);
  }
  auto at = [](const void* base, int64_t elems, int eb) {
    return static_cast<const char*>(base) + elems * eb;
  };
  // 1. Ulysses inside every ring row i_r: its P_u shards (a contiguous run of
  //    S tokens) become P_u head shares of the whole run
  for (int ir = 0; ir < P_r; ++ir) {
    const int64_t row_q = (int64_t)ir * P_u * n * H * d, row_k = (int64_t)ir * P_u * n * H_kv * d;
    const int64_t row_wk = (int64_t)ir * P_u * S * Hkl * d;
    sqkv_status st = ulysses_seq_to_head(at(q, row_q, 2), (void*)at(work_q, row_q, 2), P_u, S, H, H, d, 2, stream);
    if (st == SQKV_OK) st = ulysses_seq_to_head(at(k, row_k, 2), (void*)at(work_k, row_wk, 2), P_u, S, H_kv, Hkd, d, 2, stream);
    if (st == SQKV_OK) st = ulysses_seq_to_head(at(v, row_k, 2), (void*)at(work_v, row_wk, 2), P_u, S, H_kv, Hkd, d, 2, stream);
    if (st != SQKV_OK) return st;
  }
  // 2. a ring over the P_r rows for every head share i_u: ring rank i_r holds
  //    tokens i_r*S .. of heads i_u*H/P_u ..; chunk j of its key/value pool is
  //    row j's share i_u
  for (int iu = 0; iu < P_u; ++iu)
    for (int ir = 0; ir < P_r; ++ir) {
      const int64_t sq = ((int64_t)ir * P_u + iu) * S * Hl * d, sk = (int64_t)iu * S * Hkl * d;
      sqkv_view qv{(void*)at(work_q, sq, 2), 0, d, (int64_t)Hl * d};
      sqkv_view ov{(void*)at(work_o, sq, 2), 0, d, (int64_t)Hl * d};
      sqkv_view kv{(void*)at(work_k, sk, 2), 0, d, (int64_t)Hkl * d};
      sqkv_view vv{(void*)at(work_v, sk, 2), 0, d, (int64_t)Hkl * d};
      const int64_t cs = (int64_t)P_u * S * Hkl * d;
      sqkv_status st = ra_ring_attention(qv, kv, vv, cs, cs, ov, lse + ((int64_t)ir * P_u + iu) * Hl * S, 1, Hl, Hkl,
                                         (int)S, d, P_r, ir, SQKV_BF16, SQKV_BF16, scale, causal, stream);
      if (st != SQKV_OK) return st;
    }
  // 3. back to the sequence layout inside every ring row
  for (int ir = 0; ir < P_r; ++ir) {
    const int64_t row_q = (int64_t)ir * P_u * n * H * d;
    sqkv_status st = ulysses_head_to_seq(at(work_o, row_q, 2), (void*)at(o, row_q, 2), P_u, S, H, d, 2, stream);
    if (st != SQKV_OK) return st;
  }
  return ok();
}
