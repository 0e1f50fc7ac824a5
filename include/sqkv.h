/*
 * sqkv.h -- C ABI of libsqkv: chunked ring attention and the Ulysses
 * sequence<->head layout transform on one AMD MI355X (gfx950).
 *
 * Sources (the pages this library implements):
 *   [RA] Ring-attention Q&A "Как работает sequence parallelism в контексте LLM?"
 *        (aivaro.ru, answer 425): sections 2-3 (contiguous sequence chunks,
 *        ring of devices, P-1 exchanges) and section 5 (per-chunk scores,
 *        max, exp, normaliser, output, merged by an online softmax).
 *   [UL] "Метод контекстного параллелизма Ulysses" (Telegram channel
 *        stuffynlp, post 213): the all_to_all from [local_seqlen, global_heads,
 *        head_dim] to [global_seqlen, local_heads, head_dim] and back, the
 *        head-count limit and GQA key/value head copying.
 *   [HF] "Paralelismo de secuencias en 🤗 accelerate": section "En qué se
 *        diferencia Ulysses SP de FSDP CP" (heads divisible by the group size).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *   never allocates, frees or synchronises; each call validates its arguments
 *   on the host and then enqueues kernels on `stream` (a hipStream_t; NULL is
 *   the null stream).  Results are ready when the stream's work completes.
 * - Validation happens before any HIP call.  A non-OK status means nothing was
 *   enqueued; sqkv_last_error() then returns a message (thread-local).
 * - All calls are stateless and may be called from several host threads.
 *   Calls that overlap in time on one device must not write the same memory.
 * - Attention tensors are 4-D [B, H, n, d] views: element (b, h, t, e) sits at
 *   ptr + b*sb + h*sh + t*sn + e (strides in ELEMENTS, innermost stride 1).
 *   A [S, H, d] tensor (one Ulysses share) is the view B=1, sb=0 (unused),
 *   sh=d, sn=H*d.  Row statistics `lse` are dense float32 [B, H, n]:
 *   element (b, h, t) at lse + (b*H + h)*n + t.
 * - lse is the natural-log log-sum-exp of the scaled logits over the visible
 *   keys.  A query row with no visible key has output 0 and lse = -inf; a
 *   partial with lse = -inf is the identity of the merge.
 */
#ifndef SQKV_H_
#define SQKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sqkv_status {
  SQKV_OK = 0,
  SQKV_EINVAL = 1,       /* inconsistent sizes, null pointers, bad aliasing */
  SQKV_EUNSUPPORTED = 2, /* valid request outside what the kernels implement */
  SQKV_EHIP = 3          /* the HIP runtime reported an error on launch */
} sqkv_status;

typedef enum sqkv_dtype {
  SQKV_F32 = 0,  /* IEEE binary32 */
  SQKV_BF16 = 1  /* bfloat16 (upper half of binary32), round-to-nearest-even */
} sqkv_dtype;

/* A strided [B, H, n, d] view; strides in elements; the d stride is 1. */
typedef struct sqkv_view {
  void* ptr;
  int64_t sb, sh, sn;
} sqkv_view;

/*
 * ra_chunk_attention -- one ring step: a query chunk against one key/value
 * chunk, merged into a running result.  [RA] section 5: scores Q K^T, row
 * max, exp, row sum (normaliser) and the weighted sum of V for the chunk,
 * then the online-softmax rescale that folds this chunk's partial into the
 * running output.
 *
 *   q      [B, Hq,  n_q, d]  in_dtype          query chunk
 *   k, v   [B, Hkv, n_k, d]  in_dtype          key / value chunk
 *   o_in   [B, Hq,  n_q, d]  acc_dtype         running output, or ptr == NULL
 *   lse_in [B, Hq,  n_q]     float32           running lse (NULL iff o_in.ptr is)
 *   o_out  [B, Hq,  n_q, d]  out_dtype         merged output
 *   lse_out[B, Hq,  n_q]     float32           merged lse
 *
 * Query row t sits at global position q_pos0 + t and key u at k_pos0 + u;
 * with causal != 0 a key is visible iff its position <= the query's.
 * Logits are scale * (q . k) with scale > 0.  Query head h reads key/value
 * head h / (Hq / Hkv) (GQA).  Without o_in the call writes this chunk's
 * partial (O_j, lse_j); with o_in it writes merge((o_in, lse_in), (O_j, lse_j)).
 * o_out may be exactly o_in (same pointer, strides and dtype) and lse_out may
 * be exactly lse_in: the update is then in place.  Any other overlap between
 * an output and an input is rejected.
 *
 * Supported: d in {64, 128}; in_dtype F32 (fp32 arithmetic throughout) or
 * BF16 (bf16 MFMA products, fp32 accumulation, softmax weights rounded to
 * bf16 for the P*V product); acc_dtype, out_dtype F32 or BF16.  Pointers must
 * be 16-byte aligned, every stride a multiple of 16 bytes and key/value row
 * strides below 16 MiB; with BF16 inputs the key/value row strides must also
 * be at least d (no overlapping rows).  B and Hq at most 65535, n_q and n_k at
 * most 2^30 (F32 queries: below 2^30 - 128), B*Hq*ceil(n_q/256) below 2^31.
 * Keys a query cannot see (masked, or
 * past the chunk)
 * still pass through the P*V product with weight 0, so K and V must be
 * finite.
 * Returns SQKV_OK, SQKV_EINVAL (null pointer, Hq % Hkv != 0, negative size,
 * scale not finite and > 0, overlap, rows of o_out that share elements),
 * SQKV_EUNSUPPORTED (d, dtype, alignment, strides) or SQKV_EHIP.
 */
sqkv_status ra_chunk_attention(sqkv_view q, sqkv_view k, sqkv_view v,
                               sqkv_view o_in, const float* lse_in,
                               sqkv_view o_out, float* lse_out,
                               int B, int Hq, int Hkv, int n_q, int n_k, int d,
                               sqkv_dtype in_dtype, sqkv_dtype acc_dtype, sqkv_dtype out_dtype,
                               float scale, int causal, int64_t q_pos0, int64_t k_pos0,
                               void* stream);

/*
 * ra_ring_attention -- the whole ring for one virtual rank, with the P
 * key/value chunks resident in one HBM pool.  [RA] sections 2-3: the
 * sequence of length L = P*n is cut into P contiguous chunks (chunk j holds
 * positions j*n .. j*n + n - 1); the rank holding query chunk `rank` meets
 * every key/value chunk once, its own first and then, at step s, the chunk
 * that arrived from the previous device, j = (rank - s) mod P.  The send and
 * receive of the pages become reading chunk j in place, and [RA] section 5's
 * per-step merge is the online-softmax rescale of one running (max, sum,
 * output) state that a single launch carries across the chunks.
 *
 *   q        [B, Hq, n, d]  in_dtype      the rank's query chunk (positions
 *                                         rank*n ..)
 *   k, v     [B, Hkv, n, d] in_dtype      chunk 0 of the pool; chunk j starts
 *                                         j*k_chunk_stride (v_chunk_stride)
 *                                         elements after it
 *   o        [B, Hq, n, d]  out_dtype     result
 *   lse      [B, Hq, n]     float32       result (natural log)
 *
 * With causal != 0, chunks after the rank's own (j > rank) are skipped,
 * earlier ones are fully visible and the rank's own chunk is masked on its
 * diagonal.  Same support and status codes as ra_chunk_attention;
 * additionally EINVAL for rank outside [0, P) or P < 1, EUNSUPPORTED for
 * chunk strides that are not multiples of 16 bytes.
 */
sqkv_status ra_ring_attention(sqkv_view q, sqkv_view k, sqkv_view v,
                              int64_t k_chunk_stride, int64_t v_chunk_stride,
                              sqkv_view o, float* lse,
                              int B, int Hq, int Hkv, int n, int d, int P, int rank,
                              sqkv_dtype in_dtype, sqkv_dtype out_dtype,
                              float scale, int causal, void* stream);

/*
 * ra_ring_attention_packed -- ra_ring_attention (causal) over a sequence that
 * packs several samples one after another.  [HF], sequence-parallel
 * configuration notes: samples packed into one sequence are told apart by
 * position_ids, and an attention that treats the packed sequence as one
 * sample (as sdpa does there) lets samples see each other.  Here a query at
 * global position t sees key u iff u <= t and both lie in the same sample.
 *
 *   seg_starts  int64 [n_seg], DEVICE memory: the samples' start positions in
 *               the whole sequence of P*n tokens, strictly increasing,
 *               seg_starts[0] = 0 (what position_ids resetting to 0 marks).
 *               Shared by every batch row.
 *
 * Other arguments as ra_ring_attention (always causal).  Chunks and tiles
 * holding no key of a block's samples are skipped.  EINVAL additionally for
 * n_seg < 1 or a null seg_starts; EUNSUPPORTED for in_dtype other than BF16
 * or a seg_starts pointer not 8-byte aligned.  The contents of seg_starts
 * are not checked (they live on the device); out-of-order starts give
 * undefined attention results but no out-of-bounds access.
 */
sqkv_status ra_ring_attention_packed(sqkv_view q, sqkv_view k, sqkv_view v,
                                     int64_t k_chunk_stride, int64_t v_chunk_stride,
                                     sqkv_view o, float* lse, const int64_t* seg_starts, int n_seg,
                                     int B, int Hq, int Hkv, int n, int d, int P, int rank,
                                     sqkv_dtype in_dtype, sqkv_dtype out_dtype, float scale, void* stream);

/*
 * Backward of chunked attention.  [RA], "pet project" steps 5-7: after the
 * ring forward a loss is computed and backpropagated, and the result must
 * match full attention.  The pages give no formulas; the gradients are the
 * plain calculus of O = softmax(scale * Q K^T) V, row by row:
 *   P = exp(scale * q.k - lse),  dV = P^T dO,  dP = dO V^T,
 *   D = rowsum(dO * O),  dS = P * (dP - D),
 *   dQ = scale * dS K,  dK = scale * dS^T Q
 * (GQA: a key/value head's gradients sum over the query heads that read it).
 * With lse the rows' log-sum-exp over ALL keys -- what the forward returned --
 * P of one (query chunk, key chunk) pair is the full softmax restricted to
 * that pair, so the ring backward is a sum of per-pair contributions.
 *
 * ra_attention_bwd_preprocess: D[b,h,t] = sum_e dout[b,h,t,e] * o[b,h,t,e]
 * (o, dout [B, H, n, d] views of `dtype`, D dense float32 [B, H, n]).  Run it
 * once per query chunk on the final output before the backward calls.
 * EUNSUPPORTED also when B*H*n is 2^28 - 16 rows or more.
 */
sqkv_status ra_attention_bwd_preprocess(sqkv_view o, sqkv_view dout, float* D,
                                        int B, int H, int n, int d, sqkv_dtype dtype, void* stream);

/*
 * ra_chunk_attention_bwd -- one chunk pair: ADDS its share into the float32
 * gradients (the caller zeroes them before the first pair).
 *
 *   q, dout  [B, Hq, n_q, d]  bf16        query chunk and upstream gradient
 *   k, v     [B, Hkv, n_k, d] bf16        key/value chunk
 *   lse, D   [B, Hq, n_q]     float32     dense: the forward's lse over all
 *                                         keys (natural log) and the
 *                                         preprocess output
 *   dq       [B, Hq, n_q, d]  float32     += scale * dS K
 *   dk, dv   [B, Hkv, n_k, d] float32     += scale * dS^T Q, P^T dO
 *
 * Positions and the causal mask as in ra_chunk_attention.  Rows with
 * lse = -inf (no visible key anywhere) contribute nothing.  Supported: d in
 * {64, 128}, in_dtype BF16 (bf16 MFMA products, fp32 accumulation; P and dS
 * rounded to bf16 for the products that take them), pointers and strides
 * 16-byte aligned, row strides below 16 MiB and at least d (no overlapping
 * rows in q, k, v or dout).  Returns SQKV_OK, SQKV_EINVAL
 * (null pointer, sizes, Hq % Hkv, scale, a gradient buffer overlapping an
 * input or another gradient, rows of a gradient that share elements),
 * SQKV_EUNSUPPORTED (d, dtype, alignment,
 * strides, B*Hq*ceil(n_q/256) or B*Hkv*ceil(n_k/128) at 2^23 or more) or
 * SQKV_EHIP.
 */
sqkv_status ra_chunk_attention_bwd(sqkv_view q, sqkv_view k, sqkv_view v, sqkv_view dout,
                                   const float* lse, const float* D,
                                   sqkv_view dq, sqkv_view dk, sqkv_view dv,
                                   int B, int Hq, int Hkv, int n_q, int n_k, int d,
                                   sqkv_dtype in_dtype, float scale, int causal,
                                   int64_t q_pos0, int64_t k_pos0, void* stream);

/*
 * ra_ring_attention_bwd -- the backward of ra_ring_attention for one virtual
 * rank: the rank's query chunk against the P resident chunks in ring order
 * (own first; with causal != 0 the chunks after the rank's own are skipped).
 * dq [B, Hq, n, d] float32 receives the rank's dQ; the pool gradients dk, dv
 * (chunk 0 at dk/dv, chunk j dkv_chunk_stride elements further, float32)
 * receive the rank's share of every chunk's dK, dV -- calling it for every
 * rank accumulates the full pool gradients.  Same support and status codes
 * as ra_chunk_attention_bwd; additionally EINVAL for rank outside [0, P) or
 * pool chunks of dk or dv that share elements, and EUNSUPPORTED for chunk
 * strides that are not multiples of 16 bytes.
 */
sqkv_status ra_ring_attention_bwd(sqkv_view q, sqkv_view k, sqkv_view v,
                                  int64_t k_chunk_stride, int64_t v_chunk_stride,
                                  sqkv_view dout, const float* lse, const float* D,
                                  sqkv_view dq, sqkv_view dk, sqkv_view dv, int64_t dkv_chunk_stride,
                                  int B, int Hq, int Hkv, int n, int d, int P, int rank,
                                  sqkv_dtype in_dtype, float scale, int causal, void* stream);

/*
 * ra_zigzag_attention -- causal ring attention for one virtual rank under the
 * zigzag assignment of the sequence.  [UL], opening paragraph, names
 * Ring/ZigZag among the context-parallel methods without defining it; the
 * reading taken here is the usual one: the sequence of length L is cut into
 * 2P equal pieces of c = L/(2P) tokens and rank r holds pieces r and
 * 2P-1-r, so that under a causal mask every rank has the same work ((2P-1)
 * fully visible piece pairs and 2 diagonal ones) instead of rank P-1 doing
 * 2P-1 times the work of rank 0.  A rank's local shard is its two pieces one
 * after the other: n = 2c rows, rows 0..c-1 at positions r*c .. r*c+c-1 and
 * rows c..2c-1 at positions (2P-1-r)*c .. .
 *
 *   q        [B, Hq, n, d]  in_dtype      the rank's local shard
 *   k, v     [B, Hkv, n, d] in_dtype      shard 0 of the pool (same zigzag
 *                                         layout); shard j starts
 *                                         j*k_chunk_stride (v_chunk_stride)
 *                                         elements after it
 *   o        [B, Hq, n, d]  out_dtype     result
 *   lse      [B, Hq, n]     float32       result (natural log)
 *   work_o   [B, Hq, n/2, d] float32, dense (element (b,h,t,e) at
 *            ((b*Hq + h)*(n/2) + t)*d + e), and
 *   work_lse [B, Hq, n/2]   float32, dense: caller-owned scratch, 16- and
 *            4-byte aligned, overlapping no other argument; contents on entry
 *            are ignored and on return unspecified.
 *
 * Enqueues three launches on `stream`: the early piece against the early
 * pieces of ranks r, r-1, .., 0; the late piece against all early pieces
 * (into the scratch); the late piece against the late pieces of ranks r, r+1,
 * .., P-1, merged with the scratch.  Same support and status codes as
 * ra_ring_attention; additionally EINVAL for odd n and null or overlapping
 * scratch.
 */
sqkv_status ra_zigzag_attention(sqkv_view q, sqkv_view k, sqkv_view v,
                                int64_t k_chunk_stride, int64_t v_chunk_stride,
                                sqkv_view o, float* lse, float* work_o, float* work_lse,
                                int B, int Hq, int Hkv, int n, int d, int P, int rank,
                                sqkv_dtype in_dtype, sqkv_dtype out_dtype,
                                float scale, void* stream);

/*
 * ra_zigzag_attention_noalloc -- ra_zigzag_attention for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same three launches, with the late
 * piece's fp32 partial (what work_o / work_lse hold above) kept in a
 * file-scope device array of the library instead of caller buffers.  It calls
 * no hipMalloc, hipFree or allocating routine.
 *
 * Arguments, layouts, support and status codes as ra_zigzag_attention
 * without work_o / work_lse.  Limit: the partial needs 4*(d+1) bytes per row
 * of B*Hq*n/2 rows, plus up to 255 bytes of alignment, within
 * ra_zigzag_attention_noalloc_max_bytes() (64 MiB); larger calls return
 * SQKV_EUNSUPPORTED before any HIP call.  Each GPU holds its own copy of the
 * array from the library's first use on it until the process ends (looked up
 * once per device with hipGetSymbolAddress on the device current at the
 * call, which must be the one `stream` and the buffers belong to).  Every
 * call on a GPU shares that GPU's array, so calls that overlap on one GPU
 * (other streams, other threads) race; calls on one stream are ordered.
 * Nothing in the array needs to start at zero: launch 2 writes the whole
 * partial before launch 3 reads it.
 */
sqkv_status ra_zigzag_attention_noalloc(sqkv_view q, sqkv_view k, sqkv_view v,
                                        int64_t k_chunk_stride, int64_t v_chunk_stride,
                                        sqkv_view o, float* lse,
                                        int B, int Hq, int Hkv, int n, int d, int P, int rank,
                                        sqkv_dtype in_dtype, sqkv_dtype out_dtype,
                                        float scale, void* stream);

/* Size in bytes of the array ra_zigzag_attention_noalloc works in. */
size_t ra_zigzag_attention_noalloc_max_bytes(void);

/*
 * ra_lse_merge -- the online-softmax merge of two partial attentions over
 * disjoint key sets ([RA] section 5, the rescale of the running output and
 * normaliser by the exponent of the change in the running maximum), in the
 * log-sum-exp form: lse = log(exp(lse_a) + exp(lse_b)),
 * o = exp(lse_a - lse) * o_a + exp(lse_b - lse) * o_b, evaluated in fp32
 * with the larger lse factored out.
 *
 *   o_a, lse_a (a_dtype), o_b, lse_b (b_dtype) : [B, H, n, d] and [B, H, n]
 *   o_out, lse_out (out_dtype)                  : result
 * o_out may be exactly o_a or o_b (same pointer, strides, dtype); lse_out may
 * be exactly lse_a or lse_b.  d in {64, 128}; 16-byte alignment as above;
 * n*d/4 below 2^32 - 256 (else EUNSUPPORTED); rows of o_out that share
 * elements are refused (EINVAL).
 */
sqkv_status ra_lse_merge(sqkv_view o_a, const float* lse_a, sqkv_dtype a_dtype,
                         sqkv_view o_b, const float* lse_b, sqkv_dtype b_dtype,
                         sqkv_view o_out, float* lse_out, sqkv_dtype out_dtype,
                         int B, int H, int n, int d, void* stream);

/*
 * ulysses_seq_to_head -- the all_to_all before attention ([UL]), on one HBM
 * pool holding all P shards.  dense src [P][L/P][H_src][d] (shard p = tokens
 * p*L/P ..) becomes dense dst [P][L][H_dst/P][d] (rank r = the whole sequence
 * for heads r*H_dst/P .. (r+1)*H_dst/P - 1):
 *     dst[r][p*(L/P) + t][h'] = src[p][t][ (r*H_dst/P + h') / (H_dst/H_src) ]
 * H_dst = H_src moves query (or output) heads; H_dst = R*H_src copies every
 * key/value head R times in place (GQA: [UL] copies KV heads up to the group
 * size; use H_dst = max(H_kv, P)).  Elements are moved as raw bits of
 * elem_bytes (1, 2, 4 or 8) bytes.  src and dst must not overlap.
 * EINVAL: null pointer, P < 1, L % P, H_dst % P, H_dst % H_src ([UL], [HF]:
 * the group cannot exceed the head count and must divide it), overlap.
 */
sqkv_status ulysses_seq_to_head(const void* src, void* dst, int P, int64_t L,
                                int H_src, int H_dst, int d, int elem_bytes, void* stream);

/*
 * ulysses_head_to_seq -- the all_to_all after attention ([UL]): dense src
 * [P][L][H/P][d] becomes dense dst [P][L/P][H][d], the inverse of
 * ulysses_seq_to_head with H_src = H_dst = H:
 *     dst[p][t][r*H/P + h'] = src[r][p*(L/P) + t][h']
 * Same arguments and errors as above.
 */
sqkv_status ulysses_head_to_seq(const void* src, void* dst, int P, int64_t L,
                                int H, int d, int elem_bytes, void* stream);

/*
 * usp_attention -- the hybrid of the two methods: Ulysses inside groups of
 * P_u ranks, a ring across P_r such groups.  [HF], closing remarks of the
 * Ulysses section, points to combining sequence and context parallelism (the
 * USP scheme) for still longer sequences; [UL] gives the per-group all_to_all
 * and its head limit.  Reading: P = P_u * P_r virtual ranks, rank p = i_r*P_u
 * + i_u holds tokens p*L/P ..; the P_u ranks of ring row i_r exchange heads
 * so that each holds the row's S = L/P_r contiguous tokens for heads
 * i_u*H/P_u ..; the P_r ranks with the same i_u then run ring attention over
 * the rows; the output goes back to the sequence layout.  All on one HBM
 * pool, as three phases of the other entry points.
 *
 *   q, o     dense [P][L/P][H][d] bf16         input / output (sequence layout)
 *   k, v     dense [P][L/P][H_kv][d] bf16
 *   work_q, work_o  dense [P_r][P_u][S][H/P_u][d] bf16      caller-owned scratch
 *   work_k, work_v  dense [P_r][P_u][S][Hk][d] bf16, Hk = max(H_kv, P_u)/P_u
 *            (key/value heads copied up to P_u as in ulysses_seq_to_head)
 *   lse      dense [P_r][P_u][H/P_u][S] float32: the rows' lse, by head share
 *
 * Causal masking uses global positions (ring rows are contiguous runs).
 * EINVAL: P_u or P_r < 1, L % (P_u*P_r), H % H_kv, H % P_u, neither of H_kv,
 * P_u dividing the other, null pointers, overlapping buffers.
 * EUNSUPPORTED: d not in {64, 128}, S above 2^30 tokens, H/P_u above 65535,
 * q, k, v, o or a work buffer not 16-byte aligned, lse not 4-byte aligned.
 * These are checked before the first phase is enqueued; after that the
 * status is that of the first failing phase (a HIP launch error).
 */
sqkv_status usp_attention(const void* q, const void* k, const void* v, void* o,
                          void* work_q, void* work_k, void* work_v, void* work_o, float* lse,
                          int P_u, int P_r, int64_t L, int H, int H_kv, int d,
                          float scale, int causal, void* stream);

/* Message for the last non-OK status returned on this host thread ("" if the
 * last call succeeded).  The string stays valid until the next call. */
const char* sqkv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SQKV_H_ */
