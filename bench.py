"""Benchmark of the chunked ring-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = one GPU's share of the causal 128k ring: rank 7 of P = 8 (its
16384-row query chunk, the last of the sequence) attending to all 8 resident
key/value chunks of 16384 tokens in ring order, its own (diagonal) chunk
first, in one launch that carries the online-softmax merge across the chunks
in registers; B=1, 32 heads, d=128, bf16 in, fp32 accumulation, bf16 out.
Inputs are drawn on the device from a seeded generator and are resident in
HBM before timing starts.  W untimed warm-up steps, then exactly K timed
steps between synchronisations; every launch is also bracketed by HIP events
on the stream it runs on, which give the kernel's mean and median launch
time for the roofline.

Printed: ONE JSON line on stdout with the metric, the roofline of the
chunk-attention kernel (MFMA-bound) on that launch, and the CPU oracle timed
on a seeded sample of the same workload (16384 query rows across all heads,
extrapolated to the full share by visible pairs, with the GPU's error on
those rows).  Extra figures on the other workloads go in "extras": the whole
32k ring (8 ranks x 8 chunks of 4096, non-causal) and the causal GQA Ulysses
share at 128k (4 query heads, 1 key/value head), each with its own roofline
object; the Ulysses permutes on 8 x [16384, 32, 128] bf16 with their HBM
roofline beside the same kernel run as a plain copy of the same bytes; the
GQA key/value replication of the Ulysses exchange at 128k (1 and 2 key/value
heads copied up to 8 ranks); the whole causal 128k ring under the contiguous
and the zigzag split; the backward of the 32k ring; the USP hybrid at 128k;
the 32k ring packing 2k-token samples; the fixed cost of an attention visit
(query tiles against 1..64 key tiles); the standalone lse merge of a 128k
ring step; the tiny fp32 ring; causal attention over 1,048,576 tokens; and,
with the CPU baseline, the oracle's Ulysses copies.  Logs go to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 (published; matrix and vector alike)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (published)
METRIC = "chunked-attention TFLOP/s (% bf16 MFMA peak); Ulysses permute GB/s (% HBM)"
HEADLINE = "ring_bf16_128k_rank7_causal"
ATTN_SRC = os.path.join(ROOT, "sequence_kv_chunk_amd", "csrc", "attn_bf16.hip")
PERMUTE_SRC = os.path.join(ROOT, "sequence_kv_chunk_amd", "csrc", "ulysses.hip")
PROFILES = os.path.join(ROOT, "profiles")
# committed rocprofv3 counter summaries, per workload (used while the kernel source is unchanged)
ATTN_COUNTERS = {
    "ring_bf16_128k_rank7_causal": ("attn_bf16_rank7_128k_traffic.json", "attn_bf16_rank7_128k_mfma.json"),
    "ring_bf16_32k": ("attn_bf16_ring32k_traffic.json", "attn_bf16_ring32k_mfma.json"),
    "ulysses_share_gqa_128k_causal": ("attn_bf16_gqa_share_128k_traffic.json", "attn_bf16_gqa_share_128k_mfma.json"),
}
PERMUTE_TRAFFIC_FILE = os.path.join(PROFILES, "ulysses_permute_131k_traffic.json")
REPLICATION_TRAFFIC_FILE = os.path.join(PROFILES, "ulysses_gqa_replication_131k_traffic.json")
EXTRAS = ("ring32k", "ulysses_share", "ulysses", "gqa_replication", "packed", "visit_lengths", "backward",
          "causal_split", "usp", "lse_merge", "f32_tiny", "f32_chunk", "capacity_1m")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash(path: str = ATTN_SRC) -> str:
    """sha256[:16] of a kernel file's code: `//` comments and blank lines are
    dropped, so that editing a comment keeps the counters valid."""
    lines = []
    with open(path, encoding="utf-8") as f:
        for ln in f:
            code = ln.split("//", 1)[0].rstrip()
            if code:
                lines.append(code)
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()[:16]


def load_profile(name: str, src: str):
    """A committed rocprofv3 counter summary, if it was taken on the current
    kernel source (else None: the counters describe older code)."""
    try:
        with open(os.path.join(PROFILES, name)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash(src):
        return None
    return t


def timed_launches(torch, fn, warmup, iters, flush=None):
    """Runs fn `warmup` times, then `iters` times, each bracketed by HIP events
    on the current stream (the one the library enqueues on).  With `flush`, a
    cache-evicting fill runs before every timed launch (outside its events).
    Returns (per-launch ms list, wall ms of the timed region without flushes
    or None)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * iters)]
    t0 = time.perf_counter()
    for i in range(iters):
        if flush is not None:
            flush()
        evs[2 * i].record()
        fn()
        evs[2 * i + 1].record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 if flush is None else None
    return [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(iters)], wall


def ms_stats(ts):
    return {"ms_mean": round(sum(ts) / len(ts), 4), "ms_median": round(statistics.median(ts), 4),
            "ms_min": round(min(ts), 4), "launches_timed": len(ts)}


def attn_roofline(name, flops_per_launch, ts, kernel="attn_bf16_kernel<128, false>"):
    """Roofline object of one attention launch: algorithmic FLOPs over the mean
    launch time (events), with HBM traffic and MFMA-busy counters from the
    committed rocprofv3 summaries when they match the current kernel code."""
    mean = sum(ts) / len(ts)
    achieved = flops_per_launch / (mean * 1e-3) / 1e12
    tr_file, mf_file = ATTN_COUNTERS.get(name, (None, None))
    traffic = load_profile(tr_file, ATTN_SRC) if tr_file else None
    mfma = load_profile(mf_file, ATTN_SRC) if mf_file else None
    return {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": None if traffic is None else traffic.get("bytes_per_launch"),
            "traffic_algorithmic": None if traffic is None else traffic.get("algorithmic_bytes_per_launch"),
            "kernel": kernel, "flops_per_launch": flops_per_launch,
            "launch_ms": round(mean, 4), "launch_ms_median": round(statistics.median(ts), 4),
            "mfma_busy_pct_counters": None if mfma is None else mfma.get("MfmaUtil_pct")}


# ---------------------------------------------------------------------------
# headline: rank 7's share of the causal 128k ring
# ---------------------------------------------------------------------------
def headline(api, torch, args):
    from sequence_kv_chunk_amd.synth import WORKLOADS, device_attention_inputs
    w = WORKLOADS[HEADLINE]
    x = device_attention_inputs(w)
    rank = w.query_ranks[0]
    q, kp, vp = x["q"][0], x["k"], x["v"]
    B, H, n, d = q.shape
    o = torch.empty((B, H, n, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B * H * n, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    log(f"workload {w.name}: inputs resident ({sum(t.numel() * 2 for t in x.values()) / 2**30:.2f} GiB)")

    def step():
        api.ra_ring_attention(q, kp, vp, o, lse, rank=rank, scale=1.0, causal=True)

    ts, wall = timed_launches(torch, step, args.warmup, args.steps)
    ms_step = wall / args.steps
    flops = w.flops()
    value = flops / (ms_step * 1e-3) / 1e12
    roof = attn_roofline(w.name, flops, ts)
    log(f"{w.name}: step {ms_step:.3f} ms (wall), launches mean {roof['launch_ms']:.3f} / median "
        f"{roof['launch_ms_median']:.3f} ms, {value:.1f} TFLOP/s, roofline frac {roof['frac']}")
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) on device; Q scaled by d^-0.5)",
        "config": {"workload": "ring_bf16_128k_rank7_causal: one GPU's share of the causal 131072-token ring, "
                               "rank 7 of 8 (query chunk of 16384 tokens, positions 114688..131071) against the "
                               "8 resident KV chunks of 16384 in ring order (1 diagonal + 7 full blocks), B=1, "
                               "32 heads, d=128, one launch per step",
                   "global_batch": 1, "seq_len": w.L, "heads": w.Hq, "head_dim": w.d, "chunks": w.P,
                   "query_rank": rank, "causal": True, "parallelism": "single GPU; one virtual rank's share"},
        "roofline": roof,
    }
    return result, (w, x, o, lse)


def host_facts():
    """CPU model, BLAS library and the cores this process may run on."""
    model = platform.processor() or "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        if libs:
            blas = f"{libs[0].get('internal_api')} {libs[0].get('version')}"
    except Exception:
        pass
    return model, cores, blas


def cpu_baseline(w, x, o, lse, torch, rows_per_head=512):
    """The fp64 oracle on a seeded sample of the headline workload: in every
    head, `rows_per_head` query rows evenly spaced over the chunk (the first
    and the last included) against every key each row sees.  Its time is
    extrapolated to the whole share by the count of visible (query, key)
    pairs; the GPU output on the sampled rows is compared with it."""
    import oracle
    from sequence_kv_chunk_amd.synth import bf16_bits_to_f64
    from threadpoolctl import threadpool_limits

    def bits(t):
        return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    model, cores, blas = host_facts()
    rank, n, P, H, d = w.query_ranks[0], w.n, w.P, w.Hq, w.d
    rows = np.unique(np.linspace(0, n - 1, rows_per_head).round().astype(np.int64))
    q_pos = rank * n + rows
    k_pos = np.arange(w.L)
    o_rows = o[0][:, rows].float().cpu().numpy().astype(np.float64)            # [H, r, d]
    l_rows = lse.view(H, n)[:, rows].cpu().numpy().astype(np.float64)          # [H, r]
    secs, err_o, err_l = 0.0, 0.0, 0.0
    with threadpool_limits(limits=cores):
        for h in range(H):
            qh = bf16_bits_to_f64(bits(x["q"][0][:, h:h + 1, rows]))                     # [1, 1, r, d]
            kf = bf16_bits_to_f64(bits(x["k"][:, :, h])).reshape(1, 1, P * n, d)         # chunks in order
            vf = bf16_bits_to_f64(bits(x["v"][:, :, h])).reshape(1, 1, P * n, d)
            t0 = time.perf_counter()
            ref_o, ref_l = oracle.attention_at_positions_fp64(qh, kf, vf, q_pos, k_pos)
            secs += time.perf_counter() - t0
            err_o = max(err_o, float(np.max(np.abs(ref_o[0, 0] - o_rows[h]))))
            err_l = max(err_l, float(np.max(np.abs(ref_l[0, 0] - l_rows[h]))))
    pairs_sample = int(np.sum(q_pos + 1)) * H
    full_pairs = w.unmasked_pairs()
    flops_sample = 4 * d * pairs_sample
    return {"value": round(flops_sample / secs / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{rows.size} query rows per head (evenly spaced over rank 7's chunk, first and last "
                      f"included) x {H} heads = {rows.size * H} rows, each against all of its visible keys "
                      f"(up to {w.L}); fp64 numpy oracle",
            "sample_seconds": round(secs, 2),
            "full_share_seconds_extrapolated": round(secs * full_pairs / pairs_sample, 1),
            "extrapolation": "sample time x visible pairs of the whole share / visible pairs of the sample",
            "cpu_model": model, "blas": blas, "threads": cores,
            "gpu_max_abs_err_on_sample": {"O": float(f"{err_o:.3e}"), "lse": float(f"{err_l:.3e}")}}


# ---------------------------------------------------------------------------
# extras
# ---------------------------------------------------------------------------
def bench_ring32k(api, torch, warmup=3, iters=10):
    """The whole 32k ring: 8 virtual ranks, each a 4096-row query chunk against
    all 8 resident KV chunks (one launch per rank), 32 heads, non-causal."""
    from sequence_kv_chunk_amd.synth import WORKLOADS, device_attention_inputs
    w = WORKLOADS["ring_bf16_32k"]
    x = device_attention_inputs(w)
    qs, kp, vp = x["q"], x["k"], x["v"]
    B, H, n, d = qs.shape[1:]
    o = torch.empty((B, H, n, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B * H * n, dtype=torch.float32, device="cuda")
    launches = []
    for r in range(w.P):
        ts, _ = timed_launches(torch, lambda: api.ra_ring_attention(qs[r], kp, vp, o, lse, rank=r, scale=1.0),
                               warmup if r == 0 else 1, iters)
        launches += ts
    ring_ms = sum(launches) / len(launches) * w.P
    res = {"ring_ms": round(ring_ms, 4), "TFLOP/s": round(w.flops() / (ring_ms * 1e-3) / 1e12, 1),
           "flops": w.flops(), "roofline": attn_roofline(w.name, w.flops() // w.P, launches),
           "workload": "ring_bf16_32k: 32768 tokens as 8 chunks of 4096, all 8 query chunks x 8 resident KV "
                       "chunks, B=1, 32 heads, d=128, non-causal (one launch per rank)"}
    del x, o, lse
    torch.cuda.empty_cache()
    return res


def cpu_oracle_share(w, x, o, lse, torch, rows_per_head=512):
    """The fp64 oracle on a seeded sample of the GQA share: in every query
    head, `rows_per_head` query rows evenly spaced over the sequence (the
    first and the last included) against every key each row sees; the time
    is extrapolated to the whole share by visible (query, key) pairs, and the
    GPU output on the sampled rows is compared with it."""
    import oracle
    from sequence_kv_chunk_amd.synth import bf16_bits_to_f64
    from threadpoolctl import threadpool_limits

    def bits(t):
        return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    model, cores, blas = host_facts()
    L, Hq, Hkv, d = w.L, w.Hq, w.Hkv, w.d
    rows = np.unique(np.linspace(0, L - 1, rows_per_head).round().astype(np.int64))
    o_rows = o[rows].float().cpu().numpy().astype(np.float64)                   # [r, Hq, d]
    l_rows = lse.view(Hq, L)[:, rows].cpu().numpy().astype(np.float64)          # [Hq, r]
    secs, err_o, err_l = 0.0, 0.0, 0.0
    with threadpool_limits(limits=cores):
        for hk in range(Hkv):
            kf = bf16_bits_to_f64(bits(x["k"][:, hk])).reshape(1, 1, L, d)
            vf = bf16_bits_to_f64(bits(x["v"][:, hk])).reshape(1, 1, L, d)
            for h in range(hk * (Hq // Hkv), (hk + 1) * (Hq // Hkv)):
                qh = bf16_bits_to_f64(bits(x["q"][rows, h])).reshape(1, 1, rows.size, d)
                t0 = time.perf_counter()
                ref_o, ref_l = oracle.attention_at_positions_fp64(qh, kf, vf, rows, np.arange(L))
                secs += time.perf_counter() - t0
                err_o = max(err_o, float(np.max(np.abs(ref_o[0, 0] - o_rows[:, h]))))
                err_l = max(err_l, float(np.max(np.abs(ref_l[0, 0] - l_rows[h]))))
    pairs_sample = int(np.sum(rows + 1)) * Hq
    full_pairs = Hq * L * (L + 1) // 2
    return {"value": round(4 * d * pairs_sample / secs / 1e12, 6), "unit": "TFLOP/s", "cores": cores,
            "kind": "oracle",
            "sample": f"{rows.size} query rows per head (evenly spaced over the {L} tokens, first and last "
                      f"included) x {Hq} heads, each against all of its visible keys; fp64 numpy oracle",
            "sample_seconds": round(secs, 2),
            "full_share_seconds_extrapolated": round(secs * full_pairs / pairs_sample, 1),
            "cpu_model": model, "blas": blas, "threads": cores,
            "gpu_max_abs_err_on_sample": {"O": float(f"{err_o:.3e}"), "lse": float(f"{err_l:.3e}")}}


def bench_ulysses_share(api, torch, warmup=3, iters=10, cpu=False):
    """One Ulysses share: causal attention over 131072 tokens, 4 query heads
    on 1 key/value head, [S, H, d] layout, fp32 lse; one launch.  With `cpu`,
    also the fp64 oracle on a sample of it."""
    from sequence_kv_chunk_amd.synth import WORKLOADS, device_attention_inputs
    w = WORKLOADS["ulysses_share_gqa_128k_causal"]
    x = device_attention_inputs(w)
    o = torch.empty((w.L, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(w.Hq * w.L, dtype=torch.float32, device="cuda")
    ts, _ = timed_launches(torch, lambda: api.ra_chunk_attention(x["q"], x["k"], x["v"], o, lse, scale=1.0,
                                                                 causal=True), warmup, iters)
    res = dict(ms_stats(ts))
    res.update({"TFLOP/s": round(w.flops() / (res["ms_mean"] * 1e-3) / 1e12, 1), "flops": w.flops(),
                "roofline": attn_roofline(w.name, w.flops(), ts),
                "workload": "ulysses_share_gqa_128k_causal: L=131072, 4 query heads, 1 KV head, d=128, causal, "
                            "[S, H, d] layout, one launch"})
    if cpu:
        res["cpu_oracle"] = cpu_oracle_share(w, x, o, lse, torch)
    del x, o, lse
    torch.cuda.empty_cache()
    return res


def _flush_fill(torch):
    buf = torch.empty(768 << 20, dtype=torch.uint8, device="cuda")     # > 256 MiB last-level cache
    return buf, (lambda: buf.fill_(1))


def bench_ulysses(api, torch, iters=10):
    """Ulysses seq->head and head->seq on 8 shards of [16384, 32, 128] bf16.
    Every launch is timed on its own with HIP events on the stream it runs
    on, after a 768 MiB fill that evicts the 256 MiB last-level cache, so each
    launch reads from HBM.  The same kernel run as a plain copy of the same
    bytes (P = 1: every token's 32 heads are one contiguous 8 KiB run, so the
    permutation is the identity) is the streaming ceiling it is held
    against; torch's copy_ is shown beside it."""
    from sequence_kv_chunk_amd.synth import ULYSSES_WORKLOADS, device_ulysses_input
    w = ULYSSES_WORKLOADS["ulysses_131k_32h"]
    src = device_ulysses_input(w)
    mid = torch.empty((w.P, w.L, w.H // w.P, w.d), dtype=torch.bfloat16, device="cuda")
    back = torch.empty_like(src)
    buf, flush = _flush_fill(torch)
    nbytes = w.bytes_per_direction()
    gbs = lambda ms: nbytes / (ms * 1e-3) / 1e9
    res = {}
    for name, fn in (("seq_to_head", lambda: api.ulysses_seq_to_head(src, mid)),
                     ("head_to_seq", lambda: api.ulysses_head_to_seq(mid, back))):
        ts, _ = timed_launches(torch, fn, 1, iters, flush)
        st = ms_stats(ts)
        res[name] = {**st, "GB/s": round(gbs(st["ms_mean"]), 1), "frac_hbm": round(gbs(st["ms_mean"]) / PEAK_HBM_GBS, 4)}
    torch.cuda.synchronize()
    ok = bool(torch.equal(back.view(torch.int16), src.view(torch.int16)))
    one = src.view(1, w.L, w.H, w.d)
    dst1 = back.view(1, w.L, w.H, w.d)
    ts, _ = timed_launches(torch, lambda: api.ulysses_seq_to_head(one, dst1), 1, iters, flush)
    st = ms_stats(ts)
    res["plain_copy_same_kernel"] = {**st, "GB/s": round(gbs(st["ms_mean"]), 1),
                                     "kernel": "permute_kernel<16, 0> with P=1 (identity): a linear copy of 1 GiB "
                                               "in the permute's launch shape"}
    ts, _ = timed_launches(torch, lambda: back.copy_(src), 1, iters, flush)
    st = ms_stats(ts)
    res["torch_copy_same_bytes"] = {**st, "GB/s": round(gbs(st["ms_mean"]), 1)}
    res["round_trip_bit_exact"] = ok
    res["workload"] = "ulysses_131k_32h: 8 shards [16384, 32, 128] bf16 <-> [131072, 4, 128]"
    res["bytes_per_direction"] = nbytes
    prof = load_profile(os.path.basename(PERMUTE_TRAFFIC_FILE), PERMUTE_SRC)
    both_ms = (res["seq_to_head"]["ms_mean"] + res["head_to_seq"]["ms_mean"]) / 2
    achieved = gbs(both_ms)
    res["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                       "frac": round(achieved / PEAK_HBM_GBS, 4),
                       "traffic": None if prof is None else prof.get("bytes_per_launch"),
                       "kernel": "permute_kernel<16, *> (seq->head and head->seq, mean of the two)",
                       "bytes_per_launch": nbytes, "launch_ms": round(both_ms, 4),
                       "frac_of_same_kernel_copy": round(achieved / res["plain_copy_same_kernel"]["GB/s"], 4)}
    del src, mid, back, buf
    torch.cuda.empty_cache()
    return res


def bench_gqa_replication(api, torch, iters=10):
    """The Ulysses exchange of the key/value heads with GQA: [8][16384][H_kv][128]
    bf16 shards become [8][131072][1][128] (every key/value head copied up to
    the 8 ranks), H_kv in {1, 2}.  Bytes = read once + written 8/H_kv times;
    each launch after a cache-evicting fill."""
    P, L, d = 8, 131072, 128
    buf, flush = _flush_fill(torch)
    res = {}
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    for H_kv in (1, 2):
        src = torch.randn((P, L // P, H_kv, d), generator=g, device="cuda").to(torch.bfloat16)
        dst = torch.empty((P, L, 1, d), dtype=torch.bfloat16, device="cuda")
        fn = lambda: api.ulysses_seq_to_head(src, dst, H_dst=P)
        ts, _ = timed_launches(torch, fn, 1, iters, flush)
        nbytes = src.numel() * 2 + dst.numel() * 2
        st = ms_stats(ts)
        achieved = nbytes / (st["ms_mean"] * 1e-3) / 1e9
        prof = load_profile(os.path.basename(REPLICATION_TRAFFIC_FILE), PERMUTE_SRC)
        tr = None if prof is None else prof.get("bytes_per_launch", {}).get(f"H_kv={H_kv}")
        res[f"H_kv={H_kv}"] = {**st, "copies_per_head": P // H_kv, "bytes_per_launch": nbytes,
                               "GB/s": round(achieved, 1),
                               "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                                            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                                            "traffic": tr, "kernel": "replicate_kernel<16>"}}
        if H_kv == 1:   # write ceiling: a linear fill of the same destination bytes, timed the same way
            ts, _ = timed_launches(torch, lambda: dst.fill_(1), 1, iters, flush)
            st = ms_stats(ts)
            res["linear_fill_same_dst_bytes"] = {**st, "GB/s": round(dst.numel() * 2 / (st["ms_mean"] * 1e-3) / 1e9, 1),
                                                 "kernel": "torch fill_ of the 256 MiB destination"}
        del src, dst
    res["workload"] = ("GQA key/value exchange: 8 shards [16384, H_kv, 128] bf16 -> [131072, 1, 128] per rank "
                       "(H_dst = 8), L = 131072")
    del buf
    torch.cuda.empty_cache()
    return res


def bench_visit_lengths(api, torch, iters=5):
    """Fixed cost of one attention visit: 4096 query tiles of 256 rows (16 per
    CU, non-causal, d=128), each against T key tiles of 64 for T in 1..64;
    per-workgroup time per visit and a straight-line fit over T >= 8 (the
    slope is the steady cost of a tile, the intercept the cost of a visit's
    start and end)."""
    H, n, d = 4096, 256, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(12)
    q = (torch.randn((1, H, n, d), generator=g, device="cuda") * d ** -0.5).to(torch.bfloat16)
    o = torch.empty_like(q)
    lse = torch.empty(H * n, dtype=torch.float32, device="cuda")
    pts = {}
    for T in (1, 4, 8, 16, 32, 64):
        kv = torch.randn((1, H, 64 * T, d), generator=g, device="cuda").to(torch.bfloat16)
        ts, _ = timed_launches(torch, lambda: api.ra_chunk_attention(q, kv, kv, o, lse), 1, iters)
        pts[T] = round(statistics.median(ts) * 1e3 / (H / 256), 2)      # us per workgroup visit (16 per CU)
        del kv
    xs = [t for t in pts if t >= 8]
    mx, my = sum(xs) / len(xs), sum(pts[t] for t in xs) / len(xs)
    slope = sum((t - mx) * (pts[t] - my) for t in xs) / sum((t - mx) ** 2 for t in xs)
    del q, o, lse
    torch.cuda.empty_cache()
    return {"us_per_visit_by_key_tiles": pts, "fit_us_per_tile": round(slope, 3),
            "fit_us_per_visit": round(my - slope * mx, 2),
            "workload": "4096 query tiles of 256 rows x T key tiles of 64, d=128, non-causal, 16 visits per CU"}


def bench_lse_merge(api, torch, iters=10):
    """The standalone log-sum-exp merge (the unfused ring's step) on the
    partials of one 128k ring step: O fp32 [1, 32, 16384, 128] and lse
    [1, 32, 16384], twice in, once out.  HBM-bound: bytes = read both
    partials + write the merged one.  Each launch follows a 768 MiB fill so
    that it reads HBM."""
    B, H, n, d = 1, 32, 16384, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    oa = torch.randn((B, H, n, d), generator=g, device="cuda")
    ob = torch.randn((B, H, n, d), generator=g, device="cuda")
    la = torch.randn((B * H * n,), generator=g, device="cuda")
    lb = torch.randn((B * H * n,), generator=g, device="cuda")
    oo = torch.empty_like(oa)
    lo = torch.empty_like(la)
    buf, flush = _flush_fill(torch)
    ts, _ = timed_launches(torch, lambda: api.ra_lse_merge(oa, la, ob, lb, oo, lo), 1, iters, flush)
    st = ms_stats(ts)
    nbytes = 3 * (B * H * n * d * 4 + B * H * n * 4)
    gbs = nbytes / (st["ms_mean"] * 1e-3) / 1e9
    del oa, ob, la, lb, oo, lo, buf
    torch.cuda.empty_cache()
    return {**st, "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4), "bytes": nbytes,
            "workload": "lse merge of two fp32 partials [1, 32, 16384, 128] + lse (one 128k ring step)"}


def bench_f32_tiny(api, torch, iters=20, cpu=False):
    """The tiny fp32 ring (4 virtual ranks x 4 chunks of 256, 4 heads, d=64):
    a correctness workload; its time is reported, not held against a roofline.
    With `cpu`, also the fp64 oracle on the whole workload."""
    from sequence_kv_chunk_amd.synth import WORKLOADS, device_attention_inputs
    w = WORKLOADS["ring_f32_tiny"]
    x = device_attention_inputs(w)
    qs, kp, vp = x["q"], x["k"], x["v"]
    o = torch.empty(qs.shape[1:], dtype=torch.float32, device="cuda")
    lse = torch.empty(o.numel() // o.shape[-1], dtype=torch.float32, device="cuda")

    def step():
        for r in range(w.P):
            api.ra_ring_attention(qs[r], kp, vp, o, lse, rank=r)

    ts, _ = timed_launches(torch, step, 2, iters)
    res = {"ms": round(sum(ts) / len(ts), 4), "launches": w.P, "flops": w.flops(),
           "workload": "ring_f32_tiny: fp32, B=1, 4 heads, d=64, L=1024 as 4 chunks of 256, all 4 ranks"}
    if cpu:
        import oracle
        full = lambda t: t.permute(1, 2, 0, 3, 4).reshape(t.shape[1], t.shape[2], -1, t.shape[-1]).double().cpu().numpy()
        qf, kf, vf = full(qs), full(kp), full(vp)
        t0 = time.perf_counter()
        ref_o, _ = oracle.attention_fp64(qf, kf, vf)
        secs = time.perf_counter() - t0
        step()
        torch.cuda.synchronize()
        last = o.double().cpu().numpy()                        # rank P-1's chunk
        n = qs.shape[3]
        err = float(np.max(np.abs(last - ref_o[:, :, (w.P - 1) * n:])) / np.max(np.abs(ref_o)))
        res["cpu_oracle"] = {"ms": round(secs * 1e3, 2), "kind": "oracle", "cores": host_facts()[1],
                             "sample": "the whole workload (fp64 numpy oracle, one softmax per query row)",
                             "gpu_normwise_rel_err_last_rank": float(f"{err:.3e}")}
    return res


def bench_f32_chunk(api, torch, iters=5):
    """The exact fp32 path at a throughput size: one 4096 x 4096 chunk pair,
    B=1, 32 heads, d=128, fp32 inputs and output, non-causal (4*d FLOP per
    pair), against MI355X's fp32 peak."""
    B, H, n, d = 1, 32, 4096, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(9)
    q = torch.randn((B, H, n, d), generator=g, device="cuda") * d ** -0.5
    k = torch.randn((B, H, n, d), generator=g, device="cuda")
    v = torch.randn((B, H, n, d), generator=g, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(B * H * n, dtype=torch.float32, device="cuda")
    ts, _ = timed_launches(torch, lambda: api.ra_chunk_attention(q, k, v, o, lse), 1, iters)
    ms = sum(ts) / len(ts)
    flops = 4 * d * n * n * H * B
    tf = flops / (ms * 1e-3) / 1e12
    res = {"ms": round(ms, 3), "TFLOP/s": round(tf, 1), "flops": flops,
           "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_F32_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(tf / PEAK_F32_TFLOPS, 4)},
           "workload": "fp32 chunk pair: B=1, 32 heads, d=128, 4096 queries x 4096 keys, non-causal"}
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return res


def bench_capacity_1m(api, torch):
    """Sequence-length capacity: causal attention over 1,048,576 tokens on one
    GPU in one call, the Ulysses-share head shape (4 query heads, 1 key/value
    head, d=128, bf16).  A materialised score matrix would take L*L*2 bytes per
    head (2 TiB here); the call allocates nothing beyond its inputs/outputs."""
    L, Hq, Hkv, d = 1 << 20, 4, 1, 128
    g = torch.Generator(device="cuda")
    g.manual_seed(8)
    q = (torch.randn((L, Hq, d), generator=g, device="cuda") * d ** -0.5).to(torch.bfloat16)
    k = torch.randn((L, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((L, Hkv, d), generator=g, device="cuda").to(torch.bfloat16)
    o = torch.empty_like(q)
    lse = torch.empty(Hq * L, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    api.ra_chunk_attention(q, k, v, o, lse, scale=1.0, causal=True)
    torch.cuda.synchronize()
    extra = free0 - torch.cuda.mem_get_info()[0]
    ts, _ = timed_launches(torch, lambda: api.ra_chunk_attention(q, k, v, o, lse, scale=1.0, causal=True), 0, 1)
    ms = ts[0]
    flops = 4 * d * Hq * (L * (L + 1) // 2)
    io_bytes = sum(t.numel() * t.element_size() for t in (q, k, v, o, lse))
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return {"tokens": L, "ms": round(ms, 2), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac_mfma": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "device_bytes_inputs_outputs": io_bytes, "device_bytes_allocated_by_call": int(max(extra, 0)),
            "score_matrix_bytes_if_materialised_per_head": L * L * 2,
            "workload": "causal attention, 1048576 tokens, 4 q heads, 1 kv head, d=128, bf16, one call"}


def bench_causal_split(api, torch, iters=2):
    """The whole causal 128k ring (8 ranks x chunks of 16384, 32 heads) under the
    contiguous split and under the zigzag split: per-rank launch time, the sum
    (the ring on one GPU) and the slowest rank (what bounds a step when every
    rank has its own GPU)."""
    from sequence_kv_chunk_amd.synth import WORKLOADS, device_attention_inputs
    res = {}
    for split, name in (("contiguous", "ring_bf16_128k_causal"), ("zigzag", "zigzag_bf16_128k_causal")):
        w = WORKLOADS[name]
        x = device_attention_inputs(w)
        B, H, n, d = x["q"].shape[1:]
        o = torch.empty((B, H, n, d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(B * H * n, dtype=torch.float32, device="cuda")
        work = (torch.empty((B, H, n // 2, d), dtype=torch.float32, device="cuda"),
                torch.empty(B * H * (n // 2), dtype=torch.float32, device="cuda"))
        rank_ms = []
        for r in range(w.P):
            if split == "zigzag":
                fn = lambda: api.ra_zigzag_attention(x["q"][r], x["k"], x["v"], o, lse, rank=r, work=work)
            else:
                fn = lambda: api.ra_ring_attention(x["q"][r], x["k"], x["v"], o, lse, rank=r, causal=True)
            ts, _ = timed_launches(torch, fn, 1, iters)
            rank_ms.append(sum(ts) / len(ts))
        tot = sum(rank_ms)
        res[split] = {"rank_ms": [round(t, 3) for t in rank_ms], "ring_ms_one_gpu": round(tot, 3),
                      "slowest_rank_ms": round(max(rank_ms), 3),
                      "max_over_min": round(max(rank_ms) / min(rank_ms), 2),
                      "TFLOP/s": round(w.flops() / (tot * 1e-3) / 1e12, 1), "flops": w.flops()}
        del x, o, lse, work
        torch.cuda.empty_cache()
    res["slowest_rank_speedup_zigzag"] = round(res["contiguous"]["slowest_rank_ms"] /
                                               res["zigzag"]["slowest_rank_ms"], 2)
    res["workload"] = ("causal 131072 tokens, 8 ranks, B=1, 32 heads, d=128, bf16; contiguous chunks of 16384 "
                       "vs zigzag pieces r and 15-r of 8192")
    return res


def bench_backward(api, torch, iters=2):
    """Backward of the 32k ring: for every rank the D preprocess and the ring
    backward (dQ of the rank, its share of every chunk's dK, dV).  TFLOP/s
    counts 10*d per visible pair (scores recomputed, dV, dP, dQ, dK); the
    kernels do 14*d (the dK/dV kernel recomputes the scores and dP)."""
    from sequence_kv_chunk_amd.synth import WORKLOADS, device_attention_inputs
    w = WORKLOADS["ring_bf16_32k"]
    x = device_attention_inputs(w)
    qs, kp, vp = x["q"], x["k"], x["v"]
    P = w.P
    B, H, n, d = qs.shape[1:]
    g = torch.Generator(device="cuda")
    g.manual_seed(w.seed + 100)
    dout = torch.randn(qs.shape, generator=g, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    o = torch.empty((P, B, H, n, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((P, B * H * n), dtype=torch.float32, device="cuda")
    for r in range(P):
        api.ra_ring_attention(qs[r], kp, vp, o[r], lse[r], rank=r, causal=w.causal)
    D = torch.empty_like(lse)
    dq = torch.zeros((B, H, n, d), dtype=torch.float32, device="cuda")
    dk = torch.zeros(kp.shape, dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)

    def step():
        for r in range(P):
            api.ra_attention_bwd_preprocess(o[r], dout[r], D[r])
            api.ra_ring_attention_bwd(qs[r], kp, vp, dout[r], lse[r], D[r], dq, dk, dv, rank=r, causal=w.causal)

    ts, _ = timed_launches(torch, step, 1, iters)
    ms = sum(ts) / len(ts)
    flops = w.flops() // 4 * 10
    res = {"ms": round(ms, 3), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1),
           "frac_mfma": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "flops_10d": flops,
           "workload": "backward of ring_bf16_32k (all 8 ranks: D preprocess + ring backward)"}
    del x, dout, o, lse, D, dq, dk, dv
    torch.cuda.empty_cache()
    return res


def bench_usp(api, torch, iters=2):
    """USP hybrid at 128k: 8 virtual ranks as Ulysses groups of P_u inside a
    ring of P_r = 8 / P_u groups; B=1, 32 query heads, 8 key/value heads,
    d=128, causal, bf16.  One call runs all 8 ranks' work (permutes in,
    rings, permute out)."""
    L, H, H_kv, d, P = 131072, 32, 8, 128, 8
    n = L // P
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    q = (torch.randn((P, n, H, d), generator=g, device="cuda") * d ** -0.5).to(torch.bfloat16)
    k = torch.randn((P, n, H_kv, d), generator=g, device="cuda").to(torch.bfloat16)
    v = torch.randn((P, n, H_kv, d), generator=g, device="cuda").to(torch.bfloat16)
    o = torch.empty_like(q)
    flops = 4 * d * H * (L * (L + 1) // 2)
    res = {"workload": "USP causal, L=131072, 32 q heads, 8 kv heads, d=128, 8 virtual ranks", "flops": flops}
    for P_u in (4, 2):
        ts, _ = timed_launches(torch, lambda: api.usp_attention(q, k, v, o, P_u=P_u, causal=True), 1, iters)
        ms = sum(ts) / len(ts)
        res[f"P_u={P_u},P_r={P // P_u}"] = {"ms": round(ms, 3), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1)}
    del q, k, v, o
    torch.cuda.empty_cache()
    return res


def bench_packed(api, torch, sample_len=2048, iters=3):
    """The 32k ring with the sequence packing samples of `sample_len` tokens
    (causal inside each sample, samples blind to each other).  TFLOP/s counts
    the visible pairs only."""
    from sequence_kv_chunk_amd.synth import WORKLOADS, device_attention_inputs
    w = WORKLOADS["ring_bf16_32k"]
    x = device_attention_inputs(w)
    qs, kp, vp = x["q"], x["k"], x["v"]
    P = w.P
    B, H, n, d = qs.shape[1:]
    L = P * n
    starts = torch.arange(0, L, sample_len, dtype=torch.int64, device="cuda")
    o = torch.empty((B, H, n, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(B * H * n, dtype=torch.float32, device="cuda")

    def step():
        for r in range(P):
            api.ra_ring_attention_packed(qs[r], kp, vp, o, lse, starts, rank=r)

    ts, _ = timed_launches(torch, step, 1, iters)
    ms = sum(ts) / len(ts)
    pairs = (L // sample_len) * sample_len * (sample_len + 1) // 2
    flops = 4 * d * pairs * B * H
    del x, o, lse
    torch.cuda.empty_cache()
    return {"ms": round(ms, 3), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac_mfma": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "flops": flops,
            "workload": f"ring_bf16_32k packing {L // sample_len} causal samples of {sample_len} tokens"}


def cpu_baseline_ulysses(torch):
    """The oracle's index copies (seq->head, then head->seq) on the whole
    Ulysses workload, 8 shards [16384, 32, 128] bf16 (1 GiB), on the host: the
    CPU figure beside the permute kernel's.  The input is the same seeded
    device tensor bench_ulysses permutes, copied to host memory."""
    import oracle
    from sequence_kv_chunk_amd.synth import ULYSSES_WORKLOADS, device_ulysses_input
    w = ULYSSES_WORKLOADS["ulysses_131k_32h"]
    src = device_ulysses_input(w).cpu().view(torch.int16).numpy().view(np.uint16)
    res = {}
    t0 = time.perf_counter()
    mid = oracle.seq_to_head_naive(src, w.P)
    res["seq_to_head_s"] = round(time.perf_counter() - t0, 3)
    t0 = time.perf_counter()
    oracle.head_to_seq_naive(mid, w.P)
    res["head_to_seq_s"] = round(time.perf_counter() - t0, 3)
    secs = (res["seq_to_head_s"] + res["head_to_seq_s"]) / 2
    res.update({"value": round(w.bytes_per_direction() / secs / 1e9, 2), "unit": "GB/s", "cores": 1,
                "kind": "oracle", "sample": "the whole workload, both directions (numpy strided copies, one thread)"})
    return res


def run_extras(api, torch, chosen, cpu=False):
    """The other workloads' figures; a failure here never hides the main line.
    With `cpu`, the extras that carry an oracle figure time it too."""
    extras = {}
    runs = (("ring32k", "ring_bf16_32k", lambda: bench_ring32k(api, torch)),
            ("ulysses_share", "ulysses_share_gqa_128k_causal", lambda: bench_ulysses_share(api, torch, cpu=cpu)),
            ("ulysses", "ulysses", lambda: bench_ulysses(api, torch)),
            ("gqa_replication", "ulysses_gqa_replication_128k", lambda: bench_gqa_replication(api, torch)),
            ("packed", "ring_bf16_32k_packed_2k", lambda: bench_packed(api, torch)),
            ("visit_lengths", "attention_visit_lengths", lambda: bench_visit_lengths(api, torch)),
            ("backward", "ring_bf16_32k_backward", lambda: bench_backward(api, torch)),
            ("causal_split", "causal_128k_ring_split", lambda: bench_causal_split(api, torch)),
            ("usp", "usp_128k_causal", lambda: bench_usp(api, torch)),
            ("lse_merge", "lse_merge_128k_step", lambda: bench_lse_merge(api, torch)),
            ("f32_tiny", "ring_f32_tiny", lambda: bench_f32_tiny(api, torch, cpu=cpu)),
            ("f32_chunk", "f32_chunk_4k", lambda: bench_f32_chunk(api, torch)),
            ("capacity_1m", "capacity_1m_causal", lambda: bench_capacity_1m(api, torch)))
    for key, name, fn in runs:
        if key not in chosen:
            continue
        try:
            extras[name] = fn()
            log(f"{name}: {extras[name]}")
        except Exception as e:        # report and go on: the headline is already measured
            extras[name] = {"error": repr(e)}
            log(f"{name}: error {e!r}")
            torch.cuda.empty_cache()
    return extras


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-extras", action="store_true", help="skip the other workloads' figures")
    ap.add_argument("--extras", default="all",
                    help="comma-separated subset of " + ",".join(EXTRAS) + " (default: all)")
    ap.add_argument("--only-extras", action="store_true",
                    help="skip the headline and the CPU baseline; print the chosen extras only (for profiling)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on exactly one GPU (the ring's P chunks are resident in one HBM "
              "pool); --gpus N with N > 1 is not supported.", file=sys.stderr)
        sys.exit(2)

    chosen = () if args.no_extras else (EXTRAS if args.extras == "all" else tuple(args.extras.split(",")))
    unknown = [e for e in chosen if e not in EXTRAS]
    if unknown:
        print(f"bench.py: unknown extras {unknown}; choose from {','.join(EXTRAS)}", file=sys.stderr)
        sys.exit(2)

    import torch
    from sequence_kv_chunk_amd import api

    if args.calibrate_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    result = {}
    if not args.only_extras:
        result, kept = headline(api, torch, args)
        if not args.no_cpu:
            result["cpu_baseline"] = cpu_baseline(*kept, torch)
            log(f"cpu baseline: {result['cpu_baseline']}")
        else:
            result["cpu_baseline"] = None
        del kept
        torch.cuda.empty_cache()
    extras = run_extras(api, torch, chosen, cpu=not args.no_cpu and not args.only_extras)
    if not args.no_cpu and not args.only_extras and "ulysses" in chosen:
        extras["cpu_oracle_ulysses"] = cpu_baseline_ulysses(torch)
        log(f"cpu oracle ulysses: {extras['cpu_oracle_ulysses']}")
    if extras:
        result["extras"] = extras
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
