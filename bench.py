"""Benchmark of the chunked ring-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step = the whole 32k-token ring on one GPU: 8 virtual ranks, each
attending with its 4096-row query chunk to all 8 resident key/value chunks in
ring order (one launch per rank, the online-softmax merge carried across the
chunks in registers; bf16 in, fp32 accumulation, bf16 out), B=1, 32 heads,
d=128, non-causal.  Inputs are drawn on the device
from a seeded generator and are resident in HBM before timing starts.

Printed: ONE JSON line on stdout with the metric, the roofline of the
chunk-attention kernel (MFMA-bound) and the CPU oracle timed on a bounded
sample of the same workload.  Extra figures on the other workloads (Ulysses
permute GB/s on 8 x [16384, 32, 128] bf16 with its own HBM roofline and a
device copy of the same bytes, the causal 128k rank-7 ring share, the causal
128k GQA Ulysses share, the whole causal 128k ring under the contiguous and
the zigzag split, the backward of the 32k ring, the USP hybrid at 128k, the
32k ring packing 2k-token samples, the standalone lse merge of a 128k ring
step, the tiny fp32 ring, causal attention over 1,048,576 tokens, and with
the CPU baseline the oracle's Ulysses copies) go in "extras".  Logs go to
stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA (published)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E (published)
METRIC = "chunked-attention TFLOP/s (% bf16 MFMA peak); Ulysses permute GB/s (% HBM)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_ring32k_traffic.json")
ATTN_SRC = os.path.join(ROOT, "sequence_kv_chunk_amd", "csrc", "attn_bf16.hip")
MFMA_FILE = os.path.join(ROOT, "profiles", "attn_bf16_ring32k_mfma.json")
PERMUTE_SRC = os.path.join(ROOT, "sequence_kv_chunk_amd", "csrc", "ulysses.hip")
PERMUTE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ulysses_permute_131k_traffic.json")
EXTRAS = ("packed", "backward", "ulysses", "rank7", "ulysses_share", "causal_split", "usp", "lse_merge",
          "f32_tiny", "capacity_1m")


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


def load_profile(path: str, src: str):
    """A committed rocprofv3 counter summary, if it was taken on the current
    kernel source (else None: the counters describe older code)."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash(src):
        return None
    return t


def load_traffic():
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    passes, if they were taken on the current kernel source."""
    t = load_profile(TRAFFIC_FILE, ATTN_SRC)
    return None if t is None else t.get("bytes_per_launch")


def time_ring(api, torch, w, x, steps, warmup):
    """Times `steps` ring passes over all query ranks; returns (ms_per_step, launches/step)."""
    P = w.P
    qs, kp, vp = x["q"], x["k"], x["v"]
    B, H, n, d = qs.shape[1:]
    o = torch.empty((B, H, n, d), dtype=qs.dtype, device="cuda")     # bf16 in -> bf16 out, fp32 -> fp32
    lse = torch.empty(B * H * n, dtype=torch.float32, device="cuda")
    ranks = w.query_ranks

    def step():
        for idx, i in enumerate(ranks):
            api.ra_ring_attention(qs[idx], kp, vp, o, lse, rank=i, scale=1.0, causal=w.causal)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(steps):
        step()
    ev1.record()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    gpu = ev0.elapsed_time(ev1) / steps
    launches = len(ranks)           # one ra_ring_attention launch per virtual rank
    return wall, gpu, launches


def bench_ulysses(api, torch, iters=10):
    """Ulysses seq->head and head->seq on 8 shards of [16384, 32, 128] bf16.
    Every launch is timed on its own with HIP events on the stream it runs on,
    after a 768 MiB fill that evicts the 256 MiB last-level cache, so each
    launch reads from HBM.  A plain device copy of the same bytes, timed the
    same way, gives the streaming ceiling the permute is held against."""
    from sequence_kv_chunk_amd.synth import ULYSSES_WORKLOADS, device_ulysses_input
    w = ULYSSES_WORKLOADS["ulysses_131k_32h"]
    src = device_ulysses_input(w)
    mid = torch.empty((w.P, w.L, w.H // w.P, w.d), dtype=torch.bfloat16, device="cuda")
    back = torch.empty_like(src)
    flush = torch.empty(768 << 20, dtype=torch.uint8, device="cuda")   # > 256 MiB MALL
    nbytes = w.bytes_per_direction()

    def timed(fn):
        fn()
        ts = []
        for _ in range(iters):
            flush.zero_()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return ts

    res = {}
    for name, fn in (("seq_to_head", lambda: api.ulysses_seq_to_head(src, mid)),
                     ("head_to_seq", lambda: api.ulysses_head_to_seq(mid, back))):
        ts = timed(fn)
        avg = sum(ts) / len(ts)
        ts.sort()
        res[name] = {"ms_avg": round(avg, 4), "ms_median": round(ts[len(ts) // 2], 4), "ms_min": round(ts[0], 4),
                     "GB/s": round(nbytes / (avg * 1e-3) / 1e9, 1),
                     "frac_hbm": round(nbytes / (avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    torch.cuda.synchronize()
    ok = bool(torch.equal(back.view(torch.int16), src.view(torch.int16)))
    copy_ts = timed(lambda: back.copy_(src))
    copy_avg = sum(copy_ts) / len(copy_ts)
    res["plain_copy_same_bytes"] = {"ms_avg": round(copy_avg, 4),
                                    "GB/s": round(nbytes / (copy_avg * 1e-3) / 1e9, 1),
                                    "kernel": "torch copy_ of 1 GiB (read 1 GiB + write 1 GiB)"}
    res["round_trip_bit_exact"] = ok
    res["workload"] = "ulysses_131k_32h: 8 shards [16384, 32, 128] bf16 <-> [131072, 4, 128]"
    res["bytes_per_direction"] = nbytes
    prof = load_profile(PERMUTE_TRAFFIC_FILE, PERMUTE_SRC)
    both_ms = (res["seq_to_head"]["ms_avg"] + res["head_to_seq"]["ms_avg"]) / 2
    achieved = nbytes / (both_ms * 1e-3) / 1e9
    res["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                       "frac": round(achieved / PEAK_HBM_GBS, 4),
                       "traffic": None if prof is None else prof.get("bytes_per_launch"),
                       "kernel": "permute_kernel<16, *> (seq->head and head->seq, mean of the two)",
                       "bytes_per_launch": nbytes, "launch_ms": round(both_ms, 4)}
    del src, mid, back, flush
    torch.cuda.empty_cache()
    return res


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
    flush = torch.empty(768 << 20, dtype=torch.uint8, device="cuda")
    api.ra_lse_merge(oa, la, ob, lb, oo, lo)
    ts = []
    for _ in range(iters):
        flush.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        api.ra_lse_merge(oa, la, ob, lb, oo, lo)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    avg = sum(ts) / len(ts)
    nbytes = 3 * (B * H * n * d * 4 + B * H * n * 4)
    gbs = nbytes / (avg * 1e-3) / 1e9
    del oa, ob, la, lb, oo, lo, flush
    torch.cuda.empty_cache()
    return {"ms_avg": round(avg, 4), "GB/s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
            "bytes": nbytes, "workload": "lse merge of two fp32 partials [1, 32, 16384, 128] + lse (one 128k ring step)"}


def bench_f32_tiny(api, torch, steps=20):
    """The tiny fp32 ring (4 virtual ranks x 4 chunks of 256, 4 heads, d=64):
    a correctness workload; its time is reported, not held against a roofline."""
    from sequence_kv_chunk_amd.synth import WORKLOADS, device_attention_inputs
    w = WORKLOADS["ring_f32_tiny"]
    x = device_attention_inputs(w)
    _, ms, launches = time_ring(api, torch, w, x, steps, 2)
    return {"ms": round(ms, 4), "launches": launches, "flops": w.flops(),
            "workload": "ring_f32_tiny: fp32, B=1, 4 heads, d=64, L=1024 as 4 chunks of 256, all 4 ranks"}


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
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    api.ra_chunk_attention(q, k, v, o, lse, scale=1.0, causal=True)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    flops = 4 * d * Hq * (L * (L + 1) // 2)
    io_bytes = sum(t.numel() * t.element_size() for t in (q, k, v, o, lse))
    del q, k, v, o, lse
    torch.cuda.empty_cache()
    return {"tokens": L, "ms": round(ms, 2), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1),
            "frac_mfma": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "device_bytes_inputs_outputs": io_bytes, "device_bytes_allocated_by_call": int(max(extra, 0)),
            "score_matrix_bytes_if_materialised_per_head": L * L * 2,
            "workload": "causal attention, 1048576 tokens, 4 q heads, 1 kv head, d=128, bf16, one call"}


def bench_attention_extra(api, torch, name, steps=3):
    from sequence_kv_chunk_amd.synth import WORKLOADS, device_attention_inputs
    w = WORKLOADS[name]
    x = device_attention_inputs(w)
    if w.layout == "shd":
        o = torch.empty((w.L, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(w.Hq * w.L, dtype=torch.float32, device="cuda")
        fn = lambda: api.ra_chunk_attention(x["q"], x["k"], x["v"], o, lse, scale=1.0, causal=w.causal)
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
    else:
        _, ms, _ = time_ring(api, torch, w, x, steps, 1)
    tf = w.flops() / (ms * 1e-3) / 1e12
    del x
    torch.cuda.empty_cache()
    return {"ms": round(ms, 3), "TFLOP/s": round(tf, 1), "frac_mfma": round(tf / PEAK_BF16_TFLOPS, 4),
            "flops": w.flops()}


def bench_causal_split(api, torch, steps=2):
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
            fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            rank_ms.append(e0.elapsed_time(e1) / steps)
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


def bench_backward(api, torch, x, w, steps=2):
    """Backward of the 32k ring: for every rank the D preprocess and the ring
    backward (dQ of the rank, its share of every chunk's dK, dV).  TFLOP/s
    counts 10*d per visible pair (scores recomputed, dV, dP, dQ, dK); the
    kernels do 14*d (the dK/dV kernel recomputes the scores and dP)."""
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

    step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = w.flops() // 4 * 10
    res = {"ms": round(ms, 3), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1),
           "frac_mfma": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4), "flops_10d": flops,
           "workload": "backward of ring_bf16_32k (all 8 ranks: D preprocess + ring backward)"}
    del dout, o, lse, D, dq, dk, dv
    torch.cuda.empty_cache()
    return res


def bench_usp(api, torch, steps=2):
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
        api.usp_attention(q, k, v, o, P_u=P_u, causal=True)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            api.usp_attention(q, k, v, o, P_u=P_u, causal=True)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res[f"P_u={P_u},P_r={P // P_u}"] = {"ms": round(ms, 3), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1)}
    del q, k, v, o
    torch.cuda.empty_cache()
    return res


def bench_packed(api, torch, x, w, sample_len=2048, steps=2):
    """The 32k ring with the sequence packing samples of `sample_len` tokens
    (causal inside each sample, samples blind to each other).  TFLOP/s counts
    the visible pairs only."""
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

    step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    pairs = (L // sample_len) * sample_len * (sample_len + 1) // 2
    flops = 4 * d * pairs * B * H
    return {"ms": round(ms, 3), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 1), "flops": flops,
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


def cpu_baseline(x_dev, w, torch, budget_rows=4096, heads=16):
    """The fp64 oracle on a bounded sample of the workload: query chunk 0
    (4096 rows) of the first `heads` heads against all 32768 keys."""
    import oracle
    from sequence_kv_chunk_amd.synth import bf16_bits_to_f64

    def bits(t):
        return t.contiguous().cpu().view(torch.int16).numpy().view(np.uint16)

    q = bf16_bits_to_f64(bits(x_dev["q"][0][:, :heads, :budget_rows]))          # [B, h, rows, d]
    kp = bf16_bits_to_f64(bits(x_dev["k"][:, :, :heads]))                          # [P, B, h, n, d]
    vp = bf16_bits_to_f64(bits(x_dev["v"][:, :, :heads]))
    P, B, h, n, d = kp.shape
    k = kp.transpose(1, 2, 0, 3, 4).reshape(B, h, P * n, d)
    v = vp.transpose(1, 2, 0, 3, 4).reshape(B, h, P * n, d)
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    t0 = time.perf_counter()
    oracle.attention_fp64(q, k, v, scale=1.0, causal=False)
    dt = time.perf_counter() - t0
    flops = 4 * d * (P * n) * budget_rows * heads * B
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"query rows 0..{budget_rows - 1} (chunk 0) of heads 0..{heads - 1} against all "
                      f"{P * n} keys, fp64 numpy oracle, {dt:.1f} s",
            "seconds": round(dt, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-extras", action="store_true", help="skip the other workloads' figures")
    ap.add_argument("--extras", default="all",
                    help="comma-separated subset of " + ",".join(EXTRAS) + " (default: all)")
    ap.add_argument("--only-extras", action="store_true",
                    help="skip the ring and the CPU baseline; print the chosen extras only (for profiling)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device copy (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on exactly one GPU (the ring's P chunks are resident in one HBM "
              "pool); --gpus N with N > 1 is not supported.", file=sys.stderr)
        sys.exit(2)

    import torch
    from sequence_kv_chunk_amd import api
    from sequence_kv_chunk_amd.synth import WORKLOADS, device_attention_inputs

    chosen = () if args.no_extras else (EXTRAS if args.extras == "all" else tuple(args.extras.split(",")))
    unknown = [e for e in chosen if e not in EXTRAS]
    if unknown:
        print(f"bench.py: unknown extras {unknown}; choose from {','.join(EXTRAS)}", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        a = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    w = WORKLOADS["ring_bf16_32k"]
    x = device_attention_inputs(w)
    torch.cuda.synchronize()
    log(f"workload {w.name}: inputs resident ({sum(t.numel() * 2 for t in x.values()) / 2**30:.2f} GiB)")

    result = {}
    if not args.only_extras:
        result = ring_result(api, torch, w, x, args)
    extras = run_extras(api, torch, w, x, chosen)
    if not args.no_cpu and not args.only_extras:
        result["cpu_baseline"] = cpu_baseline(x, w, torch)
        log(f"cpu baseline: {result['cpu_baseline']}")
        extras["cpu_oracle_ulysses"] = cpu_baseline_ulysses(torch)
        log(f"cpu oracle ulysses: {extras['cpu_oracle_ulysses']}")
    elif not args.only_extras:
        result["cpu_baseline"] = None
    if extras:
        result["extras"] = extras
    print(json.dumps(result), flush=True)


def ring_result(api, torch, w, x, args):
    """The headline line: the 32k ring step, its throughput and the roofline
    of the chunk-attention kernel."""
    wall_ms, gpu_ms, launches = time_ring(api, torch, w, x, args.steps, args.warmup)
    flops = w.flops()
    value = flops / (wall_ms * 1e-3) / 1e12
    per_launch_flops = flops // launches
    launch_ms = gpu_ms / launches      # the timed region holds only chunk-attention launches
    achieved = per_launch_flops / (launch_ms * 1e-3) / 1e12
    traffic = load_traffic()
    mfma = load_profile(MFMA_FILE, ATTN_SRC)
    log(f"ring step {wall_ms:.3f} ms (events {gpu_ms:.3f} ms), {value:.1f} TFLOP/s, "
        f"{launches} launches of {launch_ms:.4f} ms")
    return {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) on device; Q scaled by d^-0.5)",
        "config": {"workload": "ring_bf16_32k: 32768 tokens as 8 chunks of 4096, all 8 query chunks x 8 "
                               "resident KV chunks, B=1, 32 heads, d=128, non-causal",
                   "global_batch": 1, "seq_len": w.L, "heads": w.Hq, "head_dim": w.d, "chunks": w.P,
                   "parallelism": "single GPU; 8 virtual ranks"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "attn_bf16_kernel<128, false>", "flops_per_launch": per_launch_flops,
                     "launch_ms": round(launch_ms, 4),
                     "mfma_busy_pct_counters": None if mfma is None else mfma.get("MfmaUtil_pct")},
    }


def run_extras(api, torch, w, x, chosen):
    """The other workloads' figures; a failure here never hides the main line."""
    extras = {}
    runs = (("packed", "ring_bf16_32k_packed_2k", lambda: bench_packed(api, torch, x, w)),
            ("backward", "ring_bf16_32k_backward", lambda: bench_backward(api, torch, x, w)),
            ("ulysses", "ulysses", lambda: bench_ulysses(api, torch)),
            ("rank7", "ring_bf16_128k_rank7_causal",
             lambda: bench_attention_extra(api, torch, "ring_bf16_128k_rank7_causal")),
            ("ulysses_share", "ulysses_share_gqa_128k_causal",
             lambda: bench_attention_extra(api, torch, "ulysses_share_gqa_128k_causal")),
            ("causal_split", "causal_128k_ring_split", lambda: bench_causal_split(api, torch)),
            ("usp", "usp_128k_causal", lambda: bench_usp(api, torch)),
            ("lse_merge", "lse_merge_128k_step", lambda: bench_lse_merge(api, torch)),
            ("f32_tiny", "ring_f32_tiny", lambda: bench_f32_tiny(api, torch)),
            ("capacity_1m", "capacity_1m_causal", lambda: bench_capacity_1m(api, torch)))
    try:
        for key, name, fn in runs:
            if key in chosen:
                extras[name] = fn()
                log(f"{name}: {extras[name]}")
    except Exception as e:
        extras["error"] = repr(e)
    return extras


if __name__ == "__main__":
    main()
