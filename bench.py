#!/usr/bin/env python3
"""Benchmark of the block-sparse attention hot path on one MI355X.

One step = bsa_pool + bsa_select + bsa_forward over one batch of synthetic
input already resident in HBM (the 768p 5s shape by default: 56 heads x
37,740 tokens, head_dim 128, top_k 64 of 295 blocks, mean summaries); with
extra tokens, bsa_select_tokens + bsa_forward_tokens in place of bsa_forward;
on the Spark-Reblock order, bsa_reblock first and the reordered calls
(bsa_pool_reordered, bsa_forward_reordered: rows read and written through the
order) in place of bsa_pool and bsa_forward.

Prints one JSON line.  `value` is the effective TFLOP/s of a whole step
counting only the selected blocks' attention FLOPs, 4 * 128 * sum_r n_r *
sum_{c in S(r)} n_c; `ms_per_step` is milliseconds per call.  The roofline
object describes the attention kernel (the dominant one), timed with HIP
events recorded on the stream it runs on.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PAGES_MS = {"768p_5s": 30.7, "768p_10s": 61.8, "2k_5s": 121.8}  # RTX PRO 6000, context only


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="768p_5s")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="approximate budget of the oracle sample")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after timing, run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--no-gemm-ref", action="store_true",
                    help="skip the dense bf16 GEMM reference timed after the steps")
    return ap.parse_args()


def gemm_reference(torch, dev, n=8192, iters=10):
    """TFLOP/s of the vendor library's dense bf16 GEMM (torch.matmul, i.e.
    hipBLASLt) at n^3 on random operands, timed after the steps on the same
    device: context for the attention kernel's rate, since the clock a chip
    holds under MFMA load differs from box to box.  Not part of the path."""
    g = torch.Generator(device=dev).manual_seed(0)
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
    for _ in range(3):
        c = torch.matmul(a, b)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        c = torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    del c
    return 2.0 * n ** 3 / (e0.elapsed_time(e1) / iters * 1e-3) / 1e12


def measured_traffic(workload):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE scaled by a copy-kernel calibration),
    or None when it was taken on another workload or another kernel source."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "attn_fwd_%s_traffic.txt" % workload)
    if not os.path.exists(path):
        return None
    fields = dict(line.split(None, 1) for line in open(path) if line.startswith(("source_sha256", "traffic_bytes")))
    src = os.path.join(ROOT, "block_sparse_attention_25_amd", "csrc", "bsa.hip")
    if hashlib.sha256(open(src, "rb").read()).hexdigest() != fields.get("source_sha256", "").strip():
        return None
    return float(fields["traffic_bytes"])


def reported_clock_peak():
    """The bf16 dense MFMA peak recomputed from the device's reported maximum
    engine clock and compute-unit count (4 SIMDs x 1024 bf16 flop per clock
    each); None when the runtime does not report them."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        clk, cus = ctypes.c_int(), ctypes.c_int()
        # hipDeviceAttributeClockRate (kHz) and hipDeviceAttributeMultiprocessorCount
        ok1 = hip.hipDeviceGetAttribute(ctypes.byref(clk), 5, 0) == 0
        ok2 = hip.hipDeviceGetAttribute(ctypes.byref(cus), 63, 0) == 0
        if not (ok1 and ok2) or clk.value <= 0 or cus.value <= 0:
            return None
        return {"clock_mhz": clk.value / 1e3, "compute_units": cus.value,
                "peak_tflops": round(cus.value * 4 * 1024 * clk.value * 1e3 / 1e12, 1)}
    except OSError:
        return None


def counted_flops(torch, idx, N, nb, H, B, dense=(), tok=None):
    """4 * d * sum over (b, h, r) of n_r * (sum_{c in S(r)} n_c + extra tokens
    of r), exactly; query blocks in `dense` (conditioning sinks) attend to all
    N keys."""
    n = torch.full((nb,), 128, dtype=torch.int64, device=idx.device)
    n[-1] = N - 128 * (nb - 1)
    k = idx.shape[-1]
    per_row = n[idx.long()].sum(-1) if k > 0 else torch.zeros((B, H, nb), dtype=torch.int64,
                                                               device=idx.device)
    if k > 0:
        # threshold selection pads rows with -1
        valid = idx >= 0
        per_row = (n[idx.clamp(min=0).long()] * valid).sum(-1)
        n_skip = nb - valid.sum(-1)
    else:
        n_skip = torch.full((B, H, nb), nb, dtype=torch.int64, device=idx.device)
    if tok is not None:
        per_row = per_row + (tok >= 0).sum(-1)
    if len(dense):
        per_row[..., list(dense)] = N
        n_skip[..., list(dense)] = 0
    exact = int((per_row * n).sum().item())
    summary = int((n * n_skip).sum().item())
    return 4 * 128 * exact, 4 * 128 * summary


def tie_zone_rows(torch, q_pool, k_pool, k, plain_topk):
    """Rows whose k-th and (k+1)-th block scores (float64 dot products of the
    pooled vectors) differ by less than 1e-4 relative: the rows where the
    selection may legitimately differ from an exact ranking.  Plain top-k
    only (None otherwise)."""
    if not plain_topk or k == 0 or k >= q_pool.shape[2]:
        return None if not plain_topk else 0
    n = 0
    for b in range(q_pool.shape[0]):
        for h in range(q_pool.shape[1]):
            s = q_pool[b, h].double() @ k_pool[b, h].double().T
            top = torch.topk(s, k + 1, dim=-1).values
            a, c = top[:, k - 1], top[:, k]
            n += int(((a - c).abs() < 1e-4 * torch.maximum(a.abs(), c.abs())).sum().item())
    return n


def cpu_baseline(w, qb, kb, vb, budget_s):
    """The oracle as it stands, on a bounded sample of the same workload: whole
    heads (pool, scores, top-k, summaries, attention of every query block) in
    order until the time budget runs out, the last head possibly cut short.
    Rate in the bench's unit: TFLOP/s of counted (selected-block) FLOPs."""
    from oracle import bsa_oracle as O
    from block_sparse_attention_25_amd.synth import bf16_to_f32
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    host = {"cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "blas_threads": cores}
    N = w.seq_len
    nb = O.n_blocks(N)
    rows = O.block_rows(N)
    top_k = w.top_k if w.top_k is not None else O.k_from_ratio(w.top_k_ratio, nb)
    sc = O.default_scale(128)
    sinks = O.sink_blocks(N, w.sink_start, w.sink_rows)
    flops, heads_done, blocks_done = 0, 0, 0
    no_tok = np.full((nb, 0), -1, dtype=np.int32)
    t0 = time.perf_counter()
    for h in range(qb.shape[1]):
        Q, K, V = (bf16_to_f32(x[0, h]).astype(np.float64) for x in (qb, kb, vb))
        if w.reblock:
            perm = O.reblock_permutation(Q, K)
            Q, K, V = Q[perm], K[perm], V[perm]
        qp, kp = O.pool_mean(Q), O.pool_mean(K)
        sc_ = O.block_scores(qp, kp)
        idx = O.select_topk(sc_, top_k, sinks) if w.tau is None else \
            O.select_threshold(sc_, w.tau, top_k, sinks)
        if w.summary == "reweight":
            sk, sv, b = O.summaries_reweight(K, V, O.anchor(Q, w.anchor_rows), sc)
        else:
            sk, sv, b = O.summaries_mean(K, V)
        for r in range(nb):
            tok = O.select_extra_tokens(qp, K, idx, w.extra, dense_blocks=sinks, query_blocks=[r]) \
                if w.extra else no_tok
            O.attention(Q, K, V, idx, sk, sv, b, sc, query_blocks=[r], dense_blocks=sinks,
                        extra=tok if w.extra else None)
            keys = N if r in sinks else sum(rows[c][1] - rows[c][0] for c in idx[r] if c >= 0) + \
                int((tok[r] >= 0).sum() if w.extra else 0)
            flops += 4 * 128 * (rows[r][1] - rows[r][0]) * keys
            blocks_done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
        heads_done += 1
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle", "host": host,
            "sample": "%d query blocks (%d whole heads of %d, each with its %spool, scores, top-k%s and "
                      "summaries) of the %s workload; %.1f s wall"
                      % (blocks_done, heads_done, qb.shape[1], "reblock order, " if w.reblock else "",
                         ", extra tokens" if w.extra else "", w.name, dt)}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(heads would shard across GPUs without communication). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import block_sparse_attention_25_amd as bsa
    from block_sparse_attention_25_amd.synth import WORKLOADS, generate
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    bsa.lib()
    w = WORKLOADS[args.workload]
    B, H, N = w.batch, w.heads, w.seq_len
    nb = -(-N // 128)
    top_k = w.top_k if w.top_k is not None else bsa.k_from_ratio(w.top_k_ratio, nb)
    t0 = time.time()
    qb, kb, vb = generate(w, threads=16)
    gen_s = time.time() - t0
    dev = torch.device("cuda:0")

    def dev_bf16(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = dev_bf16(qb), dev_bf16(kb), dev_bf16(vb)
    p = bsa.make_problem(B, H, N, top_k, None, w.summary,
                         w.anchor_rows if w.summary == "reweight" else 0,
                         sink_rows=w.sink_rows, sink_start=w.sink_start, tau=w.tau,
                         extra_tokens=w.extra)
    dense = list(range(w.sink_start // 128, (w.sink_start + w.sink_rows - 1) // 128 + 1)) \
        if w.sink_rows > 0 else []
    nb, kk = bsa.bsa_problem_blocks(p)
    f32 = torch.float32
    q_pool = torch.empty((B, H, nb, 128), dtype=f32, device=dev)
    k_pool = torch.empty_like(q_pool)
    sum_k = torch.empty((B, H, nb, 128), dtype=torch.bfloat16, device=dev)
    sum_v = torch.empty_like(sum_k)
    sum_bias = torch.empty((B, H, nb), dtype=f32, device=dev)
    idx = torch.empty((B, H, nb, kk), dtype=torch.int32, device=dev)
    ws = torch.empty(bsa.bsa_workspace_bytes(p), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    tok = torch.empty((B, H, nb, w.extra), dtype=torch.int32, device=dev) if w.extra else None
    if w.reblock:
        perm = torch.empty((B, H, N), dtype=torch.int32, device=dev)
        rws = torch.empty(bsa.bsa_reblock_workspace_bytes(p), dtype=torch.uint8, device=dev)
        kr, vr = torch.empty_like(k), torch.empty_like(v)   # keys and values in the new order
    else:
        kr, vr = k, v

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(args.steps)]

    def step(e=None):
        if e: e[0].record()
        if w.reblock:
            bsa.bsa_reblock(p, q, k, perm, rws)
        if e: e[1].record()
        if w.reblock:
            bsa.bsa_pool_reordered(p, perm, q, k, v, q_pool, k_pool, sum_k, sum_v, sum_bias, kr, vr, ws)
        else:
            bsa.bsa_pool(p, q, k, v, q_pool, k_pool, sum_k, sum_v, sum_bias, ws)
        if e: e[2].record()
        bsa.bsa_select(p, q_pool, k_pool, idx)
        if e: e[3].record()
        if tok is not None:
            bsa.bsa_select_tokens(p, q_pool, kr, idx, tok, ws)
        if e: e[4].record()
        if w.reblock:
            bsa.bsa_forward_reordered(p, perm, q, kr, vr, sum_k, sum_v, sum_bias, idx, tok, out, ws)
        elif tok is not None:
            bsa.bsa_forward_tokens(p, q, k, v, sum_k, sum_v, sum_bias, idx, tok, out, ws)
        else:
            bsa.bsa_forward(p, q, k, v, sum_k, sum_v, sum_bias, idx, out, ws)
        if e: e[5].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_start) * 1e3 / args.steps
    def span(a, b):
        return sum(e[a].elapsed_time(e[b]) for e in ev) / args.steps
    reblock_ms, pool_ms, sel_ms, tok_ms, attn_ms = (span(i, i + 1) for i in range(5))
    step_ms = span(0, 5)
    step_med = float(np.median([e[0].elapsed_time(e[5]) for e in ev]))
    flops, summary_flops = counted_flops(torch, idx, N, nb, H, B, dense, tok)
    attn_tflops = flops / (attn_ms * 1e-3) / 1e12
    value = flops / (step_ms * 1e-3) / 1e12
    # pool, algorithmic bytes: read Q, K, V once; write q_pool, k_pool (fp32),
    # sum_k, sum_v (bf16) and the bias: 1,540 B per block
    pool_bytes = 3 * B * H * N * 128 * 2 + B * H * nb * (2 * 512 + 2 * 256 + 4)
    # on a reblocked order the pool also writes K and V in the new order and
    # reads each row's perm entry twice (listed apart, not in pool_frac)
    pool_copy_bytes = B * H * N * (2 * 128 * 2 + 2 * 4) if w.reblock else 0
    sel_bytes = 2 * B * H * nb * 128 * 4 + B * H * nb * kk * 4
    tie_rows = tie_zone_rows(torch, q_pool, k_pool, kk, w.tau is None and w.sink_rows == 0)

    gemm_tflops = None if args.no_gemm_ref else gemm_reference(torch, dev)

    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        bcopy = torch.empty_like(a)
        for _ in range(3):
            bcopy.copy_(a)
        torch.cuda.synchronize()

    res = {
        "metric": "ms/call + effective TFLOP/s (% bf16 MFMA peak), 56 heads×37,740 tok, top_k=64",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(PAGES_MS[args.workload] / step_ms, 3) if args.workload in PAGES_MS else None),
        "vs_baseline_basis": "speedup over the pages' sparse attention ms/call on an RTX PRO 6000 "
                             "Blackwell (another machine; context only)",
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "heads": H, "seq_len": N, "head_dim": 128,
                   "n_blocks": nb, "top_k": kk, "summary": w.summary,
                   "sink_rows": w.sink_rows, "tau": w.tau, "extra_tokens": w.extra,
                   "reblock": w.reblock},
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "kernels_ms": {"pool": round(pool_ms, 4), "select": round(sel_ms, 4),
                       "attention": round(attn_ms, 4),
                       **({"select_tokens": round(tok_ms, 4)} if tok is not None else {}),
                       **({"reblock": round(reblock_ms, 4)} if w.reblock else {})},
        "wall_ms_per_step": round(wall_ms, 4),
        "median_ms_per_step": round(step_med, 4),
        "counted_tflop_per_step": round(flops / 1e12, 4),
        "summary_tflop_per_step": round(summary_flops / 1e12, 4),
        "pool_gbs": round(pool_bytes / (pool_ms * 1e-3) / 1e9, 1),
        "pool_frac": round(pool_bytes / (pool_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "pool_bytes": pool_bytes,
        **({"pool_reorder_copy_bytes": pool_copy_bytes,
            "pool_gbs_with_copies": round((pool_bytes + pool_copy_bytes) / (pool_ms * 1e-3) / 1e9, 1)}
           if w.reblock else {}),
        "select_gbs": round(sel_bytes / (sel_ms * 1e-3) / 1e9, 1),
        "tie_zone_rows": tie_rows,
        "roofline": {"bound": "mfma",
                     "kernel": "attn_fwd_kernel",
                     "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(w.name),
                     "traffic_unit": "bytes per launch (HBM, from rocprofv3 FETCH_SIZE + WRITE_SIZE)"},
        "peak_from_reported_clock": reported_clock_peak(),
        **({"context_gemm": {"what": "torch.matmul bf16 8192^3 (hipBLASLt), same device, after the steps",
                             "tflops": round(gemm_tflops, 1),
                             "attention_over_gemm": round(attn_tflops / gemm_tflops, 4)}}
           if gemm_tflops else {}),
        "input_gen_s": round(gen_s, 2),
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, qb, kb, vb, args.cpu_seconds)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
