"""Benchmark of the paged-KV attention hot path on one MI355X.

A step is one generate step of the long-context decode workload: append one
new token's K/V per sequence with pkv_cache_write, then attend that token
against the whole paged context with pkv_attn_forward (split kernel + fixed
order merge).  Workload: batch 16, Hq 64, Hkv 8, d 128, bf16, 131072 cached
keys per sequence, block_size 256, K/V-interleaved cache (block stride
2*256*8*128), random-permutation block table, N(0,1) values, causal.

Prints one JSON line: value = KV bytes read per second (GB/s) over the timed
steps, the roofline of the attention launch (bytes it must move / its HIP-event
duration vs 8 TB/s HBM), the oracle's throughput on a bounded sample of the
same work on the host's cores, a prefill figure (TFLOP/s of the full causal
prefill of batch 8 x 8192 tokens, Hq 16, Hkv 4), of its backward and of the
same prefill fed in 17- and 1024-token chunks, and bitwise checks.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_decode_c5_traffic.json")
MFMA_BF16_PEAK_TFLOPS = 2500.0


def settle(torch, fn, min_ms: float = 200.0, min_calls: int = 3):
    """Untimed calls of fn until at least min_calls calls and min_ms of wall time
    have passed, so the GPU clocks have settled before a timed region."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < min_calls or (time.perf_counter() - t0) * 1e3 < min_ms:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--profile", choices=["decode", "prefill", "rescore", "chunked17", "backward", "fp8"],
                    help="run one workload a few times and print its time (for rocprofv3); no JSON line")
    ap.add_argument("--calls", type=int, default=5, help="calls of the --profile workload")
    ap.add_argument("--batch", type=int, default=16)
    ap.add_argument("--seqlen-k", type=int, default=131072)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no multi-GPU sharding (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    import torch

    import invariant_paged_kv_amd as pkv
    import pkv_inputs as gen

    if args.profile:
        profile_run(torch, pkv, gen, args.profile, args.calls)
        return
    dev = "cuda"
    B, HQ, HK, D, BS = args.batch, 64, 8, 128, 256
    N = args.seqlen_k
    nb = gen.pool_num_blocks(N, BS, B)
    gdev = torch.Generator(device=dev).manual_seed(1005)
    pool = gen.new_pool(nb, BS, HK, D, "bf16", "interleaved", device=dev, generator=gdev)
    bt = gen.randperm_block_table(nb, B, generator=torch.Generator().manual_seed(1005)).to(dev)
    q = gen.randn((B, HQ, D), "bf16", generator=gdev, device=dev)
    kn = gen.randn((B, HK, D), "bf16", generator=gdev, device=dev)
    vn = gen.randn((B, HK, D), "bf16", generator=gdev, device=dev)
    pos = torch.full((B,), N - 1, dtype=torch.int32, device=dev)   # the new token's position
    seqlens = pos + 1
    cu = torch.arange(B + 1, dtype=torch.int32, device=dev)
    scale = 1.0 / math.sqrt(D)
    out = torch.empty_like(q)
    lse = torch.empty((B, HQ), dtype=torch.float32, device=dev)
    ws_bytes = pkv.workspace_size(q, pool.k, pool.v, bt, max_seqlen_q=1, max_seqlen_k=N)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    # one pair of events per timed step around the attention call, read after
    # the timed region: the steps are enqueued back to back, as a decode loop
    # would run them
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]

    def step(i=None):
        pkv.cache_write(kn, vn, pool.k, pool.v, bt, pos, cu)
        if i is not None:
            evs[i][0].record(stream)
        pkv.attn_forward(q, pool.k, pool.v, bt, seqlens, cu, True, scale, max_seqlen_q=1, max_seqlen_k=N,
                         out=out, lse=lse, workspace=ws)
        if i is not None:
            evs[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    attn_avg_ms = sum(a.elapsed_time(b) for a, b in evs) / args.steps
    ev0 = torch.cuda.Event(enable_timing=True)   # for the one-call timings below
    ev1 = torch.cuda.Event(enable_timing=True)

    kv_bytes = B * N * HK * D * 2 * 2
    attn_bytes = kv_bytes + 2 * q.numel() * 2 + lse.numel() * 4 + B * math.ceil(N / BS) * 4 + 2 * (B + 1) * 4
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = attn_bytes / (attn_avg_ms * 1e-3) / 1e9

    # the same step as one fused launch (append + attend), timed the same way
    def fused_step():
        ev0.record(stream)
        pkv.attn_forward_append(q, kn, vn, pool.k, pool.v, bt, seqlens, cu, True, scale, max_seqlen_q=1,
                                max_seqlen_k=N, out=out_f, lse=lse_f, workspace=ws)
        ev1.record(stream)

    out_f = torch.empty_like(q)
    lse_f = torch.empty_like(lse)
    for _ in range(args.warmup):
        fused_step()
    torch.cuda.synchronize()
    fused_ms = 0.0
    for _ in range(args.steps):
        fused_step()
        ev1.synchronize()
        fused_ms += ev0.elapsed_time(ev1)
    fused_ms /= args.steps
    fused_same = bool(torch.equal(out_f.view(torch.int16), out.view(torch.int16))
                      and torch.equal(lse_f.view(torch.int32), lse.view(torch.int32)))

    # bitwise: the prefill kernel on the same rows gives the same bits
    with pkv.options(path=2):
        p_out, p_lse = pkv.attn_forward(q, pool.k, pool.v, bt, seqlens, cu, True, scale, max_seqlen_q=1,
                                        max_seqlen_k=N)
    torch.cuda.synchronize()
    bitwise = bool(torch.equal(p_out.view(torch.int16), out.view(torch.int16))
                   and torch.equal(p_lse.view(torch.int32), lse.view(torch.int32)))

    result = {
        "metric": "decode KV GB/s (% HBM peak) + prefill TFLOP/s; decode==prefill bitwise",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic N(0,1), seeded",
        "config": {
            "workload": "long-context decode step: append 1 token + attend over 131072 cached keys",
            "batch": B, "num_heads_q": HQ, "num_heads_k": HK, "head_dim": D, "seqlen_k": N,
            "block_size": BS, "layout": "kv_interleaved", "block_table": "randperm", "causal": True,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(),
            "kernel": "pkv_attn_forward (split + merge)",
            "avg_ms": round(attn_avg_ms, 4),
            "bytes_per_launch": attn_bytes,
        },
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "bitwise_decode_eq_prefill_kernel": bitwise,
        "fused_append_step": {"api": "pkv_attn_forward_append", "avg_ms": round(fused_ms, 4),
                              "kv_GBs": round(kv_bytes / (fused_ms * 1e-3) / 1e9, 2),
                              "bitwise_eq_unfused": fused_same},
    }
    del p_out, p_lse

    # the default entry point, which takes the workspace from the stream-ordered
    # allocator inside every call (pkv_attn_forward without a workspace)
    def default_call():
        pkv.attn_forward(q, pool.k, pool.v, bt, seqlens, cu, True, scale, max_seqlen_q=1, max_seqlen_k=N,
                         out=out_f, lse=lse_f)

    settle(torch, default_call, min_ms=50.0)
    d_times = event_times(torch, default_call, args.steps)
    ws_times = event_times(torch, lambda: pkv.attn_forward(q, pool.k, pool.v, bt, seqlens, cu, True, scale,
                                                           max_seqlen_q=1, max_seqlen_k=N, out=out_f, lse=lse_f,
                                                           workspace=ws), args.steps)
    result["default_entry_point"] = {
        "api": "pkv_attn_forward (workspace from hipMallocAsync/hipFreeAsync inside the call)",
        "ms_median": round(d_times[len(d_times) // 2], 4),
        "ws_api_ms_median": round(ws_times[len(ws_times) // 2], 4)}
    del ws

    # The re-score of the generate-then-rescore workload: a 64-row causal
    # prefill per sequence over the same 131072-key cache (full path).
    RS = 64
    g_rs = torch.Generator(device=dev).manual_seed(1007)
    q_rs = gen.randn((B * RS, HQ, D), "bf16", generator=g_rs, device=dev)
    cu_rs = torch.arange(0, B * RS + 1, RS, dtype=torch.int32, device=dev)

    def rescore():
        return pkv.attn_forward(q_rs, pool.k, pool.v, bt, seqlens, cu_rs, True, scale, max_seqlen_q=RS,
                                max_seqlen_k=N)

    settle(torch, rescore)
    ev0.record(stream)
    for _ in range(5):
        rs_out, rs_lse = rescore()
    ev1.record(stream)
    ev1.synchronize()
    rs_ms = ev0.elapsed_time(ev1) / 5
    rs_flops = 4.0 * D * HQ * B * sum(N - RS + 1 + r for r in range(RS))
    result["rescore_prefill"] = {"workload": "64-row causal prefill per sequence over the same 131072-key cache",
                                 "ms": round(rs_ms, 3), "tflops": round(rs_flops / (rs_ms * 1e-3) / 1e12, 2),
                                 "frac": round(rs_flops / (rs_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                                 "flops": rs_flops}
    if not args.no_cpu_baseline:
        # the last row and the first of each of four sequences' 64 re-scored rows
        picks = [(b, b * RS + r, N - RS + r) for b in (0, 5, 10, 15) for r in (RS - 1, 0)]
        result["rescore_prefill"]["oracle"] = oracle_rows(torch, pool, bt, q_rs, picks, HQ, HK, D, BS, scale,
                                                          rs_out, rs_lse)
    del q_rs, rs_out, rs_lse

    if not args.no_configs:
        result["decode_configs"] = bench_decode_configs(torch, pkv, gen, want_cpu=not args.no_cpu_baseline)
    if not args.no_fp8:
        result["fp8_decode"] = bench_fp8_decode(torch, pkv, gen, B, N, args.steps, args.warmup, attn_avg_ms)
    if not args.no_prefill:
        result["prefill"], result["backward"], chunked = bench_prefill(torch, pkv, gen,
                                                                       want_cpu=not args.no_cpu_baseline)
        result["chunked_prefill"] = chunked
    if not args.no_cpu_baseline:
        result["cpu_baseline"], result["oracle_parity"] = cpu_baseline(torch, gen, pool, bt, q, N, HK, D, BS, scale,
                                                                       out, lse)
    print(json.dumps(result), flush=True)


def profile_run(torch, pkv, gen, what: str, calls: int):
    """One workload, `calls` times after one untimed call, for a profiler: the
    long-context decode call, the 8 x 8192 causal prefill, the 64-row re-score
    over 131072 keys, the 17-token chunked prefill (one graph replay), the
    prefill's backward, or the FP8 decode call."""
    dev = "cuda"
    if what in ("decode", "rescore", "fp8"):
        B, HQ, HK, D, BS, N = 16, 64, 8, 128, 256, 131072
        nb = gen.pool_num_blocks(N, BS, B)
        dt = "fp8" if what == "fp8" else "bf16"
        g = torch.Generator(device=dev).manual_seed(1005)
        pool = gen.new_pool(nb, BS, HK, D, dt, "interleaved", device=dev, generator=g)
        bt = gen.randperm_block_table(nb, B, generator=torch.Generator().manual_seed(1005)).to(dev)
        rows = 64 if what == "rescore" else 1
        q = gen.randn((B * rows, HQ, D), "bf16", generator=g, device=dev)
        sk = torch.full((B,), N, dtype=torch.int32, device=dev)
        cu = torch.arange(0, B * rows + 1, rows, dtype=torch.int32, device=dev)
        ws = torch.empty(max(256, pkv.workspace_size(q, pool.k, pool.v, bt, max_seqlen_q=rows, max_seqlen_k=N)),
                         dtype=torch.uint8, device=dev)
        ks, vs = (0.5, 1.25) if dt == "fp8" else (1.0, 1.0)

        def fn():
            pkv.attn_forward(q, pool.k, pool.v, bt, sk, cu, True, 1 / math.sqrt(D), max_seqlen_q=rows,
                             max_seqlen_k=N, workspace=ws, k_scale=ks, v_scale=vs)
    else:
        B, HQ, HK, D, BS, S = 8, 16, 4, 128, 16, 8192
        nb = gen.pool_num_blocks(S, BS, B)
        g = torch.Generator(device=dev).manual_seed(1004)
        pool = gen.new_pool(nb, BS, HK, D, "bf16", "contiguous", device=dev, generator=g)
        bt = gen.randperm_block_table(nb, B, generator=torch.Generator().manual_seed(1004)).to(dev)
        q = gen.randn((B * S, HQ, D), "bf16", generator=g, device=dev)
        sk = torch.full((B,), S, dtype=torch.int32, device=dev)
        cu = torch.arange(0, B * S + 1, S, dtype=torch.int32, device=dev)
        scale = 1 / math.sqrt(D)
        out, lse = pkv.attn_forward(q, pool.k, pool.v, bt, sk, cu, True, scale, max_seqlen_q=S, max_seqlen_k=S)
        if what == "prefill":
            def fn():
                pkv.attn_forward(q, pool.k, pool.v, bt, sk, cu, True, scale, max_seqlen_q=S, max_seqlen_k=S,
                                 out=out, lse=lse)
        elif what == "backward":
            dout = gen.randn((B * S, HQ, D), "bf16", generator=g, device=dev)

            def fn():
                pkv.attn_backward(q, pool.k, pool.v, bt, sk, cu, True, scale, out, lse, dout, max_seqlen_q=S,
                                  max_seqlen_k=S, total_k=B * S,
                                  cu_seqlens_k=torch.arange(0, B * S + 1, S, dtype=torch.int32, device=dev))
        else:   # chunked17: one replay of the captured 482-call graph
            res = bench_chunked_prefill(torch, pkv, pool, bt, q, out, lse, S, scale, 17, reps=calls)
            print(f"profile chunked17: {res['ms']} ms per replay, bitwise {res['bitwise_eq_one_shot']}", flush=True)
            return
    fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(calls):
        fn()
    torch.cuda.synchronize()
    print(f"profile {what}: {(time.perf_counter() - t0) * 1e3 / calls:.4f} ms per call (wall)", flush=True)


FLUSH_BYTES = 1 << 30   # > L2 (8 x 4 MB) + the 256 MB Infinity Cache


def event_times(torch, fn, reps: int, flush=None):
    """Per-call HIP-event times (ms) of fn on the current stream: cold (a 1 GiB
    read before each call evicts L2 and the Infinity Cache) when `flush` is
    given, else warm (calls back to back, one event pair around each).  The
    flush reads rather than writes: a written flush leaves the caches full of
    dirty lines whose write-back then lands inside the timed call."""
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i in range(reps):
        if flush is not None:
            flush.view(torch.int32).max()
        evs[i][0].record(stream)
        fn()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in evs)


def decode_workloads():
    """The decode workloads other than the long-context one, with their recipes."""
    return [
        dict(name="single sequence fp32 (339 cached + 1 appended, decode over 340 keys)", key="fp32_single",
             dtype="f32", batch=1, hq=2, hk=2, d=64, bs=16, layout="contiguous", causal=False, seed=1001,
             lens=lambda g: [340], rows=lambda g: [1]),
        dict(name="decode, Qwen3-8B-like shard: batch 64 x 4096 keys, Hq 16 / Hkv 4", key="qwen_shard",
             dtype="bf16", batch=64, hq=16, hk=4, d=128, bs=16, layout="interleaved", causal=True, seed=1002,
             lens=lambda g: [4096] * 64, rows=lambda g: [1] * 64),
        dict(name="ragged / padded decode: batch 128, keys U{1..8192}, 3-row slots, Hq 32 / Hkv 8",
             key="ragged_padded", dtype="bf16", batch=128, hq=32, hk=8, d=128, bs=256, layout="interleaved",
             causal=True, seed=1003, lens=lambda g: g.uniform_int(1, 8192, 128, generator=torch_gen(1003)),
             rows=lambda g: [3] * 128),
    ]


def torch_gen(seed):
    import torch
    return torch.Generator().manual_seed(seed)


def bench_decode_configs(torch, pkv, gen, reps: int = 30, want_cpu: bool = True):
    """Cold and warm per-call timings of the other decode workloads, each with its
    roofline (K/V bytes of the visible keys + q/out/lse/table, against 8 TB/s),
    bitwise decode == prefill, and the oracle's agreement and host throughput on
    a bounded sample of the same call."""
    dev = "cuda"
    flush = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    results = []
    for w in decode_workloads():
        B, HQ, HK, D, BS = w["batch"], w["hq"], w["hk"], w["d"], w["bs"]
        lens = [int(x) for x in w["lens"](gen)]
        rows = w["rows"](gen)
        mk = max(lens)
        nb = gen.pool_num_blocks(mk, BS, B)
        g = torch.Generator(device=dev).manual_seed(w["seed"])
        pool = gen.new_pool(nb, BS, HK, D, w["dtype"], w["layout"], device=dev, generator=g)
        bt = gen.randperm_block_table(nb, B, generator=torch.Generator().manual_seed(w["seed"])).to(dev)
        cu_l = [0]
        for r in rows:
            cu_l.append(cu_l[-1] + r)
        q = gen.randn((cu_l[-1], HQ, D), w["dtype"], generator=g, device=dev)
        sk = torch.tensor(lens, dtype=torch.int32, device=dev)
        cu = torch.tensor(cu_l, dtype=torch.int32, device=dev)
        scale = 1.0 / math.sqrt(D)
        out = torch.empty_like(q)
        lse = torch.empty((q.shape[0], HQ), dtype=torch.float32, device=dev)
        Lq = max(rows)
        ws = torch.empty(max(256, pkv.workspace_size(q, pool.k, pool.v, bt, max_seqlen_q=Lq, max_seqlen_k=mk)),
                         dtype=torch.uint8, device=dev)

        def call():
            pkv.attn_forward(q, pool.k, pool.v, bt, sk, cu, w["causal"], scale, max_seqlen_q=Lq, max_seqlen_k=mk,
                             out=out, lse=lse, workspace=ws)

        settle(torch, call, min_ms=100.0)
        cold = event_times(torch, call, reps, flush)
        warm = event_times(torch, call, reps)
        eb = 4 if w["dtype"] == "f32" else 2
        kv = sum(lens) * HK * D * eb * 2
        nbytes = kv + 2 * q.numel() * eb + lse.numel() * 4 + sum(math.ceil(n / BS) for n in lens) * 4 + (2 * B + 1) * 4
        med_c, med_w = cold[len(cold) // 2], warm[len(warm) // 2]
        with pkv.options(path=2):
            p_out, p_lse = pkv.attn_forward(q, pool.k, pool.v, bt, sk, cu, w["causal"], scale, max_seqlen_q=Lq,
                                            max_seqlen_k=mk)
        torch.cuda.synchronize()
        same = bool(torch.equal(p_out.contiguous().view(torch.int32 if eb == 4 else torch.int16),
                                out.view(torch.int32 if eb == 4 else torch.int16))
                    and torch.equal(p_lse.view(torch.int32), lse.view(torch.int32)))
        gbs = nbytes / (med_c * 1e-3) / 1e9
        res = {"workload": w["name"], "dtype": w["dtype"], "batch": B, "num_heads_q": HQ, "num_heads_k": HK,
               "head_dim": D, "block_size": BS, "layout": w["layout"], "keys_total": sum(lens),
               "rows": cu_l[-1], "bytes_per_launch": nbytes,
               "cold_ms_median": round(med_c, 4), "cold_ms_min": round(cold[0], 4),
               "warm_ms_median": round(med_w, 4), "warm_ms_min": round(warm[0], 4),
               "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": round(gbs / HBM_PEAK_GBS, 4), "timing": "cold (1 GiB flush before each call)"},
               "warm_GBs": round(nbytes / (med_w * 1e-3) / 1e9, 2),
               "tokens_per_s": round(cu_l[-1] / (med_c * 1e-3), 1),
               "bitwise_decode_eq_prefill_kernel": same}
        if want_cpu:
            res["oracle"] = oracle_sample(torch, pool, bt, q, lens, cu_l, w, out, lse, scale,
                                          budget_s=3.0 if B > 1 else 1.0, one_thread=w["key"] != "ragged_padded")
        results.append(res)
        del pool, ws, out, lse, p_out, p_lse, q
        torch.cuda.empty_cache()
    del flush
    torch.cuda.empty_cache()
    return results


def oracle_sample(torch, pool, bt, q, lens, cu_l, w, out, lse, scale, budget_s: float, one_thread: bool):
    """The float64 oracle on whole sequences of the call, until `budget_s` of host
    time is spent (all host threads; also on one thread for the small workloads):
    K/V bytes per second of host time and the max-abs agreement with the GPU."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle

    HQ, HK, D, BS = w["hq"], w["hk"], w["d"], w["bs"]
    eb = 4 if w["dtype"] == "f32" else 2
    gout = out.double().cpu().numpy()
    glse = lse.double().cpu().numpy()

    def host_seq(b):
        n = lens[b]
        nblk = math.ceil(n / BS)
        ids = bt[b, :nblk].long()
        kh = pool.k.index_select(0, ids).cpu().contiguous()
        vh = pool.v.index_select(0, ids).cpu().contiguous()
        cast = (lambda t: t.numpy().reshape(-1)) if eb == 4 else \
            (lambda t: t.view(torch.int16).numpy().view(np.uint16).reshape(-1))
        row = HK * D
        lay = oracle.Layout(w["dtype"], HQ, HK, D, BS, 0, (BS * row, row, D), 0, (BS * row, row, D))
        r0, r1 = cu_l[b], cu_l[b + 1]
        qh = q[r0:r1].cpu()
        qh = qh.numpy() if eb == 4 else qh.view(torch.int16).numpy().view(np.uint16)
        return n, nblk, cast(kh), cast(vh), lay, qh, r0, r1

    def run(threads):
        done, spent, seqs, eo, el = 0, 0.0, 0, 0.0, 0.0
        order = sorted(range(len(lens)), key=lambda b: lens[b])   # short sequences first: more of them fit
        for b in order:
            n, nblk, kf, vf, lay, qh, r0, r1 = host_seq(b)
            t0 = time.perf_counter()
            if threads is None:
                oo, ol = oracle.attention(qh, kf, vf, lay, np.arange(nblk, dtype=np.int32)[None, :], [n],
                                          [0, r1 - r0], w["causal"], scale)
            else:
                with threadpool_limits(threads):
                    oo, ol = oracle.attention(qh, kf, vf, lay, np.arange(nblk, dtype=np.int32)[None, :], [n],
                                              [0, r1 - r0], w["causal"], scale)
            spent += time.perf_counter() - t0
            fin = np.isfinite(ol)
            eo = max(eo, float(np.max(np.abs(gout[r0:r1] - oo))))
            el = max(el, float(np.max(np.abs(glse[r0:r1][fin] - ol[fin]))) if fin.any() else 0.0)
            seqs += 1
            done += n * HK * D * eb * 2
            if spent >= budget_s:
                break
        return done, spent, seqs, eo, el

    done, spent, seqs, eo, el = run(None)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    res = {"value": round(done / spent / 1e9, 5), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": f"{seqs} of {len(lens)} sequences ({spent:.2f} s)",
           "out_max_abs": eo, "lse_max_abs": el}
    if one_thread:
        d1, s1, n1, _, _ = run(1)
        res["one_thread"] = {"value": round(d1 / s1 / 1e9, 5), "unit": "GB/s", "cores": 1,
                             "sample": f"{n1} of {len(lens)} sequences ({s1:.2f} s)"}
    return res


def measured_traffic():
    """HBM bytes per attention call from the committed rocprofv3 counter summary.

    The counters (FETCH_SIZE, WRITE_SIZE, calibrated on a plain copy) were
    taken on specific kernel sources; if those have changed since, the figure
    no longer describes the compiled library and None is reported.
    """
    import hashlib
    try:
        info = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    h = hashlib.sha256()
    for f in info.get("source_files", []):
        try:
            h.update(open(os.path.join(ROOT, "invariant_paged_kv_amd", "csrc", f), "rb").read())
        except OSError:
            return None
    if h.hexdigest() != info.get("source_sha256"):
        return None
    return info.get("traffic_bytes_per_launch")


def bench_fp8_decode(torch, pkv, gen, B, N, steps, warmup, bf16_ms):
    """The same decode call over an FP8 E4M3 cache of the same shape (half the KV bytes)."""
    dev = "cuda"
    HQ, HK, D, BS = 64, 8, 128, 256
    nb = gen.pool_num_blocks(N, BS, B)
    g = torch.Generator(device=dev).manual_seed(1006)
    pool = gen.new_pool(nb, BS, HK, D, "fp8", "interleaved", device=dev, generator=g)
    bt = gen.randperm_block_table(nb, B, generator=torch.Generator().manual_seed(1006)).to(dev)
    q = gen.randn((B, HQ, D), "bf16", generator=g, device=dev)
    seqlens = torch.full((B,), N, dtype=torch.int32, device=dev)
    cu = torch.arange(B + 1, dtype=torch.int32, device=dev)
    scale, ks, vs = 1.0 / math.sqrt(D), 0.5, 1.25
    out = torch.empty_like(q)
    lse = torch.empty((B, HQ), dtype=torch.float32, device=dev)
    ws = torch.empty(pkv.workspace_size(q, pool.k, pool.v, bt, max_seqlen_q=1, max_seqlen_k=N), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)

    def call():
        ev0.record(stream)
        pkv.attn_forward(q, pool.k, pool.v, bt, seqlens, cu, True, scale, max_seqlen_q=1, max_seqlen_k=N, out=out,
                         lse=lse, workspace=ws, k_scale=ks, v_scale=vs)
        ev1.record(stream)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    total = 0.0
    for _ in range(steps):
        call()
        ev1.synchronize()
        total += ev0.elapsed_time(ev1)
    ms = total / steps
    with pkv.options(path=2):
        p_out, p_lse = pkv.attn_forward(q, pool.k, pool.v, bt, seqlens, cu, True, scale, max_seqlen_q=1,
                                        max_seqlen_k=N, k_scale=ks, v_scale=vs)
    torch.cuda.synchronize()
    same = bool(torch.equal(p_out.view(torch.int16), out.view(torch.int16))
                and torch.equal(p_lse.view(torch.int32), lse.view(torch.int32)))
    kv_bytes = B * N * HK * D * 1 * 2
    call_bytes = kv_bytes + 2 * q.numel() * 2 + lse.numel() * 4 + B * math.ceil(N / BS) * 4 + 2 * (B + 1) * 4
    gbs = call_bytes / (ms * 1e-3) / 1e9
    del pool, ws, p_out, p_lse
    torch.cuda.empty_cache()
    return {"workload": "the decode call over an FP8 E4M3 cache of the same shape (k_scale 0.5, v_scale 1.25)",
            "avg_ms": round(ms, 4), "bytes_per_launch": call_bytes, "achieved_GBs": round(gbs, 2),
            "frac": round(gbs / HBM_PEAK_GBS, 4), "keys_per_s": round(B * N / (ms * 1e-3), 1),
            "speedup_vs_bf16_call": round(bf16_ms / ms, 3), "bitwise_decode_eq_prefill_kernel": same}


def bench_prefill(torch, pkv, gen, reps: int = 5, want_cpu: bool = True):
    """Full causal prefill, batch 8 x 8192 tokens, Hq 16, Hkv 4, d 128, bs 16 (TFLOP/s of causal pairs)."""
    dev = "cuda"
    B, HQ, HK, D, BS, S = 8, 16, 4, 128, 16, 8192
    nb = gen.pool_num_blocks(S, BS, B)
    g = torch.Generator(device=dev).manual_seed(1004)
    pool = gen.new_pool(nb, BS, HK, D, "bf16", "contiguous", device=dev, generator=g)
    bt = gen.randperm_block_table(nb, B, generator=torch.Generator().manual_seed(1004)).to(dev)
    q = gen.randn((B * S, HQ, D), "bf16", generator=g, device=dev)
    sk = torch.full((B,), S, dtype=torch.int32, device=dev)
    cu = torch.arange(0, B * S + 1, S, dtype=torch.int32, device=dev)
    scale = 1.0 / math.sqrt(D)

    def call():
        return pkv.attn_forward(q, pool.k, pool.v, bt, sk, cu, True, scale, max_seqlen_q=S, max_seqlen_k=S)

    settle(torch, call)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        call()
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    flops = 4.0 * D * HQ * B * (S * (S + 1) / 2)
    tf = flops / (ms * 1e-3) / 1e12
    fwd = {"workload": "full causal prefill batch 8 x 8192, Hq 16, Hkv 4, d 128, bs 16",
           "ms": round(ms, 3), "tflops": round(tf, 2), "mfma_bf16_peak_tflops": MFMA_BF16_PEAK_TFLOPS,
           "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "flops": flops}
    if want_cpu:
        # rows spread over the causal range of every sequence, longest first
        out, lse = call()
        picks = [(b, b * S + p, p) for p in range(S - 1, 0, -256) for b in range(B)]
        fwd["oracle"] = oracle_rows(torch, pool, bt, q, picks, HQ, HK, D, BS, scale, out, lse)

    # Backward of the same prefill: dq, dk, dv for a seeded N(0,1) cotangent.
    # Algorithmic FLOPs: the five products dP, dV, dK, dQ and the recomputed S
    # over the causal pairs, 2.5x the forward's two.
    out, lse = call()
    chunked = []
    for c, fused in ((17, False), (17, True), (1024, False)):
        try:
            chunked.append(bench_chunked_prefill(torch, pkv, pool, bt, q, out, lse, S, scale, c, fused=fused))
        except (RuntimeError, ValueError) as exc:   # reported in the line; the other figures still print
            chunked.append({"chunk_tokens": c, "fused": fused, "error": str(exc)[:200]})
    dout = gen.randn((B * S, HQ, D), "bf16", generator=g, device=dev)
    cuk = torch.arange(0, B * S + 1, S, dtype=torch.int32, device=dev)
    dq = torch.empty_like(q)
    dk = torch.empty((B * S, HK, D), dtype=q.dtype, device=dev)
    dv = torch.empty_like(dk)

    def bwd():
        return pkv.attn_backward(q, pool.k, pool.v, bt, sk, cu, True, scale, out, lse, dout, max_seqlen_q=S,
                                 max_seqlen_k=S, cu_seqlens_k=cuk, total_k=B * S, dq=dq, dk=dk, dv=dv)

    settle(torch, bwd)
    e0.record()
    for _ in range(reps):
        bwd()
    e1.record()
    e1.synchronize()
    bms = e0.elapsed_time(e1) / reps
    bflops = 2.5 * flops
    btf = bflops / (bms * 1e-3) / 1e12
    bwd_res = {"workload": "backward of the same prefill (dq, dk, dv)", "ms": round(bms, 3),
               "tflops": round(btf, 2), "frac": round(btf / MFMA_BF16_PEAK_TFLOPS, 4), "flops": bflops}
    del pool, out, lse, dout, dq, dk, dv
    torch.cuda.empty_cache()
    return fwd, bwd_res, chunked


def bench_chunked_prefill(torch, pkv, pool, bt, q, ref_out, ref_lse, S, scale, chunk, reps: int = 3,
                          fused: bool = False):
    """The same prefill fed in chunks of `chunk` tokens per sequence.

    Each call appends the chunk's K/V with pkv_cache_write (the bits the pool
    already holds at those positions, so the cache is unchanged) and attends
    the chunk's rows over every key up to the chunk's end.  The calls are
    captured once as a HIP graph and replayed, as a serving loop would run
    them; the chunked out/lse must equal the one-shot prefill's bit for bit.
    With `fused`, each call is one pkv_attn_forward_append instead.
    """
    dev = q.device
    B, HK, D = bt.shape[0], pool.k.shape[2], pool.k.shape[3]
    BS, HQ = pool.k.shape[1], q.shape[1]
    used = bt[:, :S // BS].long()
    kd = pool.k[used].reshape(B, S, HK, D)   # each sequence's keys and values, dense
    vd = pool.v[used].reshape(B, S, HK, D)
    qv = q.view(B, S, HQ, D)
    calls = []
    for lo in range(0, S, chunk):
        hi = min(lo + chunk, S)
        n = hi - lo
        qc = qv[:, lo:hi].reshape(B * n, HQ, D).contiguous()
        calls.append({
            "lo": lo, "hi": hi, "q": qc,
            "k": kd[:, lo:hi].reshape(B * n, HK, D).contiguous(),
            "v": vd[:, lo:hi].reshape(B * n, HK, D).contiguous(),
            "pos": torch.full((B,), lo, dtype=torch.int32, device=dev),
            "sk": torch.full((B,), hi, dtype=torch.int32, device=dev),
            "cu": torch.arange(0, B * n + 1, n, dtype=torch.int32, device=dev),
            "out": torch.empty_like(qc),
            "lse": torch.empty((B * n, HQ), dtype=torch.float32, device=dev),
        })
    del kd, vd
    # the largest split-path workspace any call needs: B * chunk rows over all S keys
    ws_bytes = pkv.workspace_size(q[:B * chunk], pool.k, pool.v, bt, max_seqlen_q=chunk, max_seqlen_k=S)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    def run_all():
        for c in calls:
            if fused:
                pkv.attn_forward_append(c["q"], c["k"], c["v"], pool.k, pool.v, bt, c["sk"], c["cu"], True, scale,
                                        max_seqlen_q=c["hi"] - c["lo"], max_seqlen_k=c["hi"], out=c["out"],
                                        lse=c["lse"], workspace=ws)
                continue
            pkv.cache_write(c["k"], c["v"], pool.k, pool.v, bt, c["pos"], c["cu"])
            pkv.attn_forward(c["q"], pool.k, pool.v, bt, c["sk"], c["cu"], True, scale,
                             max_seqlen_q=c["hi"] - c["lo"], max_seqlen_k=c["hi"], out=c["out"], lse=c["lse"],
                             workspace=ws)

    def same_as_one_shot():
        ro, rl = ref_out.view(B, S, HQ, D), ref_lse.view(B, S, HQ)
        ok = True
        for c in calls:
            n = c["hi"] - c["lo"]
            ok = ok and torch.equal(c["out"].view(B, n, HQ, D).view(torch.int16),
                                    ro[:, c["lo"]:c["hi"]].view(torch.int16))
            ok = ok and torch.equal(c["lse"].view(B, n, HQ).view(torch.int32), rl[:, c["lo"]:c["hi"]].view(torch.int32))
        return bool(ok)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        run_all()                      # eager pass on the capture stream
        torch.cuda.synchronize()
        eager_same = same_as_one_shot()
        with torch.cuda.graph(graph, stream=side):
            run_all()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for c in calls:
        c["out"].fill_(float("nan"))
        c["lse"].fill_(float("nan"))
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    replay_same = same_as_one_shot()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1) / reps
    timed_same = same_as_one_shot()
    flops = 4.0 * D * HQ * B * (S * (S + 1) / 2)
    kv_bytes = sum(B * c["hi"] * HK * D * 2 * 2 for c in calls)   # every call re-reads the keys it sees
    per_call = "pkv_attn_forward_append" if fused else "cache_write + attention"
    res = {"workload": f"the same prefill in {len(calls)} chunks of {chunk} tokens per sequence "
                       f"({per_call} per chunk, replayed as one HIP graph)",
           "chunk_tokens": chunk, "fused": fused, "calls": len(calls), "ms": round(ms, 3),
           "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
           "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
           "kv_reread_bytes": kv_bytes, "kv_GBs": round(kv_bytes / (ms * 1e-3) / 1e9, 2),
           "hbm_frac": round(kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "bitwise_eq_one_shot": eager_same and replay_same and timed_same}
    del graph, calls, ws
    torch.cuda.empty_cache()
    return res


def cpu_baseline(torch, gen, pool, bt, q, N, HK, D, BS, scale, out, lse, budget_s: float = 12.0):
    """The float64 oracle on whole sequences of the same decode step, timed on the host.

    The oracle's results for those sequences are also compared with the GPU's
    out / lse of the same step (max-abs errors reported next to the timing).
    """
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle

    nblk = math.ceil(N / BS)
    done, spent, seqs = 0, 0.0, 0
    err_o = err_l = 0.0
    gout = out.double().cpu().numpy()
    glse = lse.double().cpu().numpy()
    B, HQ = q.shape[0], q.shape[1]
    for b in range(B):
        ids = bt[b, :nblk].long()
        kh = pool.k.index_select(0, ids).cpu().contiguous()
        vh = pool.v.index_select(0, ids).cpu().contiguous()
        kf = kh.view(torch.int16).numpy().view(np.uint16).reshape(-1)
        vf = vh.view(torch.int16).numpy().view(np.uint16).reshape(-1)
        row = HK * D
        lay = oracle.Layout("bf16", HQ, HK, D, BS, 0, (BS * row, row, D), 0, (BS * row, row, D))
        qh = q[b:b + 1].cpu().view(torch.int16).numpy().view(np.uint16)
        t0 = time.perf_counter()
        oo, ol = oracle.attention(qh, kf, vf, lay, np.arange(nblk, dtype=np.int32)[None, :], [N], [0, 1], True, scale)
        spent += time.perf_counter() - t0
        err_o = max(err_o, float(np.max(np.abs(gout[b] - oo[0]))))
        err_l = max(err_l, float(np.max(np.abs(glse[b] - ol[0]))))
        seqs += 1
        done += N * HK * D * 2 * 2
        if spent >= budget_s:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(done / spent / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{seqs} of {B} sequences of one decode step (all {HQ} heads, {N} keys each), "
                      f"{spent:.1f} s"}, {"out_max_abs": err_o, "lse_max_abs": err_l, "sequences": seqs,
                                           "tolerance": {"out": 2e-2, "lse": 1e-3}}


def oracle_rows(torch, pool, bt, q, picks, HQ, HK, D, BS, scale, out, lse, budget_s: float = 4.0):
    """The float64 oracle on sampled causal rows of a prefill, timed on the host.

    ``picks`` lists (sequence, row of q, key position p): each row is the
    oracle's one-row call over that sequence's keys 0..p (a causal row at
    position p sees exactly those), taken in order until ``budget_s`` of host
    time is spent.  Returns the oracle's TFLOP/s (4 * d * Hq * (p + 1) per row)
    and its max-abs agreement with the GPU's out / lse of those rows."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle

    gout = out.double().cpu().numpy()
    glse = lse.double().cpu().numpy()
    row = HK * D
    lay = oracle.Layout("bf16", HQ, HK, D, BS, 0, (BS * row, row, D), 0, (BS * row, row, D))
    spent, flops, rows, eo, el = 0.0, 0.0, 0, 0.0, 0.0
    for b, r, p in picks:
        n = p + 1
        nblk = math.ceil(n / BS)
        ids = bt[b, :nblk].long()
        kf = pool.k.index_select(0, ids).cpu().contiguous().view(torch.int16).numpy().view(np.uint16).reshape(-1)
        vf = pool.v.index_select(0, ids).cpu().contiguous().view(torch.int16).numpy().view(np.uint16).reshape(-1)
        qh = q[r:r + 1].cpu().view(torch.int16).numpy().view(np.uint16)
        t0 = time.perf_counter()
        oo, ol = oracle.attention(qh, kf, vf, lay, np.arange(nblk, dtype=np.int32)[None, :], [n], [0, 1], True, scale)
        spent += time.perf_counter() - t0
        eo = max(eo, float(np.max(np.abs(gout[r] - oo[0]))))
        el = max(el, float(np.max(np.abs(glse[r] - ol[0]))))
        flops += 4.0 * D * HQ * n
        rows += 1
        if spent >= budget_s:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {len(picks)} sampled rows, all {HQ} heads ({spent:.1f} s)",
            "out_max_abs": eo, "lse_max_abs": el, "tolerance": {"out": 2e-2, "lse": 1e-3}}


if __name__ == "__main__":
    main()
