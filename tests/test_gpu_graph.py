"""Decode and chunked-prefill steps inside a captured HIP graph.

pkv_attn_forward_ws and pkv_cache_write allocate nothing and enqueue only
kernels (no memset), so a decode step can be captured once and replayed.
Each replay, with eager work and synchronisations between replays, must give
the eager result bit for bit.
"""

from __future__ import annotations

import math

import pytest
import torch

import invariant_paged_kv_amd as pkv
import pkv_inputs as gen
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_decode_step_replays_bitwise(dtype):
    announce(f"graph replay decode step {dtype}")
    B, HQ, HK, D, BS, N = 4, 32, 8, 128, 256, 3000
    g = torch.Generator().manual_seed(9300)
    nb = gen.pool_num_blocks(N, BS, B)
    pool = gc.to_device(gen.new_pool(nb, BS, HK, D, dtype, "interleaved", generator=g))
    bt = gen.randperm_block_table(nb, B, generator=g).to(gc.DEV)
    qdt = "bf16"
    q = gen.randn((B, HQ, D), qdt, generator=g).to(gc.DEV)
    kn = gen.randn((B, HK, D), dtype, generator=g).to(gc.DEV)
    vn = gen.randn((B, HK, D), dtype, generator=g).to(gc.DEV)
    pos = torch.full((B,), N - 1, dtype=torch.int32, device=gc.DEV)
    seqlens = pos + 1
    cu = torch.arange(B + 1, dtype=torch.int32, device=gc.DEV)
    scale = 1.0 / math.sqrt(D)
    out = torch.empty_like(q)
    lse = torch.empty((B, HQ), dtype=torch.float32, device=gc.DEV)
    ws = torch.empty(pkv.workspace_size(q, pool.k, pool.v, bt, max_seqlen_q=1, max_seqlen_k=N), dtype=torch.uint8,
                     device=gc.DEV)

    def step():
        pkv.cache_write(kn, vn, pool.k, pool.v, bt, pos, cu)
        pkv.attn_forward(q, pool.k, pool.v, bt, seqlens, cu, True, scale, max_seqlen_q=1, max_seqlen_k=N, out=out,
                         lse=lse, workspace=ws, k_scale=0.5 if dtype == "fp8" else 1.0)

    step()
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()                       # warm up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=gc.DEV).sum()   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        gc.assert_bitwise((out, lse), ref, f"replay {i}")
        del junk


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_prefill_chunk_replays_bitwise(dtype):
    """A chunked-prefill step (append the chunk, attend through the full path) captured once."""
    announce(f"graph replay prefill chunk {dtype}")
    B, HQ, HK, D, BS, N, LC = 2, 16, 4, 128, 16, 2300, 96
    g = torch.Generator().manual_seed(9310)
    nb = gen.pool_num_blocks(N, BS, B)
    pool = gc.to_device(gen.new_pool(nb, BS, HK, D, dtype, "contiguous", generator=g))
    bt = gen.randperm_block_table(nb, B, generator=g).to(gc.DEV)
    q = gen.randn((B * LC, HQ, D), "bf16", generator=g).to(gc.DEV)
    kn = gen.randn((B * LC, HK, D), dtype, generator=g).to(gc.DEV)
    vn = gen.randn((B * LC, HK, D), dtype, generator=g).to(gc.DEV)
    pos = torch.full((B,), N - LC, dtype=torch.int32, device=gc.DEV)
    seqlens = pos + LC
    cu = torch.arange(0, B * LC + 1, LC, dtype=torch.int32, device=gc.DEV)
    scale = 1.0 / math.sqrt(D)
    out = torch.empty_like(q)
    lse = torch.empty((B * LC, HQ), dtype=torch.float32, device=gc.DEV)

    def step():
        pkv.cache_write(kn, vn, pool.k, pool.v, bt, pos, cu)
        with pkv.options(path=2):
            pkv.attn_forward(q, pool.k, pool.v, bt, seqlens, cu, True, scale, max_seqlen_q=LC, max_seqlen_k=N,
                             out=out, lse=lse, k_scale=0.5 if dtype == "fp8" else 1.0)

    step()
    torch.cuda.synchronize()
    ref = (out.clone(), lse.clone())
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        junk = torch.randn(1 << 20, device=gc.DEV).sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        gc.assert_bitwise((out, lse), ref, f"replay {i}")
        del junk
