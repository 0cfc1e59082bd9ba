"""GPU edge cases: unusual block sizes, degenerate batches, the caller-owned
workspace entry point, and large head counts per KV head.

aiter commit d293d61bbf19 parametrises block_size over {16, 256}; the library
accepts any block size >= 1 (key j of a sequence is in table entry j / block_size),
so odd sizes are checked against the oracle here too.
"""

from __future__ import annotations

import math

import pytest
import torch

import invariant_paged_kv_amd as pkv
import pkv_inputs as gen
from tests import gpu_cases as gc
from tests.oracle_bridge import oracle_pool, storage_np

import numpy as np
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("bs", [1, 3, 7, 48, 100, 1024])
@pytest.mark.parametrize("layout", ["contiguous", "interleaved"])
def test_odd_block_sizes(bs, layout):
    announce(f"block_size {bs} {layout}")
    case = gc.make_case(4000 + bs, "bf16", 3, 8, 2, 128, bs, 1500, layout, True, [1, 5, 2])
    out, lse = gc.run(case)
    gc.check_oracle(case, out, lse)
    other = gen.relayout(case.pool, "contiguous" if layout == "interleaved" else "interleaved")
    gc.assert_bitwise(gc.run(case, pool=other), (out, lse), "layouts")
    for path in (1, 2):
        gc.assert_bitwise(gc.run(case, path=path), (out, lse), f"path {path}")
    for fk in (1, 3):   # the other full-path kernels (per-row block ids when bs % 16 != 0)
        gc.assert_bitwise(gc.run(case, path=2, full_kernel=fk), (out, lse), f"full kernel {fk}")


@pytest.mark.parametrize("bs", [1, 7, 100])
def test_cache_write_odd_block_sizes(bs):
    announce(f"cache_write block_size {bs}")
    g = torch.Generator().manual_seed(4100 + bs)
    hk, d, batch = 2, 64, 2
    nb = gen.pool_num_blocks(300, bs, batch)
    host = gen.new_pool(nb, bs, hk, d, "bf16", "interleaved", generator=g)
    bt = gen.randperm_block_table(nb, batch, generator=g)
    seqlens, lens = [13, 250], [40, 1]
    cu = gen.cu_from_lengths(lens)
    kn = gen.randn((41, hk, d), "bf16", generator=g)
    vn = gen.randn((41, hk, d), "bf16", generator=g)
    kf, vf, lay = oracle_pool(host, hk)
    ek, ev = oracle.cache_write(kf, vf, lay, storage_np(kn), storage_np(vn), bt.numpy(), seqlens, cu.tolist())
    pool = gc.to_device(host)
    pkv.cache_write(kn.to(gc.DEV), vn.to(gc.DEV), pool.k, pool.v, bt.to(gc.DEV),
                    torch.tensor(seqlens, dtype=torch.int32, device=gc.DEV), cu.to(gc.DEV))
    torch.cuda.synchronize()
    gk, gv, _ = oracle_pool(gc.host_pool(pool), hk)
    assert np.array_equal(gk, ek) and np.array_equal(gv, ev)


def test_caller_workspace_matches_internal():
    announce("pkv_attn_forward_ws vs pkv_attn_forward")
    case = gc.make_case(4200, "bf16", 4, 16, 4, 128, 16, 3000, "interleaved", True, [1, 1, 1, 1])
    ref = gc.run(case, path=1)
    sk, cu = case.seqlens_d(), case.cu_d()
    need = pkv.workspace_size(case.q, case.pool.k, case.pool.v, case.block_table, max_seqlen_q=1,
                              max_seqlen_k=case.max_seqlen_k)
    assert need > 0
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=gc.DEV)   # garbage-filled workspace
    with pkv.options(path=1):
        out, lse = pkv.attn_forward(case.q, case.pool.k, case.pool.v, case.block_table, sk, cu, True, case.scale,
                                    max_seqlen_q=1, max_seqlen_k=case.max_seqlen_k, workspace=ws)
        torch.cuda.synchronize()
        gc.assert_bitwise((out, lse), ref, "caller workspace")
        with pytest.raises(pkv.PkvError):
            pkv.attn_forward(case.q, case.pool.k, case.pool.v, case.block_table, sk, cu, True, case.scale,
                             max_seqlen_q=1, max_seqlen_k=case.max_seqlen_k, workspace=ws[: need // 2])


def test_degenerate_batches():
    """Empty sequences, sequences with no keys, and a batch whose only rows see nothing."""
    announce("degenerate batches")
    case = gc.make_case(4300, "bf16", 4, 8, 2, 128, 16, 600, "interleaved", True, [0, 3, 2, 0],
                        seqlens=[5, 0, 1, 600])
    out, lse = gc.run(case)
    gc.check_oracle(case, out, lse)
    r = case.cu
    assert torch.all(lse[r[1]:r[2]] == -math.inf) and torch.all(out[r[1]:r[2]] == 0)   # n = 0
    assert torch.all(lse[r[2]:r[2] + 1] == -math.inf)      # n = 1, L = 2: first row at position -1
    for path in (1, 2):
        gc.assert_bitwise(gc.run(case, path=path), (out, lse), f"path {path}")
    # the first sequence has rows but no keys: no path may read its block-table row
    # (a read before the table) -- its rows see nothing, the other sequence is normal
    first = gc.make_case(4310, "bf16", 2, 8, 2, 128, 16, 700, "contiguous", True, [4, 2], seqlens=[0, 700])
    fo, fl = gc.run(first)
    gc.check_oracle(first, fo, fl)
    assert torch.all(fl[0:4] == -math.inf) and torch.all(fo[0:4] == 0)
    for path in (1, 2):
        gc.assert_bitwise(gc.run(first, path=path), (fo, fl), f"first empty, path {path}")
    # a zero-row call is a no-op
    empty = torch.empty((0, 8, 128), dtype=torch.bfloat16, device=gc.DEV)
    o, l = pkv.attn_forward(empty, case.pool.k, case.pool.v, case.block_table, case.seqlens_d(),
                            torch.zeros(5, dtype=torch.int32, device=gc.DEV), True, 0.1, max_seqlen_q=0)
    assert o.shape == (0, 8, 128) and l.shape == (0, 8)


@pytest.mark.parametrize("hq,hk,L", [(64, 8, 2), (48, 2, 1), (32, 32, 5), (16, 1, 3)])
def test_gqa_groups_and_rows(hq, hk, L):
    """Column blocks of the decode kernel: g*L below, at and above 16 columns per KV head."""
    announce(f"GQA hq={hq} hk={hk} L={L}")
    case = gc.make_case(4400 + hq + hk + L, "bf16", 2, hq, hk, 128, 256, 2200, "interleaved", True, [L, L])
    out, lse = gc.run(case)
    gc.check_oracle(case, out, lse)
    for path in (1, 2):
        for split in (1, 3):
            gc.assert_bitwise(gc.run(case, path=path, split_chunks=split), (out, lse), f"path {path} split {split}")


def test_fp32_head_dim_128():
    announce("fp32 d=128")
    case = gc.make_case(4500, "f32", 2, 4, 2, 128, 16, 700, "interleaved", True, [1, 9])
    out, lse = gc.run(case)
    gc.check_oracle(case, out, lse)
    for path in (1, 2):
        gc.assert_bitwise(gc.run(case, path=path), (out, lse), f"path {path}")
