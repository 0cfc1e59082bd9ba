"""Split path with every sequence within one 1024-key chunk.

A row's ascending fold then has a single term, so the split kernels apply the
merge's operations to it and write out / lse themselves: no partials, no
workspace, no merge launch.  The bits must be those of the full (prefill)
path, which folds the same chunk result the same way; rows without a visible
key get out = 0 and lse = -inf; the oracle agrees on the rows.  Covers the
one-wave decode kernels (16 columns or fewer per KV head), the 8-wave split
kernel (17 rows x 4 heads = 68 columns), fp32 and bf16, and the fused append.
"""

from __future__ import annotations

import math

import pytest
import torch

import invariant_paged_kv_amd as pkv
import pkv_inputs as gen
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


def single_chunk_case(seed, dtype, rows, bs=16):
    B = 6
    lens_q = [rows] * B
    lens_q[1] = 0                       # a sequence without rows
    d = 128 if dtype == "bf16" else 64
    case = gc.make_case(seed, dtype, B, 16, 4, d, bs, 1024, "interleaved", True, lens_q)
    sl = list(case.seqlens)
    sl[0] = 1024                        # exactly one full chunk
    sl[2] = 0                           # rows but no keys
    sl[3] = 1
    sl[4] = max(1, rows - 2)            # fewer keys than rows: the first causal rows see nothing
    case.seqlens = sl
    return case


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows", [1, 3, 17])
def test_single_chunk_writes_directly(dtype, rows):
    announce(f"single-chunk direct write {dtype} rows={rows}")
    case = single_chunk_case(9900 + rows + (dtype == "f32"), dtype, rows)
    need = pkv.workspace_size(case.q, case.pool.k, case.pool.v, case.block_table, max_seqlen_q=rows,
                              max_seqlen_k=max(case.seqlens))
    assert need == 0
    out, lse = gc.run(case)             # NaN-filled outputs: every row must be written
    gc.assert_bitwise(gc.run(case, path=2), (out, lse), "full path")
    for r in range(case.cu[2], case.cu[3]):          # sequence 2: rows, no keys
        assert torch.all(lse[r] == -math.inf) and torch.all(out[r] == 0), r
    if rows > 2:                                     # sequence 4: its first rows see no key
        r = case.cu[4]
        assert torch.all(lse[r] == -math.inf) and torch.all(out[r] == 0)
    assert not torch.isnan(lse).any() and not torch.isnan(out.float()).any()
    gc.check_oracle(case, out, lse, seq_ids=[0, 3, 4, 5])


def test_single_chunk_fused_append():
    announce("single-chunk direct write, fused append")
    B, HK, D = 6, 4, 128
    case = gc.make_case(9950, "bf16", B, 16, HK, D, 16, 1024, "interleaved", True, [1] * B)
    sl = list(case.seqlens)
    sl[0] = 1024
    case.seqlens = sl
    g = torch.Generator().manual_seed(9951)
    kn = gen.randn((B, HK, D), "bf16", generator=g).to(gc.DEV)
    vn = gen.randn((B, HK, D), "bf16", generator=g).to(gc.DEV)
    sk = torch.tensor(sl, dtype=torch.int32, device=gc.DEV)
    cu = torch.arange(B + 1, dtype=torch.int32, device=gc.DEV)
    pk, pv = case.pool.k.clone(), case.pool.v.clone()
    pkv.cache_write(kn, vn, pk, pv, case.block_table, sk - 1, cu)
    ref = pkv.attn_forward(case.q, pk, pv, case.block_table, sk, cu, True, case.scale, max_seqlen_q=1,
                           max_seqlen_k=1024, **gc.nan_outputs(case.q))
    with pkv.options(path=2):
        full = pkv.attn_forward(case.q, pk, pv, case.block_table, sk, cu, True, case.scale, max_seqlen_q=1,
                                max_seqlen_k=1024, **gc.nan_outputs(case.q))
    fk, fv = case.pool.k.clone(), case.pool.v.clone()
    got = pkv.attn_forward_append(case.q, kn, vn, fk, fv, case.block_table, sk, cu, True, case.scale,
                                  max_seqlen_q=1, max_seqlen_k=1024, **gc.nan_outputs(case.q))
    torch.cuda.synchronize()
    gc.assert_bitwise(ref, full, "split (direct) vs full path")
    gc.assert_bitwise(got, ref, "fused append vs unfused")
    assert torch.equal(fk.view(torch.int16), pk.view(torch.int16)) and torch.equal(fv.view(torch.int16), pv.view(torch.int16))
