"""Rows of many 1024-key chunks through the split path and the merge.

A row's chunk partials are folded in ascending chunk index, in rounds of
loads; rows here span more chunks than one round holds and end at ragged
points (a partial last chunk, a last round with one chunk), with decode rows
and 2- and 3-row slots, d 64 and 128, bf16 and fp32, and through the
context-parallel merge entry point with its chunk-major layout.  The fold is
fixed by global chunk index (RL-Kernel PR #284, section Changes: a fixed
merge order by global block index), so the split path must equal the full
(prefill) path bit for bit; the oracle checks a few rows.
"""

from __future__ import annotations

import pytest
import torch

import invariant_paged_kv_amd as pkv
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("dtype,d,rows", [("bf16", 128, [1, 2, 1, 3]), ("bf16", 64, [1, 1, 1, 1]),
                                          ("f32", 64, [2, 1, 1, 1])])
def test_many_chunks_split_equals_full_path(dtype, d, rows):
    announce(f"many chunks {dtype} d={d} rows={rows}")
    # 150,000 keys: 147 chunks; 24,577: 25 (one key in the last chunk);
    # 131,072: 128 full chunks; 66,000: 65
    case = gc.make_case(8200 + d + len(dtype), dtype, 4, 8, 2, d, 256, 150000, "interleaved", True, rows,
                        seqlens=[150000, 24577, 131072, 66000])
    split = gc.run(case, path=1)      # decode (split) kernels + merge
    full = gc.run(case, path=2)       # prefill kernel, in-register fold
    gc.assert_bitwise(split, full, "split path vs full path")
    gc.check_oracle(case, split[0], split[1], seq_ids=[1, 3])


def test_many_chunks_context_parallel_merge():
    announce("many chunks through pkv_attn_merge_partials (chunk-major partials)")
    case = gc.make_case(8250, "bf16", 2, 8, 2, 128, 256, 40000, "interleaved", True, [1, 2],
                        seqlens=[40000, 30000])
    ref = gc.run(case, path=2)
    maxc = (40000 + 1023) // 1024     # 40 chunks
    rows, hq = case.q.shape[0], case.q.shape[1]
    part_o = torch.empty((maxc, rows * hq, 128), dtype=torch.float32, device=gc.DEV)
    part_ml = torch.empty((maxc, rows * hq, 2), dtype=torch.float32, device=gc.DEV)
    sk, cu = case.seqlens_d(), case.cu_d()
    pkv.attn_chunk_partials(case.q, case.pool.k, case.pool.v, case.block_table, sk, cu, True, case.scale,
                            chunk_begin=0, chunk_end=maxc, max_chunks=maxc, part_o=part_o, part_ml=part_ml,
                            max_seqlen_q=2, max_seqlen_k=40000)
    out, lse = pkv.attn_merge_partials(part_o, part_ml, case.q, case.pool.k, case.pool.v, case.block_table, sk, cu,
                                       True, max_seqlen_q=2, max_seqlen_k=40000, **gc.nan_outputs(case.q))
    torch.cuda.synchronize()
    gc.assert_bitwise((out, lse), ref, "context-parallel merge vs full path")
