"""Decode over two chunks in one round of wave slots: the chunk fold in the work group.

The one-wave bf16 decode kernel then runs one work group per (sequence, KV
head) whose two waves take one 1024-key chunk each, leave their chunk results in
LDS and fold them in ascending chunk order before writing out / lse -- the
merge's operations on the same values, without partials in HBM or a merge
launch.  Compared bit for bit with the same call through the partials and the
merge (two chunks per work item, which keeps the fold off) and with the full
(prefill) path, against the oracle on sampled rows, with ragged lengths,
sequences without keys, causal multi-row slots, d = 64 and a block size that
is not a multiple of 16 (per-lane block ids).
"""

from __future__ import annotations

import math

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


@pytest.mark.parametrize("d,bs,rows", [(128, 16, 1), (64, 256, 3), (128, 24, 3)])
def test_fold_in_group_matches_merge(d, bs, rows):
    announce(f"decode fold in the work group: 2048 keys, d={d}, bs={bs}, rows={rows}")
    B, HK = 64, 4                                   # 256 (sequence, KV head) groups: one per CU
    lens_q = [rows] * B
    lens_q[6] = 0                                   # a sequence without rows
    case = gc.make_case(9600 + d + bs + rows, "bf16", B, 16, HK, d, bs, 2048, "interleaved", True, lens_q)
    sl = list(case.seqlens)
    sl[0] = 2048                                    # both waves of its group have a chunk
    sl[1] = 1024                                    # exactly one chunk: the other wave only joins the fold
    sl[2] = 1025                                    # a one-key second chunk
    sl[3] = 0                                       # rows but no keys
    sl[4] = max(1, rows - 2)                        # fewer keys than rows
    case.seqlens = sl
    need = pkv.workspace_size(case.q, case.pool.k, case.pool.v, case.block_table, max_seqlen_q=rows,
                              max_seqlen_k=max(sl))
    assert need == 0                                # no partials: nothing to hold
    out, lse = gc.run(case)                         # NaN-filled outputs: every row must be written
    gc.assert_bitwise(gc.run(case, split_chunks=2), (out, lse), "partials + merge")
    gc.assert_bitwise(gc.run(case, path=2), (out, lse), "full path")
    for r in range(case.cu[3], case.cu[4]):
        assert torch.all(lse[r] == -math.inf) and torch.all(out[r] == 0), r
    assert not torch.isnan(lse).any() and not torch.isnan(out.float()).any()
    gc.check_oracle(case, out, lse, seq_ids=[0, 1, 2, 4, 63])
