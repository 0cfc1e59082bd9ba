"""The split kernel's tile staging with and without loader waves.

With more than 16 columns per KV head (query rows x heads per KV head) the
split path runs 8 waves x 16 columns per work group.  When a column block
leaves the last two waves without a column (at most 96 columns) those two
load and stage every tile and the others only compute; with 97-128 columns
every wave stages its share.  The staging moves bytes only: the split path
must equal the full (prefill) path bit for bit in every case (RL-Kernel issue
#152, Acceptance criteria: chunked prefill equals full prefill), at d 64 and
128, over an FP8 cache, and under the fused append (which keeps the shared
staging); the oracle checks a sequence.
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


# rows per sequence x 4 query heads per KV head: 68 and 84 columns (loader
# waves), 120 (none), 200 (a block of 128 without and one of 72 with them)
@pytest.mark.parametrize("rows", [17, 21, 30, 50])
@pytest.mark.parametrize("d", [64, 128])
def test_split_staging_equals_full_path(rows, d):
    announce(f"split staging: {rows} rows x 4 heads, d={d}")
    case = gc.make_case(8600 + rows + d, "bf16", 3, 16, 4, d, 16, 3000, "interleaved", True, [rows, rows - 3, rows],
                        seqlens=[3000, 1500, 2100])
    split = gc.run(case, path=1)
    full = gc.run(case, path=2)
    gc.assert_bitwise(split, full, "split vs full path")
    gc.check_oracle(case, split[0], split[1], seq_ids=[1])


def test_split_staging_fused_append_and_fp8():
    announce("split staging: 17-row chunk with fused append, and over an FP8 cache")
    from tests.test_gpu_fp8 import fp8_case
    case = fp8_case(8650, 3, 16, 4, 128, 16, 3000, "interleaved", True, [17, 17, 17], seqlens=[3000, 1800, 2500],
                    k_scale=1.0, v_scale=1.0)
    sk, cu = case.seqlens_d(), case.cu_d()
    outs = []
    for path in (1, 2):
        with pkv.options(path=path):
            outs.append(pkv.attn_forward(case.q, case.pool.k, case.pool.v, case.block_table, sk, cu, True, case.scale,
                                         max_seqlen_q=17, max_seqlen_k=3000, **gc.nan_outputs(case.q)))
    torch.cuda.synchronize()
    gc.assert_bitwise(outs[0], outs[1], "fp8 split vs full path")
    # fused append of the chunk's own rows (bf16 cache), against the separate write + attention
    case = gc.make_case(8660, "bf16", 3, 16, 4, 128, 16, 3000, "interleaved", True, [17, 17, 17],
                        seqlens=[3000, 1800, 2500])
    g = torch.Generator().manual_seed(8661)
    kn = torch.randn((51, 4, 128), generator=g).to(torch.bfloat16).to(gc.DEV)
    vn = torch.randn((51, 4, 128), generator=g).to(torch.bfloat16).to(gc.DEV)
    sk, cu = case.seqlens_d(), case.cu_d()
    pk, pv = case.pool.k.clone(), case.pool.v.clone()
    pkv.cache_write(kn, vn, pk, pv, case.block_table, sk - 17, cu)
    ref = pkv.attn_forward(case.q, pk, pv, case.block_table, sk, cu, True, case.scale, max_seqlen_q=17,
                           max_seqlen_k=3000, **gc.nan_outputs(case.q))
    fk, fv = case.pool.k.clone(), case.pool.v.clone()
    got = pkv.attn_forward_append(case.q, kn, vn, fk, fv, case.block_table, sk, cu, True, case.scale,
                                  max_seqlen_q=17, max_seqlen_k=3000, **gc.nan_outputs(case.q))
    torch.cuda.synchronize()
    gc.assert_bitwise(got, ref, "fused append vs separate write + attention")
    assert torch.equal(fk.view(torch.int16), pk.view(torch.int16)) and torch.equal(fv.view(torch.int16),
                                                                                  pv.view(torch.int16))
