"""``flash_attn_with_kvcache``: the pages' call shape over the library.

aiter commit d293d61bbf19 tests paged attention through
``flash_attn_with_kvcache(q [B, Lq, Hq, d], k_cache, v_cache, cache_seqlens=,
page_table=, causal=)``.  The adapter only reshapes and builds the packed
row offsets, so its out / lse must equal ``attn_forward``'s bit for bit, and
match the oracle at the stated tolerances.
"""

from __future__ import annotations

import pytest
import torch

import invariant_paged_kv_amd as pkv
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("layout,bs", [("interleaved", 16), ("contiguous", 256)])
def test_flash_attn_with_kvcache_matches_attn_forward(causal, layout, bs):
    announce(f"flash_attn_with_kvcache causal={causal} {layout} bs={bs}")
    B, Lq = 3, 4
    case = gc.make_case(9800 + bs + causal, "bf16", B, 8, 2, 128, bs, 1500, layout, causal, [Lq] * B,
                        seqlens=[1500, 4, 777])
    sk = torch.tensor(case.seqlens, dtype=torch.int32, device=gc.DEV)
    q4 = case.q.view(B, Lq, 8, 128)
    out4, lse4 = pkv.flash_attn_with_kvcache(q4, case.pool.k, case.pool.v, cache_seqlens=sk,
                                             page_table=case.block_table, causal=causal, return_softmax_lse=True)
    torch.cuda.synchronize()
    assert out4.shape == (B, Lq, 8, 128) and lse4.shape == (B, 8, Lq)
    out, lse = gc.run(case)
    gc.assert_bitwise((out4.reshape(B * Lq, 8, 128), lse4.permute(0, 2, 1).reshape(B * Lq, 8)), (out, lse),
                      "adapter vs attn_forward")
    gc.check_oracle(case, out, lse)
    # out alone by default
    o = pkv.flash_attn_with_kvcache(q4, case.pool.k, case.pool.v, cache_seqlens=sk, page_table=case.block_table,
                                    causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), out4.view(torch.int16))
