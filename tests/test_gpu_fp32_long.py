"""fp32 caches at long contexts: the LSE bound of 1e-6 where |LSE| passes 8.

RL-Kernel PR #284, "feat(attention): add CP backward drift validation",
section Changes: the forward reports an attention-domain (natural-log) LSE
with the output.  With N(0,1) data and scale 1/sqrt(d) a row over n keys has
an LSE near ln(n) + 1/2: about 9 at 5000 keys and 10.9 at 32768, where
neighbouring fp32 values are 9.5e-7 apart, so the stated 1e-6 bound leaves
about one ulp for everything the kernel does.  Decode rows (one query per
sequence, split path) and prefill rows (the last rows of a causal prefill,
full path) are compared with the float64 oracle at the stated fp32
tolerances, and with each other bit for bit.
"""

from __future__ import annotations

import math

import pytest
import torch

from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [5000, 32768])
def test_fp32_long_context_lse(n, d):
    print(f"[case] fp32 n={n} d={d}", flush=True)
    rows = 6
    # two sequences of n keys: the last `rows` rows of a causal prefill of each
    case = gc.make_case(5200 + n + d, "f32", 2, 8, 2, d, 16, n, "interleaved", True, [rows, rows],
                        seqlens=[n, n])
    pre_out, pre_lse = gc.run(case, path=2)
    eo, el = gc.check_oracle(case, pre_out, pre_lse)
    assert float(pre_lse.min()) > 8.0, "the case must reach |LSE| > 8"
    # the same rows on the split path, bit for bit
    gc.assert_bitwise(gc.run(case, path=1), (pre_out, pre_lse), "split path vs full path")
    # each prefill row alone, as a decode call (one query row over its visible keys)
    for r in (0, rows - 1):
        sel = [r, rows + r]
        q = case.q[torch.tensor(sel, device=gc.DEV)].contiguous()
        sk = [n - rows + 1 + r] * 2
        out, lse = gc.run(case, q=q, seqlens=sk, cu=[0, 1, 2])
        gc.assert_bitwise((out, lse), (pre_out[sel], pre_lse[sel]), f"decode row {r} vs prefill row")
    print(f"  out max-abs {eo:.2e} (tol 1e-5), lse max-abs {el:.2e} (tol 1e-6), "
          f"lse range [{float(pre_lse.min()):.2f}, {float(pre_lse.max()):.2f}]", flush=True)
