"""pkv_attn_forward_noalloc: the forward for callers that cannot allocate.

Called through the C ABI (ctypes) and checked bit for bit against
pkv_attn_forward, which takes its workspace from the stream-ordered
allocator; both run the same kernels, so the bits must be equal.  Two decode
calls in a row (the second smaller, so it runs over the scratch contents the
first one left), an fp32 decode and prefill-shaped rows (the 4-wave split
kernel).  The rejection of a split path larger than the scratch is a host
check, tested on the CPU (tests/test_abi.py).
"""

from __future__ import annotations

import ctypes

import pytest
import torch

import invariant_paged_kv_amd as pkv
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu


def c_call(entry, case, out, lse, max_seqlen_k=0):
    lay = pkv.make_layout(case.pool.k, case.pool.v, case.block_table, case.q.shape[1], case.max_seqlen_q,
                          case.q.shape[0], max_seqlen_k)
    sk, cu = case.seqlens_d(), case.cu_d()
    fn = getattr(pkv.lib(), entry)
    rc = fn(case.q.data_ptr(), case.pool.k.data_ptr(), case.pool.v.data_ptr(), ctypes.byref(lay),
            case.block_table.data_ptr(), sk.data_ptr(), cu.data_ptr(), 1 if case.causal else 0,
            ctypes.c_float(case.scale), out.data_ptr(), lse.data_ptr(),
            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    return rc, lay


def both(case, max_seqlen_k=0):
    ref = gc.nan_outputs(case.q)
    got = gc.nan_outputs(case.q)
    rc, _ = c_call("pkv_attn_forward", case, ref["out"], ref["lse"], max_seqlen_k)
    assert rc == 0, pkv.lib().pkv_last_error()
    rc, lay = c_call("pkv_attn_forward_noalloc", case, got["out"], got["lse"], max_seqlen_k)
    assert rc == 0, pkv.lib().pkv_last_error()
    gc.assert_bitwise((got["out"], got["lse"]), (ref["out"], ref["lse"]), "noalloc vs pkv_attn_forward")
    return got, lay


def test_noalloc_matches_forward_on_consecutive_calls():
    print("[case] noalloc: 2 decode calls (large, then small), then a prefill", flush=True)
    big = gc.make_case(7101, "bf16", 24, 16, 4, 128, 16, 9000, "interleaved", True, [1] * 24)
    got, lay = both(big)
    ws = pkv.lib().pkv_attn_workspace_size(ctypes.byref(lay))
    assert 0 < ws <= pkv.NOALLOC_MAX_BYTES
    gc.check_oracle(big, got["out"], got["lse"], seq_ids=[0, 23])
    small = gc.make_case(7102, "bf16", 3, 8, 2, 64, 256, 2500, "contiguous", True, [1, 3, 2])
    got, _ = both(small)
    gc.check_oracle(small, got["out"], got["lse"])
    # an fp32 decode, and prefill rows (few work groups: the 4-wave split path, also over the scratch)
    f32 = gc.make_case(7103, "f32", 2, 4, 2, 64, 16, 1500, "interleaved", False, [1, 1])
    both(f32)
    pre = gc.make_case(7104, "bf16", 2, 8, 2, 128, 16, 700, "interleaved", True, [300, 200], seqlens=[600, 700])
    both(pre)
