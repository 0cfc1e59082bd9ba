"""Debug mode on the GPU: the check kernel before a call's kernels.

With PKV_OPT_DEBUG set, each call first checks its index data on the device
(csrc/pkv_checks.h); on a violation its kernels return without touching
memory and pkv_check_device_errors reports it.  Valid inputs must give the
same bits as without debug mode and leave no error.  Every bad case here
stays inside the allocated buffers (block ids beyond the *declared* pool but
inside the real one, a declared table narrower than the real one, counts
above the declared bounds): even an unchecked launch would only compute
wrong values, never touch memory outside the allocations.
"""

from __future__ import annotations

import pytest
import torch

import invariant_paged_kv_amd as pkv
import pkv_inputs as gen
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _debug_off_after():
    yield
    torch.cuda.synchronize()
    pkv.set_option(pkv.PKV_OPT_DEBUG, 0)
    try:
        pkv.check_device_errors()
    except pkv.PkvError:
        pass


def case():
    return gc.make_case(7301, "bf16", 3, 8, 2, 128, 16, 3000, "interleaved", True, [1, 2, 1])


def fwd(c, pool=None, **kw):
    p = pool or c.pool
    o = gc.nan_outputs(c.q)
    sk = kw.pop("seqlens", c.seqlens)
    cu = kw.pop("cu", c.cu)
    out, lse = pkv.attn_forward(c.q, p.k, p.v, kw.pop("block_table", c.block_table),
                                torch.tensor(sk, dtype=torch.int32, device=gc.DEV),
                                torch.tensor(cu, dtype=torch.int32, device=gc.DEV), True, c.scale,
                                max_seqlen_q=kw.pop("max_seqlen_q", 2), max_seqlen_k=kw.pop("max_seqlen_k", 0), **o)
    torch.cuda.synchronize()
    return out, lse


def expect_error(text):
    with pytest.raises(pkv.PkvError) as ei:
        pkv.check_device_errors()
    assert ei.value.code == pkv.PKV_ERR_DEVICE_DATA and text in str(ei.value), str(ei.value)
    pkv.check_device_errors()   # collected: clear now


def untouched(out, lse):
    return bool(torch.isnan(out.float()).all()) and bool(torch.isnan(lse).all())


def test_debug_mode_valid_inputs_same_bits():
    print("[case] debug mode on valid inputs", flush=True)
    c = case()
    ref = fwd(c)
    for path in (1, 2):
        with pkv.options(debug=1, path=path):
            got = fwd(c)
        gc.assert_bitwise(got, ref, f"debug mode, path {path}")
    pkv.check_device_errors()


def test_block_id_beyond_declared_pool():
    print("[case] debug mode: block id beyond the declared pool", flush=True)
    c = case()
    used = int(c.block_table[:, :188].max())     # 3000 keys / 16 = 188 blocks per sequence
    small = used // 2                            # declare a pool that ends before some used blocks
    pool = gen.PagedKV(c.pool.k[:small], c.pool.v[:small], "interleaved", c.pool.storage)
    with pkv.options(debug=1):
        out, lse = fwd(c, pool=pool)
    assert untouched(out, lse)
    expect_error("block_id")


def test_counts_beyond_declared_bounds_and_sticky_word():
    print("[case] debug mode: seqlens above max_seqlen_k, rows above max_seqlen_q, cu total", flush=True)
    c = case()
    with pkv.options(debug=1):
        assert untouched(*fwd(c, max_seqlen_k=2048))            # seqlens 3000 > declared 2048
        expect_error("seqlens_k")
        assert untouched(*fwd(c, max_seqlen_q=1))               # a sequence has 2 rows
        expect_error("rows>max_seqlen_q")
        assert untouched(*fwd(c, cu=[0, 1, 2, 3]))              # cu[batch] = 3 != total_q = 4
        expect_error("cu_seqlens")
        # the word is sticky: a valid call after a violation does nothing until it is collected
        assert untouched(*fwd(c, max_seqlen_k=2048))
        assert untouched(*fwd(c))
        expect_error("seqlens_k")
        ref = fwd(c)
    pkv.check_device_errors()
    gc.assert_bitwise(ref, fwd(c), "after the error was collected")


def test_cache_write_beyond_declared_table():
    print("[case] debug mode: cache write past the declared table", flush=True)
    c = case()
    bt_full = c.block_table                      # [3, mbps] real table
    narrow = bt_full.reshape(-1)[: 3 * 100].view(3, 100)   # declared 100 entries per row, same memory
    kn = torch.randn(4, 2, 128, dtype=torch.bfloat16, device=gc.DEV)
    before = c.pool.storage[0].clone()
    with pkv.options(debug=1):
        pkv.cache_write(kn, kn, c.pool.k, c.pool.v, narrow, torch.tensor([0, 1599, 0], dtype=torch.int32,
                        device=gc.DEV), torch.tensor([0, 1, 3, 4], dtype=torch.int32, device=gc.DEV))
        torch.cuda.synchronize()
        expect_error("write_position")                        # position 1599 + 1 >= 100 * 16
    assert torch.equal(before.view(torch.int16), c.pool.storage[0].view(torch.int16)), "the cache changed"


def test_backward_cu_seqlens_k():
    print("[case] debug mode: backward with a wrong cu_seqlens_k", flush=True)
    c = gc.make_case(7302, "bf16", 2, 4, 2, 64, 16, 300, "contiguous", True, [5, 3], seqlens=[200, 300])
    out, lse = gc.run(c)
    dout = torch.randn_like(c.q)
    cuk = torch.tensor([0, 200, 499], dtype=torch.int32, device=gc.DEV)   # should end at 500
    with pkv.options(debug=1):
        dq, dk, dv = pkv.attn_backward(c.q, c.pool.k, c.pool.v, c.block_table, c.seqlens_d(), c.cu_d(), True, c.scale,
                                       out, lse, dout, max_seqlen_q=5, cu_seqlens_k=cuk, total_k=500,
                                       dq=torch.full_like(c.q, float("nan")),
                                       dk=torch.full((500, 2, 64), float("nan"), dtype=torch.bfloat16, device=gc.DEV),
                                       dv=torch.full((500, 2, 64), float("nan"), dtype=torch.bfloat16, device=gc.DEV))
        torch.cuda.synchronize()
        expect_error("cu_seqlens_k")
    assert bool(torch.isnan(dq.float()).all()) and bool(torch.isnan(dk.float()).all())
