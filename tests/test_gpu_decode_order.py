"""The one-wave decode kernels' longest-first job list.

With sequences spanning few chunks and more (sequence, KV head, chunk) jobs
than one round of wave slots, the decode kernels take their work in a
longest-first order (every full 1024-key chunk, then the partial last
chunks), from prefix counts computed on the device.  A job is the same
(sequence, KV head, chunk) as in the plain grid order, so the bits must not
change: compared here with two chunks per work item (which keeps the plain
order), with the full (prefill) path, and with the oracle on sampled
sequences; the fused append under the same order against the unfused pair.
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


def ragged(seed, dtype, bs):
    # 48 sequences x 8 KV heads x 8 chunks = 3072 job slots (> 2048): the job list is used
    case = gc.make_case(seed, dtype if dtype != "fp8" else "bf16", 48, 32, 8, 128, bs, 8192,
                        "interleaved", True, [1] * 48)
    if dtype == "fp8":
        g = torch.Generator().manual_seed(seed + 1)
        nb = gen.pool_num_blocks(8192, bs, 48)
        case.pool = gc.to_device(gen.new_pool(nb, bs, 8, 128, "fp8", "interleaved", generator=g))
    # a mix of lengths: exact chunk multiples, one-key tails and one-key sequences
    sl = list(case.seqlens)
    sl[0], sl[1], sl[2], sl[3] = 1024, 1025, 1, 8192
    case.seqlens = sl
    return case


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("bs", [256, 24])
def test_longest_first_order_keeps_bits(dtype, bs):
    announce(f"decode job order {dtype} bs={bs}")
    case = ragged(9700 + bs + (dtype == "fp8"), dtype, bs)
    if dtype == "fp8":
        from tests import test_gpu_fp8 as f8
        case.extra = {"k_scale": 0.5, "v_scale": 1.25}
        run = lambda **kw: f8.run(case, path=kw.get("path"), split=kw.get("split_chunks"))
    else:
        run = lambda **kw: gc.run(case, **kw)
    out, lse = run()
    gc.assert_bitwise(run(split_chunks=2), (out, lse), "plain order (2 chunks per item)")
    gc.assert_bitwise(run(path=2), (out, lse), "full path")
    if dtype == "fp8":
        f8.check_oracle(case, out, lse, seq_ids=[0, 1, 2, 3, 17])
    else:
        gc.check_oracle(case, out, lse, seq_ids=[0, 1, 2, 3, 17])


def test_longest_first_order_fused_append():
    announce("decode job order, fused append")
    case = ragged(9750, "bf16", 256)
    B, HK, D = 48, 8, 128
    g = torch.Generator().manual_seed(9751)
    kn = gen.randn((B, HK, D), "bf16", generator=g).to(gc.DEV)
    vn = gen.randn((B, HK, D), "bf16", generator=g).to(gc.DEV)
    sk = torch.tensor(case.seqlens, dtype=torch.int32, device=gc.DEV)
    cu = torch.arange(B + 1, dtype=torch.int32, device=gc.DEV)
    # unfused: write the new rows, then attend (plain order via 2 chunks per item)
    pk, pv = case.pool.k.clone(), case.pool.v.clone()
    pkv.cache_write(kn, vn, pk, pv, case.block_table, sk - 1, cu)
    with pkv.options(split_chunks=2):
        ref = pkv.attn_forward(case.q, pk, pv, case.block_table, sk, cu, True, case.scale, max_seqlen_q=1,
                               max_seqlen_k=8192, **gc.nan_outputs(case.q))
    # fused, longest-first order
    fk, fv = case.pool.k.clone(), case.pool.v.clone()
    got = pkv.attn_forward_append(case.q, kn, vn, fk, fv, case.block_table, sk, cu, True, case.scale,
                                  max_seqlen_q=1, max_seqlen_k=8192, **gc.nan_outputs(case.q))
    torch.cuda.synchronize()
    gc.assert_bitwise(got, ref, "fused append vs unfused")
    assert torch.equal(fk.view(torch.int16), pk.view(torch.int16)) and torch.equal(fv.view(torch.int16), pv.view(torch.int16))


def test_longest_first_order_with_empty_sequences():
    """Sequences without rows or without keys take no job; their rows get out = 0, lse = -inf."""
    announce("decode job order, empty sequences")
    B = 48
    lens = [1] * B
    for b in (5, 6, 30):          # no query rows
        lens[b] = 0
    case = gc.make_case(9760, "bf16", B, 32, 8, 128, 64, 8192, "interleaved", True, lens)
    sl = list(case.seqlens)
    for b in (7, 8, 47):          # rows but no keys
        sl[b] = 0
    sl[0], sl[9] = 1024, 1025
    case.seqlens = sl
    out, lse = gc.run(case)
    gc.assert_bitwise(gc.run(case, split_chunks=2), (out, lse), "plain order")
    gc.assert_bitwise(gc.run(case, path=2), (out, lse), "full path")
    for b in (7, 8, 47):
        r = case.cu[b]
        assert torch.all(lse[r] == -math.inf) and torch.all(out[r] == 0), b
    gc.check_oracle(case, out, lse, seq_ids=[0, 4, 7, 9, 31])


@pytest.mark.parametrize("batch", [63, 64, 300])
def test_many_sequences_lookups(batch):
    """The row -> sequence lookups of the merge and the append take every lane's own sequence
    values in the probe's round below 64 sequences and a separate round from 64 on; the job list's
    search counts 256 prefix entries per round (300 sequences x 8 KV heads x 2 chunks = 4800 jobs:
    two rounds).  Same bits as the plain order and the full path, the oracle on sampled sequences,
    and the appended rows exactly where host indexing puts them."""
    announce(f"decode lookups, batch {batch}")
    B, HK, D, BS = batch, 8, 128, 16
    case = gc.make_case(9800 + batch, "bf16", B, 16, HK, D, BS, 2048, "interleaved", True, [1] * B)
    out, lse = gc.run(case)
    gc.assert_bitwise(gc.run(case, split_chunks=2), (out, lse), "plain order (2 chunks per item)")
    gc.assert_bitwise(gc.run(case, path=2), (out, lse), "full path")
    gc.check_oracle(case, out, lse, seq_ids=[0, B // 2, B - 1])
    g = torch.Generator().manual_seed(9801 + batch)
    kn = gen.randn((B, HK, D), "bf16", generator=g).to(gc.DEV)
    vn = gen.randn((B, HK, D), "bf16", generator=g).to(gc.DEV)
    sk = torch.tensor(case.seqlens, dtype=torch.int32, device=gc.DEV)
    cu = torch.arange(B + 1, dtype=torch.int32, device=gc.DEV)
    pk, pv = case.pool.k.clone(), case.pool.v.clone()
    want_k, want_v = pk.clone(), pv.clone()
    pkv.cache_write(kn, vn, pk, pv, case.block_table, sk - 1, cu)   # token b at position seqlens[b] - 1
    pos = (sk - 1).long()
    blk = case.block_table.long()[torch.arange(B, device=gc.DEV), pos // BS]
    want_k[blk, pos % BS] = kn
    want_v[blk, pos % BS] = vn
    torch.cuda.synchronize()
    assert torch.equal(pk.view(torch.int16), want_k.view(torch.int16))
    assert torch.equal(pv.view(torch.int16), want_v.view(torch.int16))


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("shape", [(16, 16, 4, 16, 5000), (24, 32, 8, 256, 6000), (40, 8, 2, 24, 3000)])
def test_dispatch_orders_keep_bits(dtype, shape):
    """Both dispatch orders of the plain decode grid (items of one (sequence,
    KV head) consecutive, or the sequence fastest) run the same jobs: same bits,
    for both one-wave decode kernels (a grid within one round of wave slots and
    one beyond it), and the oracle on two sequences."""
    B, hq, hk, bs, n = shape
    announce(f"decode dispatch orders {dtype} {shape}")
    case = gc.make_case(9800 + B, "bf16", B, hq, hk, 128, bs, n, "interleaved", True, [1] * B)
    kw = {}
    if dtype == "fp8":
        g = torch.Generator().manual_seed(9801 + B)
        case.pool = gc.to_device(gen.new_pool(gen.pool_num_blocks(n, bs, B), bs, hk, 128, "fp8", "interleaved",
                                              generator=g))
        kw = dict(k_scale=0.5, v_scale=1.25)
    res = []
    for order in (1, 2):
        with pkv.options(decode_order=order):
            o = gc.nan_outputs(case.q)
            out, lse = pkv.attn_forward(case.q, case.pool.k, case.pool.v, case.block_table, case.seqlens_d(),
                                        case.cu_d(), True, case.scale, max_seqlen_q=1,
                                        max_seqlen_k=case.max_seqlen_k, **o, **kw)
            torch.cuda.synchronize()
            res.append((out, lse))
    gc.assert_bitwise(res[0], res[1], "dispatch order 1 vs 2")
    with pkv.options(path=2):
        full = pkv.attn_forward(case.q, case.pool.k, case.pool.v, case.block_table, case.seqlens_d(), case.cu_d(),
                                True, case.scale, max_seqlen_q=1, max_seqlen_k=case.max_seqlen_k, **kw)
    torch.cuda.synchronize()
    gc.assert_bitwise(res[0], full, "decode vs full path")
    if dtype == "bf16":
        gc.check_oracle(case, *res[0], seq_ids=[0, B - 1])


@pytest.mark.parametrize("batch", [65, 100, 128])
def test_ragged_rows_lookups(batch):
    """Between 64 and 128 sequences the merge's and the append's row -> sequence lookups take the
    wave-wide search; ragged row counts (0 to 3 rows per sequence, empty ones among them), bitwise
    against the full path, the oracle on sampled sequences, and 0-3 appended rows per sequence
    exactly where host indexing puts them."""
    announce(f"ragged-row lookups, batch {batch}")
    B, HK, D, BS = batch, 4, 64, 16
    rows = [(b * 7) % 4 for b in range(B)]
    rows[-1] = 3                                  # the last sequence has rows
    case = gc.make_case(9900 + batch, "bf16", B, 8, HK, D, BS, 3000, "interleaved", True, rows)
    sl = [max(int(x), 3) for x in case.seqlens]
    sl[1] = 1025
    case.seqlens = sl
    out, lse = gc.run(case)
    gc.assert_bitwise(gc.run(case, path=2), (out, lse), "full path")
    gc.check_oracle(case, out, lse, seq_ids=[1, B // 2 + 1, B - 1])
    g = torch.Generator().manual_seed(9901 + batch)
    total = case.cu[-1]
    kn = gen.randn((total, HK, D), "bf16", generator=g).to(gc.DEV)
    vn = gen.randn((total, HK, D), "bf16", generator=g).to(gc.DEV)
    before = torch.tensor([s - r for s, r in zip(sl, rows)], dtype=torch.int32, device=gc.DEV)
    cu = case.cu_d()
    pk, pv = case.pool.k.clone(), case.pool.v.clone()
    want_k, want_v = pk.clone(), pv.clone()
    pkv.cache_write(kn, vn, pk, pv, case.block_table, before, cu)
    seq = torch.repeat_interleave(torch.arange(B, device=gc.DEV), torch.tensor(rows, device=gc.DEV))
    pos = before.long()[seq] + (torch.arange(total, device=gc.DEV) - cu.long()[seq])
    blk = case.block_table.long()[seq, pos // BS]
    want_k[blk, pos % BS] = kn
    want_v[blk, pos % BS] = vn
    torch.cuda.synchronize()
    assert torch.equal(pk.view(torch.int16), want_k.view(torch.int16))
    assert torch.equal(pv.view(torch.int16), want_v.view(torch.int16))
