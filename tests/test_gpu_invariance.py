"""GPU invariances: results that must not change, bit for bit, when the work is
split, scheduled or laid out differently, and the cache write's bit copy.

RL-Kernel issue #152 "[WS1] KV-cache path consistency (prefill & decode)",
sections Scope and Acceptance criteria: the same reductions for the same
effective context across batch sizes and padding layouts, and no drift added
by the stored-KV layout.  aiter commit d293d61bbf19: the same data in a
contiguous and a K/V-interleaved paged cache gives the same result, and a
kernel that assumes the contiguous block stride must be caught.
"""

from __future__ import annotations

import math

import pytest
import torch

import invariant_paged_kv_amd as pkv
import pkv_inputs as gen
from tests import gpu_cases as gc
from tests.oracle_bridge import oracle_attention, oracle_pool, storage_np

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


def mixed_case(seed=3001, dtype="bf16", layout="interleaved", lens_q=(1, 3, 1, 2), hq=8, hk=2, d=128, bs=16,
               seqlen_k=3000, causal=True):
    return gc.make_case(seed, dtype, len(lens_q), hq, hk, d, bs, seqlen_k, layout, causal, list(lens_q))


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_split_count_and_path_invariance(dtype, d):
    announce(f"split counts {dtype} d={d}")
    case = mixed_case(dtype=dtype, d=d)
    ref = gc.run(case)
    gc.check_oracle(case, *ref)
    for path in (1, 2):
        for split in (1, 2, 3, 7, 64):
            gc.assert_bitwise(gc.run(case, path=path, split_chunks=split), ref, f"path {path} split {split}")
    for fk in (1, 2, 3):
        gc.assert_bitwise(gc.run(case, path=2, full_kernel=fk), ref, f"full path, kernel {fk}")


@pytest.mark.parametrize("layout", ["interleaved", "contiguous"])
def test_full_path_kernels_agree(layout):
    """The two bf16 full-path kernels (pipelined 8-wave, single-buffered 4-wave) and
    the split path give the same bits on a chunked prefill with ragged rows."""
    announce(f"full-path kernels {layout}")
    lens, seqlens = [300, 17, 129, 64], [900, 17, 700, 1030]
    case = gc.make_case(3010, "bf16", 4, 16, 4, 128, 16, max(seqlens), layout, True, lens, seqlens)
    ref = gc.run(case, path=2, full_kernel=1)
    gc.check_oracle(case, *ref, seq_ids=[1, 3])
    gc.assert_bitwise(gc.run(case, path=2, full_kernel=2), ref, "4-wave vs 8-wave full kernel")
    gc.assert_bitwise(gc.run(case, path=1), ref, "split vs full")


def test_chunked_prefill_rows_split_kernel():
    """17-row chunks of a GQA-4 group (68 columns per KV head, the 4-wave split
    kernel, whose staged tiles cross chunk boundaries inside a work item when it
    takes several chunks) over contexts of one to five 1024-key chunks: every
    grouping of chunks into work items and the full path give the same bits."""
    announce("chunked-prefill rows, split kernel")
    lens, seqlens = [17, 17, 17, 17], [4100, 2049, 1041, 17]
    case = gc.make_case(3020, "bf16", 4, 16, 4, 128, 16, max(seqlens), "contiguous", True, lens, seqlens)
    ref = gc.run(case, path=1)
    gc.check_oracle(case, *ref, seq_ids=[1, 3])
    for split in (2, 3, 5):
        gc.assert_bitwise(gc.run(case, path=1, split_chunks=split), ref, f"split {split}")
    gc.assert_bitwise(gc.run(case, path=2), ref, "full path")


def test_permuted_block_table():
    announce("permuted block table")
    case = mixed_case(seed=3002, layout="contiguous")
    ref = gc.run(case)
    nb = case.pool.num_blocks
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(9)).to(gc.DEV)
    inv = torch.argsort(perm)
    k2, v2 = case.pool.k[inv].contiguous(), case.pool.v[inv].contiguous()
    moved = gen.PagedKV(k2, v2, "contiguous", [k2, v2])
    bt2 = perm[case.block_table.long()].to(torch.int32)
    gc.assert_bitwise(gc.run(case, pool=moved, block_table=bt2), ref, "permuted table")


def test_unread_memory_is_never_read():
    """NaN in every slot no sequence may read, -1 in unused table entries: no change."""
    announce("poisoned unused memory")
    case = mixed_case(seed=3003)
    ref = gc.run(case)
    gen.poison_unused(case.pool, case.block_table, case.seqlens)
    bt2 = gen.poison_table_tail(case.block_table, case.seqlens, case.pool.block_size, -1)
    gc.assert_bitwise(gc.run(case, block_table=bt2), ref, "poisoned pool and table tail")
    for path in (1, 2):
        gc.assert_bitwise(gc.run(case, block_table=bt2, path=path), ref, f"poisoned, path {path}")
    for fk in (1, 2, 3):
        gc.assert_bitwise(gc.run(case, block_table=bt2, path=2, full_kernel=fk), ref, f"poisoned, full kernel {fk}")


def test_run_to_run_determinism():
    announce("10 repeats")
    case = mixed_case(seed=3004, lens_q=(1,) * 6, seqlen_k=5000)
    ref = gc.run(case)
    for _ in range(10):
        gc.assert_bitwise(gc.run(case), ref, "repeat")


def test_power_of_two_scaling():
    """V*2 gives out*2 exactly; (2q, scale/2) gives identical bits."""
    announce("power-of-two scaling")
    case = mixed_case(seed=3005, layout="contiguous")
    out, lse = gc.run(case)
    v2 = (case.pool.v.float() * 2).to(case.pool.v.dtype)
    p2 = gen.PagedKV(case.pool.k, v2, "contiguous", [case.pool.k, v2])
    o2, l2 = gc.run(case, pool=p2)
    gc.assert_bitwise((o2, l2), ((out.float() * 2).to(out.dtype), lse), "V * 2")
    q2 = (case.q.float() * 2).to(case.q.dtype)
    gc.assert_bitwise(gc.run(case, q=q2, scale=case.scale / 2), (out, lse), "(2q, scale/2)")


def test_batch_permutation():
    """Permuting the sequences of a batch permutes the outputs, bit for bit."""
    announce("batch permutation")
    case = mixed_case(seed=3006, lens_q=(1, 3, 2, 1, 3))
    out, lse = gc.run(case)
    order = [3, 0, 4, 2, 1]
    rows, cu = [], [0]
    for b in order:
        rows.extend(range(case.cu[b], case.cu[b + 1]))
        cu.append(cu[-1] + case.cu[b + 1] - case.cu[b])
    idx = torch.tensor(rows, dtype=torch.long, device=gc.DEV)
    o2, l2 = gc.run(case, q=case.q.index_select(0, idx).contiguous(),
                    block_table=case.block_table[torch.tensor(order, device=gc.DEV)].contiguous(),
                    seqlens=[case.seqlens[b] for b in order], cu=cu)
    gc.assert_bitwise((o2, l2), (out.index_select(0, idx), lse.index_select(0, idx)), "batch permutation")


def test_gqa_group_permutation():
    """Permuting the query heads inside each GQA group permutes the outputs."""
    announce("GQA group permutation")
    case = mixed_case(seed=3007, hq=8, hk=2)
    out, lse = gc.run(case)
    perm = torch.tensor([2, 0, 3, 1, 5, 7, 4, 6], device=gc.DEV)   # stays within groups {0..3}, {4..7}
    o2, l2 = gc.run(case, q=case.q[:, perm].contiguous())
    gc.assert_bitwise((o2, l2), (out[:, perm], lse[:, perm]), "head permutation")


def test_wrong_block_stride_is_caught():
    """Negative control: reading the interleaved cache with the contiguous block stride breaks parity."""
    announce("negative control: contiguous block stride on an interleaved cache")
    case = mixed_case(seed=3008, lens_q=(1, 1))
    good = gc.run(case)
    gc.check_oracle(case, *good)
    k_bad = case.pool.k.as_strided(case.pool.k.shape, (case.pool.k.stride(0) // 2,) + case.pool.k.stride()[1:])
    v_bad = case.pool.v.as_strided(case.pool.v.shape, (case.pool.v.stride(0) // 2,) + case.pool.v.stride()[1:])
    bad = gc.run(case, pool=gen.PagedKV(k_bad, v_bad, "interleaved", case.pool.storage))
    with pytest.raises(AssertionError):
        gc.check_oracle(case, *bad)


@pytest.mark.parametrize("layout", ["contiguous", "interleaved"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cache_write_is_a_bit_copy(layout, dtype):
    announce(f"cache_write {layout} {dtype}")
    g = torch.Generator().manual_seed(3100)
    bs, hk, d, batch = 16, 4, 128, 3
    nb = gen.pool_num_blocks(200, bs, batch)
    host = gen.new_pool(nb, bs, hk, d, dtype, layout, generator=g)
    bt = gen.randperm_block_table(nb, batch, generator=g)
    seqlens = [5, 0, 177]
    lens_new = [17, 40, 23]
    cu = gen.cu_from_lengths(lens_new)
    kn = gen.randn((int(cu[-1]), hk, d), dtype, generator=g)
    vn = gen.randn((int(cu[-1]), hk, d), dtype, generator=g)
    # expected: the oracle's write on host copies
    kf, vf, lay = oracle_pool(host, hk)
    ek, ev = oracle.cache_write(kf, vf, lay, storage_np(kn), storage_np(vn), bt.numpy(), seqlens, cu.tolist())
    pool = gc.to_device(host)
    pkv.cache_write(kn.to(gc.DEV), vn.to(gc.DEV), pool.k, pool.v, bt.to(gc.DEV),
                    torch.tensor(seqlens, dtype=torch.int32, device=gc.DEV), cu.to(gc.DEV))
    torch.cuda.synchronize()
    gk, gv, _ = oracle_pool(gc.host_pool(pool), hk)
    assert np.array_equal(gk, ek) and np.array_equal(gv, ev), "cache_write differs from the bit copy"
    # in pieces of 17 tokens == all at once
    pool2 = gc.to_device(host)
    done = [0, 0, 0]
    while any(done[b] < lens_new[b] for b in range(batch)):
        take = [min(17, lens_new[b] - done[b]) for b in range(batch)]
        rows = [int(cu[b]) + done[b] + i for b in range(batch) for i in range(take[b])]
        idx = torch.tensor(rows, dtype=torch.long)
        pkv.cache_write(kn[idx].to(gc.DEV), vn[idx].to(gc.DEV), pool2.k, pool2.v, bt.to(gc.DEV),
                        torch.tensor([seqlens[b] + done[b] for b in range(batch)], dtype=torch.int32, device=gc.DEV),
                        gen.cu_from_lengths(take).to(gc.DEV))
        done = [done[b] + take[b] for b in range(batch)]
    torch.cuda.synchronize()
    for s1, s2 in zip(pool.storage, pool2.storage):
        assert torch.equal(gc.bits(s1), gc.bits(s2)), "pieces of 17 differ from one write"
