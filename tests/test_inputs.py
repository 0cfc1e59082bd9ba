"""Checks of the seeded generators (layouts, strides, tables, poisoning)."""

import math

import torch

import pkv_inputs as gen


def test_interleaved_views_are_noncontiguous_with_double_block_stride():
    """aiter commit d293d61bbf19, test preconditions: K/V views really non-contiguous."""
    bs, hk, d = 16, 3, 64
    pool = gen.new_pool(gen.pool_num_blocks(339, bs, 2), bs, hk, d, "bf16", "interleaved",
                        generator=torch.Generator().manual_seed(0))
    assert not pool.k.is_contiguous() and not pool.v.is_contiguous()
    assert pool.k.stride(0) == 2 * bs * hk * d
    assert pool.v.storage_offset() - pool.k.storage_offset() == bs * hk * d
    assert pool.num_blocks == math.ceil(339 / 16) * 2 * 3


def test_relayout_preserves_bits():
    pool = gen.new_pool(12, 4, 2, 8, "bf16", "interleaved", generator=torch.Generator().manual_seed(1))
    c = gen.relayout(pool, "contiguous")
    assert c.k.is_contiguous() and torch.equal(c.k.view(torch.int16), pool.k.view(torch.int16))
    back = gen.relayout(c, "interleaved")
    assert torch.equal(back.v.view(torch.int16), pool.v.view(torch.int16))


def test_block_table_is_a_permutation():
    bt = gen.randperm_block_table(48, 4, generator=torch.Generator().manual_seed(2))
    assert bt.shape == (4, 12) and bt.dtype == torch.int32
    assert sorted(bt.flatten().tolist()) == list(range(48))


def test_seeded_generation_is_reproducible():
    a = gen.randn((3, 4, 8), "bf16", generator=torch.Generator().manual_seed(7))
    b = gen.randn((3, 4, 8), "bf16", generator=torch.Generator().manual_seed(7))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_rope_depends_only_on_global_position():
    x = gen.randn((10, 2, 8), "f32", generator=torch.Generator().manual_seed(3))
    full = gen.rope_rotate_half(x, torch.arange(100, 110))
    part = gen.rope_rotate_half(x[4:7], torch.arange(104, 107))
    assert torch.equal(full[4:7], part)
    # position 0 is the identity
    assert torch.equal(gen.rope_rotate_half(x, torch.zeros(10, dtype=torch.long)), x)


def test_poison_touches_only_unreadable_slots():
    pool = gen.new_pool(12, 4, 1, 2, "f32", "contiguous", generator=torch.Generator().manual_seed(4))
    bt = gen.randperm_block_table(12, 2, generator=torch.Generator().manual_seed(5))
    before = pool.k.clone()
    gen.poison_unused(pool, bt, [5, 0])
    # sequence 0 reads blocks bt[0,0] (4 slots) and bt[0,1] slot 0 only
    assert torch.equal(pool.k[bt[0, 0].long()], before[bt[0, 0].long()])
    assert torch.equal(pool.k[bt[0, 1].long(), 0], before[bt[0, 1].long(), 0])
    assert torch.isnan(pool.k[bt[0, 1].long(), 1:]).all()
    assert int(torch.isnan(pool.k).any(dim=(1, 2, 3)).sum()) == 11
