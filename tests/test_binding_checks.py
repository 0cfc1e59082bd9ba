"""The binding rejects bad arguments before anything reaches the library.

The C ABI takes raw addresses and sizes; it cannot see a tensor's device or
its allocated size.  So the binding checks every tensor's shape, dtype,
contiguity and device before the first call into ``libpkv.so``: a host tensor
or an undersized buffer would otherwise become a host-pointer or out-of-bounds
access inside a kernel.  These tests run on the CPU: each one breaks a single
argument of an otherwise well-formed call and checks that the call raises,
naming that argument; the well-formed call itself (all tensors on the host)
raises for the device.
"""

from __future__ import annotations

import pytest
import torch

import invariant_paged_kv_amd as pkv


def base(dtype=torch.bfloat16, batch=2, hq=4, hk=2, d=64, bs=16, nblk=3, rows=(1, 2)):
    nb = nblk * batch
    pool = torch.zeros(nb, 2, bs, hk, d, dtype=dtype)
    total = sum(rows)
    cu = [0]
    for r in rows:
        cu.append(cu[-1] + r)
    return dict(
        q=torch.zeros(total, hq, d, dtype=pkv.query_dtype(dtype)),
        k_cache=pool[:, 0], v_cache=pool[:, 1],
        block_table=torch.arange(nb, dtype=torch.int32).view(batch, nblk),
        seqlens_k=torch.tensor([5, 7], dtype=torch.int32)[:batch],
        cu_seqlens_q=torch.tensor(cu, dtype=torch.int32),
    )


def call_forward(a, **over):
    a = dict(a, **over)
    return pkv.attn_forward(a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seqlens_k"], a["cu_seqlens_q"],
                            True, 0.125, max_seqlen_q=2, out=a.get("out"), lse=a.get("lse"),
                            workspace=a.get("workspace"))


def test_well_formed_host_call_raises_for_the_device():
    with pytest.raises(ValueError, match="GPU"):
        call_forward(base())


@pytest.mark.parametrize("bad, what", [
    (dict(out=torch.zeros(2, 4, 64, dtype=torch.bfloat16)), "out"),                 # too few rows
    (dict(out=torch.zeros(3, 4, 64, dtype=torch.float32)), "out"),                  # wrong dtype
    (dict(out=torch.zeros(3, 4, 128, dtype=torch.bfloat16)[..., :64]), "out"),      # not contiguous
    (dict(lse=torch.zeros(3, 3, dtype=torch.float32)), "lse"),
    (dict(lse=torch.zeros(3, 4, dtype=torch.float64)), "lse"),
    (dict(seqlens_k=torch.tensor([5], dtype=torch.int32)), "seqlens_k"),
    (dict(seqlens_k=torch.tensor([5, 7], dtype=torch.int64)), "seqlens_k"),
    (dict(cu_seqlens_q=torch.tensor([0, 1], dtype=torch.int32)), "cu_seqlens_q"),
    (dict(block_table=torch.arange(6, dtype=torch.int32)), "block_table"),
    (dict(block_table=torch.arange(6, dtype=torch.int64).view(2, 3)), "block_table"),
    (dict(workspace=torch.zeros(64, 2, dtype=torch.uint8)[:, 0]), "workspace"),
    (dict(q=torch.zeros(3, 4, 32, dtype=torch.bfloat16)), "head_dim"),
    (dict(q=torch.zeros(3, 4, 64, dtype=torch.float32)), "q dtype"),
])
def test_forward_rejects_each_bad_argument(bad, what):
    with pytest.raises((ValueError, TypeError), match=what):
        call_forward(base(), **bad)


def test_append_rejects_bad_new_rows():
    a = base()
    kn = torch.zeros(3, 2, 64, dtype=torch.bfloat16)
    for name, k_new, v_new in (("k_new", kn[:2], kn), ("v_new", kn, torch.zeros(3, 1, 64, dtype=torch.bfloat16)),
                               ("k_new", kn.float(), kn)):
        with pytest.raises(ValueError, match=name):
            pkv.attn_forward_append(a["q"], k_new, v_new, a["k_cache"], a["v_cache"], a["block_table"],
                                    a["seqlens_k"], a["cu_seqlens_q"], True, 0.125, max_seqlen_q=2)
    with pytest.raises(ValueError, match="GPU"):
        pkv.attn_forward_append(a["q"], kn, kn, a["k_cache"], a["v_cache"], a["block_table"], a["seqlens_k"],
                                a["cu_seqlens_q"], True, 0.125, max_seqlen_q=2)


def test_cache_write_rejects_bad_arguments():
    a = base()
    kn = torch.zeros(4, 2, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 2, 4], dtype=torch.int32)
    args = (a["k_cache"], a["v_cache"], a["block_table"], a["seqlens_k"], cu)
    with pytest.raises(ValueError, match="total_new"):
        pkv.cache_write(kn, kn, *args, total_new=5)            # more rows than k_new holds
    with pytest.raises(ValueError, match="total_new"):
        pkv.cache_write(kn, kn, *args, total_new=-1)
    with pytest.raises(ValueError, match="k_new"):
        pkv.cache_write(torch.zeros(4, 2, 32, dtype=torch.bfloat16), kn, *args)   # head_dim differs from the cache
    with pytest.raises(ValueError, match="v_new"):
        pkv.cache_write(kn, torch.zeros(4, 3, 64, dtype=torch.bfloat16), *args)   # Hkv differs
    with pytest.raises(ValueError, match="same number of rows"):
        pkv.cache_write(kn, kn[:3], *args)
    with pytest.raises(ValueError, match="cu_seqlens_new"):
        pkv.cache_write(kn, kn, a["k_cache"], a["v_cache"], a["block_table"], a["seqlens_k"], cu[:2])
    with pytest.raises(ValueError, match="GPU"):
        pkv.cache_write(kn, kn, *args)


def test_partials_and_merge_reject_bad_buffers():
    a = base()
    args = (a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seqlens_k"], a["cu_seqlens_q"], True, 0.125)
    rows = 3 * 4
    with pytest.raises(ValueError, match="part_o"):
        pkv.attn_chunk_partials(*args, 0, 1, max_seqlen_q=2, max_chunks=1,
                                part_o=torch.zeros(1, rows - 1, 64), part_ml=torch.zeros(1, rows, 2))
    with pytest.raises(ValueError, match="part_ml"):
        pkv.attn_chunk_partials(*args, 0, 1, max_seqlen_q=2, max_chunks=1,
                                part_o=torch.zeros(1, rows, 64), part_ml=torch.zeros(1, rows, 3))
    with pytest.raises(ValueError, match="GPU"):
        pkv.attn_chunk_partials(*args, 0, 1, max_seqlen_q=2, max_chunks=1)
    mk = dict(max_seqlen_q=2)
    with pytest.raises(ValueError, match="part_ml"):
        pkv.attn_merge_partials(torch.zeros(2, rows, 64), torch.zeros(1, rows, 2), a["q"], a["k_cache"],
                                a["v_cache"], a["block_table"], a["seqlens_k"], a["cu_seqlens_q"], True, **mk)
    with pytest.raises(ValueError, match="out"):
        pkv.attn_merge_partials(torch.zeros(2, rows, 64), torch.zeros(2, rows, 2), a["q"], a["k_cache"],
                                a["v_cache"], a["block_table"], a["seqlens_k"], a["cu_seqlens_q"], True,
                                out=torch.zeros(1, 4, 64, dtype=torch.bfloat16), **mk)
    with pytest.raises(ValueError, match="GPU"):
        pkv.attn_merge_partials(torch.zeros(2, rows, 64), torch.zeros(2, rows, 2), a["q"], a["k_cache"],
                                a["v_cache"], a["block_table"], a["seqlens_k"], a["cu_seqlens_q"], True, **mk)


def test_backward_rejects_bad_buffers():
    a = base(dtype=torch.float32)
    q = a["q"]
    out = torch.zeros_like(q)
    lse = torch.zeros(q.shape[:2])
    cuk = torch.tensor([0, 5, 12], dtype=torch.int32)
    common = (a["q"], a["k_cache"], a["v_cache"], a["block_table"], a["seqlens_k"], a["cu_seqlens_q"], True, 0.1,
              out, lse, torch.zeros_like(q))
    with pytest.raises(ValueError, match="dk"):
        pkv.attn_backward(*common, max_seqlen_q=2, cu_seqlens_k=cuk, total_k=12, dk=torch.zeros(11, 2, 64))
    with pytest.raises(ValueError, match="dq"):
        pkv.attn_backward(*common, max_seqlen_q=2, cu_seqlens_k=cuk, total_k=12, dq=torch.zeros(2, 4, 64))
    with pytest.raises(ValueError, match="cu_seqlens_k"):
        pkv.attn_backward(*common, max_seqlen_q=2, cu_seqlens_k=cuk[:2], total_k=12)
    with pytest.raises(ValueError, match="GPU"):
        pkv.attn_backward(*common, max_seqlen_q=2, cu_seqlens_k=cuk, total_k=12)
