"""Fused append-then-attend (pkv_attn_forward_append) against the unfused pair.

The fused call writes each query row's K/V at the row's own key position and
attends in one launch; it must leave the cache and return out/lse bit for bit
as pkv_cache_write followed by pkv_attn_forward (aiter commit d293d61bbf19:
flash_attn_with_kvcache with new_kv; RL-Kernel issue #152, section Scope: no
precision difference between the path that writes the cache and the one that
reads it).
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


def clone_pool(pool: gen.PagedKV) -> gen.PagedKV:
    if pool.layout == "interleaved":
        buf = pool.storage[0].clone()
        return gen.PagedKV(buf[:, 0], buf[:, 1], "interleaved", [buf])
    k, v = pool.k.clone(), pool.v.clone()
    return gen.PagedKV(k, v, "contiguous", [k, v])


def unfused(q, kn, vn, pool, bt, seqlens, cu, causal, scale, max_q, max_k, path=None):
    L = torch.tensor([cu[i + 1] - cu[i] for i in range(len(cu) - 1)], dtype=torch.int32, device=gc.DEV)
    sk = torch.tensor(seqlens, dtype=torch.int32, device=gc.DEV)
    cu_d = torch.tensor(cu, dtype=torch.int32, device=gc.DEV)
    pkv.cache_write(kn, vn, pool.k, pool.v, bt, sk - L, cu_d)
    with pkv.options(path=path):
        return pkv.attn_forward(q, pool.k, pool.v, bt, sk, cu_d, causal, scale, max_seqlen_q=max_q, max_seqlen_k=max_k,
                                **gc.nan_outputs(q))


def fused(q, kn, vn, pool, bt, seqlens, cu, causal, scale, max_q, max_k, path=None, split=None):
    sk = torch.tensor(seqlens, dtype=torch.int32, device=gc.DEV)
    cu_d = torch.tensor(cu, dtype=torch.int32, device=gc.DEV)
    with pkv.options(path=path, split_chunks=split):
        return pkv.attn_forward_append(q, kn, vn, pool.k, pool.v, bt, sk, cu_d, causal, scale,
                                       max_seqlen_q=max_q, max_seqlen_k=max_k)


def check_same(case_kw, paths=(None, 1, 2), splits=(None,)):
    g = torch.Generator().manual_seed(case_kw["seed"])
    hq, hk, d, bs, layout = case_kw["hq"], case_kw["hk"], case_kw["d"], case_kw["bs"], case_kw["layout"]
    seqlens, lens = case_kw["seqlens"], case_kw["lens"]
    batch = len(seqlens)
    nb = gen.pool_num_blocks(max(seqlens), bs, batch)
    base = gc.to_device(gen.new_pool(nb, bs, hk, d, case_kw.get("dtype", "bf16"), layout, generator=g))
    bt = gen.randperm_block_table(nb, batch, generator=g).to(gc.DEV)
    cu = [0]
    for x in lens:
        cu.append(cu[-1] + x)
    dt = case_kw.get("dtype", "bf16")
    q = gen.randn((cu[-1], hq, d), dt, generator=g).to(gc.DEV)
    kn = gen.randn((cu[-1], hk, d), dt, generator=g).to(gc.DEV)
    vn = gen.randn((cu[-1], hk, d), dt, generator=g).to(gc.DEV)
    scale = 1.0 / math.sqrt(d)
    max_q, max_k = max(lens), max(seqlens)
    ref_pool = clone_pool(base)
    ref = unfused(q, kn, vn, ref_pool, bt, seqlens, cu, True, scale, max_q, max_k)
    torch.cuda.synchronize()
    for path in paths:
        for split in splits:
            p = clone_pool(base)
            got = fused(q, kn, vn, p, bt, seqlens, cu, True, scale, max_q, max_k, path=path, split=split)
            torch.cuda.synchronize()
            gc.assert_bitwise(got, ref, f"fused vs unfused (path {path}, split {split})")
            for s1, s2 in zip(p.storage, ref_pool.storage):
                assert torch.equal(gc.bits(s1), gc.bits(s2)), f"cache bytes differ (path {path}, split {split})"
    return ref


@pytest.mark.parametrize("layout", ["interleaved", "contiguous"])
@pytest.mark.parametrize("bs", [16, 256, 7])
def test_append_decode_rows(layout, bs):
    announce(f"append decode {layout} bs={bs}")
    check_same(dict(seed=5000 + bs, hq=16, hk=4, d=128, bs=bs, layout=layout,
                    seqlens=[1, 700, 513, 1030], lens=[1, 1, 3, 2]), splits=(None, 3))


def test_append_chunk_rows_cross_chunk_boundary():
    """17 new rows straddling a chunk boundary (1024 and 2048 keys), several KV heads per column block."""
    announce("append 17 rows across a chunk boundary")
    check_same(dict(seed=5100, hq=16, hk=4, d=128, bs=16, layout="interleaved",
                    seqlens=[1030, 2060], lens=[17, 17]))


def test_append_long_prefill_rows():
    announce("append 300 rows (prefill kernel)")
    check_same(dict(seed=5200, hq=8, hk=2, d=64, bs=32, layout="contiguous",
                    seqlens=[300, 900], lens=[300, 300]))


def test_append_fp32():
    announce("append fp32")
    check_same(dict(seed=5300, hq=2, hk=2, d=64, bs=16, layout="contiguous", dtype="f32",
                    seqlens=[340, 50], lens=[1, 4]))


def test_generate_with_fused_append_equals_rescore():
    """The generate-then-rescore check with the fused step: 64 steps vs one 64-row prefill."""
    announce("fused generate vs re-score")
    batch, hq, hk, d, bs, n_final, steps = 2, 64, 8, 128, 256, 4096, 64
    nb = gen.pool_num_blocks(n_final, bs, batch)
    pool = gc.device_pool(5400, nb, bs, hk, d, "bf16", "interleaved")
    bt = gen.randperm_block_table(nb, batch, generator=torch.Generator().manual_seed(5400)).to(gc.DEV)
    g = torch.Generator(device=gc.DEV).manual_seed(5401)
    q = gen.randn((steps, batch, hq, d), "bf16", generator=g, device=gc.DEV)
    kn = gen.randn((steps, batch, hk, d), "bf16", generator=g, device=gc.DEV)
    vn = gen.randn((steps, batch, hk, d), "bf16", generator=g, device=gc.DEV)
    scale = 1.0 / math.sqrt(d)
    cu1 = torch.arange(batch + 1, dtype=torch.int32, device=gc.DEV)
    outs, lses = [], []
    for t in range(steps):
        sk = torch.full((batch,), n_final - steps + t + 1, dtype=torch.int32, device=gc.DEV)
        o, l = pkv.attn_forward_append(q[t].contiguous(), kn[t].contiguous(), vn[t].contiguous(), pool.k, pool.v,
                                       bt, sk, cu1, True, scale, max_seqlen_q=1, max_seqlen_k=n_final)
        outs.append(o)
        lses.append(l)
    qp = q.transpose(0, 1).reshape(batch * steps, hq, d).contiguous()
    case = gc.Case(qp, pool, bt, [n_final] * batch, [steps * b for b in range(batch + 1)], True, scale, "bf16")
    p_out, p_lse = gc.run(case)
    d_out = torch.stack(outs, dim=1).reshape(batch * steps, hq, d)
    d_lse = torch.stack(lses, dim=1).reshape(batch * steps, hq)
    gc.assert_bitwise((d_out, d_lse), (p_out, p_lse), "fused generate vs re-score")
    gc.check_oracle(case, p_out, p_lse, seq_ids=[1])
