"""FP8 E4M3 KV cache (PKV_FP8_E4M3) on the GPU.

The FP8 cache is the step RL-Kernel issue #152 defers (section Out of scope):
half the decode bytes.  Stored bytes are widened exactly to bf16 in the
loaders, k_scale enters the score multiplier and v_scale the final write, so
the computation after the load is the bf16 one: the same tolerances against
the oracle (out 2e-2 in the units of the stored V, i.e. on out / v_scale; lse
1e-3) and the same bitwise invariances between paths, splits, batches and
layouts.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import invariant_paged_kv_amd as pkv
import pkv_inputs as gen
from tests import gpu_cases as gc
from tests.oracle_bridge import oracle_attention

pytestmark = pytest.mark.gpu

TOL_OUT, TOL_LSE = gc.TOL["bf16"]


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


def fp8_case(seed, batch, hq, hk, d, bs, seqlen_k, layout, causal, lens_q, seqlens=None,
             k_scale=0.5, v_scale=1.25):
    g = torch.Generator().manual_seed(seed)
    nb = gen.pool_num_blocks(seqlen_k, bs, batch)
    pool = gen.new_pool(nb, bs, hk, d, "fp8", layout, generator=g)
    bt = gen.randperm_block_table(nb, batch, generator=g)
    if seqlens is None:
        seqlens = gen.uniform_int(1, seqlen_k, batch, generator=g)
    cu = [0]
    for x in lens_q:
        cu.append(cu[-1] + int(x))
    q = gen.randn((cu[-1], hq, d), "bf16", generator=g)
    case = gc.Case(q.to(gc.DEV), gc.to_device(pool), bt.to(gc.DEV), list(map(int, seqlens)), cu, causal,
                   1.0 / math.sqrt(d), "bf16")
    case.extra = {"k_scale": k_scale, "v_scale": v_scale}
    return case


def run(case, pool=None, block_table=None, q=None, seqlens=None, cu=None, path=None, split=None, full_kernel=None):
    pool = pool or case.pool
    bt = case.block_table if block_table is None else block_table
    q = case.q if q is None else q
    sl = case.seqlens if seqlens is None else seqlens
    cul = case.cu if cu is None else cu
    out0 = torch.full_like(q, float("nan"))   # unwritten elements stay NaN
    lse0 = torch.full((q.shape[0], q.shape[1]), float("nan"), dtype=torch.float32, device=q.device)
    with pkv.options(path=path, split_chunks=split, full_kernel=full_kernel):
        out, lse = pkv.attn_forward(
            q, pool.k, pool.v, bt, torch.tensor(sl, dtype=torch.int32, device=gc.DEV),
            torch.tensor(cul, dtype=torch.int32, device=gc.DEV), case.causal, case.scale,
            max_seqlen_q=max(cul[i + 1] - cul[i] for i in range(len(cul) - 1)), max_seqlen_k=max(sl),
            k_scale=case.extra["k_scale"], v_scale=case.extra["v_scale"], out=out0, lse=lse0)
    torch.cuda.synchronize()
    return out, lse


def check_oracle(case, out, lse, seq_ids=None):
    if seq_ids is None:
        seq_ids = list(range(len(case.seqlens)))
    q, pool, bt, seqlens, cu, rows = gc.subset_for_oracle(case, seq_ids)
    if not rows:
        return
    oout, olse = oracle_attention(q, pool, bt, seqlens, cu, case.causal, case.scale,
                                  case.extra["k_scale"], case.extra["v_scale"])
    # v_scale multiplies every output; the bf16 out tolerance (an absolute bound
    # for N(0,1) values) applies in the units of the stored V, i.e. to out / v_scale.
    vs = case.extra["v_scale"]
    idx = torch.tensor(rows, dtype=torch.long, device=out.device)
    eo = gc.max_err(out.index_select(0, idx).double() / vs, oout / vs)
    el = gc.max_err(lse.index_select(0, idx), olse)
    assert eo <= TOL_OUT, f"out max-abs {eo:.3e}"
    assert el <= TOL_LSE, f"lse max-abs {el:.3e}"
    print(f"oracle: out {eo:.2e}, lse {el:.2e}")


CASES = [
    # name, hq, hk, d, bs, layout, causal, lens, seqlens, scales
    ("decode-gqa4", 16, 4, 128, 16, "interleaved", True, [1, 1, 1, 1], [3000, 1, 513, 2048], (0.5, 1.25)),
    ("padded-decode-3", 32, 8, 128, 256, "contiguous", True, [3, 3, 3], [700, 2, 5000], (1.0, 1.0)),
    ("chunked-prefill", 16, 4, 128, 16, "interleaved", True, [300, 17], [900, 17], (0.25, 3.0)),
    ("d64-bs7-noncausal", 8, 2, 64, 7, "contiguous", False, [5, 1, 40], [100, 333, 40], (2.0, 0.0625)),
]


@pytest.mark.parametrize("spec", CASES, ids=[c[0] for c in CASES])
def test_fp8_parity_and_paths(spec):
    name, hq, hk, d, bs, layout, causal, lens, seqlens, (ks, vs) = spec
    announce(f"fp8 {name}")
    case = fp8_case(8000 + CASES.index(spec), len(lens), hq, hk, d, bs, max(seqlens), layout, causal, lens,
                    seqlens, ks, vs)
    ref = run(case)
    check_oracle(case, *ref)
    for path in (1, 2):
        for split in (None, 1, 3):
            gc.assert_bitwise(run(case, path=path, split=split), ref, f"path {path} split {split}")
    for fk in (1, 2, 3):
        gc.assert_bitwise(run(case, path=2, full_kernel=fk), ref, f"full kernel {fk}")
    other = gc.to_device(gen.relayout(gc.host_pool(case.pool), "contiguous" if layout == "interleaved" else "interleaved"))
    gc.assert_bitwise(run(case, pool=other), ref, "layout")


def test_fp8_batch_invariance_and_poison():
    announce("fp8 batch invariance + poisoned unused memory")
    lens, seqlens = [1, 3, 1, 2], [2500, 70, 1, 1030]
    case = fp8_case(8100, 4, 16, 4, 128, 16, max(seqlens), "interleaved", True, lens, seqlens)
    ref = run(case)
    for s in range(4):
        r0, r1 = case.cu[s], case.cu[s + 1]
        one = run(case, block_table=case.block_table[s:s + 1].contiguous(), q=case.q[r0:r1].contiguous(),
                  seqlens=[seqlens[s]], cu=[0, r1 - r0])
        gc.assert_bitwise(one, (ref[0][r0:r1], ref[1][r0:r1]), f"sequence {s} alone")
    gen.poison_unused(case.pool, case.block_table, case.seqlens)
    bt2 = gen.poison_table_tail(case.block_table, case.seqlens, case.pool.block_size, -1)
    gc.assert_bitwise(run(case, block_table=bt2), ref, "poisoned")


def test_fp8_generate_then_rescore_and_fused_append():
    """16 generate steps (one FP8 K/V row written, then decode) equal one
    16-row causal prefill bitwise; the fused append gives the same bits and cache bytes."""
    announce("fp8 generate vs re-score, fused append")
    batch, hq, hk, d, bs, n_final, steps = 2, 16, 4, 128, 16, 1300, 16
    nb = gen.pool_num_blocks(n_final, bs, batch)
    g = torch.Generator().manual_seed(8200)
    pool = gc.to_device(gen.new_pool(nb, bs, hk, d, "fp8", "interleaved", generator=g))
    pool_f = gc.to_device(gen.relayout(gc.host_pool(pool), "interleaved"))
    bt = gen.randperm_block_table(nb, batch, generator=g).to(gc.DEV)
    q = gen.randn((steps, batch, hq, d), "bf16", generator=g).to(gc.DEV)
    kn = gen.randn((steps, batch, hk, d), "fp8", generator=g).to(gc.DEV)
    vn = gen.randn((steps, batch, hk, d), "fp8", generator=g).to(gc.DEV)
    scale, ks, vs = 1.0 / math.sqrt(d), 0.75, 1.5
    cu1 = torch.arange(batch + 1, dtype=torch.int32, device=gc.DEV)
    outs, lses = [], []
    for t in range(steps):
        n = n_final - steps + t
        sk_old = torch.full((batch,), n, dtype=torch.int32, device=gc.DEV)
        pkv.cache_write(kn[t].contiguous(), vn[t].contiguous(), pool.k, pool.v, bt, sk_old, cu1)
        o, l = pkv.attn_forward(q[t].contiguous(), pool.k, pool.v, bt, sk_old + 1, cu1, True, scale,
                                max_seqlen_q=1, max_seqlen_k=n_final, k_scale=ks, v_scale=vs, **gc.nan_outputs(q[t]))
        of, lf = pkv.attn_forward_append(q[t].contiguous(), kn[t].contiguous(), vn[t].contiguous(), pool_f.k,
                                         pool_f.v, bt, sk_old + 1, cu1, True, scale, max_seqlen_q=1,
                                         max_seqlen_k=n_final, k_scale=ks, v_scale=vs)
        gc.assert_bitwise((of, lf), (o, l), f"fused append step {t}")
        outs.append(o)
        lses.append(l)
    torch.cuda.synchronize()
    assert torch.equal(pool.storage[0].view(torch.uint8), pool_f.storage[0].view(torch.uint8)), "cache bytes differ"
    qp = q.transpose(0, 1).reshape(batch * steps, hq, d).contiguous()
    case = gc.Case(qp, pool, bt, [n_final] * batch, [steps * b for b in range(batch + 1)], True, scale, "bf16")
    case.extra = {"k_scale": ks, "v_scale": vs}
    p_out, p_lse = run(case)
    d_out = torch.stack(outs, dim=1).reshape(batch * steps, hq, d)
    d_lse = torch.stack(lses, dim=1).reshape(batch * steps, hq)
    gc.assert_bitwise((d_out, d_lse), (p_out, p_lse), "generate vs re-score")
    check_oracle(case, p_out, p_lse, seq_ids=[1])


def test_fp8_cache_write_is_a_byte_copy():
    announce("fp8 cache_write bytes")
    g = torch.Generator().manual_seed(8300)
    nb, bs, hk, d = 24, 16, 4, 128
    pool = gc.to_device(gen.new_pool(nb, bs, hk, d, "fp8", "contiguous", generator=g))
    before = [t.view(torch.uint8).clone() for t in (pool.k, pool.v)]
    bt = gen.randperm_block_table(nb, 2, generator=g).to(gc.DEV)
    kn = gen.randn((7, hk, d), "fp8", generator=g).to(gc.DEV)
    vn = gen.randn((7, hk, d), "fp8", generator=g).to(gc.DEV)
    sk = torch.tensor([30, 5], dtype=torch.int32, device=gc.DEV)
    cu = torch.tensor([0, 4, 7], dtype=torch.int32, device=gc.DEV)
    pkv.cache_write(kn, vn, pool.k, pool.v, bt, sk, cu)
    torch.cuda.synchronize()
    btc = bt.cpu()
    for t, new, old in ((pool.k, kn, before[0]), (pool.v, vn, before[1])):
        got = t.view(torch.uint8).clone()
        want = old.clone()
        for b, (n0, r0, r1) in enumerate(((30, 0, 4), (5, 4, 7))):
            for i in range(r1 - r0):
                pos = n0 + i
                want[int(btc[b, pos // bs]), pos % bs] = new.view(torch.uint8)[r0 + i]
        assert torch.equal(got, want), "FP8 cache_write changed other bytes or wrote wrong ones"


@pytest.mark.large
def test_fp8_long_context_decode():
    """Long-context FP8 decode: batch 16, Hq 64, Hkv 8, d 128, 131072 keys, bs 256, interleaved;
    one sequence against the oracle and bitwise through the prefill kernel."""
    announce("fp8 long-context decode 16 x 131072")
    B, HQ, HK, D, BS, N = 16, 64, 8, 128, 256, 131072
    nb = gen.pool_num_blocks(N, BS, B)
    pool = gc.device_pool(8400, nb, BS, HK, D, "fp8", "interleaved")
    bt = gen.randperm_block_table(nb, B, generator=torch.Generator().manual_seed(8400)).to(gc.DEV)
    g = torch.Generator(device=gc.DEV).manual_seed(8401)
    q = gen.randn((B, HQ, D), "bf16", generator=g, device=gc.DEV)
    case = gc.Case(q, pool, bt, [N] * B, list(range(B + 1)), True, 1.0 / math.sqrt(D), "bf16")
    case.extra = {"k_scale": 0.5, "v_scale": 1.25}
    out, lse = run(case)
    check_oracle(case, out, lse, seq_ids=[3])
    full = run(case, path=2, block_table=bt[3:4].contiguous(), q=q[3:4].contiguous(), seqlens=[N], cu=[0, 1])
    gc.assert_bitwise(full, (out[3:4], lse[3:4]), "decode row vs prefill kernel")
