"""GPU parity: the HIP path against the float64 oracle, element by element, and
the bitwise identities the pages ask for, on every workload shape.

Workloads (seeded synthetic inputs, shapes of the pages' tests):
  C1  fp32 MHA Hq=Hkv=2, d=64, one sequence, bs=16, contiguous pool of
      ceil(339/16)*3 blocks: decode of token 339 after appending it with
      pkv_cache_write, and the same token as row 339 of a 340-row causal prefill.
  aiter grid  mha/gqa (6 q heads, 6 or 3 KV heads), causal on/off, bs 16/256,
      (seqlen_q, seqlen_k) in {(1,339), (3,1024), (17,156)}, d 64/128, batch 2,
      bf16, K/V-interleaved pool (aiter commit d293d61bbf19, test
      test_flash_attn_kvcache_noncontiguous_paged).
  C2  decode, Hq=16, Hkv=4, d=128, bf16, seqlen_k=4096, bs=16, interleaved.
  C3  ragged/padded decode, Hq=32, Hkv=8, bs=256, seqlen_k ~ U[1, 8192], 1 or 3
      real query rows left-padded into 3-row slots, causal.
  C4  chunked vs full prefill, Hq=16, Hkv=4, bs=16, post-RoPE-like Q/K, cache
      written by pkv_cache_write chunk by chunk.
  C5  long-context decode, Hq=64, Hkv=8, bs=256, interleaved: 64 generate steps
      (append one token, decode it) against a one-shot 64-row prefill.
Reduced sizes run always; the full sizes are marked ``large``.
"""

from __future__ import annotations

import math

import pytest
import torch

import invariant_paged_kv_amd as pkv
import pkv_inputs as gen
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

FORCE_SPLIT, FORCE_FULL = 1, 2


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


# ---------------------------------------------------------------------------
# C1: fp32, decode == row 339 of the 340-row causal prefill
# ---------------------------------------------------------------------------

def c1_case():
    g = torch.Generator().manual_seed(1001)
    bs, hk, d = 16, 2, 64
    nb = gen.pool_num_blocks(339, bs, 1)                  # 22 * 3 = 66
    pool = gc.to_device(gen.new_pool(nb, bs, hk, d, "f32", "contiguous", generator=g))
    bt = gen.randperm_block_table(nb, 1, generator=g).to(gc.DEV)
    q_all = gen.randn((340, 2, d), "f32", generator=g).to(gc.DEV)
    k_new = gen.randn((1, hk, d), "f32", generator=g).to(gc.DEV)
    v_new = gen.randn((1, hk, d), "f32", generator=g).to(gc.DEV)
    return pool, bt, q_all, k_new, v_new


def test_c1_fp32_decode_equals_prefill_row():
    announce("C1 fp32 decode vs prefill row 339")
    pool, bt, q_all, k_new, v_new = c1_case()
    assert pool.k.shape == (66, 16, 2, 64) and pool.k.stride(0) == 2048
    # token 339 is appended by the library's cache write
    pkv.cache_write(k_new, v_new, pool.k, pool.v, bt, torch.tensor([339], dtype=torch.int32, device=gc.DEV),
                    torch.tensor([0, 1], dtype=torch.int32, device=gc.DEV))
    torch.cuda.synchronize()
    assert torch.equal(pool.k[bt[0, 339 // 16].long(), 339 % 16], k_new[0])
    scale = 1.0 / 8.0
    dec = gc.Case(q_all[339:340].contiguous(), pool, bt, [340], [0, 1], False, scale, "f32")
    pre = gc.Case(q_all, pool, bt, [340], [0, 340], True, scale, "f32")
    d_out, d_lse = gc.run(dec)
    p_out, p_lse = gc.run(pre)
    gc.check_oracle(dec, d_out, d_lse)
    gc.check_oracle(pre, p_out, p_lse)
    gc.assert_bitwise((d_out[0], d_lse[0]), (p_out[339], p_lse[339]), "C1 decode vs prefill row 339")
    # causal decode of the same token, and the forced-path variants
    dc_out, dc_lse = gc.run(dec, causal=True)
    gc.assert_bitwise((dc_out, dc_lse), (d_out, d_lse), "causal decode")
    for path in (FORCE_SPLIT, FORCE_FULL):
        gc.assert_bitwise(gc.run(pre, path=path), (p_out, p_lse), f"prefill forced path {path}")
        gc.assert_bitwise(gc.run(dec, path=path), (d_out, d_lse), f"decode forced path {path}")
    # the other reading: token 338 over 339 keys == prefill row 338
    alt = gc.Case(q_all[338:339].contiguous(), pool, bt, [339], [0, 1], False, scale, "f32")
    a_out, a_lse = gc.run(alt)
    gc.check_oracle(alt, a_out, a_lse)
    gc.assert_bitwise((a_out[0], a_lse[0]), (p_out[338], p_lse[338]), "C1 token 338 vs prefill row 338")


# ---------------------------------------------------------------------------
# The aiter test grid: oracle parity, interleaved == contiguous, decode == prefill paths
# ---------------------------------------------------------------------------

GRID = [(mha, causal, bs, sq, sk, d)
        for mha in ("mha", "gqa") for causal in (False, True) for bs in (16, 256)
        for (sq, sk) in ((1, 339), (3, 1024), (17, 156)) for d in (64, 128)]


@pytest.mark.parametrize("mha,causal,bs,sq,sk,d", GRID)
def test_aiter_grid(mha, causal, bs, sq, sk, d):
    announce(f"aiter grid {mha} causal={causal} bs={bs} sq={sq} sk={sk} d={d}")
    hk = 6 if mha == "mha" else 3
    seed = 2000 + GRID.index((mha, causal, bs, sq, sk, d))
    case = gc.make_case(seed, "bf16", 2, 6, hk, d, bs, sk, "interleaved", causal, [sq, sq])
    assert not case.pool.k.is_contiguous() and case.pool.k.stride(0) == 2 * bs * hk * d
    out, lse = gc.run(case)
    gc.check_oracle(case, out, lse)
    contig = gen.relayout(case.pool, "contiguous")
    gc.assert_bitwise(gc.run(case, pool=contig), (out, lse), "interleaved vs contiguous")
    for path in (FORCE_SPLIT, FORCE_FULL):
        gc.assert_bitwise(gc.run(case, path=path), (out, lse), f"forced path {path}")


# ---------------------------------------------------------------------------
# C2: decode, Qwen3-8B-like shard
# ---------------------------------------------------------------------------

def c2_case(batch: int, seed: int = 1002):
    bs, hq, hk, d, n = 16, 16, 4, 128, 4096
    nb = gen.pool_num_blocks(n, bs, batch)
    pool = gc.device_pool(seed, nb, bs, hk, d, "bf16", "interleaved")
    bt = gen.randperm_block_table(nb, batch, generator=torch.Generator().manual_seed(seed)).to(gc.DEV)
    q = gen.randn((batch, hq, d), "bf16", generator=torch.Generator().manual_seed(seed + 1)).to(gc.DEV)
    return gc.Case(q, pool, bt, [n] * batch, list(range(batch + 1)), False, 1.0 / math.sqrt(128), "bf16")


def test_c2_decode_reduced():
    announce("C2 reduced batch=8")
    case = c2_case(8)
    out, lse = gc.run(case)
    gc.check_oracle(case, out, lse)
    gc.assert_bitwise(gc.run(case, causal=True), (out, lse), "causal == non-causal for the last row")
    gc.assert_bitwise(gc.run(case, path=FORCE_FULL), (out, lse), "decode vs prefill kernel")


@pytest.mark.large
def test_c2_decode_full_size():
    announce("C2 full batch=64")
    case = c2_case(64)
    assert case.pool.num_blocks == 256 * 64 * 3 and case.pool.k.stride(0) == 2 * 16 * 4 * 128
    out, lse = gc.run(case)
    gc.check_oracle(case, out, lse, seq_ids=[0, 31, 63])
    gc.assert_bitwise(gc.run(case, path=FORCE_FULL), (out, lse), "decode vs prefill kernel")


# ---------------------------------------------------------------------------
# C3: ragged / padded decode; batch invariance
# ---------------------------------------------------------------------------

def c3_case(batch: int, seed: int = 1003, maxk: int = 8192):
    bs, hq, hk, d = 256, 32, 8, 128
    g = torch.Generator().manual_seed(seed)
    seqlens = gen.uniform_int(1, maxk, batch, generator=g)
    real = [1 if x == 0 else 3 for x in gen.uniform_int(0, 1, batch, generator=g)]
    nb = gen.pool_num_blocks(maxk, bs, batch)
    pool = gc.device_pool(seed, nb, bs, hk, d, "bf16", "interleaved")
    bt = gen.randperm_block_table(nb, batch, generator=g).to(gc.DEV)
    q = gen.randn((3 * batch, hq, d), "bf16", generator=g).to(gc.DEV)
    cu = [3 * i for i in range(batch + 1)]
    case = gc.Case(q, pool, bt, seqlens, cu, True, 1.0 / math.sqrt(128), "bf16")
    case.extra["real"] = real
    return case


def c3_checks(case: gc.Case, oracle_ids):
    out, lse = gc.run(case)
    gc.check_oracle(case, out, lse, seq_ids=oracle_ids)
    contig = gen.relayout(case.pool, "contiguous")
    gc.assert_bitwise(gc.run(case, pool=contig), (out, lse), "C3 interleaved vs contiguous")
    del contig
    # unpadded batch: only the real rows of each slot
    real = case.extra["real"]
    keep = [3 * b + (3 - real[b]) + i for b in range(len(real)) for i in range(real[b])]
    idx = torch.tensor(keep, dtype=torch.long, device=gc.DEV)
    cu = [0]
    for r in real:
        cu.append(cu[-1] + r)
    u_out, u_lse = gc.run(case, q=case.q.index_select(0, idx).contiguous(), cu=cu)
    gc.assert_bitwise((u_out, u_lse), (out.index_select(0, idx), lse.index_select(0, idx)), "padded vs unpadded")
    # batch = 1 per sequence
    for b in range(len(real)):
        r0 = 3 * b
        one = gc.run(case, q=case.q[r0:r0 + 3].contiguous(), block_table=case.block_table[b:b + 1].contiguous(),
                     seqlens=[case.seqlens[b]], cu=[0, 3])
        gc.assert_bitwise(one, (out[r0:r0 + 3], lse[r0:r0 + 3]), f"batch=1 vs batched, sequence {b}")
    return out, lse


def test_c3_ragged_reduced():
    announce("C3 reduced batch=16")
    case = c3_case(16)
    c3_checks(case, list(range(16)))


@pytest.mark.large
def test_c3_ragged_full_size():
    announce("C3 full batch=128")
    case = c3_case(128)
    c3_checks(case, [0, 1, 77, 127])


# ---------------------------------------------------------------------------
# C4: chunked prefill (cache written chunk by chunk) vs full prefill
# ---------------------------------------------------------------------------

def c4_inputs(batch: int, seqlen: int, seed: int = 1004):
    hq, hk, d = 16, 4, 128
    g = torch.Generator().manual_seed(seed)
    pos = torch.arange(seqlen)
    qs, ks, vs = [], [], []
    for _ in range(batch):
        q = gen.rope_rotate_half(torch.randn((seqlen, hq, d), generator=g), pos).to(torch.bfloat16)
        k = gen.rope_rotate_half(torch.randn((seqlen, hk, d), generator=g), pos).to(torch.bfloat16)
        v = torch.randn((seqlen, hk, d), generator=g).to(torch.bfloat16)
        qs.append(q), ks.append(k), vs.append(v)
    return qs, ks, vs


def c4_run(qs, ks, vs, chunk: int, layout: str = "contiguous", seed: int = 1004):
    """Write the cache chunk by chunk with pkv_cache_write, attending each chunk's rows."""
    batch, seqlen = len(qs), qs[0].shape[0]
    bs, hk, d, hq = 16, 4, 128, 16
    nb = gen.pool_num_blocks(seqlen, bs, batch)
    pool = gen.new_pool(nb, bs, hk, d, "bf16", layout, device=gc.DEV, fill="nan")
    bt = gen.randperm_block_table(nb, batch, generator=torch.Generator().manual_seed(seed)).to(gc.DEV)
    outs, lses = [], []
    for s0 in range(0, seqlen, chunk):
        s1 = min(seqlen, s0 + chunk)
        L = s1 - s0
        cu = [L * b for b in range(batch + 1)]
        kn = torch.cat([k[s0:s1] for k in ks]).to(gc.DEV)
        vn = torch.cat([v[s0:s1] for v in vs]).to(gc.DEV)
        pkv.cache_write(kn, vn, pool.k, pool.v, bt, torch.full((batch,), s0, dtype=torch.int32, device=gc.DEV),
                        torch.tensor(cu, dtype=torch.int32, device=gc.DEV))
        q = torch.cat([x[s0:s1] for x in qs]).to(gc.DEV)
        case = gc.Case(q, pool, bt, [s1] * batch, cu, True, 1.0 / math.sqrt(d), "bf16")
        o, l = gc.run(case)
        outs.append(o.view(batch, L, hq, d))
        lses.append(l.view(batch, L, hq))
    out = torch.cat(outs, dim=1).reshape(batch * seqlen, hq, d)
    lse = torch.cat(lses, dim=1).reshape(batch * seqlen, hq)
    full_case = gc.Case(torch.cat(qs).to(gc.DEV), pool, bt, [seqlen] * batch,
                        [seqlen * b for b in range(batch + 1)], True, 1.0 / math.sqrt(d), "bf16")
    return out, lse, full_case


def test_c4_chunked_vs_full_reduced():
    announce("C4 reduced batch=2 seqlen=2100")
    qs, ks, vs = c4_inputs(2, 2100)
    full_out, full_lse, case = c4_run(qs, ks, vs, 2100)
    gc.check_oracle(case, full_out, full_lse)
    for chunk in (17, 1024):
        out, lse, _ = c4_run(qs, ks, vs, chunk)
        gc.assert_bitwise((out, lse), (full_out, full_lse), f"chunk {chunk} vs full")
    out, lse, _ = c4_run(qs, ks, vs, 1024, layout="interleaved")
    gc.assert_bitwise((out, lse), (full_out, full_lse), "chunk 1024 interleaved vs full contiguous")


@pytest.mark.large
def test_c4_chunked_vs_full_size():
    announce("C4 full batch=8 seqlen=8192")
    qs, ks, vs = c4_inputs(8, 8192)
    full_out, full_lse, case = c4_run(qs, ks, vs, 8192)
    # sampled oracle rows: the last 64 rows of two sequences
    sub = gc.Case(torch.cat([qs[0][-64:], qs[5][-64:]]).to(gc.DEV), case.pool, case.block_table[[0, 5]].contiguous(),
                  [8192, 8192], [0, 64, 128], True, case.scale, "bf16")
    o, l = gc.run(sub)
    gc.check_oracle(sub, o, l)
    rows = torch.cat([torch.arange(8192 - 64, 8192), torch.arange(5 * 8192 + 8192 - 64, 6 * 8192)]).to(gc.DEV)
    gc.assert_bitwise((o, l), (full_out[rows], full_lse[rows]), "64-row tail vs full prefill rows")
    for chunk in (17, 1024):
        out, lse, _ = c4_run(qs, ks, vs, chunk)
        gc.assert_bitwise((out, lse), (full_out, full_lse), f"chunk {chunk} vs full")


# ---------------------------------------------------------------------------
# C5: long-context decode, generate-then-rescore
# ---------------------------------------------------------------------------

def c5_generate_rescore(batch: int, n_final: int, seed: int = 1005, steps: int = 64, oracle_ids=(0,)):
    bs, hq, hk, d = 256, 64, 8, 128
    nb = gen.pool_num_blocks(n_final, bs, batch)
    pool = gc.device_pool(seed, nb, bs, hk, d, "bf16", "interleaved")
    bt = gen.randperm_block_table(nb, batch, generator=torch.Generator().manual_seed(seed)).to(gc.DEV)
    g = torch.Generator(device=gc.DEV).manual_seed(seed + 1)
    q = gen.randn((steps, batch, hq, d), "bf16", generator=g, device=gc.DEV)
    kn = gen.randn((steps, batch, hk, d), "bf16", generator=g, device=gc.DEV)
    vn = gen.randn((steps, batch, hk, d), "bf16", generator=g, device=gc.DEV)
    prefix = n_final - steps
    scale = 1.0 / math.sqrt(d)
    cu1 = torch.arange(batch + 1, dtype=torch.int32, device=gc.DEV)
    dec_out, dec_lse = [], []
    for t in range(steps):
        pos = torch.full((batch,), prefix + t, dtype=torch.int32, device=gc.DEV)
        pkv.cache_write(kn[t].contiguous(), vn[t].contiguous(), pool.k, pool.v, bt, pos, cu1)
        o, l = pkv.attn_forward(q[t].contiguous(), pool.k, pool.v, bt, pos + 1, cu1, True, scale,
                                max_seqlen_q=1, max_seqlen_k=prefix + t + 1, **gc.nan_outputs(q[t]))
        dec_out.append(o)
        dec_lse.append(l)
    torch.cuda.synchronize()
    # one-shot prefill of the last `steps` tokens over the whole context
    qp = q.transpose(0, 1).reshape(batch * steps, hq, d).contiguous()
    case = gc.Case(qp, pool, bt, [n_final] * batch, [steps * b for b in range(batch + 1)], True, scale, "bf16")
    p_out, p_lse = gc.run(case)
    d_out = torch.stack(dec_out, dim=1).reshape(batch * steps, hq, d)
    d_lse = torch.stack(dec_lse, dim=1).reshape(batch * steps, hq)
    gc.assert_bitwise((d_out, d_lse), (p_out, p_lse), "generate (decode) vs re-score (prefill)")
    gc.check_oracle(case, p_out, p_lse, seq_ids=list(oracle_ids))


def test_c5_generate_then_rescore_reduced():
    announce("C5 reduced batch=2 n=8192")
    c5_generate_rescore(2, 8192, oracle_ids=(0, 1))


@pytest.mark.large
def test_c5_generate_then_rescore_full_size():
    announce("C5 full batch=16 n=131072")
    c5_generate_rescore(16, 131072, oracle_ids=(0, 15))
