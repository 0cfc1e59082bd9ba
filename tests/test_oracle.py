"""Pins for the float64 oracle: it is checked against things other than itself.

* a pure-Python ``decimal`` brute force (50 digits) that reads K/V from a
  nested-list copy of the pool through the logical ``[block][slot][head][elem]``
  index, with no max subtraction and explicit visibility sets;
* PyTorch's float64 ``scaled_dot_product_attention`` on a dense cache gathered by
  torch advanced indexing, the recipe of the aiter commit's reference;
* ``torch.logsumexp`` of the masked scores;
* closed forms (q = 0, one visible key, constant V, one-hot V);
* the invariances the pages state: interleaved == contiguous, a permuted block
  table with the data moved to match, decode row == causal prefill row,
  chunked == full prefill, GQA == MHA on repeated K/V;
* ``cache_write`` against a per-element nested-list write.

``test_planted_mistakes_are_caught`` plants plausible mistakes in the oracle
(wrong GQA map, off-by-one causal alignment, contiguous block stride assumed,
dropped softmax scale, log base 2 for the LSE) and checks that the pins fail.
"""

from __future__ import annotations

import decimal
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.paged_kv as oa
import pkv_inputs as gen
from tests.oracle_bridge import oracle_attention, oracle_pool, storage_np


# ----------------------------------------------------------------------------
# small seeded cases
# ----------------------------------------------------------------------------

def tiny_case(seed, dtype="f32", layout="interleaved", batch=2, hq=4, hk=2, d=8,
              bs=4, seqlen_k=11, lens_q=None, seqlens=None):
    g = torch.Generator().manual_seed(seed)
    nb = gen.pool_num_blocks(seqlen_k, bs, batch)
    pool = gen.new_pool(nb, bs, hk, d, dtype, layout, generator=g)
    bt = gen.randperm_block_table(nb, batch, generator=g)
    if seqlens is None:
        seqlens = gen.uniform_int(1, seqlen_k, batch, generator=g)
    if lens_q is None:
        lens_q = [1] * batch
    cu = gen.cu_from_lengths(lens_q)
    q = gen.randn((int(cu[-1]), hq, d), dtype, generator=g)
    return q, pool, bt, list(seqlens), cu


def _to_list(t):
    return t.to(torch.float64).tolist()


def brute_force(q, pool, bt, seqlens, cu, causal, scale):
    """Pure-Python decimal attention straight from the definition."""
    ctx = decimal.Context(prec=50)
    D = decimal.Decimal
    K = _to_list(pool.k)   # logical [block][slot][head][elem]
    V = _to_list(pool.v)
    Q = _to_list(q)
    hq, d = q.shape[1], q.shape[2]
    hk = pool.k.shape[2]
    bs = pool.k.shape[1]
    g = hq // hk
    total = q.shape[0]
    out = [[[0.0] * d for _ in range(hq)] for _ in range(total)]
    lse = [[-math.inf] * hq for _ in range(total)]
    table = bt.tolist()
    for b in range(len(seqlens)):
        n = seqlens[b]
        r0, r1 = int(cu[b]), int(cu[b + 1])
        L = r1 - r0
        for r in range(L):
            pos = n - L + r
            J = [j for j in range(n) if (not causal or j <= pos)]
            for h in range(hq):
                kvh = h // g
                if not J:
                    continue
                es = []
                for j in J:
                    blk, slot = table[b][j // bs], j % bs
                    dot = sum((D(Q[r0 + r][h][e]) * D(K[blk][slot][kvh][e]) for e in range(d)), D(0))
                    es.append(ctx.exp(ctx.multiply(D(scale), dot)))
                z = sum(es, D(0))
                lse[r0 + r][h] = float(ctx.ln(z))
                for e in range(d):
                    acc = D(0)
                    for w, j in zip(es, J):
                        blk, slot = table[b][j // bs], j % bs
                        acc += w * D(V[blk][slot][kvh][e])
                    out[r0 + r][h][e] = float(acc / z)
    return np.array(out), np.array(lse)


def assert_close(a, b, tol, what=""):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    fin = np.isfinite(b)
    assert np.array_equal(np.isfinite(a), fin), f"{what}: finiteness differs"
    assert np.array_equal(a[~fin], b[~fin]), f"{what}: non-finite values differ"
    if fin.any():
        err = np.max(np.abs(a[fin] - b[fin]))
        assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


# ----------------------------------------------------------------------------
# pin checks (each returns normally on success, raises AssertionError on failure)
# ----------------------------------------------------------------------------

BRUTE_CASES = [
    # seed, dtype, layout, hq, hk, d, bs, seqlen_k, lens_q, seqlens, causal
    (1, "f32", "interleaved", 4, 2, 8, 4, 11, [1, 1], None, False),
    (2, "bf16", "contiguous", 4, 2, 8, 4, 11, [3, 3], None, True),
    (3, "f32", "interleaved", 2, 2, 4, 3, 10, [4, 2], [7, 10], True),
    (4, "bf16", "interleaved", 6, 3, 8, 16, 20, [3, 1], [2, 17], True),   # L > n: padded rows
    (5, "f32", "contiguous", 3, 1, 4, 2, 9, [2, 0, 3], [5, 3, 9], False),
    (6, "f32", "interleaved", 2, 1, 4, 4, 8, [2, 1], [0, 5], True),       # n = 0
]


def check_brute_force():
    for seed, dt, lay, hq, hk, d, bs, sk, lq, sl, causal in BRUTE_CASES:
        q, pool, bt, seqlens, cu = tiny_case(seed, dt, lay, len(lq), hq, hk, d, bs, sk, lq, sl)
        scale = 1.0 / math.sqrt(d) if seed % 2 else 0.3
        out, lse = oracle_attention(q, pool, bt, seqlens, cu, causal, scale)
        bout, blse = brute_force(q, pool, bt, seqlens, cu, causal, scale)
        assert_close(out, bout, 1e-12, f"out case {seed}")
        assert_close(lse, blse, 1e-12, f"lse case {seed}")


def dense_reference_torch(q, pool, bt, seqlens, cu, causal, scale):
    """Dense K/V by torch advanced indexing of the paged views, then SDPA in float64."""
    bs = pool.block_size
    hq = q.shape[1]
    hk = pool.k.shape[2]
    g = hq // hk
    outs, lses = [], []
    for b, n in enumerate(seqlens):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        L = r1 - r0
        kd = pool.k[bt[b].long()].reshape(-1, hk, pool.k.shape[3])[:n].to(torch.float64)
        vd = pool.v[bt[b].long()].reshape(-1, hk, pool.v.shape[3])[:n].to(torch.float64)
        kd = kd.repeat_interleave(g, dim=1).transpose(0, 1)   # [hq, n, d]
        vd = vd.repeat_interleave(g, dim=1).transpose(0, 1)
        qq = q[r0:r1].to(torch.float64).transpose(0, 1)        # [hq, L, d]
        pos = torch.arange(L) + (n - L)
        mask = torch.ones(L, n, dtype=torch.bool)
        if causal:
            mask &= torch.arange(n)[None, :] <= pos[:, None]
        o = F.scaled_dot_product_attention(qq, kd, vd, attn_mask=mask, scale=scale)
        s = (qq @ kd.transpose(1, 2)) * scale
        s = s.masked_fill(~mask, -math.inf)
        l = torch.logsumexp(s, dim=-1)
        outs.append(o.transpose(0, 1))
        lses.append(l.transpose(0, 1))
    return torch.cat(outs).numpy(), torch.cat(lses).numpy()


def check_torch_sdpa():
    for seed in (11, 12, 13):
        lq = [1, 5, 2]
        q, pool, bt, seqlens, cu = tiny_case(seed, "bf16" if seed % 2 else "f32",
                                             "interleaved", 3, 8, 2, 16, 8, 40, lq)
        seqlens = [max(s, 5) for s in seqlens]   # rows fully masked are excluded here
        for causal in (False, True):
            out, lse = oracle_attention(q, pool, bt, seqlens, cu, causal, 0.25)
            rout, rlse = dense_reference_torch(q, pool, bt, seqlens, cu, causal, 0.25)
            assert_close(out, rout, 1e-12, "out vs SDPA")
            assert_close(lse, rlse, 1e-12, "lse vs logsumexp")


def check_interleaved_equals_contiguous():
    for seed in (21, 22):
        q, pool, bt, seqlens, cu = tiny_case(seed, "bf16", "interleaved", 2, 4, 2, 8, 4, 13, [2, 1])
        other = gen.relayout(pool, "contiguous")
        a = oracle_attention(q, pool, bt, seqlens, cu, True, 0.5)
        b = oracle_attention(q, other, bt, seqlens, cu, True, 0.5)
        for x, y in zip(a, b):
            assert np.array_equal(x, y), "interleaved != contiguous"


def check_permuted_table():
    q, pool, bt, seqlens, cu = tiny_case(31, "f32", "contiguous", 2, 4, 2, 8, 4, 13, [1, 3])
    perm = torch.randperm(pool.num_blocks, generator=torch.Generator().manual_seed(5))
    inv = torch.argsort(perm)
    moved = gen.PagedKV(pool.k[inv].clone(), pool.v[inv].clone(), "contiguous", [])
    moved.storage = [moved.k, moved.v]
    bt2 = perm[bt.long()].to(torch.int32)   # block x now lives at perm[x]
    a = oracle_attention(q, pool, bt, seqlens, cu, False, 0.5)
    b = oracle_attention(q, moved, bt2, seqlens, cu, False, 0.5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y), "permuted table changed the result"


def check_gqa_equals_repeated_mha():
    q, pool, bt, seqlens, cu = tiny_case(41, "bf16", "interleaved", 2, 6, 2, 8, 4, 13, [2, 3])
    g = 3
    rep = gen.PagedKV(pool.k.repeat_interleave(g, dim=2), pool.v.repeat_interleave(g, dim=2),
                      "contiguous", [])
    rep.storage = [rep.k.contiguous(), rep.v.contiguous()]
    rep.k, rep.v = rep.storage
    a = oracle_attention(q, pool, bt, seqlens, cu, True, 0.5)
    b = oracle_attention(q, rep, bt, seqlens, cu, True, 0.5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y), "GQA != MHA on repeated K/V"


def check_decode_equals_prefill():
    """One decode query over n keys equals row n-1 of an n-row causal prefill.

    The oracle batches rows through BLAS, whose summation order depends on the
    matrix shapes, so equality here is to float64 rounding (1e-13), not bitwise.
    """
    g = torch.Generator().manual_seed(51)
    n, hq, hk, d, bs = 37, 4, 2, 8, 8
    nb = gen.pool_num_blocks(n, bs, 1)
    pool = gen.new_pool(nb, bs, hk, d, "f32", "interleaved", generator=g)
    bt = gen.randperm_block_table(nb, 1, generator=g)
    qall = gen.randn((n, hq, d), "f32", generator=g)
    full = oracle_attention(qall, pool, bt, [n], [0, n], True, 0.3)
    for t in (0, 1, 15, n - 1):
        for causal in (False, True):
            dec = oracle_attention(qall[t:t + 1], pool, bt, [t + 1], [0, 1], causal, 0.3)
            assert_close(dec[0][0], full[0][t], 1e-13, "decode out vs prefill row")
            assert_close(dec[1][0], full[1][t], 1e-13, "decode lse vs prefill row")
    # chunked prefill: rows [a, b) against n = b keys equal the full prefill rows
    for a, b in ((0, 17), (17, 34), (34, 37)):
        ch = oracle_attention(qall[a:b], pool, bt, [b], [0, b - a], True, 0.3)
        assert_close(ch[0], full[0][a:b], 1e-13, "chunked out vs full")
        assert_close(ch[1], full[1][a:b], 1e-13, "chunked lse vs full")


def check_closed_forms():
    g = torch.Generator().manual_seed(61)
    n, hq, hk, d, bs = 9, 2, 1, 16, 4
    nb = gen.pool_num_blocks(n, bs, 1)
    pool = gen.new_pool(nb, bs, hk, d, "f32", "contiguous", generator=g)
    bt = gen.randperm_block_table(nb, 1, generator=g)
    # q = 0: uniform weights over the visible keys
    q0 = torch.zeros((3, hq, d))
    out, lse = oracle_attention(q0, pool, bt, [n], [0, 3], True, 0.7)
    kd = pool.v[bt[0].long()].reshape(-1, hk, d)[:n].to(torch.float64).numpy()
    for r in range(3):
        cnt = n - 3 + r + 1
        assert abs(lse[r, 0] - math.log(cnt)) <= 1e-15 * 4
        assert np.max(np.abs(out[r, 0] - kd[:cnt, 0].mean(axis=0))) <= 1e-15 * 8
    # one visible key: out = v_0, lse = s_0
    q1 = gen.randn((1, hq, d), "f32", generator=g)
    out, lse = oracle_attention(q1, pool, bt, [1], [0, 1], True, 0.7)
    k0 = pool.k[bt[0, 0].long(), 0, 0].to(torch.float64).numpy()
    assert np.array_equal(out[0, 0], pool.v[bt[0, 0].long(), 0, 0].to(torch.float64).numpy())
    assert abs(lse[0, 0] - 0.7 * float(q1[0, 0].double() @ torch.from_numpy(k0))) <= 1e-15
    # constant V: out = that constant
    cpool = gen.PagedKV(pool.k, torch.full_like(pool.v, 1.25), "contiguous", [])
    cpool.storage = [cpool.k, cpool.v]
    qq = gen.randn((2, hq, d), "f32", generator=g)
    out, _ = oracle_attention(qq, cpool, bt, [n], [0, 2], False, 0.7)
    assert np.max(np.abs(out - 1.25)) <= 1e-15 * 4
    # one-hot V rows (v_j = e_j): out is the weight vector; it sums to 1, is >= 0
    vh = torch.zeros_like(pool.v)
    flat = vh.view(-1, bs, hk, d)
    for j in range(n):
        flat[bt[0, j // bs].long(), j % bs, 0, j] = 1.0
    hpool = gen.PagedKV(pool.k, vh, "contiguous", [pool.k, vh])
    out, lse = oracle_attention(qq, hpool, bt, [n], [0, 2], True, 0.7)
    w = out[:, 0, :]
    assert np.all(w >= 0)
    assert np.max(np.abs(w.sum(axis=1) - 1.0)) <= 1e-12
    assert np.all(w[0, n - 1:] == 0)          # row 0 sits at n-2: key n-1 invisible
    # w_j = exp(s_j - lse): softmax definition for each visible key
    kd = pool.k[bt[0].long()].reshape(-1, hk, d)[:n, 0].to(torch.float64).numpy()
    s = 0.7 * (qq[:, 0].double().numpy() @ kd.T)
    assert np.max(np.abs(w[1, :n] - np.exp(s[1] - lse[1, 0]))) <= 1e-12


def check_fully_masked_rows():
    q, pool, bt, seqlens, cu = tiny_case(71, "bf16", "interleaved", 2, 2, 1, 8, 4, 9, [3, 2], [1, 0])
    out, lse = oracle_attention(q, pool, bt, seqlens, cu, True, 0.5)
    # seq 0: n=1, L=3 -> rows at positions -2, -1 see nothing, row at 0 sees key 0
    assert np.all(lse[0:2] == -np.inf) and np.all(out[0:2] == 0)
    assert np.all(np.isfinite(lse[2]))
    # seq 1: n=0 -> nothing visible, causal or not
    assert np.all(lse[3:5] == -np.inf) and np.all(out[3:5] == 0)
    out2, lse2 = oracle_attention(q, pool, bt, seqlens, cu, False, 0.5)
    assert np.all(lse2[3:5] == -np.inf) and np.all(out2[3:5] == 0)
    assert np.all(np.isfinite(lse2[0:3]))        # non-causal: all 3 rows see key 0


PINS = [check_brute_force, check_torch_sdpa, check_interleaved_equals_contiguous,
        check_permuted_table, check_gqa_equals_repeated_mha, check_decode_equals_prefill,
        check_closed_forms, check_fully_masked_rows]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin()


# ----------------------------------------------------------------------------
# gather and cache write
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("layout", ["contiguous", "interleaved"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gather_matches_advanced_indexing(layout, dtype):
    """The flat-index gather equals the aiter recipe (pool[table.flatten()] cut to n), bit for bit."""
    q, pool, bt, seqlens, cu = tiny_case(81, dtype, layout, 3, 4, 2, 8, 5, 23, [1, 1, 1])
    kf, vf, lay = oracle_pool(pool, 4)
    for b, n in enumerate(seqlens):
        for flat, off, st, view in ((kf, lay.k_offset, lay.k_strides, pool.k),
                                    (vf, lay.v_offset, lay.v_strides, pool.v)):
            got = oracle.gather_sequence(flat, dtype, off, st, bt[b].numpy(), n, 5, 2, 8)
            ref = view[bt[b].long()].reshape(-1, 2, 8)[:n].to(torch.float64).numpy()
            assert np.array_equal(got, ref)


def test_gather_reads_only_visible_slots():
    """NaN in every slot no sequence may read leaves the result unchanged."""
    q, pool, bt, seqlens, cu = tiny_case(82, "bf16", "interleaved", 3, 4, 2, 8, 4, 21, [2, 1, 3])
    a = oracle_attention(q, pool, bt, seqlens, cu, True, 0.5)
    gen.poison_unused(pool, bt, seqlens)
    bt2 = gen.poison_table_tail(bt, seqlens, pool.block_size, -1)
    b = oracle_attention(q, pool, bt2, seqlens, cu, True, 0.5)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def _nested_write(pool, bt, seqlens, cu, kn, vn):
    """Per-element write through the logical [block][slot][head][elem] view."""
    k = pool.k.clone()
    v = pool.v.clone()
    bs = pool.block_size
    for b in range(len(seqlens)):
        for t in range(int(cu[b + 1] - cu[b])):
            pos = seqlens[b] + t
            blk, slot = int(bt[b, pos // bs]), pos % bs
            for h in range(k.shape[2]):
                for e in range(k.shape[3]):
                    k[blk, slot, h, e] = kn[int(cu[b]) + t, h, e]
                    v[blk, slot, h, e] = vn[int(cu[b]) + t, h, e]
    return k, v


@pytest.mark.parametrize("layout", ["contiguous", "interleaved"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_cache_write_oracle(layout, dtype):
    g = torch.Generator().manual_seed(91)
    q, pool, bt, _, _ = tiny_case(91, dtype, layout, 2, 4, 2, 8, 4, 15, [1, 1])
    seqlens = [3, 0]
    lens_new = [5, 4]
    cu = gen.cu_from_lengths(lens_new)
    kn = gen.randn((9, 2, 8), dtype, generator=g)
    vn = gen.randn((9, 2, 8), dtype, generator=g)
    kf, vf, lay = oracle_pool(pool, 4)
    k2, v2 = oracle.cache_write(kf, vf, lay, storage_np(kn), storage_np(vn), bt.numpy(),
                                seqlens, cu.tolist())
    ek, ev = _nested_write(pool, bt, seqlens, cu, kn, vn)
    want = gen.PagedKV(ek, ev, "contiguous", [ek, ev])
    wk, wv, wlay = oracle_pool(gen.relayout(want, layout), 4)
    assert np.array_equal(k2, wk) and np.array_equal(v2, wv)
    # writing in pieces equals writing at once
    kf_a, vf_a = kf, vf
    kf_b, vf_b = oracle.cache_write(kf, vf, lay, storage_np(kn[[0, 1, 5]]), storage_np(vn[[0, 1, 5]]),
                                    bt.numpy(), seqlens, [0, 2, 3])
    kf_b, vf_b = oracle.cache_write(kf_b, vf_b, lay, storage_np(kn[[2, 3, 4, 6, 7, 8]]),
                                    storage_np(vn[[2, 3, 4, 6, 7, 8]]), bt.numpy(),
                                    [5, 1], [0, 3, 6])
    assert np.array_equal(kf_b, k2) and np.array_equal(vf_b, v2)
    assert kf_a is kf  # inputs are not modified in place


# ----------------------------------------------------------------------------
# planted mistakes must be caught
# ----------------------------------------------------------------------------

def _wrong_gqa(h, hq, hk):
    return h % hk


def _off_by_one_rows(n, L):
    return n - L + 1 + np.arange(L, dtype=np.int64)


_ORIG_GATHER = oa.gather_sequence
_ORIG_SOFTMAX = oa.masked_softmax


def _assume_contiguous_block_stride(flat, dtype, offset, strides, row, n, bs, hk, d):
    """The aiter pre-fix bug: block stride taken as block_size * slot_stride."""
    return _ORIG_GATHER(flat, dtype, offset, (bs * strides[1], strides[1], strides[2]),
                        row, n, bs, hk, d)


def _no_scale(q_rows, k_rows, softmax_scale):
    return q_rows @ k_rows.T


def _log2_lse(s, vis):
    w, lse = _ORIG_SOFTMAX(s, vis)
    return w, lse / math.log(2.0)


MISTAKES = {
    "gqa_modulo": ("kv_head_of", _wrong_gqa),
    "causal_off_by_one": ("row_positions", _off_by_one_rows),
    "block_stride_contiguous": ("gather_sequence", _assume_contiguous_block_stride),
    "scale_dropped": ("scores", _no_scale),
    "lse_log2": ("masked_softmax", _log2_lse),
}


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_mistakes_are_caught(name, monkeypatch):
    attr, fn = MISTAKES[name]
    monkeypatch.setattr(oa, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, IndexError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"


# ----------------------------------------------------------------------------
# per-chunk attention (the context-parallel partials)
# ----------------------------------------------------------------------------

def _chunks(q, pool, bt, seqlens, cu, causal, scale, ck, nc, k_scale=1.0, v_scale=1.0):
    from tests.oracle_bridge import oracle_pool
    kf, vf, lay = oracle_pool(pool, q.shape[1], k_scale, v_scale)
    return oracle.attention_chunks(storage_np(q).reshape(q.shape), kf, vf, lay, np.asarray(bt),
                                   list(seqlens), [int(x) for x in cu], causal, scale, ck, nc)


@pytest.mark.parametrize("causal", [False, True])
def test_chunk_attention_recombines_to_full(causal):
    """log-sum-exp over chunks is the full LSE and the LSE-weighted chunk outputs are the full output."""
    for seed, dt in ((91, "f32"), (92, "bf16")):
        q, pool, bt, seqlens, cu = tiny_case(seed, dt, "interleaved", 3, 4, 2, 8, 4, 37, [1, 4, 2])
        out, lse = oracle_attention(q, pool, bt, seqlens, cu, causal, 0.4)
        for ck in (4, 7, 16):
            nc = -(-max(seqlens) // ck)
            oc, lc = _chunks(q, pool, bt, seqlens, cu, causal, 0.4, ck, nc)
            m = np.max(lc, axis=2, initial=-np.inf)
            fin = np.isfinite(m)
            tot = np.where(fin, m + np.log(np.sum(np.exp(lc - np.where(fin, m, 0)[..., None]), axis=2)), -np.inf)
            assert_close(tot, lse, 1e-12, "recombined lse")
            wts = np.where(np.isfinite(lc), np.exp(lc - np.where(np.isfinite(tot), tot, 0)[..., None]), 0.0)
            assert_close(np.sum(wts[..., None] * oc, axis=2), out, 1e-12, "recombined out")
            # chunks that start past a row's last visible key are empty
            for b, n in enumerate(seqlens):
                r0, r1 = int(cu[b]), int(cu[b + 1])
                for r in range(r1 - r0):
                    lim = min(n - (r1 - r0) + r + 1, n) if causal else n
                    for c in range(nc):
                        if c * ck >= lim:
                            assert np.all(lc[r0 + r, :, c] == -np.inf) and np.all(oc[r0 + r, :, c] == 0)


def test_one_chunk_is_full_attention():
    q, pool, bt, seqlens, cu = tiny_case(93, "f32", "contiguous", 2, 4, 2, 8, 4, 20, [3, 1])
    out, lse = oracle_attention(q, pool, bt, seqlens, cu, True, 0.5)
    oc, lc = _chunks(q, pool, bt, seqlens, cu, True, 0.5, 512, 1)
    assert np.array_equal(oc[:, :, 0], out) and np.array_equal(lc[:, :, 0], lse)


def test_chunk_attention_brute_force():
    """Each chunk against the decimal brute force run on the chunk's keys alone (a sequence
    whose keys are that chunk's: the chunk's keys moved to positions 0.. of a fresh cache)."""
    q, pool, bt, seqlens, cu = tiny_case(94, "f32", "interleaved", 1, 2, 1, 8, 4, 12, [1], [12])
    ck = 5
    oc, lc = _chunks(q, pool, bt, seqlens, cu, False, 0.5, ck, 3)
    kd = pool.k[bt[0].long()].reshape(-1, 1, 8)[:12]
    vd = pool.v[bt[0].long()].reshape(-1, 1, 8)[:12]
    for c in range(3):
        keys = list(range(c * ck, min((c + 1) * ck, 12)))
        sub = gen.PagedKV(kd[keys].reshape(-1, 1, 1, 8).contiguous(), vd[keys].reshape(-1, 1, 1, 8).contiguous(),
                          "contiguous", [])
        sub.storage = [sub.k, sub.v]
        sbt = torch.arange(len(keys), dtype=torch.int32)[None, :]
        bo, bl = brute_force(q, sub, sbt, [len(keys)], cu, False, 0.5)
        assert_close(oc[:, :, c], bo, 1e-12, f"chunk {c} out")
        assert_close(lc[:, :, c], bl, 1e-12, f"chunk {c} lse")
