"""Pins for the float64 backward oracle (``oracle.attention_backward``).

It is checked against things other than itself:

* PyTorch's float64 autograd through ``scaled_dot_product_attention`` on a
  dense cache gathered by torch advanced indexing (the GQA repeat done by
  ``repeat_interleave``, so autograd itself sums the heads of a group);
* central finite differences of the pinned forward oracle, in float64, along
  random directions of q, of the K storage and of the V storage;
* the identities of the softmax gradient: the weights of a row sum to one, so
  the keys' gradients of a sequence and KV head sum to zero and the values'
  gradients sum to the rows' output cotangents; a single visible key passes
  all of dout to that value and nothing to q or k; q = 0 gives dk = 0;
* the pages' invariances: GQA equals MHA on repeated K/V (summed over the
  group), a decode row's dq equals the same row's dq in a causal prefill,
  interleaved equals contiguous, fully masked rows have zero gradients;
* the error bound: every gradient's magnitude is at most its term bound, and
  the term bound equals the sum of the absolute values of the monomials of
  the chain-rule expansion, enumerated one by one in 40-digit decimal
  arithmetic (so an inflated bound fails as well as a deflated one).

``test_planted_backward_mistakes_are_caught`` plants plausible mistakes in
the oracle (the row term dropped, the scale dropped from dq, P used where dS
belongs, dS used where P belongs, the GQA map taken modulo; and in the term
bound: the scale dropped, the row-term bound F counted twice, a stray factor
of the group size) and checks that the pins fail.
"""

from __future__ import annotations

import decimal
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import oracle.backward as ob
import pkv_inputs as gen
from tests.oracle_bridge import oracle_attention, oracle_backward, oracle_pool, storage_np


def case(seed, dtype="f32", layout="interleaved", batch=2, hq=4, hk=2, d=8, bs=4,
         seqlen_k=13, lens_q=(2, 3), seqlens=None):
    g = torch.Generator().manual_seed(seed)
    nb = gen.pool_num_blocks(seqlen_k, bs, batch)
    pool = gen.new_pool(nb, bs, hk, d, dtype, layout, generator=g)
    bt = gen.randperm_block_table(nb, batch, generator=g)
    if seqlens is None:
        seqlens = [max(x, max(lens_q)) for x in gen.uniform_int(1, seqlen_k, batch, generator=g)]
    cu = gen.cu_from_lengths(list(lens_q))
    q = gen.randn((int(cu[-1]), hq, d), dtype, generator=g)
    dout = gen.randn((int(cu[-1]), hq, d), dtype, generator=g)
    return q, pool, bt, list(seqlens), cu, dout


def close(a, b, rel, what):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    scale = max(1.0, float(np.max(np.abs(b))) if b.size else 1.0)
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= rel * scale, f"{what}: max err {err:.3e} > {rel:.1e} * {scale:.3e}"


# ----------------------------------------------------------------------------
# pins
# ----------------------------------------------------------------------------

def torch_autograd(q, pool, bt, seqlens, cu, causal, scale, dout):
    """Gradients by torch float64 autograd through SDPA on a dense gathered cache."""
    bs = pool.block_size
    hq, d = q.shape[1], q.shape[2]
    hk = pool.k.shape[2]
    g = hq // hk
    dq = torch.zeros(q.shape, dtype=torch.float64)
    dks, dvs = [], []
    for b, n in enumerate(seqlens):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        L = r1 - r0
        kd = pool.k[bt[b].long()].reshape(-1, hk, d)[:n].to(torch.float64).requires_grad_(True)
        vd = pool.v[bt[b].long()].reshape(-1, hk, d)[:n].to(torch.float64).requires_grad_(True)
        qq = q[r0:r1].to(torch.float64).requires_grad_(True)
        if L == 0 or n == 0:
            dks.append(torch.zeros(n, hk, d, dtype=torch.float64))
            dvs.append(torch.zeros(n, hk, d, dtype=torch.float64))
            continue
        pos = torch.arange(L) + (n - L)
        mask = torch.ones(L, n, dtype=torch.bool)
        if causal:
            mask &= torch.arange(n)[None, :] <= pos[:, None]
        o = F.scaled_dot_product_attention(qq.transpose(0, 1),
                                           kd.repeat_interleave(g, dim=1).transpose(0, 1),
                                           vd.repeat_interleave(g, dim=1).transpose(0, 1),
                                           attn_mask=mask, scale=scale)
        o.transpose(0, 1).backward(dout[r0:r1].to(torch.float64))
        dq[r0:r1] = qq.grad
        dks.append(kd.grad)
        dvs.append(vd.grad)
    return dq.numpy(), torch.cat(dks).numpy(), torch.cat(dvs).numpy()


def check_torch_autograd():
    for seed, dt, lay, hq, hk in ((101, "f32", "interleaved", 4, 2), (102, "bf16", "contiguous", 6, 3),
                                  (103, "bf16", "interleaved", 4, 4), (104, "f32", "contiguous", 8, 2)):
        q, pool, bt, seqlens, cu, dout = case(seed, dt, lay, 3, hq, hk, 16, 8, 40, (1, 6, 3))
        for causal in (False, True):
            got = oracle_backward(q, pool, bt, seqlens, cu, causal, 0.25, dout)
            ref = torch_autograd(q, pool, bt, seqlens, cu, causal, 0.25, dout)
            for name, a, b in zip(("dq", "dk", "dv"), got, ref):
                close(a, b, 1e-12, f"{name} vs autograd (seed {seed}, causal {causal})")


def _f64_inputs(seed, hq=4, hk=2, d=4, bs=4, seqlens=(7, 5), lens=(3, 2)):
    """A case in exact float64 storage (flat arrays + oracle Layout)."""
    rng = np.random.default_rng(seed)
    batch = len(seqlens)
    nb = gen.pool_num_blocks(max(seqlens), bs, batch)
    row = hk * d
    lay = oracle.Layout("f64", hq, hk, d, bs, 0, (2 * bs * row, row, d), bs * row, (2 * bs * row, row, d))
    flat = rng.standard_normal(nb * 2 * bs * row)
    bt = rng.permutation(nb).reshape(batch, -1)
    cu = np.concatenate([[0], np.cumsum(lens)])
    q = rng.standard_normal((int(cu[-1]), hq, d))
    dout = rng.standard_normal(q.shape)
    return q, flat, lay, bt, list(seqlens), cu, dout


def check_finite_differences():
    """Directional derivatives of sum(dout * out) by central differences."""
    for seed, causal in ((111, True), (112, False), (113, True)):
        q, flat, lay, bt, seqlens, cu, dout = _f64_inputs(seed)
        scale = 0.6
        dq, dk, dv = oracle.attention_backward(q, flat, flat, lay, bt, seqlens, cu, causal, scale, dout)
        rng = np.random.default_rng(seed + 1000)

        def phi(qq, ff):
            out, _ = oracle.attention(qq, ff, ff, lay, bt, seqlens, cu, causal, scale)
            return float(np.sum(out * dout))

        eps = 1e-6
        # along q
        dirq = rng.standard_normal(q.shape)
        fd = (phi(q + eps * dirq, flat) - phi(q - eps * dirq, flat)) / (2 * eps)
        assert abs(fd - float(np.sum(dq * dirq))) <= 1e-7 * max(1.0, abs(fd)), ("q", fd, np.sum(dq * dirq))
        # along K storage and V storage (a direction on the whole flat array;
        # the gathered slots of every sequence carry it into K or V)
        cuk = oracle.cu_seqlens_k_of(seqlens)
        for which, grad in (("k", dk), ("v", dv)):
            dirf = np.zeros_like(flat)
            off, st = (lay.k_offset, lay.k_strides) if which == "k" else (lay.v_offset, lay.v_strides)
            proj = 0.0
            for b, n in enumerate(seqlens):
                dirs = rng.standard_normal((n, lay.num_heads_k, lay.head_dim))
                j = np.arange(n)
                idx = oracle.paged_kv.flat_index(off, st, bt[b][j // lay.block_size][:, None, None],
                                                 (j % lay.block_size)[:, None, None],
                                                 np.arange(lay.num_heads_k)[None, :, None],
                                                 np.arange(lay.head_dim)[None, None, :])
                dirf[idx] = dirs
                proj += float(np.sum(grad[cuk[b]:cuk[b] + n] * dirs))
            fd = (phi(q, flat + eps * dirf) - phi(q, flat - eps * dirf)) / (2 * eps)
            assert abs(fd - proj) <= 1e-7 * max(1.0, abs(fd)), (which, fd, proj)


def check_softmax_identities():
    for seed, causal in ((121, True), (122, False)):
        q, pool, bt, seqlens, cu, dout = case(seed, "f32", "interleaved", 3, 6, 2, 8, 4, 30, (4, 1, 5))
        dq, dk, dv = oracle_backward(q, pool, bt, seqlens, cu, causal, 0.4, dout)
        cuk = oracle.cu_seqlens_k_of(seqlens)
        g = 3
        do = dout.to(torch.float64).numpy()
        for b in range(3):
            k0, k1 = cuk[b], cuk[b + 1]
            r0, r1 = int(cu[b]), int(cu[b + 1])
            # every row sees at least one key here (seqlens >= rows)
            assert np.max(np.abs(dk[k0:k1].sum(axis=0))) <= 1e-12 * max(1.0, np.max(np.abs(dk[k0:k1])))
            for hk in range(2):
                want = do[r0:r1, hk * g:(hk + 1) * g].sum(axis=(0, 1))
                assert np.max(np.abs(dv[k0:k1, hk].sum(axis=0) - want)) <= 1e-12 * max(1.0, np.max(np.abs(want)))


def check_closed_forms():
    # a single visible key: P = 1, so dS = 0 -> dq = 0, dk = 0, dv = dout summed over rows and the group's heads
    q, pool, bt, _, cu, dout = case(131, "f32", "contiguous", 1, 4, 2, 8, 4, 8, (1,), seqlens=[1])
    dq, dk, dv = oracle_backward(q, pool, bt, [1], cu, True, 0.5, dout)
    assert np.max(np.abs(dq)) <= 1e-15 and np.max(np.abs(dk)) <= 1e-15
    do = dout.to(torch.float64).numpy()
    assert np.max(np.abs(dv[0] - do[0].reshape(2, 2, 8).sum(axis=1))) <= 1e-15
    # q = 0: every key of a row weighs the same and dk = scale * sum_i dS_ij q_i = 0
    q, pool, bt, seqlens, cu, dout = case(132, "f32", "contiguous", 2, 4, 2, 8, 4, 12, (3, 2))
    q0 = torch.zeros_like(q)
    dq, dk, dv = oracle_backward(q0, pool, bt, seqlens, cu, False, 0.5, dout)
    assert np.max(np.abs(dk)) <= 1e-15
    # uniform weights: dv_j = sum over rows and heads of dout / n (non-causal)
    cuk = oracle.cu_seqlens_k_of(seqlens)
    do = dout.to(torch.float64).numpy()
    for b, n in enumerate(seqlens):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        want = do[r0:r1].reshape(r1 - r0, 2, 2, 8).sum(axis=(0, 2)) / n
        got = dv[cuk[b]:cuk[b + 1]]
        assert np.max(np.abs(got - want[None])) <= 1e-14


def check_gqa_equals_repeated_mha():
    q, pool, bt, seqlens, cu, dout = case(141, "bf16", "interleaved", 2, 6, 2, 8, 4, 13, (2, 3))
    g = 3
    rep = gen.PagedKV(pool.k.repeat_interleave(g, dim=2).contiguous(),
                      pool.v.repeat_interleave(g, dim=2).contiguous(), "contiguous", [])
    rep.storage = [rep.k, rep.v]
    a = oracle_backward(q, pool, bt, seqlens, cu, True, 0.5, dout)
    b = oracle_backward(q, rep, bt, seqlens, cu, True, 0.5, dout)
    assert np.array_equal(a[0], b[0]), "dq: GQA != MHA"
    for i in (1, 2):
        summed = b[i].reshape(b[i].shape[0], 2, g, -1).sum(axis=2)
        close(a[i], summed, 1e-14, "dk/dv: GQA != MHA summed over the group")


def check_decode_row_dq_equals_prefill_row():
    g = torch.Generator().manual_seed(151)
    n, hq, hk, d, bs = 21, 4, 2, 8, 4
    nb = gen.pool_num_blocks(n, bs, 1)
    pool = gen.new_pool(nb, bs, hk, d, "f32", "interleaved", generator=g)
    bt = gen.randperm_block_table(nb, 1, generator=g)
    qall = gen.randn((n, hq, d), "f32", generator=g)
    dall = gen.randn((n, hq, d), "f32", generator=g)
    full = oracle_backward(qall, pool, bt, [n], [0, n], True, 0.3, dall)
    for t in (0, 7, n - 1):
        dec = oracle_backward(qall[t:t + 1], pool, bt, [t + 1], [0, 1], True, 0.3, dall[t:t + 1])
        close(dec[0][0], full[0][t], 1e-13, "decode dq vs prefill row dq")
    # the last row alone: its dk/dv equal the full prefill's only when the other rows add nothing,
    # so compare the sum over row chunks instead: dk of rows [a,b) over n keys add up to the full dk
    parts = [oracle_backward(qall[a:b], pool, bt, [b], [0, b - a], True, 0.3, dall[a:b]) for a, b in ((0, 8), (8, 21))]
    dk = np.zeros_like(full[1])
    dv = np.zeros_like(full[2])
    for (a, b), p in zip(((0, 8), (8, 21)), parts):
        dk[:b] += p[1]
        dv[:b] += p[2]
    close(dk, full[1], 1e-13, "chunked dk sum")
    close(dv, full[2], 1e-13, "chunked dv sum")


def check_layout_and_masking():
    q, pool, bt, _, cu, dout = case(161, "bf16", "interleaved", 2, 2, 1, 8, 4, 9, (3, 2), seqlens=[1, 0])
    a = oracle_backward(q, pool, bt, [1, 0], cu, True, 0.5, dout)
    b = oracle_backward(q, gen.relayout(pool, "contiguous"), bt, [1, 0], cu, True, 0.5, dout)
    for x, y in zip(a, b):
        assert np.array_equal(x, y), "interleaved != contiguous"
    dq, dk, dv = a
    # seq 0: n=1, L=3 -> rows at positions -2, -1 see nothing; seq 1: n=0 -> nothing at all
    assert np.all(dq[0:2] == 0) and np.all(dq[3:5] == 0)
    assert dk.shape[0] == 1 and np.all(dk == 0)    # one visible key: dS = 0
    do = dout.to(torch.float64).numpy()
    assert np.max(np.abs(dv[0, 0] - do[2].sum(axis=0))) <= 1e-15


def check_bound():
    for seed, dt in ((171, "f32"), (172, "bf16")):
        q, pool, bt, seqlens, cu, dout = case(seed, dt, "interleaved", 3, 6, 2, 16, 4, 30, (4, 1, 5))
        for causal in (False, True):
            ref = oracle_backward(q, pool, bt, seqlens, cu, causal, 0.4, dout)
            bnd = oracle_backward(q, pool, bt, seqlens, cu, causal, 0.4, dout, bound=True)
            for r, a in zip(ref, bnd):
                assert np.all(np.abs(r) <= a * (1 + 1e-12) + 1e-300)


def _nested(t):
    return t.to(torch.float64).tolist()


def brute_force_bound(q, pool, bt, seqlens, cu, causal, scale, dout):
    """Term bounds by enumeration, in 40-digit decimal arithmetic.

    Expanding the chain rule down to the softmax weights P, every gradient
    element is a sum of monomials:

        dq[i, h, e]  =  scale * sum_j sum_f P_ij dO_if V_jf K_je
                      - scale * sum_j sum_k sum_f P_ij P_ik dO_if V_kf K_je
        dk[j, hk, e] =  scale * sum_(h, i) sum_f P_ij dO_if V_jf Q_ie
                      - scale * sum_(h, i) sum_k sum_f P_ij P_ik dO_if V_kf Q_ie
        dv[j, hk, e] =  sum_(h, i) P_ij dO_ie

    (h runs over the query heads of KV head hk).  The bound of an element is
    the sum of the absolute values of its monomials, enumerated one by one
    here.  P is computed from its definition (exp of the scaled score over the
    sum of exps of the row's visible keys, no max subtraction); K/V are read
    from a nested-list copy of the pool through the block table.
    """
    ctx = decimal.Context(prec=40)
    D = decimal.Decimal
    Kp, Vp, Q, dO = _nested(pool.k), _nested(pool.v), _nested(q), _nested(dout)
    hq, d = q.shape[1], q.shape[2]
    hk_n, bs = pool.k.shape[2], pool.k.shape[1]
    g = hq // hk_n
    table = bt.tolist()
    cuk = [0]
    for n in seqlens:
        cuk.append(cuk[-1] + n)
    aq = [[[D(0)] * d for _ in range(hq)] for _ in range(q.shape[0])]
    ak = [[[D(0)] * d for _ in range(hk_n)] for _ in range(cuk[-1])]
    av = [[[D(0)] * d for _ in range(hk_n)] for _ in range(cuk[-1])]
    sc = abs(D(scale))
    for b, n in enumerate(seqlens):
        r0, r1 = int(cu[b]), int(cu[b + 1])
        L = r1 - r0

        def kv(tab, j, hk, e):
            return D(tab[table[b][j // bs]][j % bs][hk][e])

        for r in range(L):
            i = r0 + r
            J = [j for j in range(n) if not causal or j <= n - L + r]
            if not J:
                continue
            for h in range(hq):
                hk = h // g
                ex = {j: ctx.exp(D(scale) * sum((D(Q[i][h][e]) * kv(Kp, j, hk, e) for e in range(d)), D(0)))
                      for j in J}
                z = sum(ex.values(), D(0))
                P = {j: ex[j] / z for j in J}
                for e in range(d):
                    tq = D(0)
                    for j in J:
                        for f in range(d):
                            tq += abs(P[j] * D(dO[i][h][f]) * kv(Vp, j, hk, f) * kv(Kp, j, hk, e))
                            for k in J:
                                tq += abs(P[j] * P[k] * D(dO[i][h][f]) * kv(Vp, k, hk, f) * kv(Kp, j, hk, e))
                    aq[i][h][e] += sc * tq
                    for j in J:
                        tk = D(0)
                        for f in range(d):
                            tk += abs(P[j] * D(dO[i][h][f]) * kv(Vp, j, hk, f) * D(Q[i][h][e]))
                            for k in J:
                                tk += abs(P[j] * P[k] * D(dO[i][h][f]) * kv(Vp, k, hk, f) * D(Q[i][h][e]))
                        ak[cuk[b] + j][hk][e] += sc * tk
                        av[cuk[b] + j][hk][e] += abs(P[j] * D(dO[i][h][e]))
    to = lambda x: np.array([[[float(v) for v in row] for row in m] for m in x]).reshape(len(x), -1, d)
    return to(aq), to(ak), to(av)


def check_bound_brute_force():
    """The oracle's term bound equals the enumerated sum of |monomials| (two-sided pin)."""
    for seed, dt, hq, hk, lens, sl, causal, scale in ((181, "f32", 4, 2, (2, 3), [5, 6], True, 0.4),
                                                      (182, "bf16", 4, 1, (3, 1), [4, 6], False, 0.7),
                                                      (183, "f32", 2, 2, (3, 2), [2, 5], True, 1.3)):
        q, pool, bt, seqlens, cu, dout = case(seed, dt, "interleaved", 2, hq, hk, 3, 2, 6, lens, seqlens=sl)
        got = oracle_backward(q, pool, bt, seqlens, cu, causal, scale, dout, bound=True)
        want = brute_force_bound(q, pool, bt, seqlens, cu, causal, scale, dout)
        for name, a, w in zip(("Aq", "Ak", "Av"), got, want):
            assert a.shape == w.shape, (name, a.shape, w.shape)
            err = float(np.max(np.abs(a - w) / np.maximum(np.abs(w), 1e-300)))
            assert err <= 1e-12, f"{name} bound vs enumerated monomials (seed {seed}): rel err {err:.3e}"


PINS = [check_torch_autograd, check_finite_differences, check_softmax_identities, check_closed_forms,
        check_gqa_equals_repeated_mha, check_decode_row_dq_equals_prefill_row, check_layout_and_masking,
        check_bound, check_bound_brute_force]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_backward_oracle_pin(pin):
    pin()


# ----------------------------------------------------------------------------
# planted mistakes: each must make at least one pin fail
# ----------------------------------------------------------------------------

def _grads_with(mistake):
    def head_gradients(Q, K, V, dO, vis, softmax_scale):
        P, _ = oracle.masked_softmax(oracle.scores(Q, K, softmax_scale), vis)
        dP = dO @ V.T
        row = np.sum(P * dP, axis=1)
        dS = P * (dP - row[:, None])
        if mistake == "no_row_term":
            dS = P * dP
        dq = softmax_scale * (dS @ K)
        if mistake == "dq_no_scale":
            dq = dS @ K
        dk = softmax_scale * (dS.T @ Q)
        if mistake == "dk_uses_P":
            dk = softmax_scale * (P.T @ Q)
        dv = P.T @ dO
        if mistake == "dv_uses_dS":
            dv = dS.T @ dO
        return dq, dk, dv
    return head_gradients


def _bound_with(mistake):
    """Inflated term bounds: the scale dropped, F counted twice, a stray factor g."""
    def head_bound(Q, K, V, dO, vis, softmax_scale):
        P, _ = oracle.masked_softmax(oracle.scores(Q, K, softmax_scale), vis)
        G = np.abs(dO) @ np.abs(V).T
        F = np.sum(P * G, axis=1)
        W = P * (G + (2 if mistake == "F_twice" else 1) * F[:, None])
        s = 1.0 if mistake == "no_scale" else abs(softmax_scale)
        return s * (W @ np.abs(K)), s * (W.T @ np.abs(Q)), P.T @ np.abs(dO)

    if mistake != "extra_g":
        return head_bound
    real = ob.attention_backward_bound

    def attention_backward_bound(q, k_flat, v_flat, layout, *args):
        aq, ak, av = real(q, k_flat, v_flat, layout, *args)
        g = layout.num_heads_q // layout.num_heads_k
        return aq, g * ak, g * av
    return attention_backward_bound


MISTAKES = {
    "no_row_term": ("head_gradients", _grads_with("no_row_term")),
    "dq_no_scale": ("head_gradients", _grads_with("dq_no_scale")),
    "dk_uses_P": ("head_gradients", _grads_with("dk_uses_P")),
    "dv_uses_dS": ("head_gradients", _grads_with("dv_uses_dS")),
    "gqa_modulo": ("kv_head_of", lambda h, hq, hk: h % hk),
    "bound_no_scale": ("head_bound", _bound_with("no_scale")),
    "bound_F_twice": ("head_bound", _bound_with("F_twice")),
    "bound_extra_g": ("attention_backward_bound", _bound_with("extra_g")),
}


@pytest.mark.parametrize("name", sorted(MISTAKES))
def test_planted_backward_mistakes_are_caught(name, monkeypatch):
    attr, fn = MISTAKES[name]
    # the test bridge calls the bound through the package namespace
    monkeypatch.setattr(oracle if attr == "attention_backward_bound" else ob, attr, fn)
    failed = []
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
    print(name, "caught by", failed)
