"""Backward (pkv_attn_backward) on the GPU against the float64 oracle.

RL-Kernel PR #284, "feat(attention): add CP backward drift validation",
sections Summary and Changes: dq, dk and dv of causal prefill and chunked
prefill over the same forward, deterministic.

Tolerance (derived from the arithmetic): each gradient element is a sum of
terms whose absolute values add up to the oracle's bound A (the same formulas
with every quantity replaced by its absolute value).  In bf16 the kernels
round P and dS to bf16 once as MFMA operands and use the bf16-rounded forward
output for delta = <dout, out>, each a relative error of at most 2^-9 on terms
bounded by A, and round the result once (2^-9 relative); so
|gpu - oracle| <= 2^-6 A + 2^-8 |oracle| leaves a margin of about 3.  In fp32
the errors come from expf, the forward's LSE and fp32 sums (~1e-6 relative):
2^-15 A + 2^-20 |oracle|.  Between GPU runs and paths: bitwise.
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import invariant_paged_kv_amd as pkv
import pkv_inputs as gen
from tests import gpu_cases as gc
from tests.oracle_bridge import oracle_backward

pytestmark = pytest.mark.gpu

BWD_TOL = {"bf16": (2.0 ** -6, 2.0 ** -8), "f32": (2.0 ** -15, 2.0 ** -20)}


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


def make_dout(case: gc.Case, seed: int) -> torch.Tensor:
    g = torch.Generator().manual_seed(seed)
    return gen.randn(tuple(case.q.shape), case.dtype, generator=g).to(gc.DEV)


def cu_k_of(seqlens):
    cu = [0]
    for n in seqlens:
        cu.append(cu[-1] + n)
    return cu


def run_bwd(case: gc.Case, dout, out=None, lse=None, pool=None, block_table=None, q=None, seqlens=None, cu=None):
    pool = pool or case.pool
    bt = case.block_table if block_table is None else block_table
    q = case.q if q is None else q
    sl = case.seqlens if seqlens is None else seqlens
    cul = case.cu if cu is None else cu
    if out is None:
        out, lse = gc.run(case, pool=pool, block_table=bt, q=q, seqlens=sl, cu=cul)
    dq, dk, dv = pkv.attn_backward(
        q, pool.k, pool.v, bt, torch.tensor(sl, dtype=torch.int32, device=gc.DEV),
        torch.tensor(cul, dtype=torch.int32, device=gc.DEV), case.causal, case.scale, out, lse, dout,
        max_seqlen_q=max(cul[i + 1] - cul[i] for i in range(len(cul) - 1)), max_seqlen_k=max(sl))
    torch.cuda.synchronize()
    return dq, dk, dv


def within(got: torch.Tensor, ref: np.ndarray, bound: np.ndarray, dtype: str, what: str) -> float:
    g = got.detach().cpu().to(torch.float64).numpy()
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    c1, c2 = BWD_TOL[dtype]
    allow = c1 * bound + c2 * np.abs(ref) + 1e-30
    ratio = np.abs(g - ref) / allow
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > 1.0:
        i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(f"{what}: error {abs(g[i] - ref[i]):.3e} at {i} exceeds {allow[i]:.3e} "
                             f"(ref {ref[i]:.4e}, bound {bound[i]:.3e})")
    return worst


def check_bwd_oracle(case: gc.Case, dout, dq, dk, dv, seq_ids=None):
    """Compare the gradients of some sequences with the oracle; returns the worst error/allowance ratio."""
    if seq_ids is None:
        seq_ids = list(range(len(case.seqlens)))
    q, pool, bt, seqlens, cu, rows = gc.subset_for_oracle(case, seq_ids)
    d_rows = dout[torch.tensor(rows, dtype=torch.long, device=gc.DEV)].cpu() if rows else dout[:0].cpu()
    ref = oracle_backward(q, pool, bt, seqlens, cu, case.causal, case.scale, d_rows)
    bnd = oracle_backward(q, pool, bt, seqlens, cu, case.causal, case.scale, d_rows, bound=True)
    worst = 0.0
    if rows:
        idx = torch.tensor(rows, dtype=torch.long, device=gc.DEV)
        worst = max(worst, within(dq.index_select(0, idx), ref[0], bnd[0], case.dtype, "dq"))
    cuk = cu_k_of(case.seqlens)
    ocuk = cu_k_of(seqlens)
    krows = [r for s, b in enumerate(seq_ids) for r in range(cuk[b], cuk[b] + case.seqlens[b])]
    orows = [r for s, b in enumerate(seq_ids) for r in range(ocuk[s], ocuk[s] + case.seqlens[b])]
    if krows:
        kidx = torch.tensor(krows, dtype=torch.long, device=gc.DEV)
        worst = max(worst, within(dk.index_select(0, kidx), ref[1][orows], bnd[1][orows], case.dtype, "dk"))
        worst = max(worst, within(dv.index_select(0, kidx), ref[2][orows], bnd[2][orows], case.dtype, "dv"))
    return worst


# (name, dtype, hq, hk, d, bs, layout, causal, lens_q, seqlens)
CASES = [
    ("bf16-gqa4-full", "bf16", 16, 4, 128, 16, "interleaved", True, [200, 37, 129], [200, 37, 129]),
    ("bf16-gqa4-chunked", "bf16", 16, 4, 128, 16, "interleaved", True, [200, 37, 129], [300, 37, 700]),
    ("bf16-mha-noncausal-d64-bs7", "bf16", 8, 8, 64, 7, "contiguous", False, [65, 3], [100, 260]),
    ("bf16-gqa8-long-chunk", "bf16", 64, 8, 128, 256, "interleaved", True, [100], [1500]),
    ("f32-c1-like", "f32", 2, 2, 64, 16, "contiguous", True, [340], [340]),
    ("f32-gqa2-d128", "f32", 4, 2, 128, 16, "interleaved", True, [33, 70], [33, 200]),
    ("bf16-edges", "bf16", 8, 2, 128, 16, "interleaved", True, [0, 5, 3, 1], [10, 0, 2, 9]),
    ("f32-noncausal-edges", "f32", 4, 4, 64, 5, "contiguous", False, [0, 4, 1], [6, 0, 77]),
]


@pytest.mark.parametrize("spec", CASES, ids=[c[0] for c in CASES])
def test_backward_parity(spec):
    name, dt, hq, hk, d, bs, layout, causal, lens, seqlens = spec
    announce(f"backward parity {name}")
    seed = 7000 + CASES.index(spec)
    case = gc.make_case(seed, dt, len(lens), hq, hk, d, bs, max(seqlens), layout, causal, lens, seqlens)
    dout = make_dout(case, seed + 1)
    dq, dk, dv = run_bwd(case, dout)
    worst = check_bwd_oracle(case, dout, dq, dk, dv)
    print(f"{name}: worst error / allowance = {worst:.3f}")


def test_backward_deterministic_and_batch_invariant():
    announce("backward determinism + batch invariance")
    lens, seqlens = [150, 1, 64, 90], [150, 513, 64, 400]
    case = gc.make_case(7100, "bf16", 4, 16, 4, 128, 16, max(seqlens), "interleaved", True, lens, seqlens)
    dout = make_dout(case, 7101)
    out, lse = gc.run(case)
    a = run_bwd(case, dout, out, lse)
    b = run_bwd(case, dout, out, lse)
    gc.assert_bitwise(a, b, "two runs")
    cuk = cu_k_of(seqlens)
    for s in range(4):
        r0, r1 = case.cu[s], case.cu[s + 1]
        one = run_bwd(case, dout[r0:r1].contiguous(), out[r0:r1].contiguous(), lse[r0:r1].contiguous(),
                      block_table=case.block_table[s:s + 1].contiguous(), q=case.q[r0:r1].contiguous(),
                      seqlens=[seqlens[s]], cu=[0, r1 - r0])
        gc.assert_bitwise((one[0],), (a[0][r0:r1],), f"dq of sequence {s} alone vs in batch")
        gc.assert_bitwise((one[1], one[2]), (a[1][cuk[s]:cuk[s + 1]], a[2][cuk[s]:cuk[s + 1]]),
                          f"dk/dv of sequence {s} alone vs in batch")


def test_backward_layout_and_table_invariance():
    announce("backward interleaved == contiguous, permuted table")
    lens, seqlens = [70, 130], [90, 130]
    case = gc.make_case(7200, "bf16", 2, 8, 2, 128, 16, max(seqlens), "interleaved", True, lens, seqlens)
    dout = make_dout(case, 7201)
    out, lse = gc.run(case)
    a = run_bwd(case, dout, out, lse)
    other = gc.to_device(gen.relayout(gc.host_pool(case.pool), "contiguous"))
    b = run_bwd(case, dout, out, lse, pool=other)
    gc.assert_bitwise(a, b, "contiguous vs interleaved")
    nb = case.pool.num_blocks
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(7202)).to(gc.DEV)
    inv = torch.argsort(perm)
    buf = case.pool.storage[0][inv].contiguous()
    moved = gen.PagedKV(buf[:, 0], buf[:, 1], "interleaved", [buf])
    bt2 = perm[case.block_table.long()].to(torch.int32)
    c = run_bwd(case, dout, out, lse, pool=moved, block_table=bt2)
    gc.assert_bitwise(a, c, "permuted block table")


def test_backward_dq_chunked_equals_full():
    """A row's dq is the same bits whether its rows were one call or several (chunked prefill)."""
    announce("backward dq chunked == full")
    n = 600
    case = gc.make_case(7300, "bf16", 1, 16, 4, 128, 16, n, "interleaved", True, [n], [n])
    dout = make_dout(case, 7301)
    full = run_bwd(case, dout)
    for a, b in ((0, 17), (17, 300), (300, 600)):
        part = run_bwd(case, dout[a:b].contiguous(), q=case.q[a:b].contiguous(), seqlens=[b], cu=[0, b - a])
        gc.assert_bitwise((part[0],), (full[0][a:b],), f"dq rows [{a},{b})")


def test_backward_decode_row_dq_equals_prefill_row():
    announce("backward decode row dq == prefill row dq")
    n = 777
    case = gc.make_case(7400, "f32", 1, 4, 2, 64, 16, n, "contiguous", True, [n], [n])
    dout = make_dout(case, 7401)
    full = run_bwd(case, dout)
    for t in (0, 511, 512, n - 1):
        one = run_bwd(case, dout[t:t + 1].contiguous(), q=case.q[t:t + 1].contiguous(), seqlens=[t + 1], cu=[0, 1])
        gc.assert_bitwise((one[0],), (full[0][t:t + 1],), f"dq of row {t}")


@pytest.mark.large
def test_backward_full_size_prefill():
    """Causal prefill batch 8 x 8192, Hq 16, Hkv 4, d 128, bs 16: sampled rows of dq
    and one KV head of one sequence's dk/dv against the oracle; determinism;
    the gradient identities (sum of dk over keys = 0, sum of dv = sum of dout)."""
    announce("backward full size 8 x 8192")
    B, HQ, HK, D, BS, S = 8, 16, 4, 128, 16, 8192
    nb = gen.pool_num_blocks(S, BS, B)
    pool = gc.device_pool(7500, nb, BS, HK, D, "bf16", "contiguous")
    bt = gen.randperm_block_table(nb, B, generator=torch.Generator().manual_seed(7500)).to(gc.DEV)
    g = torch.Generator(device=gc.DEV).manual_seed(7501)
    q = gen.randn((B * S, HQ, D), "bf16", generator=g, device=gc.DEV)
    dout = gen.randn((B * S, HQ, D), "bf16", generator=g, device=gc.DEV)
    case = gc.Case(q, pool, bt, [S] * B, [S * b for b in range(B + 1)], True, 1.0 / math.sqrt(D), "bf16")
    out, lse = gc.run(case)
    a = run_bwd(case, dout, out, lse)
    b = run_bwd(case, dout, out, lse)
    gc.assert_bitwise(a, b, "two runs at full size")
    dq, dk, dv = a
    # dq rows: a row's dq needs only that row, so the oracle runs it as a one-row call
    for s, t in ((0, 0), (0, 1), (0, 777), (3, 4096), (7, 8191), (7, 5000)):
        r = s * S + t
        sub = gc.Case(q[r:r + 1].contiguous(), pool, bt[s:s + 1].contiguous(), [t + 1], [0, 1], True, case.scale, "bf16")
        qh, ph, bth, sl, cu, rows = gc.subset_for_oracle(sub, [0])
        ref = oracle_backward(qh, ph, bth, sl, cu, True, case.scale, dout[r:r + 1].cpu())
        bnd = oracle_backward(qh, ph, bth, sl, cu, True, case.scale, dout[r:r + 1].cpu(), bound=True)
        within(dq[r:r + 1], ref[0], bnd[0], "bf16", f"dq row {t} of sequence {s}")
    # dk/dv of sequence 5, KV head 1 (query heads 4..7): the oracle on that head group alone
    s, hk = 5, 1
    sub = gc.Case(q[s * S:(s + 1) * S, 4 * hk:4 * hk + 4].contiguous(), pool, bt[s:s + 1].contiguous(), [S], [0, S],
                  True, case.scale, "bf16")
    qh, ph, bth, sl, cu, rows = gc.subset_for_oracle(sub, [0])
    ph = gen.PagedKV(ph.k[:, :, hk:hk + 1].contiguous(), ph.v[:, :, hk:hk + 1].contiguous(), "contiguous", [])
    ph.storage = [ph.k, ph.v]
    dh = dout[s * S:(s + 1) * S, 4 * hk:4 * hk + 4].cpu().contiguous()
    ref = oracle_backward(qh, ph, bth, sl, cu, True, case.scale, dh)
    bnd = oracle_backward(qh, ph, bth, sl, cu, True, case.scale, dh, bound=True)
    within(dk[s * S:(s + 1) * S, hk:hk + 1], ref[1], bnd[1], "bf16", "dk of sequence 5, KV head 1")
    within(dv[s * S:(s + 1) * S, hk:hk + 1], ref[2], bnd[2], "bf16", "dv of sequence 5, KV head 1")
    # identities over every sequence and KV head, to the bf16 rounding of the stored gradients
    dk64 = dk.double().view(B, S, HK, D)
    dv64 = dv.double().view(B, S, HK, D)
    ksum = dk64.sum(1)
    assert float((ksum.abs() - 2.0 ** -7 * dk64.abs().sum(1)).max()) <= 0, "sum of dk over keys is not ~0"
    want = dout.double().view(B, S, HK, HQ // HK, D).sum((1, 3))
    assert float(((dv64.sum(1) - want).abs() - 2.0 ** -7 * dv64.abs().sum(1)).max()) <= 0, "sum of dv != sum of dout"
