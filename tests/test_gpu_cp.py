"""Context-parallel share and fold on one GPU (pkv_attn_chunk_partials,
pkv_attn_merge_partials).

RL-Kernel PR #284, "feat(attention): add CP backward drift validation",
section Changes: with context parallelism each rank handles a range of KV
chunks and the partials are merged in fixed ascending global block order, so
the result does not depend on the CP world size.  Here each "rank" is one call
over a contiguous chunk range writing its slab of a shared chunk-major buffer
(what an all-gather would assemble); the fold must give pkv_attn_forward's
bits for every split, and each chunk partial must match the oracle's attention
restricted to that chunk (out 2e-2 / lse 1e-3 in bf16, 1e-5 / 1e-6 in fp32).
"""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import invariant_paged_kv_amd as pkv
import pkv_inputs as gen
from tests import gpu_cases as gc
from tests.oracle_bridge import oracle_pool, storage_np

import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


def make(seed, dtype, hq, hk, d, bs, layout, causal, lens, seqlens, scales=(1.0, 1.0)):
    g = torch.Generator().manual_seed(seed)
    batch = len(lens)
    nb = gen.pool_num_blocks(max(seqlens), bs, batch)
    pool = gen.new_pool(nb, bs, hk, d, dtype, layout, generator=g)
    bt = gen.randperm_block_table(nb, batch, generator=g)
    cu = [0]
    for x in lens:
        cu.append(cu[-1] + x)
    qdt = "bf16" if dtype == "fp8" else dtype
    q = gen.randn((cu[-1], hq, d), qdt, generator=g)
    case = gc.Case(q.to(gc.DEV), gc.to_device(pool), bt.to(gc.DEV), list(seqlens), cu, causal, 1.0 / math.sqrt(d), qdt)
    case.extra = {"k_scale": scales[0], "v_scale": scales[1]}
    return case


def kw(case):
    return dict(max_seqlen_q=case.max_seqlen_q, max_seqlen_k=case.max_seqlen_k)


def forward(case):
    out, lse = pkv.attn_forward(case.q, case.pool.k, case.pool.v, case.block_table, case.seqlens_d(), case.cu_d(),
                                case.causal, case.scale, k_scale=case.extra["k_scale"],
                                v_scale=case.extra["v_scale"], **kw(case), **gc.nan_outputs(case.q))
    torch.cuda.synchronize()
    return out, lse


def shares(case, bounds, max_chunks):
    """Partials computed rank by rank (chunk ranges [bounds[i], bounds[i+1])) into one buffer."""
    rows = case.q.shape[0] * case.q.shape[1]
    d = case.q.shape[2]
    po = torch.full((max_chunks, rows, d), float("nan"), dtype=torch.float32, device=gc.DEV)
    pm = torch.full((max_chunks, rows, 2), float("nan"), dtype=torch.float32, device=gc.DEV)
    for c0, c1 in zip(bounds[:-1], bounds[1:]):
        pkv.attn_chunk_partials(case.q, case.pool.k, case.pool.v, case.block_table, case.seqlens_d(), case.cu_d(),
                                case.causal, case.scale, c0, c1, max_chunks=max_chunks, part_o=po, part_ml=pm,
                                k_scale=case.extra["k_scale"], v_scale=case.extra["v_scale"], **kw(case))
    torch.cuda.synchronize()
    return po, pm


def merge(case, po, pm):
    out, lse = pkv.attn_merge_partials(po, pm, case.q, case.pool.k, case.pool.v, case.block_table,
                                       case.seqlens_d(), case.cu_d(), case.causal,
                                       v_scale=case.extra["v_scale"], **kw(case), **gc.nan_outputs(case.q))
    torch.cuda.synchronize()
    return out, lse


CASES = [
    ("bf16-decode-gqa", "bf16", 16, 4, 128, 16, "interleaved", True, [1, 1, 1], [3000, 700, 1]),
    ("bf16-chunked-rows", "bf16", 16, 4, 128, 16, "contiguous", True, [40, 7], [2100, 1500]),
    ("f32-c1-like", "f32", 2, 2, 64, 16, "contiguous", True, [1, 3], [1340, 600]),
    ("fp8-decode", "fp8", 32, 8, 128, 256, "interleaved", True, [1, 3], [5000, 2600]),
]


def row_limits(case):
    lims = []
    for b, n in enumerate(case.seqlens):
        L = case.cu[b + 1] - case.cu[b]
        for r in range(L):
            lims.append(min(n - L + r + 1, n) if case.causal else n)
    return lims


@pytest.mark.parametrize("spec", CASES, ids=[c[0] for c in CASES])
def test_any_split_of_the_chunks_folds_to_the_forward(spec):
    name, dt, hq, hk, d, bs, layout, causal, lens, seqlens = spec
    announce(f"cp fold {name}")
    case = make(9000 + CASES.index(spec), dt, hq, hk, d, bs, layout, causal, lens, seqlens,
                (0.5, 1.25) if dt == "fp8" else (1.0, 1.0))
    ref = forward(case)
    nc = -(-max(seqlens) // pkv.CHUNK_KEYS)
    splits = [[0, nc], [0, nc // 2, nc], [0, 1, 2, nc], [0, 0, nc], list(range(nc + 1)), [0, nc - 1, nc]]
    for bounds in splits:   # each list: rank i computes chunks [bounds[i], bounds[i+1]); [0, 0, nc] has an idle rank
        assert bounds == sorted(bounds) and bounds[0] == 0 and bounds[-1] == nc
        po, pm = shares(case, bounds, nc + 2)
        gc.assert_bitwise(merge(case, po, pm), ref, f"ranks {bounds}")


@pytest.mark.parametrize("spec", CASES, ids=[c[0] for c in CASES])
def test_chunk_partials_match_the_oracle(spec):
    name, dt, hq, hk, d, bs, layout, causal, lens, seqlens = spec
    announce(f"cp partials vs oracle {name}")
    ks, vs = (0.5, 1.25) if dt == "fp8" else (1.0, 1.0)
    case = make(9100 + CASES.index(spec), dt, hq, hk, d, bs, layout, causal, lens, seqlens, (ks, vs))
    nc = -(-max(seqlens) // pkv.CHUNK_KEYS)
    po, pm = shares(case, [0, nc], nc)
    qh, ph, bth, sl, cu, rows = gc.subset_for_oracle(case, list(range(len(seqlens))))
    kf, vf, lay = oracle_pool(ph, hq, ks, vs)
    oo, ol = oracle.attention_chunks(storage_np(qh).reshape(qh.shape), kf, vf, lay, np.asarray(bth), sl, cu,
                                     causal, case.scale, pkv.CHUNK_KEYS, nc)
    m = pm[..., 0].double().cpu().numpy()          # [nc, rows*hq]
    l = pm[..., 1].double().cpu().numpy()
    o = po.double().cpu().numpy()                   # [nc, rows*hq, d]
    base2 = dt != "f32"
    tol_o, tol_l = gc.TOL["f32" if dt == "f32" else "bf16"]
    lims = row_limits(case)
    worst_o = worst_l = 0.0
    for r, lim in enumerate(lims):
        nck = -(-lim // pkv.CHUNK_KEYS) if lim > 0 else 0
        for h in range(hq):
            w = r * hq + h
            for c in range(nck):
                if m[c, w] == -np.inf:
                    assert ol[r, h, c] == -np.inf, (r, h, c)
                    continue
                lse_c = (m[c, w] + np.log2(l[c, w])) * math.log(2.0) if base2 else m[c, w] + np.log(l[c, w])
                out_c = o[c, w] / l[c, w] * vs
                worst_l = max(worst_l, abs(lse_c - ol[r, h, c]))
                # the out bound applies in the units of the stored V
                worst_o = max(worst_o, float(np.max(np.abs(out_c - oo[r, h, c]))) / vs)
    assert worst_o <= tol_o, f"chunk out max-abs {worst_o:.3e}"
    assert worst_l <= tol_l, f"chunk lse max-abs {worst_l:.3e}"
    print(f"{name}: chunk out {worst_o:.2e}, chunk lse {worst_l:.2e}")
