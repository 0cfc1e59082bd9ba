"""Shared helpers of the GPU tests: seeded cases on the device, calls through
the C ABI, bitwise comparison, and oracle comparison on host copies.

The oracle only ever sees host copies of the generator's tensors (moved with
torch, never produced by the library); expected values never come from the
HIP path.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np
import torch

import invariant_paged_kv_amd as pkv
import pkv_inputs as gen
from tests.oracle_bridge import oracle_attention

DEV = "cuda"
TOL = {"bf16": (2e-2, 1e-3), "f32": (1e-5, 1e-6)}   # (out max-abs, lse max-abs)


@dataclass
class Case:
    q: torch.Tensor                 # device [total_q, Hq, d]
    pool: gen.PagedKV               # device
    block_table: torch.Tensor       # device int32
    seqlens: List[int]
    cu: List[int]
    causal: bool
    scale: float
    dtype: str
    extra: dict = field(default_factory=dict)

    @property
    def max_seqlen_q(self) -> int:
        return max([self.cu[i + 1] - self.cu[i] for i in range(len(self.cu) - 1)] + [0])

    @property
    def max_seqlen_k(self) -> int:
        return max(self.seqlens + [0])

    def seqlens_d(self) -> torch.Tensor:
        return torch.tensor(self.seqlens, dtype=torch.int32, device=DEV)

    def cu_d(self) -> torch.Tensor:
        return torch.tensor(self.cu, dtype=torch.int32, device=DEV)


def run(case: Case, pool: Optional[gen.PagedKV] = None, block_table=None, q=None, path=None,
        split_chunks=None, scale=None, seqlens=None, cu=None, causal=None, full_kernel=None):
    pool = pool or case.pool
    bt = case.block_table if block_table is None else block_table
    q = case.q if q is None else q
    sl = case.seqlens if seqlens is None else seqlens
    cul = case.cu if cu is None else cu
    # NaN-filled outputs: an element a kernel does not write cannot pass as the
    # stale copy of an earlier run's result
    out0 = torch.full_like(q, float("nan"))
    lse0 = torch.full((q.shape[0], q.shape[1]), float("nan"), dtype=torch.float32, device=q.device)
    with pkv.options(path=path, split_chunks=split_chunks, full_kernel=full_kernel):
        out, lse = pkv.attn_forward(
            q, pool.k, pool.v, bt, torch.tensor(sl, dtype=torch.int32, device=DEV),
            torch.tensor(cul, dtype=torch.int32, device=DEV),
            case.causal if causal is None else causal, case.scale if scale is None else scale,
            max_seqlen_q=max(cul[i + 1] - cul[i] for i in range(len(cul) - 1)),
            max_seqlen_k=max(sl), out=out0, lse=lse0)
    torch.cuda.synchronize()
    return out, lse


def nan_outputs(q: torch.Tensor) -> dict:
    """out / lse buffers for q, filled with NaN (every element must be written)."""
    return dict(out=torch.full_like(q, float("nan")),
                lse=torch.full((q.shape[0], q.shape[1]), float("nan"), dtype=torch.float32, device=q.device))


def bits(t: torch.Tensor) -> torch.Tensor:
    t = t.contiguous()
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def assert_bitwise(a, b, what=""):
    """Same bit patterns (so -inf == -inf, +0 != -0)."""
    for x, y in zip(a, b):
        bx, by = bits(x), bits(y)
        if not torch.equal(bx, by):
            diff = (bx != by).nonzero()
            raise AssertionError(f"{what}: {diff.shape[0]} elements differ, first at {diff[0].tolist()}: "
                                 f"{x.flatten()[0].item() if x.numel() else None}")


def host_pool(pool: gen.PagedKV) -> gen.PagedKV:
    if pool.layout == "interleaved":
        buf = pool.storage[0].cpu()
        return gen.PagedKV(buf[:, 0], buf[:, 1], "interleaved", [buf])
    k, v = pool.k.cpu(), pool.v.cpu()
    return gen.PagedKV(k, v, "contiguous", [k, v])


def subset_for_oracle(case: Case, seq_ids: Sequence[int]):
    """Host copy of just the blocks and query rows of some sequences.

    Returns ``(q, pool, block_table, seqlens, cu, row_index)``: a compact
    contiguous pool holding the sequences' visible blocks in table order,
    and the original row numbers of the kept query rows.
    """
    bs = case.pool.block_size
    bt = case.block_table.cpu()
    ks, vs, rows, tables, seqlens, cu = [], [], [], [], [], [0]
    nxt = 0
    maxblk = max(max(1, (case.seqlens[b] + bs - 1) // bs) for b in seq_ids)
    fp8 = case.pool.k.dtype == torch.float8_e4m3fn
    kview = case.pool.k.view(torch.uint8) if fp8 else case.pool.k   # byte view: index FP8 as raw bytes
    vview = case.pool.v.view(torch.uint8) if fp8 else case.pool.v
    for b in seq_ids:
        n = case.seqlens[b]
        nblk = (n + bs - 1) // bs
        ids = bt[b, :nblk].long().to(DEV)
        ks.append(kview.index_select(0, ids).cpu())
        vs.append(vview.index_select(0, ids).cpu())
        row = list(range(nxt, nxt + nblk)) + [0] * (maxblk - nblk)
        tables.append(row)
        nxt += nblk
        r0, r1 = case.cu[b], case.cu[b + 1]
        rows.extend(range(r0, r1))
        seqlens.append(n)
        cu.append(cu[-1] + r1 - r0)
    k = torch.cat(ks) if nxt else torch.zeros((1,) + tuple(kview.shape[1:]), dtype=kview.dtype)
    v = torch.cat(vs) if nxt else torch.zeros_like(k)
    if fp8:
        k, v = k.view(torch.float8_e4m3fn), v.view(torch.float8_e4m3fn)
    if nxt == 0:
        tables = [[0] * maxblk for _ in seq_ids]
    pool = gen.PagedKV(k.contiguous(), v.contiguous(), "contiguous", [])
    pool.storage = [pool.k, pool.v]
    q = case.q[torch.tensor(rows, dtype=torch.long, device=DEV)].cpu() if rows else case.q[:0].cpu()
    return q, pool, torch.tensor(tables, dtype=torch.int32), seqlens, cu, rows


def oracle_for(case: Case, seq_ids: Optional[Sequence[int]] = None):
    """Oracle (out, lse) float64 for the given sequences (default: all); plus row ids."""
    if seq_ids is None:
        seq_ids = list(range(len(case.seqlens)))
    q, pool, bt, seqlens, cu, rows = subset_for_oracle(case, seq_ids)
    out, lse = oracle_attention(q, pool, bt, seqlens, cu, case.causal, case.scale)
    return out, lse, rows


def max_err(got: torch.Tensor, want: np.ndarray) -> float:
    g = got.detach().cpu().to(torch.float64).numpy()
    fin = np.isfinite(want)
    assert np.array_equal(np.isfinite(g), fin), "finite/-inf pattern differs from the oracle"
    assert np.array_equal(g[~fin], want[~fin]), "non-finite values differ from the oracle"
    return float(np.max(np.abs(g[fin] - want[fin]))) if fin.any() else 0.0


def check_oracle(case: Case, out: torch.Tensor, lse: torch.Tensor, seq_ids=None):
    """Compare GPU out/lse rows of the given sequences with the oracle, at the stated tolerances."""
    oout, olse, rows = oracle_for(case, seq_ids)
    if not rows:
        return 0.0, 0.0
    idx = torch.tensor(rows, dtype=torch.long, device=out.device)
    eo = max_err(out.index_select(0, idx), oout)
    el = max_err(lse.index_select(0, idx), olse)
    to, tl = TOL[case.dtype]
    assert eo <= to, f"out max-abs {eo:.3e} > {to:.0e}"
    assert el <= tl, f"lse max-abs {el:.3e} > {tl:.0e}"
    return eo, el


def make_case(seed: int, dtype: str, batch: int, hq: int, hk: int, d: int, bs: int, seqlen_k: int,
              layout: str, causal: bool, lens_q: Sequence[int], seqlens: Optional[Sequence[int]] = None,
              scale: Optional[float] = None) -> Case:
    """A case from the aiter recipe: pool ceil(seqlen_k/bs)*batch*3 blocks of N(0,1), randperm table."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    nb = gen.pool_num_blocks(seqlen_k, bs, batch)
    pool = gen.new_pool(nb, bs, hk, d, dtype, layout, generator=g)
    bt = gen.randperm_block_table(nb, batch, generator=g)
    if seqlens is None:
        seqlens = gen.uniform_int(1, seqlen_k, batch, generator=g)
    cu = [0]
    for x in lens_q:
        cu.append(cu[-1] + int(x))
    q = gen.randn((cu[-1], hq, d), dtype, generator=g)
    dev_pool = to_device(pool)
    return Case(q.to(DEV), dev_pool, bt.to(DEV), list(map(int, seqlens)), cu, causal,
                scale if scale is not None else 1.0 / math.sqrt(d), dtype)


def to_device(pool: gen.PagedKV) -> gen.PagedKV:
    if pool.layout == "interleaved":
        buf = pool.storage[0].to(DEV)
        return gen.PagedKV(buf[:, 0], buf[:, 1], "interleaved", [buf])
    k, v = pool.k.to(DEV), pool.v.to(DEV)
    return gen.PagedKV(k, v, "contiguous", [k, v])


def device_pool(seed: int, num_blocks: int, bs: int, hk: int, d: int, dtype: str, layout: str) -> gen.PagedKV:
    """Large pools drawn directly on the device (seeded device generator)."""
    g = torch.Generator(device=DEV).manual_seed(seed)
    return gen.new_pool(num_blocks, bs, hk, d, dtype, layout, device=DEV, generator=g)
