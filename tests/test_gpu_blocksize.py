"""Block-size invariance: the same keys and values stored in caches of different
block sizes give the same bits.

The block size only decides where a key's row is stored (key j of a sequence
sits in table entry j / block_size, slot j % block_size); it enters no
arithmetic.  So for every path -- the split decode kernels, the 4-wave and
8-wave full kernels and the 4-wave split kernel -- out and lse must be bitwise identical
across block sizes.  The sizes cover every way the kernels address a tile:
multiples of 16 (one block id per 16-row group, read with a scalar load; for
a tile below the sequence's end, one id per tile when the block size is a
multiple of the 64-key tile -- 64, 256 -- and four consecutive ids with
16-key blocks) and other sizes (a block id per row).  Slots the tables do not reference hold NaN,
and sequence lengths are not multiples of the tile, so a read of a wrong slot
or a missed clamp at a sequence's end shows up as NaN or changed bits.  One
configuration per dtype is also checked against the oracle.
"""

from __future__ import annotations

import math

import pytest
import torch

import invariant_paged_kv_amd as pkv
import pkv_inputs as gen
from tests import gpu_cases as gc

pytestmark = pytest.mark.gpu

BLOCK_SIZES = [8, 16, 24, 32, 64, 256]
SEQLENS = [1000, 333, 1, 2049]
HQ, HK, D = 16, 4, 128


@pytest.fixture(autouse=True)
def _free():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def announce(msg: str) -> None:
    print(f"[case] {msg}", flush=True)


def dense_kv(seed: int, dtype: str):
    g = torch.Generator().manual_seed(seed)
    ks = [gen.randn((n, HK, D), dtype, generator=g) for n in SEQLENS]
    vs = [gen.randn((n, HK, D), dtype, generator=g) for n in SEQLENS]
    return ks, vs, g


def paged(ks, vs, bs: int, dtype: str, layout: str, seed: int):
    """The dense rows placed in a NaN-filled pool of block size bs under a random block table."""
    nblk = [-(-n // bs) for n in SEQLENS]
    total = sum(nblk) + 3
    pool = gen.new_pool(total, bs, HK, D, dtype, layout, fill="nan")
    perm = torch.randperm(total, generator=torch.Generator().manual_seed(seed))
    width = max(nblk)
    table = torch.zeros((len(SEQLENS), width), dtype=torch.int32)
    raw = (lambda t: t.view(torch.uint8)) if dtype == "fp8" else (lambda t: t)
    used = 0
    for b, n in enumerate(SEQLENS):
        ids = perm[used:used + nblk[b]]
        used += nblk[b]
        table[b, :nblk[b]] = ids.to(torch.int32)
        for i, blk in enumerate(ids.tolist()):
            lo, hi = i * bs, min((i + 1) * bs, n)
            raw(pool.k)[blk, :hi - lo] = raw(ks[b][lo:hi])
            raw(pool.v)[blk, :hi - lo] = raw(vs[b][lo:hi])
    return gc.to_device(pool), table.to(gc.DEV)


def case_for(pool, table, q, lens, dtype):
    cu = [0]
    for x in lens:
        cu.append(cu[-1] + x)
    qdt = "bf16" if dtype == "fp8" else dtype
    return gc.Case(q.to(gc.DEV), pool, table, list(SEQLENS), cu, True, 1.0 / math.sqrt(D), qdt)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("mode", ["decode", "prefill-full", "prefill-full8", "prefill-split"])
def test_block_size_invariance(dtype, mode):
    announce(f"block-size invariance {dtype} {mode}")
    ks, vs, g = dense_kv(9500 + (dtype == "fp8"), dtype)
    lens = [1, 1, 1, 1] if mode == "decode" else [min(n, 150) for n in SEQLENS]
    qdt = "bf16" if dtype == "fp8" else dtype
    q = gen.randn((sum(lens), HQ, D), qdt, generator=g)
    path = {"decode": None, "prefill-full": 2, "prefill-full8": 2, "prefill-split": 1}[mode]
    fk = 3 if mode == "prefill-full8" else None
    ref = None
    for i, bs in enumerate(BLOCK_SIZES):
        layout = "interleaved" if i % 2 == 0 else "contiguous"
        pool, table = paged(ks, vs, bs, dtype, layout, seed=9600 + bs)
        case = case_for(pool, table, q, lens, dtype)
        got = gc.run(case, path=path, full_kernel=fk)
        assert not torch.isnan(got[0].float()).any(), f"NaN in out at block size {bs}"
        if ref is None:
            ref = got
            if mode not in ("prefill-split", "prefill-full8"):
                # anchor the shared result to the oracle (bf16 tolerances; FP8 queries are bf16)
                gc.check_oracle(case, *got)
        else:
            gc.assert_bitwise(got, ref, f"block size {bs} vs {BLOCK_SIZES[0]}")
