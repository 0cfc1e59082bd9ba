"""Seeded synthetic inputs for the paged-KV attention tests and benchmark.

This module is shared by the GPU path's tests and by the oracle's tests.  It
holds none of the attention method's arithmetic: it draws random values, lays
them out as paged caches, and builds block tables, sequence lengths and packed
query offsets.  Everything is driven by an explicit ``torch.Generator`` so each
input is reproducible from its seed.

Recipes follow the pages:

* ROCm/aiter commit d293d61bbf19, "test(triton/decode): pin non-contiguous
  paged KV block stride", helper ``_generate_interleaved_block_kvcache``: pool
  size ``ceil(seqlen_k / block_size) * batch * 3`` blocks of N(0, 1) values,
  the K/V-interleaved layout ``[num_blocks, 2, block_size, nheads_k, d]``, and a
  block table that is a random permutation of all blocks reshaped to
  ``[batch, num_blocks // batch]``; test ``test_flash_attn_kvcache_noncontiguous_paged``:
  ``cache_seqlens`` drawn uniformly in ``1 .. seqlen_k``.
* RL-Kernel PR #284, "feat(attention): add CP backward drift validation",
  section "RoPE / TE Boundary": Q/K are post-RoPE with shared global position
  offsets.  ``rope_rotate_half`` builds such inputs; the library itself never
  applies a positional transform.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import List, Optional, Sequence

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}
FP8_NAN_BYTE = 0x7F  # an OCP FP8 E4M3 NaN


@dataclass
class PagedKV:
    """A paged K/V cache: ``k``/``v`` are ``[num_blocks, block_size, nheads_k, d]``.

    ``layout`` is ``"contiguous"`` (two separate contiguous tensors) or
    ``"interleaved"`` (one ``[num_blocks, 2, block_size, nheads_k, d]`` tensor
    whose ``[:, 0]`` and ``[:, 1]`` views are K and V).  ``storage`` lists the
    backing tensors.
    """

    k: torch.Tensor
    v: torch.Tensor
    layout: str
    storage: List[torch.Tensor]

    @property
    def num_blocks(self) -> int:
        return self.k.shape[0]

    @property
    def block_size(self) -> int:
        return self.k.shape[1]


def pool_num_blocks(seqlen_k: int, block_size: int, batch: int) -> int:
    """Pool size used by the aiter test: three times what the batch needs."""
    return math.ceil(seqlen_k / block_size) * batch * 3


def new_pool(num_blocks: int, block_size: int, nheads_k: int, d: int, dtype: str,
             layout: str, device="cpu", generator: Optional[torch.Generator] = None,
             fill: str = "randn") -> PagedKV:
    """Allocate a paged cache; ``fill`` is ``randn`` (N(0,1)), ``zeros`` or ``nan``."""
    tdt = DTYPES[dtype]
    if layout == "interleaved":
        shape = (num_blocks, 2, block_size, nheads_k, d)
    elif layout == "contiguous":
        shape = (2, num_blocks, block_size, nheads_k, d)
    else:
        raise ValueError(layout)
    if fill == "randn":
        buf = torch.randn(shape, dtype=torch.float32, device=device,
                          generator=generator).to(tdt)
    elif fill == "zeros":
        buf = torch.zeros(shape, dtype=torch.float32, device=device).to(tdt)
    elif fill == "nan":
        buf = torch.full(shape, float("nan"), dtype=torch.float32, device=device).to(tdt)
    else:
        raise ValueError(fill)
    if layout == "interleaved":
        return PagedKV(buf[:, 0], buf[:, 1], layout, [buf])
    k, v = buf[0].clone(), buf[1].clone()
    del buf
    return PagedKV(k, v, layout, [k, v])


def relayout(pool: PagedKV, layout: str) -> PagedKV:
    """The same K/V values in another layout (a pure copy)."""
    nb, bs, hk, d = pool.k.shape
    dt = pool.k.dtype
    # copy FP8 as raw bytes (byte views copy on every device)
    raw = (lambda t: t.view(torch.uint8)) if dt == torch.float8_e4m3fn else (lambda t: t)
    if layout == "interleaved":
        buf = torch.empty((nb, 2, bs, hk, d), dtype=dt, device=pool.k.device)
        raw(buf)[:, 0].copy_(raw(pool.k))
        raw(buf)[:, 1].copy_(raw(pool.v))
        return PagedKV(buf[:, 0], buf[:, 1], layout, [buf])
    k = raw(pool.k).contiguous().clone().view(dt)
    v = raw(pool.v).contiguous().clone().view(dt)
    return PagedKV(k, v, "contiguous", [k, v])


def randperm_block_table(num_blocks: int, batch: int,
                         generator: Optional[torch.Generator] = None,
                         device="cpu") -> torch.Tensor:
    """``randperm(num_blocks)`` reshaped to ``[batch, num_blocks // batch]``, int32."""
    perm = torch.randperm(num_blocks, generator=generator, device="cpu").to(torch.int32)
    return perm[: (num_blocks // batch) * batch].reshape(batch, -1).to(device)


def cu_from_lengths(lengths: Sequence[int], device="cpu") -> torch.Tensor:
    cu = [0]
    for x in lengths:
        cu.append(cu[-1] + int(x))
    return torch.tensor(cu, dtype=torch.int32, device=device)


def randn(shape, dtype: str, generator: Optional[torch.Generator] = None,
          device="cpu") -> torch.Tensor:
    """N(0, 1) values drawn in float32 and rounded to ``dtype`` (round to nearest even)."""
    return torch.randn(shape, dtype=torch.float32, generator=generator,
                       device=device).to(DTYPES[dtype])


def rope_rotate_half(x: torch.Tensor, positions: torch.Tensor,
                     theta: float = 10000.0) -> torch.Tensor:
    """Rotate-half RoPE at the given global positions, in float32.

    ``x`` is ``[tokens, heads, d]``; returns float32.  Used only to make
    post-RoPE-like test inputs whose values depend on the global position of a
    token and not on how a sequence is chunked.
    """
    d = x.shape[-1]
    half = d // 2
    inv = theta ** (-torch.arange(half, dtype=torch.float64) * 2.0 / d)
    ang = positions.to(torch.float64)[:, None] * inv[None, :]
    cos = torch.cos(ang).to(torch.float32)[:, None, :]
    sin = torch.sin(ang).to(torch.float32)[:, None, :]
    xf = x.to(torch.float32)
    x1, x2 = xf[..., :half], xf[..., half:]
    return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1)


def uniform_int(lo: int, hi: int, count: int,
                generator: Optional[torch.Generator] = None) -> List[int]:
    """``count`` integers uniform in ``lo .. hi`` inclusive."""
    return torch.randint(lo, hi + 1, (count,), generator=generator).tolist()


def poison_unused(pool: PagedKV, block_table: torch.Tensor,
                  seqlens_k: Sequence[int], value: float = float("nan")) -> None:
    """Write ``value`` into every slot of the pool that no sequence may read.

    Slots at positions ``>= seqlens_k[b]`` in a sequence's last used block and
    all blocks not referenced by the first ``ceil(seqlens_k[b] / block_size)``
    table entries of any sequence are overwritten, for K and V.
    """
    bs = pool.block_size
    used = torch.zeros(pool.num_blocks, dtype=torch.bool)
    tail = []
    bt = block_table.cpu()
    for b, n in enumerate(seqlens_k):
        nblk = (int(n) + bs - 1) // bs
        if nblk:
            used[bt[b, :nblk].long()] = True
            if n % bs:
                tail.append((int(bt[b, nblk - 1]), int(n) % bs))
    unused = (~used).nonzero().flatten().to(pool.k.device)
    for t in (pool.k, pool.v):
        if t.dtype == torch.float8_e4m3fn:   # fill the bytes: FP8 NaN for a NaN value
            t = t.view(torch.uint8)
            value_t = FP8_NAN_BYTE if math.isnan(value) else int(torch.tensor(value).to(torch.float8_e4m3fn).view(torch.uint8))
        else:
            value_t = value
        t.index_fill_(0, unused, value_t)
        for blk, start in tail:
            t[blk, start:].fill_(value_t)


def poison_table_tail(block_table: torch.Tensor, seqlens_k: Sequence[int],
                      block_size: int, value: int = -1) -> torch.Tensor:
    """Copy of ``block_table`` with every entry past ``ceil(n / block_size)`` set to ``value``."""
    bt = block_table.clone().cpu()
    for b, n in enumerate(seqlens_k):
        nblk = (int(n) + block_size - 1) // block_size
        bt[b, nblk:] = value
    return bt.to(block_table.device)
