"""Writes the stored expected values of ``tests/golden/*.json``.

Run from the repository root: ``python -m tests.golden.make_golden``.  The
inputs come from the seeded generators (``pkv_inputs``); the expected values
come from the float64 oracle alone (``oracle.attention``), never from the
library.  Each case stores its recipe, a SHA-256 of the generated input bytes
(so a change in the generators is caught before values are compared), every
LSE and a fixed sample of output elements.

What is computed: attention of packed query rows over a paged KV cache read
through a block table with the real block stride (aiter commit d293d61bbf19,
"pin non-contiguous paged KV block stride": the K and V of block i sit at
i * block_stride, and query head h reads KV head h // (Hq / Hkv)); a row of a
sequence with n keys and L rows sits at position n - L + r and, when causal,
sees the keys at positions <= its own -- the bottom-right reading under which
a decode row equals the same row of the equivalent prefill (RL-Kernel issue
#152 "[WS1] KV-cache path consistency (prefill & decode)", section Scope).
"""

from __future__ import annotations

import hashlib
import json
import math
import os

import numpy as np
import torch

import pkv_inputs as gen
from tests.oracle_bridge import oracle_attention, storage_np

HERE = os.path.dirname(os.path.abspath(__file__))

# name: (seed, dtype, batch, hq, hk, d, bs, layout, causal, seqlens_k, rows per sequence)
CASES = {
    "gqa_decode_bf16_interleaved": (7101, "bf16", 3, 8, 2, 64, 16, "interleaved", True, [37, 1, 70], [1, 1, 1]),
    "chunked_rows_bf16_contiguous": (7102, "bf16", 2, 2, 1, 64, 16, "contiguous", True, [1100, 300], [5, 3]),
    "noncausal_f32_interleaved": (7103, "f32", 2, 4, 4, 64, 8, "interleaved", False, [19, 45], [2, 4]),
}
SAMPLES = 96  # output elements stored per case


def build_inputs(spec):
    """The case's tensors (CPU), rebuilt identically from its seed."""
    seed, dtype, batch, hq, hk, d, bs, layout, causal, seqlens, lens = spec
    g = torch.Generator().manual_seed(seed)
    nb = gen.pool_num_blocks(max(seqlens), bs, batch)
    pool = gen.new_pool(nb, bs, hk, d, dtype, layout, generator=g)
    bt = gen.randperm_block_table(nb, batch, generator=g)
    cu = [0]
    for x in lens:
        cu.append(cu[-1] + x)
    q = gen.randn((cu[-1], hq, d), dtype, generator=g)
    return q, pool, bt, cu


def input_digest(q, pool, bt) -> str:
    h = hashlib.sha256()
    for t in (q, pool.k, pool.v, bt):
        h.update(storage_np(t).tobytes() if t.dtype != torch.int32 else t.numpy().tobytes())
    return h.hexdigest()


def sample_indices(spec, rows: int):
    """Fixed (row, head, element) sample, drawn from a generator of its own."""
    seed, _, _, hq, _, d = spec[:6]
    rng = np.random.default_rng(seed + 1)
    return [[int(rng.integers(rows)), int(rng.integers(hq)), int(rng.integers(d))] for _ in range(SAMPLES)]


def expected(spec):
    seed, dtype, batch, hq, hk, d, bs, layout, causal, seqlens, lens = spec
    q, pool, bt, cu = build_inputs(spec)
    out, lse = oracle_attention(q, pool, bt, seqlens, cu, causal, 1.0 / math.sqrt(d))
    idx = sample_indices(spec, cu[-1])
    return {
        "recipe": {"seed": seed, "dtype": dtype, "batch": batch, "num_heads_q": hq, "num_heads_k": hk,
                   "head_dim": d, "block_size": bs, "layout": layout, "causal": causal,
                   "seqlens_k": seqlens, "rows": lens, "softmax_scale": "1/sqrt(head_dim)",
                   "pool": "pkv_inputs.new_pool(pool_num_blocks(max(seqlens_k), bs, batch), ...) of N(0,1)",
                   "block_table": "pkv_inputs.randperm_block_table", "q": "pkv_inputs.randn"},
        "input_sha256": input_digest(q, pool, bt),
        "lse": [[float(x) for x in row] for row in lse],
        "out_samples": [[r, h, e, float(out[r, h, e])] for r, h, e in idx],
    }


def main():
    for name, spec in CASES.items():
        path = os.path.join(HERE, name + ".json")
        with open(path, "w") as f:
            json.dump(expected(spec), f, indent=1)
            f.write("\n")
        print("wrote", path)


if __name__ == "__main__":
    main()
