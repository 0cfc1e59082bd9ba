"""Turn the generators' torch tensors into the oracle's NumPy inputs.

Test code only.  The oracle's layout (offsets and element strides) is derived
here from the layout's *name* and shape, by the formulas the aiter commit
states, not from torch's stride machinery, so the oracle's view of the pool is
independent of the one the library binding computes from ``tensor.stride()``.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from pkv_inputs import PagedKV


def storage_np(t: torch.Tensor) -> np.ndarray:
    """Flat NumPy copy of a tensor's elements: uint16 bits for bf16, float32 otherwise."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16).reshape(-1).copy()
    if t.dtype == torch.float32:
        return t.numpy().reshape(-1).copy()
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy().reshape(-1).copy()
    raise TypeError(t.dtype)


def dtype_name(t: torch.Tensor) -> str:
    return {torch.bfloat16: "bf16", torch.float32: "f32", torch.float8_e4m3fn: "fp8e4m3"}[t.dtype]


def oracle_pool(pool: PagedKV, num_heads_q: int, k_scale: float = 1.0, v_scale: float = 1.0):
    """``(k_flat, v_flat, Layout)`` for the oracle.  An FP8 pool goes with bf16 queries."""
    nb, bs, hk, d = pool.k.shape
    dt = dtype_name(pool.k)
    qdt, kvdt = ("bf16", dt) if dt == "fp8e4m3" else (dt, None)
    row = hk * d
    extra = dict(kv_dtype=kvdt, k_scale=k_scale, v_scale=v_scale)
    if pool.layout == "interleaved":
        flat = storage_np(pool.storage[0])
        lay = oracle.Layout(qdt, num_heads_q, hk, d, bs,
                            k_offset=0, k_strides=(2 * bs * row, row, d),
                            v_offset=bs * row, v_strides=(2 * bs * row, row, d), **extra)
        return flat, flat, lay
    lay = oracle.Layout(qdt, num_heads_q, hk, d, bs,
                        k_offset=0, k_strides=(bs * row, row, d),
                        v_offset=0, v_strides=(bs * row, row, d), **extra)
    return storage_np(pool.k), storage_np(pool.v), lay


def oracle_attention(q: torch.Tensor, pool: PagedKV, block_table, seqlens_k,
                     cu_seqlens_q, causal: bool, softmax_scale: float,
                     k_scale: float = 1.0, v_scale: float = 1.0):
    """Run the oracle on generator tensors; returns float64 ``(out, lse)``."""
    hq = q.shape[1]
    kf, vf, lay = oracle_pool(pool, hq, k_scale, v_scale)
    return oracle.attention(storage_np(q).reshape(q.shape), kf, vf, lay,
                            np.asarray(torch.as_tensor(block_table).cpu()),
                            [int(x) for x in torch.as_tensor(seqlens_k).cpu()],
                            [int(x) for x in torch.as_tensor(cu_seqlens_q).cpu()],
                            causal, softmax_scale)


def oracle_backward(q: torch.Tensor, pool: PagedKV, block_table, seqlens_k,
                    cu_seqlens_q, causal: bool, softmax_scale: float,
                    dout: torch.Tensor, bound: bool = False):
    """Run the backward oracle on generator tensors; float64 ``(dq, dk, dv)``.

    With ``bound=True`` the term-magnitude bounds ``(Aq, Ak, Av)`` come back
    instead (used to scale the GPU tolerances).
    """
    hq = q.shape[1]
    kf, vf, lay = oracle_pool(pool, hq)
    fn = oracle.attention_backward_bound if bound else oracle.attention_backward
    return fn(storage_np(q).reshape(q.shape), kf, vf, lay,
              np.asarray(torch.as_tensor(block_table).cpu()),
              [int(x) for x in torch.as_tensor(seqlens_k).cpu()],
              [int(x) for x in torch.as_tensor(cu_seqlens_q).cpu()],
              causal, softmax_scale, storage_np(dout).reshape(dout.shape))
