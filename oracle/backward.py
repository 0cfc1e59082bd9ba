"""Float64 reference for the backward pass of paged-KV attention.

TEST INFRASTRUCTURE (see the package docstring): never imported by the library.

Source, cited by page title and section: RL-Kernel PR #284, "feat(attention):
add CP backward drift validation", sections "Summary" and "Changes": a
deterministic training backward for causal prefill and chunked prefill that
reports the gradients of the query, key and value tensors (dq, dk, dv) over
the same forward graph, with decode backward unsupported.

What is differentiated (readings where the pages are silent):

* The function is ``out`` of the forward (``paged_kv.attention``); its
  attention-domain ``lse`` is an auxiliary output whose cotangent is zero.
* ``dk``/``dv`` are the gradients with respect to each sequence's visible keys
  and values, positions ``0 .. seqlens_k[b] - 1``, packed as
  ``[sum_b seqlens_k[b], nheads_k, d]`` with sequence ``b`` starting at row
  ``cu_seqlens_k[b]`` (the exclusive prefix sum of ``seqlens_k``).  Query heads
  that share a KV head (GQA) add their contributions.

With ``P`` the softmax weights of a row (zero for invisible keys), ``dO`` the
cotangent of ``out``, and ``s`` the scaled scores, the chain rule gives, per
sequence and query head ``h`` reading KV head ``hk``::

    dV[j, hk] += sum_i P[i, j] dO[i]
    dP[i, j]   = <dO[i], V[j]>
    dS[i, j]   = P[i, j] (dP[i, j] - sum_k P[i, k] dP[i, k])
    dQ[i, h]   = scale * sum_j dS[i, j] K[j]
    dK[j, hk] += scale * sum_i dS[i, j] Q[i, h]

The row term ``sum_k P[i, k] dP[i, k]`` equals ``<dO[i], out[i]>`` in exact
arithmetic.  Everything is float64; nothing is blocked, chunked or reordered.
"""

from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np

from .paged_kv import Layout, _as_f64, gather_kv, kv_head_of, masked_softmax, scores, visible_keys


def cu_seqlens_k_of(seqlens_k: Sequence[int]) -> np.ndarray:
    """Row offsets of each sequence's keys in the packed dk/dv: exclusive prefix sum."""
    cu = np.zeros(len(seqlens_k) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(seqlens_k, dtype=np.int64))
    return cu


def _sequences(q, k_flat, v_flat, layout, block_table, seqlens_k, cu_seqlens_q, causal):
    """Yield per sequence: (b, r0, r1, n, K [n,Hk,d], V [n,Hk,d], vis [L,n])."""
    Hq, Hk, d, bs = layout.num_heads_q, layout.num_heads_k, layout.head_dim, layout.block_size
    if Hq % Hk != 0:
        raise ValueError("num_heads_q must be a multiple of num_heads_k")
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    if np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens_q must be non-decreasing")
    bt = np.asarray(block_table)
    for b in range(len(cu) - 1):
        n = int(seqlens_k[b])
        r0, r1 = int(cu[b]), int(cu[b + 1])
        if n > bt.shape[1] * bs:
            raise ValueError(f"seqlens_k[{b}]={n} exceeds the block table")
        K, V = gather_kv(k_flat, v_flat, layout, bt[b], n)
        yield b, r0, r1, n, K, V, visible_keys(n, r1 - r0, causal)


def head_gradients(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray,
                   vis: np.ndarray, softmax_scale: float):
    """Chain rule through one head of one sequence: ``(dQ [L,d], dK [n,d], dV [n,d])``.

    ``Q``/``dO`` are the head's rows, ``K``/``V`` its KV head's keys, ``vis``
    the ``[L, n]`` visibility mask; the formulas are the ones in the module
    docstring, with the softmax weights recomputed from the scores.
    """
    P, _ = masked_softmax(scores(Q, K, softmax_scale), vis)   # [L, n]
    dP = dO @ V.T                                              # [L, n]
    row_term = np.sum(P * dP, axis=1)                          # [L]
    dS = P * (dP - row_term[:, None])
    return softmax_scale * (dS @ K), softmax_scale * (dS.T @ Q), P.T @ dO


def attention_backward(q: np.ndarray, k_flat: np.ndarray, v_flat: np.ndarray,
                       layout: Layout, block_table: np.ndarray,
                       seqlens_k: Sequence[int], cu_seqlens_q: Sequence[int],
                       causal: bool, softmax_scale: float,
                       dout: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Gradients of ``out`` (cotangent ``dout``) w.r.t. q and the visible K/V.

    ``q`` and ``dout`` are ``[total_q, nheads, d]`` in the layout's dtype
    (float32 values or bf16 bits).  Returns float64 ``(dq [total_q, nheads, d],
    dk [total_k, nheads_k, d], dv [total_k, nheads_k, d])`` with ``total_k =
    sum(seqlens_k)`` and sequence ``b``'s keys at rows ``cu_seqlens_k_of(
    seqlens_k)[b] ..``.  Rows with no visible key get ``dq = 0`` and add
    nothing to dk/dv.
    """
    Hq, Hk, d = layout.num_heads_q, layout.num_heads_k, layout.head_dim
    qf = _as_f64(q, layout.dtype).reshape(-1, Hq, d)
    dof = _as_f64(dout, layout.dtype).reshape(-1, Hq, d)
    cuk = cu_seqlens_k_of(seqlens_k)
    dq = np.zeros_like(qf)
    dk = np.zeros((int(cuk[-1]), Hk, d), dtype=np.float64)
    dv = np.zeros_like(dk)
    for b, r0, r1, n, K, V, vis in _sequences(q, k_flat, v_flat, layout, block_table,
                                              seqlens_k, cu_seqlens_q, causal):
        if r1 == r0 or n == 0:
            continue
        k0 = int(cuk[b])
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hk)
            gq, gk, gv = head_gradients(qf[r0:r1, h], K[:, hk], V[:, hk], dof[r0:r1, h], vis, softmax_scale)
            dq[r0:r1, h] = gq
            dk[k0:k0 + n, hk] += gk
            dv[k0:k0 + n, hk] += gv
    return dq, dk, dv


def head_bound(Q: np.ndarray, K: np.ndarray, V: np.ndarray, dO: np.ndarray,
               vis: np.ndarray, softmax_scale: float):
    """Term bounds of one head of one sequence: ``(Aq [L,d], Ak [n,d], Av [n,d])``.

    With ``G[i, j] = sum_e |dO[i, e]| |V[j, e]|`` (a bound of ``|dP[i, j]|``)
    and ``F[i] = sum_j P[i, j] G[i, j]`` (a bound of the row term)::

        Aq[i] = |scale| * sum_j P[i, j] (G[i, j] + F[i]) |K[j]|
        Ak[j] = |scale| * sum_i P[i, j] (G[i, j] + F[i]) |Q[i]|
        Av[j] = sum_i P[i, j] |dO[i]|

    Expanding dS into its monomials (``P dO V`` and ``P P dO V``), each bound
    is exactly the sum of the absolute values of the monomials its gradient
    element adds up.
    """
    P, _ = masked_softmax(scores(Q, K, softmax_scale), vis)
    G = np.abs(dO) @ np.abs(V).T
    F = np.sum(P * G, axis=1)
    W = P * (G + F[:, None])
    return (abs(softmax_scale) * (W @ np.abs(K)), abs(softmax_scale) * (W.T @ np.abs(Q)),
            P.T @ np.abs(dO))


def attention_backward_bound(q: np.ndarray, k_flat: np.ndarray, v_flat: np.ndarray,
                             layout: Layout, block_table: np.ndarray,
                             seqlens_k: Sequence[int], cu_seqlens_q: Sequence[int],
                             causal: bool, softmax_scale: float,
                             dout: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Magnitude of the terms each gradient element sums, for error bounds.

    The same formulas as ``attention_backward`` with every quantity replaced by
    an upper bound of its absolute value (``head_bound``), the heads of a GQA
    group adding up in ``Ak``/``Av`` as their gradients do.  By the triangle
    inequality each gradient's absolute value is at most its bound, and the
    rounding error of any evaluation that rounds its operands and sums in
    finite precision is a small multiple of the unit roundoff times the bound
    (the usual forward error analysis of a dot product).
    """
    Hq, Hk, d = layout.num_heads_q, layout.num_heads_k, layout.head_dim
    qs = _as_f64(q, layout.dtype).reshape(-1, Hq, d)
    dof = _as_f64(dout, layout.dtype).reshape(-1, Hq, d)
    cuk = cu_seqlens_k_of(seqlens_k)
    aq = np.zeros_like(qs)
    ak = np.zeros((int(cuk[-1]), Hk, d), dtype=np.float64)
    av = np.zeros_like(ak)
    for b, r0, r1, n, K, V, vis in _sequences(q, k_flat, v_flat, layout, block_table,
                                              seqlens_k, cu_seqlens_q, causal):
        if r1 == r0 or n == 0:
            continue
        k0 = int(cuk[b])
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hk)
            bq, bk, bv = head_bound(qs[r0:r1, h], K[:, hk], V[:, hk], dof[r0:r1, h], vis, softmax_scale)
            aq[r0:r1, h] = bq
            ak[k0:k0 + n, hk] += bk
            av[k0:k0 + n, hk] += bv
    return aq, ak, av
