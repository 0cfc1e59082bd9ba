"""Float64 reference for paged-KV attention and for appending K/V to the cache.

TEST INFRASTRUCTURE (see the package docstring): never imported by the library.

Sources, cited by page title and section:

* RL-Kernel issue #152, "[WS1] KV-cache path consistency (prefill & decode)",
  section "Scope": decode (one query against N cached keys/values) must give the
  result of the equivalent prefill over the full sequence; cache writes and
  reads must not change the stored values.
* ROCm/aiter commit d293d61bbf19, "test(triton/decode): pin non-contiguous paged
  KV block stride": the paged cache ``[num_blocks, block_size, nheads_k, d]``,
  its K/V-interleaved variant ``[num_blocks, 2, block_size, nheads_k, d]`` whose
  K and V views have block stride ``2*block_size*nheads_k*d`` (helper
  ``_generate_interleaved_block_kvcache``), the dense reference gathered from
  the paged buffer through the block table, the ``cache_seqlens`` key padding
  mask, and the GQA rule that query head ``h`` uses KV head ``h // (nheads //
  nheads_k)`` (test ``test_flash_attn_kvcache_noncontiguous_paged``).
* RL-Kernel PR #284, "feat(attention): add CP backward drift validation",
  section "Changes": the forward reports an attention-domain LSE next to the
  output; section "RoPE / TE Boundary": Q/K arrive attention-ready (post-RoPE),
  so no positional transform happens here.
* AstrAI commit list: queries of several requests are packed and addressed
  through cumulative query lengths.

Readings taken where the pages are silent:

* Causal alignment is bottom-right: with ``n`` visible keys and ``L`` query rows
  for a sequence, row ``r`` sits at key position ``n - L + r`` and sees keys
  ``0 .. n - L + r``.  This is the only alignment under which one decode query
  against ``n`` cached keys equals row ``n - 1`` of an ``n``-row causal prefill.
* ``lse`` is the natural-log log-sum-exp of the scaled, masked scores.
* A row with no visible key has ``out = 0`` and ``lse = -inf``.
* ``seqlens_k[b]`` counts every key the call may see, including the keys of the
  call's own query rows.

Everything is float64.  bf16 storage is passed as raw ``uint16`` bit patterns
and FP8 E4M3 storage as raw ``uint8`` bytes; both are widened exactly.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import numpy as np


@dataclass(frozen=True)
class Layout:
    """Where the K and V elements of a paged cache live in flat storage.

    ``k_offset``/``v_offset`` are element offsets into the flat arrays that hold
    K and V; ``k_strides``/``v_strides`` are element strides
    ``(block, slot, head)``; the head-dim stride is 1.  For the interleaved
    layout of the aiter commit, K and V live in the same flat array, ``v_offset
    = block_size*nheads_k*d`` and the block stride is ``2*block_size*nheads_k*d``.
    """

    dtype: str  # "f32" or "bf16" ("f64" for exact float64 inputs)
    num_heads_q: int
    num_heads_k: int
    head_dim: int
    block_size: int
    k_offset: int
    k_strides: Tuple[int, int, int]
    v_offset: int
    v_strides: Tuple[int, int, int]
    # Stored K/V element type if it differs from the queries' ("fp8e4m3": OCP
    # FP8 E4M3 bytes), and the per-tensor factors that turn stored values into
    # K and V (K = stored * k_scale, V = stored * v_scale).
    kv_dtype: Optional[str] = None
    k_scale: float = 1.0
    v_scale: float = 1.0

    @property
    def stored_dtype(self) -> str:
        return self.kv_dtype or self.dtype


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64.

    A bf16 value is the upper half of an IEEE float32, so shifting its bits up
    by 16 gives that float32 exactly.
    """
    u32 = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u32.view(np.float32).astype(np.float64)


def fp8e4m3_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of OCP FP8 E4M3 bytes (uint8) as float64.

    The format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
    infinities; exponent 0 encodes subnormals m * 2^-9, and exponent 15 with
    mantissa 7 is NaN (so the largest finite magnitude is 1.75 * 2^8 = 448).
    """
    b = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = sign * m * 2.0 ** -9
    out = np.where(e == 0, sub, normal)
    return np.where((e == 15) & (m == 7), np.nan, out)


def _as_f64(values: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f64(values)
    if dtype == "fp8e4m3":
        return fp8e4m3_bits_to_f64(values)
    if dtype == "f32":
        return np.asarray(values, dtype=np.float32).astype(np.float64)
    if dtype == "f64":  # exact float64 inputs (finite-difference checks)
        return np.asarray(values, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def kv_head_of(h: int, num_heads_q: int, num_heads_k: int) -> int:
    """Query head ``h`` reads KV head ``h // g`` with ``g = nheads // nheads_k``.

    aiter commit d293d61bbf19, test ``test_flash_attn_kvcache_noncontiguous_paged``:
    the dense reference repeats each KV head ``g`` times as ``(h g)``.
    """
    return h // (num_heads_q // num_heads_k)


def flat_index(offset: int, strides: Tuple[int, int, int], block: np.ndarray,
               slot: np.ndarray, head: np.ndarray, elem: np.ndarray) -> np.ndarray:
    """Element index of (block, slot, head, elem) in flat storage.

    The block term uses the real block stride, which is what the aiter commit
    pins: for the interleaved layout it is twice the contiguous one.
    """
    sb, ss, sh = strides
    return offset + block * sb + slot * ss + head * sh + elem


def gather_sequence(flat: np.ndarray, dtype: str, offset: int,
                    strides: Tuple[int, int, int], block_table_row: np.ndarray,
                    n: int, block_size: int, num_heads_k: int,
                    head_dim: int) -> np.ndarray:
    """Dense ``[n, nheads_k, d]`` float64 K (or V) of one sequence.

    Key ``j`` lives in block ``block_table_row[j // block_size]`` at slot
    ``j % block_size`` (aiter commit d293d61bbf19, helper
    ``_generate_interleaved_block_kvcache``: the pool indexed by the flattened
    block table and cut to ``seqlen_k``).  Only the first ``ceil(n /
    block_size)`` table entries and the first ``n`` slots are read.
    """
    if n == 0:
        return np.zeros((0, num_heads_k, head_dim), dtype=np.float64)
    j = np.arange(n, dtype=np.int64)
    blocks = np.asarray(block_table_row, dtype=np.int64)[j // block_size]
    slots = j % block_size
    idx = flat_index(offset, strides,
                     blocks[:, None, None], slots[:, None, None],
                     np.arange(num_heads_k, dtype=np.int64)[None, :, None],
                     np.arange(head_dim, dtype=np.int64)[None, None, :])
    return _as_f64(np.asarray(flat)[idx], dtype)


def gather_kv(k_flat: np.ndarray, v_flat: np.ndarray, layout: Layout,
              block_table_row: np.ndarray, n: int) -> Tuple[np.ndarray, np.ndarray]:
    """Dense float64 ``K, V`` (``[n, nheads_k, d]``) of one sequence.

    Stored values are widened exactly and multiplied by the layout's K and V
    scales (1 unless the cache stores scaled values, e.g. FP8).
    """
    args = (block_table_row, n, layout.block_size, layout.num_heads_k, layout.head_dim)
    K = gather_sequence(k_flat, layout.stored_dtype, layout.k_offset, layout.k_strides, *args)
    V = gather_sequence(v_flat, layout.stored_dtype, layout.v_offset, layout.v_strides, *args)
    return K * layout.k_scale, V * layout.v_scale


def row_positions(n: int, L: int) -> np.ndarray:
    """Key position of each of the ``L`` query rows: bottom-right alignment."""
    return n - L + np.arange(L, dtype=np.int64)


def visible_keys(n: int, L: int, causal: bool) -> np.ndarray:
    """Boolean ``[L, n]``: key ``j`` is visible to row ``r``.

    Keys at or past ``seqlens_k`` are padding (aiter commit d293d61bbf19: the
    ``key_padding_mask = arange < cache_seqlens``); with ``causal`` a row also
    sees no key after its own position.
    """
    j = np.arange(n, dtype=np.int64)[None, :]
    vis = np.ones((L, n), dtype=bool)
    if causal:
        vis &= j <= row_positions(n, L)[:, None]
    return vis


def attention(q: np.ndarray, k_flat: np.ndarray, v_flat: np.ndarray,
              layout: Layout, block_table: np.ndarray, seqlens_k: Sequence[int],
              cu_seqlens_q: Sequence[int], causal: bool,
              softmax_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Exact attention of packed queries against a paged K/V cache, float64.

    ``q`` is ``[total_q, nheads, d]`` (float32 values or bf16 bits); rows
    ``cu_seqlens_q[b] .. cu_seqlens_q[b+1]`` belong to sequence ``b``, whose
    keys are ``0 .. seqlens_k[b] - 1``.  For each row and query head::

        s_j = softmax_scale * <q, k_j>            (j visible)
        lse = log(sum_j exp(s_j))
        out = sum_j exp(s_j - lse) * v_j

    Returns ``(out [total_q, nheads, d], lse [total_q, nheads])`` in float64.
    This is softmax(Q K^T * scale + mask) V written out per (sequence, KV head):
    RL-Kernel issue #152, "Scope" (decode equals the equivalent prefill), and
    RL-Kernel PR #284, "Changes" (out and attention-domain lse).
    """
    Hq, Hk, d, bs = layout.num_heads_q, layout.num_heads_k, layout.head_dim, layout.block_size
    if Hq % Hk != 0:
        raise ValueError("num_heads_q must be a multiple of num_heads_k")
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    batch = len(cu) - 1
    if np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens_q must be non-decreasing")
    qf = _as_f64(q, layout.dtype).reshape(-1, Hq, d)
    total_q = qf.shape[0]
    out = np.zeros((total_q, Hq, d), dtype=np.float64)
    lse = np.full((total_q, Hq), -np.inf, dtype=np.float64)
    bt = np.asarray(block_table)
    for b in range(batch):
        n = int(seqlens_k[b])
        r0, r1 = int(cu[b]), int(cu[b + 1])
        L = r1 - r0
        if L == 0:
            continue
        if n > bt.shape[1] * bs:
            raise ValueError(f"seqlens_k[{b}]={n} exceeds the block table")
        K, V = gather_kv(k_flat, v_flat, layout, bt[b], n)
        vis = visible_keys(n, L, causal)                    # [L, n]
        for h in range(Hq):
            hk = kv_head_of(h, Hq, Hk)
            s = scores(qf[r0:r1, h, :], K[:, hk, :], softmax_scale)
            weights, row_lse = masked_softmax(s, vis)
            out[r0:r1, h, :] = weights @ V[:, hk, :]
            lse[r0:r1, h] = row_lse
    return out, lse


def attention_chunks(q: np.ndarray, k_flat: np.ndarray, v_flat: np.ndarray,
                     layout: Layout, block_table: np.ndarray, seqlens_k: Sequence[int],
                     cu_seqlens_q: Sequence[int], causal: bool, softmax_scale: float,
                     chunk_keys: int, num_chunks: int) -> Tuple[np.ndarray, np.ndarray]:
    """Attention restricted to each fixed chunk of global key positions, float64.

    RL-Kernel PR #284, "feat(attention): add CP backward drift validation",
    section Changes: context parallelism splits the keys into chunks of a fixed
    size by global position and merges the chunk results in ascending global
    block index.  For chunk ``c`` (keys ``c*chunk_keys .. (c+1)*chunk_keys - 1``)
    and each row and query head this is the plain attention over the row's
    visible keys inside the chunk::

        lse_c = log(sum_{j in J_c} exp(s_j)),   out_c = sum_{j in J_c} exp(s_j - lse_c) v_j

    (``lse_c = -inf``, ``out_c = 0`` when ``J_c`` is empty).  Returns
    ``(out_c [total_q, nheads, num_chunks, d], lse_c [total_q, nheads, num_chunks])``.
    The full result follows from them: ``lse = log sum_c exp(lse_c)`` and
    ``out = sum_c exp(lse_c - lse) out_c``.
    """
    Hq, Hk, d = layout.num_heads_q, layout.num_heads_k, layout.head_dim
    cu = np.asarray(cu_seqlens_q, dtype=np.int64)
    qf = _as_f64(q, layout.dtype).reshape(-1, Hq, d)
    total_q = qf.shape[0]
    out = np.zeros((total_q, Hq, num_chunks, d), dtype=np.float64)
    lse = np.full((total_q, Hq, num_chunks), -np.inf, dtype=np.float64)
    bt = np.asarray(block_table)
    for b in range(len(cu) - 1):
        n = int(seqlens_k[b])
        r0, r1 = int(cu[b]), int(cu[b + 1])
        L = r1 - r0
        if L == 0:
            continue
        K, V = gather_kv(k_flat, v_flat, layout, bt[b], n)
        vis = visible_keys(n, L, causal)
        chunk_of = np.arange(n, dtype=np.int64) // chunk_keys
        for c in range(num_chunks):
            vis_c = vis & (chunk_of == c)[None, :]
            for h in range(Hq):
                hk = kv_head_of(h, Hq, Hk)
                w, row_lse = masked_softmax(scores(qf[r0:r1, h, :], K[:, hk, :], softmax_scale), vis_c)
                out[r0:r1, h, c, :] = w @ V[:, hk, :]
                lse[r0:r1, h, c] = row_lse
    return out, lse


def scores(q_rows: np.ndarray, k_rows: np.ndarray, softmax_scale: float) -> np.ndarray:
    """``[L, n]`` scaled dot products ``softmax_scale * <q_r, k_j>`` in float64."""
    return softmax_scale * (q_rows @ k_rows.T)


def masked_softmax(s: np.ndarray, vis: np.ndarray):
    """Row softmax over the visible entries, and each row's log-sum-exp.

    Returns ``(weights [L, n], lse [L])``; invisible entries get weight 0.  The
    row maximum is subtracted before ``exp`` only to avoid overflow; it cancels
    in exact arithmetic.  A row with no visible entry has all-zero weights and
    ``lse = -inf``.
    """
    s = np.where(vis, s, -np.inf)
    m = np.max(s, axis=1, initial=-np.inf)
    has = np.isfinite(m)
    w = np.where(vis, np.exp(s - np.where(has, m, 0.0)[:, None]), 0.0)
    z = np.sum(w, axis=1)
    lse = np.where(has, m + np.log(np.where(has, z, 1.0)), -np.inf)
    return w / np.where(has, z, 1.0)[:, None], lse


def cache_write(k_flat: np.ndarray, v_flat: np.ndarray, layout: Layout,
                k_new: np.ndarray, v_new: np.ndarray, block_table: np.ndarray,
                seqlens_k: Sequence[int],
                cu_seqlens_new: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Append new K/V rows to the paged cache; returns new flat storage.

    Token ``t`` of sequence ``b`` (rows ``cu_seqlens_new[b] + t`` of ``k_new`` /
    ``v_new``, each ``[nheads_k, d]``) goes to key position ``seqlens_k[b] + t``:
    block ``block_table[b][pos // block_size]``, slot ``pos % block_size``.  The
    stored elements are the given ones bit for bit (RL-Kernel issue #152,
    "Scope": a cache write must add no precision difference between writer and
    reader).  No other element changes.  If K and V share one storage array
    (interleaved layout), pass the same array twice; the result is then one
    array returned twice.
    """
    Hk, d, bs = layout.num_heads_k, layout.head_dim, layout.block_size
    same = k_flat is v_flat
    k_out = np.array(k_flat, copy=True)
    v_out = k_out if same else np.array(v_flat, copy=True)
    kn = np.asarray(k_new).reshape(-1, Hk, d)
    vn = np.asarray(v_new).reshape(-1, Hk, d)
    cu = np.asarray(cu_seqlens_new, dtype=np.int64)
    bt = np.asarray(block_table, dtype=np.int64)
    heads = np.arange(Hk, dtype=np.int64)[:, None]
    elems = np.arange(d, dtype=np.int64)[None, :]
    for b in range(len(cu) - 1):
        for t in range(int(cu[b + 1] - cu[b])):
            pos = int(seqlens_k[b]) + t
            if pos >= bt.shape[1] * bs:
                raise ValueError(f"sequence {b}: position {pos} is past the block table")
            blk, slot = bt[b, pos // bs], pos % bs
            row = int(cu[b]) + t
            k_out[flat_index(layout.k_offset, layout.k_strides, blk, slot, heads, elems)] = kn[row]
            v_out[flat_index(layout.v_offset, layout.v_strides, blk, slot, heads, elems)] = vn[row]
    return k_out, v_out
