"""Python binding of libpkv, the batch-invariant paged-KV attention library.

Argument marshalling only: shapes and strides are read from torch tensors,
pointers and the current HIP stream are passed to the C ABI of ``libpkv.so``
(``include/pkv.h``), and every step of the computation runs in its HIP kernels.
PyTorch provides device memory and streams.  There is no fallback: if the
library is not built, every call raises.

    out, lse = attn_forward(q, k_cache, v_cache, block_table, seqlens_k,
                            cu_seqlens_q, causal=True, softmax_scale=d**-0.5,
                            max_seqlen_q=...)
    cache_write(k_new, v_new, k_cache, v_cache, block_table, seqlens_k,
                cu_seqlens_new, total_new)
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")

PKV_F32, PKV_BF16, PKV_FP8_E4M3 = 0, 1, 2
PKV_OK, PKV_ERR_NULL, PKV_ERR_SHAPE, PKV_ERR_DTYPE, PKV_ERR_ALIGN, PKV_ERR_WORKSPACE, PKV_ERR_HIP, PKV_ERR_OPTION = \
    0, -1, -2, -3, -4, -5, -6, -7
PKV_ERR_DEVICE_DATA = -8
PKV_OPT_PATH, PKV_OPT_SPLIT_CHUNKS, PKV_OPT_FULL_KERNEL, PKV_OPT_DEBUG, PKV_OPT_DECODE_ORDER = 1, 2, 3, 4, 5
PKV_CHECK_ATTENTION, PKV_CHECK_APPEND, PKV_CHECK_CACHE_WRITE = 0, 1, 2
CHUNK_KEYS = 1024
TILE_KEYS = 64
NOALLOC_MAX_BYTES = 96 << 20   # PKV_NOALLOC_MAX_BYTES: the static scratch of pkv_attn_forward_noalloc

# Every symbol include/pkv.h declares.
EXPORTS = (
    "pkv_attn_forward",
    "pkv_attn_forward_ws",
    "pkv_attn_forward_noalloc",
    "pkv_attn_forward_append",
    "pkv_attn_workspace_size",
    "pkv_attn_chunk_partials",
    "pkv_attn_merge_partials",
    "pkv_attn_backward",
    "pkv_attn_backward_workspace_size",
    "pkv_cache_write",
    "pkv_validate_layout",
    "pkv_set_option",
    "pkv_check_device_errors",
    "pkv_check_inputs",
    "pkv_get_option",
    "pkv_error_string",
    "pkv_last_error",
    "pkv_abi_version",
)


class PkvLayout(ctypes.Structure):
    """Mirror of ``pkv_layout`` in include/pkv.h."""

    _fields_ = [
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("num_heads_q", ctypes.c_int32),
        ("num_heads_k", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_k", ctypes.c_int64),
        ("total_q", ctypes.c_int64),
        ("num_blocks", ctypes.c_int64),
        ("k_block_stride", ctypes.c_int64),
        ("k_slot_stride", ctypes.c_int64),
        ("k_head_stride", ctypes.c_int64),
        ("v_block_stride", ctypes.c_int64),
        ("v_slot_stride", ctypes.c_int64),
        ("v_head_stride", ctypes.c_int64),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


class PkvError(RuntimeError):
    def __init__(self, code: int, where: str, msg: str):
        super().__init__(f"{where}: {msg} (code {code})")
        self.code = code


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded ``libpkv.so``; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m invariant_paged_kv_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lay = ctypes.POINTER(PkvLayout)
    L.pkv_attn_forward.argtypes = [vp, vp, vp, lay, vp, vp, vp, i32, f32, vp, vp, vp]
    L.pkv_attn_forward.restype = i32
    L.pkv_attn_forward_ws.argtypes = [vp, vp, vp, lay, vp, vp, vp, i32, f32, vp, vp, vp, sz, vp]
    L.pkv_attn_forward_ws.restype = i32
    L.pkv_attn_forward_noalloc.argtypes = [vp, vp, vp, lay, vp, vp, vp, i32, f32, vp, vp, vp]
    L.pkv_attn_forward_noalloc.restype = i32
    L.pkv_attn_forward_append.argtypes = [vp, vp, vp, vp, vp, lay, vp, vp, vp, i32, f32, vp, vp, vp, sz, vp]
    L.pkv_attn_forward_append.restype = i32
    L.pkv_attn_workspace_size.argtypes = [lay]
    L.pkv_attn_workspace_size.restype = sz
    L.pkv_attn_chunk_partials.argtypes = [vp, vp, vp, lay, vp, vp, vp, i32, f32, i32, i32, i32, vp, vp, vp]
    L.pkv_attn_chunk_partials.restype = i32
    L.pkv_attn_merge_partials.argtypes = [vp, vp, i32, lay, vp, vp, i32, vp, vp, vp]
    L.pkv_attn_merge_partials.restype = i32
    L.pkv_attn_backward.argtypes = [vp, vp, vp, lay, vp, vp, vp, vp, i64, i32, f32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.pkv_attn_backward.restype = i32
    L.pkv_attn_backward_workspace_size.argtypes = [lay]
    L.pkv_attn_backward_workspace_size.restype = sz
    L.pkv_cache_write.argtypes = [vp, vp, vp, vp, lay, vp, vp, vp, i64, vp]
    L.pkv_cache_write.restype = i32
    L.pkv_validate_layout.argtypes = [lay]
    L.pkv_validate_layout.restype = i32
    L.pkv_check_device_errors.argtypes = [vp]
    L.pkv_check_device_errors.restype = i32
    L.pkv_check_inputs.argtypes = [lay, vp, vp, vp, i64, i32]
    L.pkv_check_inputs.restype = i32
    L.pkv_set_option.argtypes = [i32, i64]
    L.pkv_set_option.restype = i32
    L.pkv_get_option.argtypes = [i32]
    L.pkv_get_option.restype = i64
    L.pkv_error_string.argtypes = [i32]
    L.pkv_error_string.restype = ctypes.c_char_p
    L.pkv_last_error.argtypes = []
    L.pkv_last_error.restype = ctypes.c_char_p
    L.pkv_abi_version.argtypes = []
    L.pkv_abi_version.restype = i32
    _lib = L
    return L


def _check(rc: int, where: str) -> None:
    if rc != 0:
        L = lib()
        raise PkvError(rc, where, (L.pkv_last_error() or L.pkv_error_string(rc)).decode())


def _dtype_code(t: torch.dtype) -> int:
    """pkv_dtype of a cache: its storage type (an FP8 cache goes with bf16 queries)."""
    if t == torch.bfloat16:
        return PKV_BF16
    if t == torch.float32:
        return PKV_F32
    if t == torch.float8_e4m3fn:
        return PKV_FP8_E4M3
    raise TypeError(f"unsupported dtype {t}")


def query_dtype(cache_dtype: torch.dtype) -> torch.dtype:
    """Element type of q/out for a cache of ``cache_dtype``."""
    return torch.bfloat16 if cache_dtype == torch.float8_e4m3fn else cache_dtype


def make_layout(k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                num_heads_q: int, max_seqlen_q: int, total_q: int, max_seqlen_k: int = 0,
                batch: Optional[int] = None, k_scale: float = 1.0, v_scale: float = 1.0) -> PkvLayout:
    """``pkv_layout`` from the cache views' shapes and strides.

    ``k_cache``/``v_cache`` are ``[num_blocks, block_size, Hkv, d]`` views with
    unit stride in the last dimension; any block/slot/head strides (e.g. the
    K/V-interleaved layout) are passed through as they are.  ``k_scale`` /
    ``v_scale`` turn stored values into K / V (FP8 caches).
    """
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must be [num_blocks, block_size, Hkv, d] with equal shapes")
    if k_cache.stride(3) != 1 or v_cache.stride(3) != 1:
        raise ValueError("the head-dim stride of k_cache and v_cache must be 1")
    if k_cache.dtype != v_cache.dtype:
        raise TypeError("k_cache and v_cache dtypes differ")
    if block_table.dim() != 2:
        raise ValueError("block_table must be [batch, max_blocks_per_seq]")
    nb, bs, hk, d = k_cache.shape
    L = PkvLayout()
    L.dtype = _dtype_code(k_cache.dtype)
    L.batch = block_table.shape[0] if batch is None else batch
    L.num_heads_q = num_heads_q
    L.num_heads_k = hk
    L.head_dim = d
    L.block_size = bs
    L.max_blocks_per_seq = block_table.shape[1]
    L.max_seqlen_q = max_seqlen_q
    L.max_seqlen_k = max_seqlen_k
    L.total_q = total_q
    L.num_blocks = nb
    L.k_block_stride, L.k_slot_stride, L.k_head_stride = k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)
    L.v_block_stride, L.v_slot_stride, L.v_head_stride = v_cache.stride(0), v_cache.stride(1), v_cache.stride(2)
    L.k_scale = float(k_scale)
    L.v_scale = float(v_scale)
    return L


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _int32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.int32 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous int32 tensor")
    return t


# Argument checks.  The C ABI receives raw addresses and cannot see a tensor's
# device or size, so an undersized buffer or a host tensor would become an
# out-of-bounds or host-pointer access inside a kernel; every public call
# checks shapes and dtypes first, then devices, before the library is touched.

def _check_index(block_table: torch.Tensor, seqlens_k: torch.Tensor, cu: torch.Tensor, cu_name: str) -> int:
    """int32 block table [batch, max_blocks], seqlens [batch], cumulative lengths [batch + 1]; returns batch."""
    _int32(block_table, "block_table")
    _int32(seqlens_k, "seqlens_k")
    _int32(cu, cu_name)
    if block_table.dim() != 2:
        raise ValueError("block_table must be [batch, max_blocks_per_seq]")
    batch = block_table.shape[0]
    if seqlens_k.dim() != 1 or seqlens_k.numel() != batch:
        raise ValueError(f"seqlens_k must have batch = {batch} elements")
    if cu.dim() != 1 or cu.numel() != batch + 1:
        raise ValueError(f"{cu_name} must have batch + 1 = {batch + 1} elements")
    return batch


def _check_like(t: Optional[torch.Tensor], name: str, shape, dtype: torch.dtype) -> None:
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)} "
                         f"(got {t.dtype} {tuple(t.shape)})")


def _check_workspace(ws: Optional[torch.Tensor]) -> None:
    if ws is not None and not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")


def _check_devices(ref: torch.Tensor, **named: Optional[torch.Tensor]) -> None:
    """Every tensor on ref's GPU."""
    if not ref.is_cuda:
        raise ValueError(f"tensors must be on a GPU (got {ref.device}); the library takes device addresses")
    for name, t in named.items():
        if t is not None and (not t.is_cuda or t.device != ref.device):
            raise ValueError(f"{name} is on {t.device}; every tensor must be on {ref.device}")


def _check_new_rows(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor, rows: Optional[int],
                    what: str) -> None:
    """k_new / v_new: contiguous [rows, Hkv, d] in the cache's dtype."""
    hk, d = k_cache.shape[2], k_cache.shape[3]
    for t, name in ((k_new, "k_new"), (v_new, "v_new")):
        if (t.dim() != 3 or not t.is_contiguous() or t.dtype != k_cache.dtype or tuple(t.shape[1:]) != (hk, d)
                or (rows is not None and t.shape[0] != rows)):
            raise ValueError(f"{name} must be a contiguous [{what}, {hk}, {d}] tensor of the cache dtype")


def attn_forward(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                 block_table: torch.Tensor, seqlens_k: torch.Tensor, cu_seqlens_q: torch.Tensor,
                 causal: bool, softmax_scale: float, *, max_seqlen_q: int, max_seqlen_k: int = 0,
                 out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None, k_scale: float = 1.0,
                 v_scale: float = 1.0, noalloc: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention of packed queries ``q [total_q, Hq, d]`` against the paged cache.

    ``seqlens_k[b]`` keys are visible to sequence ``b`` (including its own new
    rows); rows ``cu_seqlens_q[b] .. cu_seqlens_q[b+1]`` are its queries, row
    ``r`` at key position ``seqlens_k[b] - L + r``.  ``max_seqlen_q`` (and
    optionally ``max_seqlen_k``) are host-side bounds.  Returns ``(out, lse)``:
    ``out`` like ``q``, ``lse [total_q, Hq]`` fp32 natural-log LSE.
    """
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [total_q, Hq, d] tensor")
    if q.dtype != query_dtype(k_cache.dtype):
        raise TypeError("q dtype does not match the cache (bf16 queries for an FP8 cache)")
    lay = make_layout(k_cache, v_cache, block_table, q.shape[1], max_seqlen_q, q.shape[0], max_seqlen_k,
                      k_scale=k_scale, v_scale=v_scale)
    if lay.head_dim != q.shape[2]:
        raise ValueError("q head_dim differs from the cache's")
    _check_index(block_table, seqlens_k, cu_seqlens_q, "cu_seqlens_q")
    _check_like(out, "out", q.shape, q.dtype)
    _check_like(lse, "lse", q.shape[:2], torch.float32)
    _check_workspace(workspace)
    _check_devices(q, k_cache=k_cache, v_cache=v_cache, block_table=block_table, seqlens_k=seqlens_k,
                   cu_seqlens_q=cu_seqlens_q, out=out, lse=lse, workspace=workspace)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=q.device)
    bt, sk, cu = block_table, seqlens_k, cu_seqlens_q
    L = lib()
    args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), ctypes.byref(lay), bt.data_ptr(),
            sk.data_ptr(), cu.data_ptr(), 1 if causal else 0, float(softmax_scale), out.data_ptr(),
            lse.data_ptr())
    if noalloc:
        if workspace is not None:
            raise ValueError("noalloc uses the library's static scratch; pass no workspace")
        rc = L.pkv_attn_forward_noalloc(*args, _stream_handle(q.device))
        _check(rc, "pkv_attn_forward_noalloc")
        return out, lse
    if workspace is None:
        rc = L.pkv_attn_forward(*args, _stream_handle(q.device))
    else:
        rc = L.pkv_attn_forward_ws(*args, workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                   _stream_handle(q.device))
    _check(rc, "pkv_attn_forward")
    return out, lse


def attn_forward_noalloc(*args, **kwargs) -> Tuple[torch.Tensor, torch.Tensor]:
    """``attn_forward`` through ``pkv_attn_forward_noalloc``: no device allocation
    by the library (the split path uses its static per-GPU scratch; calls that
    may overlap on one GPU must not be issued).  Pass ``out``/``lse`` to keep the
    binding from allocating them."""
    return attn_forward(*args, noalloc=True, **kwargs)


def flash_attn_with_kvcache(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            cache_seqlens: torch.Tensor, page_table: torch.Tensor, causal: bool = False,
                            softmax_scale: Optional[float] = None, return_softmax_lse: bool = False,
                            k_scale: float = 1.0, v_scale: float = 1.0):
    """The call shape of the pages' paged-cache interface, over ``attn_forward``.

    aiter commit d293d61bbf19 ("pin non-contiguous paged KV block stride")
    calls ``flash_attn_with_kvcache(q, k_cache, v_cache, cache_seqlens=...,
    page_table=..., causal=...)`` with batch-major queries ``q [B, Lq, Hq, d]``,
    caches ``[num_blocks, block_size, Hkv, d]`` (views of an interleaved pool
    allowed) and a page table ``[B, max_blocks]``; ``cache_seqlens[b]`` keys are
    visible to sequence b and its Lq query rows are the last Lq positions
    (bottom-right).  This packs q to ``[B * Lq, Hq, d]`` (a view), builds
    ``cu_seqlens_q = [0, Lq, 2 Lq, ...]`` and calls ``attn_forward`` -- argument
    marshalling only.  Returns ``out [B, Lq, Hq, d]``, and with
    ``return_softmax_lse`` also ``lse [B, Hq, Lq]`` (natural log, fp32).
    """
    if q.dim() != 4:
        raise ValueError("q must be [batch, seqlen_q, num_heads, head_dim]")
    B, Lq, Hq, d = q.shape
    qp = q.contiguous().view(B * Lq, Hq, d)
    cu = torch.arange(0, B * Lq + 1, Lq, dtype=torch.int32, device=q.device) if Lq > 0 else \
        torch.zeros(B + 1, dtype=torch.int32, device=q.device)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    bs = k_cache.shape[1]
    out, lse = attn_forward(qp, k_cache, v_cache, page_table, cache_seqlens, cu, causal, scale,
                            max_seqlen_q=Lq, max_seqlen_k=page_table.shape[1] * bs,
                            k_scale=k_scale, v_scale=v_scale)
    out = out.view(B, Lq, Hq, d)
    if return_softmax_lse:
        return out, lse.view(B, Lq, Hq).permute(0, 2, 1)
    return out


def attn_forward_append(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor,
                        v_cache: torch.Tensor, block_table: torch.Tensor, seqlens_k: torch.Tensor,
                        cu_seqlens_q: torch.Tensor, causal: bool, softmax_scale: float, *, max_seqlen_q: int,
                        max_seqlen_k: int = 0, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None, k_scale: float = 1.0,
                        v_scale: float = 1.0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Write ``k_new``/``v_new`` (one row per query row, at the row's own key
    position ``seqlens_k[b] - L + r``) into the cache and attend, in one launch.

    Bitwise the same cache and ``(out, lse)`` as ``cache_write`` (at
    ``seqlens_k - L``) followed by ``attn_forward``.
    """
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [total_q, Hq, d] tensor")
    if q.dtype != query_dtype(k_cache.dtype):
        raise TypeError("q dtype does not match the cache (bf16 queries for an FP8 cache)")
    lay = make_layout(k_cache, v_cache, block_table, q.shape[1], max_seqlen_q, q.shape[0], max_seqlen_k,
                      k_scale=k_scale, v_scale=v_scale)
    if lay.head_dim != q.shape[2]:
        raise ValueError("q head_dim differs from the cache's")
    _check_new_rows(k_new, v_new, k_cache, q.shape[0], "total_q")
    _check_index(block_table, seqlens_k, cu_seqlens_q, "cu_seqlens_q")
    _check_like(out, "out", q.shape, q.dtype)
    _check_like(lse, "lse", q.shape[:2], torch.float32)
    _check_workspace(workspace)
    _check_devices(q, k_new=k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                   seqlens_k=seqlens_k, cu_seqlens_q=cu_seqlens_q, out=out, lse=lse, workspace=workspace)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().pkv_attn_forward_append(
        q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), ctypes.byref(lay),
        _int32(block_table, "block_table").data_ptr(), _int32(seqlens_k, "seqlens_k").data_ptr(),
        _int32(cu_seqlens_q, "cu_seqlens_q").data_ptr(), 1 if causal else 0, float(softmax_scale), out.data_ptr(),
        lse.data_ptr(), ws_ptr, ws_bytes, _stream_handle(q.device))
    _check(rc, "pkv_attn_forward_append")
    return out, lse


def attn_chunk_partials(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                        seqlens_k: torch.Tensor, cu_seqlens_q: torch.Tensor, causal: bool, softmax_scale: float,
                        chunk_begin: int, chunk_end: int, *, max_seqlen_q: int, max_seqlen_k: int = 0,
                        max_chunks: Optional[int] = None, part_o: Optional[torch.Tensor] = None,
                        part_ml: Optional[torch.Tensor] = None, k_scale: float = 1.0,
                        v_scale: float = 1.0) -> Tuple[torch.Tensor, torch.Tensor]:
    """Chunk partials of global chunks ``[chunk_begin, chunk_end)`` (one rank's share).

    ``part_o [max_chunks, total_q * Hq, d]`` and ``part_ml [max_chunks, total_q * Hq, 2]``
    fp32, chunk-major; allocated (uninitialised) when not given.
    """
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [total_q, Hq, d] tensor")
    if q.dtype != query_dtype(k_cache.dtype):
        raise TypeError("q dtype does not match the cache (bf16 queries for an FP8 cache)")
    lay = make_layout(k_cache, v_cache, block_table, q.shape[1], max_seqlen_q, q.shape[0], max_seqlen_k,
                      k_scale=k_scale, v_scale=v_scale)
    if lay.head_dim != q.shape[2]:
        raise ValueError("q head_dim differs from the cache's")
    if max_chunks is None:
        mk = max_seqlen_k or block_table.shape[1] * k_cache.shape[1]
        max_chunks = max(1, -(-mk // CHUNK_KEYS))
    rows = q.shape[0] * q.shape[1]
    _check_index(block_table, seqlens_k, cu_seqlens_q, "cu_seqlens_q")
    _check_like(part_o, "part_o", (max_chunks, rows, q.shape[2]), torch.float32)
    _check_like(part_ml, "part_ml", (max_chunks, rows, 2), torch.float32)
    _check_devices(q, k_cache=k_cache, v_cache=v_cache, block_table=block_table, seqlens_k=seqlens_k,
                   cu_seqlens_q=cu_seqlens_q, part_o=part_o, part_ml=part_ml)
    if part_o is None:
        part_o = torch.empty((max_chunks, rows, q.shape[2]), dtype=torch.float32, device=q.device)
    if part_ml is None:
        part_ml = torch.empty((max_chunks, rows, 2), dtype=torch.float32, device=q.device)
    rc = lib().pkv_attn_chunk_partials(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), ctypes.byref(lay),
        _int32(block_table, "block_table").data_ptr(), _int32(seqlens_k, "seqlens_k").data_ptr(),
        _int32(cu_seqlens_q, "cu_seqlens_q").data_ptr(), 1 if causal else 0, float(softmax_scale), int(chunk_begin),
        int(chunk_end), int(max_chunks), part_o.data_ptr(), part_ml.data_ptr(), _stream_handle(q.device))
    _check(rc, "pkv_attn_chunk_partials")
    return part_o, part_ml


def attn_merge_partials(part_o: torch.Tensor, part_ml: torch.Tensor, q: torch.Tensor, k_cache: torch.Tensor,
                        v_cache: torch.Tensor, block_table: torch.Tensor, seqlens_k: torch.Tensor,
                        cu_seqlens_q: torch.Tensor, causal: bool, *, max_seqlen_q: int, max_seqlen_k: int = 0,
                        v_scale: float = 1.0, out: Optional[torch.Tensor] = None,
                        lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Fold chunk partials in ascending chunk order into ``(out, lse)`` (shapes from ``q``)."""
    if q.dim() != 3:
        raise ValueError("q must be [total_q, Hq, d]")
    lay = make_layout(k_cache, v_cache, block_table, q.shape[1], max_seqlen_q, q.shape[0], max_seqlen_k,
                      v_scale=v_scale)
    if lay.head_dim != q.shape[2]:
        raise ValueError("q head_dim differs from the cache's")
    rows = q.shape[0] * q.shape[1]
    if part_o.dim() != 3 or part_o.shape[0] < 1:
        raise ValueError("part_o must be [max_chunks, total_q * Hq, d]")
    _check_like(part_o, "part_o", (part_o.shape[0], rows, q.shape[2]), torch.float32)
    _check_like(part_ml, "part_ml", (part_o.shape[0], rows, 2), torch.float32)
    _check_index(block_table, seqlens_k, cu_seqlens_q, "cu_seqlens_q")
    _check_like(out, "out", q.shape, q.dtype)
    _check_like(lse, "lse", q.shape[:2], torch.float32)
    _check_devices(part_o, part_ml=part_ml, seqlens_k=seqlens_k, cu_seqlens_q=cu_seqlens_q, out=out, lse=lse)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=q.device)
    rc = lib().pkv_attn_merge_partials(part_o.data_ptr(), part_ml.data_ptr(), int(part_o.shape[0]), ctypes.byref(lay),
                                       _int32(seqlens_k, "seqlens_k").data_ptr(),
                                       _int32(cu_seqlens_q, "cu_seqlens_q").data_ptr(), 1 if causal else 0,
                                       out.data_ptr(), lse.data_ptr(), _stream_handle(q.device))
    _check(rc, "pkv_attn_merge_partials")
    return out, lse


def attn_backward(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                  seqlens_k: torch.Tensor, cu_seqlens_q: torch.Tensor, causal: bool, softmax_scale: float,
                  out: torch.Tensor, lse: torch.Tensor, dout: torch.Tensor, *, max_seqlen_q: int,
                  max_seqlen_k: int = 0, cu_seqlens_k: Optional[torch.Tensor] = None,
                  total_k: Optional[int] = None, dq: Optional[torch.Tensor] = None,
                  dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Gradients ``(dq, dk, dv)`` of ``out`` for cotangent ``dout``.

    ``out``/``lse`` are the forward's outputs for the same inputs.  ``dk``/``dv``
    are ``[total_k, Hkv, d]``: row ``cu_seqlens_k[b] + j`` is key position ``j``
    of sequence ``b``.  Without ``cu_seqlens_k``/``total_k`` they are computed
    from ``seqlens_k`` (``total_k`` then needs one device-to-host copy).
    """
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [total_q, Hq, d] tensor")
    for t, name in ((out, "out"), (dout, "dout")):
        if t.shape != q.shape or t.dtype != q.dtype or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor of q's shape and dtype")
    if lse.shape != q.shape[:2] or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [total_q, Hq] tensor")
    if q.dtype != k_cache.dtype:
        raise TypeError("q and the cache must share the dtype (bf16 or float32)")
    batch = _check_index(block_table, seqlens_k, cu_seqlens_q, "cu_seqlens_q")
    if cu_seqlens_k is not None and (_int32(cu_seqlens_k, "cu_seqlens_k").dim() != 1
                                     or cu_seqlens_k.numel() != batch + 1):
        raise ValueError(f"cu_seqlens_k must have batch + 1 = {batch + 1} elements")
    _check_like(dq, "dq", q.shape, q.dtype)
    if total_k is not None:
        for t, name in ((dk, "dk"), (dv, "dv")):
            _check_like(t, name, (total_k, k_cache.shape[2], k_cache.shape[3]), q.dtype)
    _check_workspace(workspace)
    _check_devices(q, k_cache=k_cache, v_cache=v_cache, block_table=block_table, seqlens_k=seqlens_k,
                   cu_seqlens_q=cu_seqlens_q, out=out, lse=lse, dout=dout, cu_seqlens_k=cu_seqlens_k, dq=dq,
                   dk=dk, dv=dv, workspace=workspace)
    sk = _int32(seqlens_k, "seqlens_k")
    if cu_seqlens_k is None:
        cu_seqlens_k = torch.zeros(sk.numel() + 1, dtype=torch.int32, device=sk.device)
        cu_seqlens_k[1:] = torch.cumsum(sk, 0)
    cuk = _int32(cu_seqlens_k, "cu_seqlens_k")
    if total_k is None:
        total_k = int(cuk[-1].item())
    lay = make_layout(k_cache, v_cache, block_table, q.shape[1], max_seqlen_q, q.shape[0], max_seqlen_k)
    hk, d = k_cache.shape[2], k_cache.shape[3]
    if lay.head_dim != q.shape[2]:
        raise ValueError("q head_dim differs from the cache's")
    _check_like(dk, "dk", (total_k, hk, d), q.dtype)
    _check_like(dv, "dv", (total_k, hk, d), q.dtype)
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.empty((total_k, hk, d), dtype=q.dtype, device=q.device)
    if dv is None:
        dv = torch.empty((total_k, hk, d), dtype=q.dtype, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib().pkv_attn_backward(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), ctypes.byref(lay),
        _int32(block_table, "block_table").data_ptr(), sk.data_ptr(), _int32(cu_seqlens_q, "cu_seqlens_q").data_ptr(),
        cuk.data_ptr(), int(total_k), 1 if causal else 0, float(softmax_scale), out.data_ptr(), lse.data_ptr(),
        dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws_ptr, ws_bytes, _stream_handle(q.device))
    _check(rc, "pkv_attn_backward")
    return dq, dk, dv


def backward_workspace_size(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                            block_table: torch.Tensor, max_seqlen_q: int) -> int:
    lay = make_layout(k_cache, v_cache, block_table, q.shape[1], max_seqlen_q, q.shape[0], 0)
    return int(lib().pkv_attn_backward_workspace_size(ctypes.byref(lay)))


def workspace_size(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                   *, max_seqlen_q: int, max_seqlen_k: int = 0) -> int:
    lay = make_layout(k_cache, v_cache, block_table, q.shape[1], max_seqlen_q, q.shape[0], max_seqlen_k)
    return int(lib().pkv_attn_workspace_size(ctypes.byref(lay)))


def cache_write(k_new: torch.Tensor, v_new: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                block_table: torch.Tensor, seqlens_k: torch.Tensor, cu_seqlens_new: torch.Tensor,
                total_new: Optional[int] = None) -> None:
    """Bit-copy ``k_new``/``v_new`` ``[total_new, Hkv, d]`` into the paged cache.

    Token ``t`` of sequence ``b`` goes to key position ``seqlens_k[b] + t``;
    ``seqlens_k`` is not advanced.
    """
    if total_new is None:
        total_new = k_new.shape[0]
    lay = make_layout(k_cache, v_cache, block_table, k_cache.shape[2], 0, 0)
    _check_new_rows(k_new, v_new, k_cache, None, "total_new")
    if v_new.shape[0] != k_new.shape[0]:
        raise ValueError("k_new and v_new must have the same number of rows")
    if not 0 <= int(total_new) <= k_new.shape[0]:
        raise ValueError(f"total_new = {total_new} must be in [0, {k_new.shape[0]}] (the rows of k_new)")
    _check_index(block_table, seqlens_k, cu_seqlens_new, "cu_seqlens_new")
    _check_devices(k_new, v_new=v_new, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
                   seqlens_k=seqlens_k, cu_seqlens_new=cu_seqlens_new)
    L = lib()
    rc = L.pkv_cache_write(k_new.data_ptr(), v_new.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                           ctypes.byref(lay), _int32(block_table, "block_table").data_ptr(),
                           _int32(seqlens_k, "seqlens_k").data_ptr(),
                           _int32(cu_seqlens_new, "cu_seqlens_new").data_ptr(), int(total_new),
                           _stream_handle(k_new.device))
    _check(rc, "pkv_cache_write")


def check_device_errors(device: Optional[torch.device] = None) -> None:
    """Synchronise the current stream and raise ``PkvError`` if a launch failed or a
    debug-mode check (``options(debug=1)`` / ``PKV_DEBUG=1``) recorded bad index
    data since the last call (the record is then cleared)."""
    dev = torch.device("cuda") if device is None else device
    _check(lib().pkv_check_device_errors(_stream_handle(dev)), "pkv_check_device_errors")


def check_inputs(k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
                 seqlens_k: torch.Tensor, cu_seqlens: torch.Tensor, *, num_heads_q: int, max_seqlen_q: int,
                 total_rows: int, op: int = PKV_CHECK_ATTENTION, max_seqlen_k: int = 0) -> None:
    """The debug-mode precondition checks on host copies of the index data (no
    device call); raises ``PkvError`` (``PKV_ERR_DEVICE_DATA``) naming the violations."""
    lay = make_layout(k_cache, v_cache, block_table, num_heads_q, max_seqlen_q, total_rows, max_seqlen_k)
    bt = block_table.detach().to("cpu", torch.int32).contiguous()
    sk = seqlens_k.detach().to("cpu", torch.int32).contiguous()
    cu = cu_seqlens.detach().to("cpu", torch.int32).contiguous()
    if sk.numel() != bt.shape[0] or cu.numel() != bt.shape[0] + 1:
        raise ValueError("seqlens_k needs batch and cu_seqlens batch + 1 elements")
    _check(lib().pkv_check_inputs(ctypes.byref(lay), bt.data_ptr(), sk.data_ptr(), cu.data_ptr(), int(total_rows),
                                  int(op)), "pkv_check_inputs")


def set_option(option: int, value: int) -> None:
    _check(lib().pkv_set_option(option, value), "pkv_set_option")


def get_option(option: int) -> int:
    return int(lib().pkv_get_option(option))


class options:
    """Context manager that sets library options and restores them on exit."""

    def __init__(self, path: Optional[int] = None, split_chunks: Optional[int] = None,
                 full_kernel: Optional[int] = None, debug: Optional[int] = None,
                 decode_order: Optional[int] = None):
        self._want = {}
        if decode_order is not None:
            self._want[PKV_OPT_DECODE_ORDER] = decode_order
        if debug is not None:
            self._want[PKV_OPT_DEBUG] = debug
        if path is not None:
            self._want[PKV_OPT_PATH] = path
        if split_chunks is not None:
            self._want[PKV_OPT_SPLIT_CHUNKS] = split_chunks
        if full_kernel is not None:
            self._want[PKV_OPT_FULL_KERNEL] = full_kernel
        self._old = {}

    def __enter__(self):
        for k, v in self._want.items():
            self._old[k] = get_option(k)
            set_option(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self._old.items():
            set_option(k, v)
        return False
