"""C-ABI checks that need no GPU: the library loads, exports what include/pkv.h
declares, and rejects bad arguments on the host before any launch."""

import ctypes
import os
import re

import pytest

import invariant_paged_kv_amd as pkv

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_]+)\s*\(", text)))


def test_library_is_built_and_loads():
    assert os.path.exists(pkv.LIB_PATH), "run python -m invariant_paged_kv_amd.build"
    L = pkv.lib()
    assert L.pkv_abi_version() == 2


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(pkv.EXPORTS), (names, pkv.EXPORTS)
    L = pkv.lib()
    for n in names:
        assert hasattr(L, n), f"{n} not exported"


def good_layout(**over):
    lay = pkv.PkvLayout()
    vals = dict(dtype=pkv.PKV_BF16, batch=2, num_heads_q=16, num_heads_k=4, head_dim=128, block_size=16,
                max_blocks_per_seq=8, max_seqlen_q=1, max_seqlen_k=0, total_q=2, num_blocks=16,
                k_block_stride=2 * 16 * 4 * 128, k_slot_stride=4 * 128, k_head_stride=128,
                v_block_stride=2 * 16 * 4 * 128, v_slot_stride=4 * 128, v_head_stride=128)
    vals.update(over)
    for k, v in vals.items():
        setattr(lay, k, v)
    return lay


@pytest.mark.parametrize("over,code", [
    ({}, 0),
    ({"dtype": 7}, -3),
    ({"num_heads_q": 6}, -2),
    ({"num_heads_k": 0}, -2),
    ({"head_dim": 96}, -2),
    ({"block_size": 0}, -2),
    ({"k_slot_stride": 4 * 128 + 4}, -4),        # 8-byte multiple only: breaks 128-bit loads
    ({"v_head_stride": -128}, -2),
    ({"dtype": pkv.PKV_F32, "k_head_stride": 132}, 0),
    ({"dtype": pkv.PKV_F32, "k_head_stride": 130}, -4),
    ({"max_seqlen_q": -1}, -2),
    ({"dtype": pkv.PKV_FP8_E4M3}, 0),
    ({"dtype": pkv.PKV_FP8_E4M3, "k_slot_stride": 4 * 128 + 8}, -4),   # 8 bytes: not a 16-byte multiple
    ({"dtype": 3}, -3),
    ({"k_scale": -1.0}, -2),
    ({"v_scale": float("nan")}, -2),
    ({"k_scale": 0.5, "v_scale": 0.0}, 0),
    ({"batch": 65535}, 0),                     # launch-grid limits
    ({"batch": 65536}, -2),
    ({"num_heads_q": 65536 * 2, "num_heads_k": 65536}, -2),
    ({"total_q": ((1 << 31) - 1) // 16}, 0),
    ({"total_q": ((1 << 31) - 1) // 16 + 1}, -2),   # total_q * num_heads_q past 2^31 - 1
])
def test_validate_layout(over, code):
    L = pkv.lib()
    assert L.pkv_validate_layout(ctypes.byref(good_layout(**over))) == code
    if code:
        assert L.pkv_last_error().decode()


def test_null_and_misaligned_pointers_fail_before_launch():
    L = pkv.lib()
    lay = good_layout()
    rc = L.pkv_attn_forward(None, None, None, ctypes.byref(lay), None, None, None, 1, 0.1, None, None, None)
    assert rc == -1 and "NULL" in L.pkv_last_error().decode()
    rc = L.pkv_attn_forward(8, 16, 32, ctypes.byref(lay), 64, 64, 64, 1, 0.1, 48, 64, None)
    assert rc == -4
    rc = L.pkv_attn_forward(16, 16, 32, ctypes.byref(lay), 64, 64, 64, 1, float("nan"), 48, 64, None)
    assert rc == -2
    rc = L.pkv_cache_write(None, None, None, None, ctypes.byref(lay), None, None, None, 3, None)
    assert rc == -1
    rc = L.pkv_attn_forward(16, 16, 32, None, 64, 64, 64, 1, 0.1, 48, 64, None)
    assert rc == -1


def test_workspace_size_matches_partial_buffers():
    L = pkv.lib()
    lay = good_layout(max_seqlen_k=4096, total_q=64, batch=64, max_blocks_per_seq=768)
    chunks = 4096 // pkv.CHUNK_KEYS
    parts = 64 * 16 * chunks
    want = -(-parts * 128 * 4 // 256) * 256 + -(-parts * 2 * 4 // 256) * 256
    assert L.pkv_attn_workspace_size(ctypes.byref(lay)) == want   # 64 x 4 x 4 jobs: no job list
    # 128 sequences x 8 KV heads x 8 chunks: the decode kernels' longest-first job list adds its prefix counts
    lay2 = good_layout(max_seqlen_k=8192, total_q=128, batch=128, max_blocks_per_seq=512, num_heads_q=32,
                       num_heads_k=8, k_block_stride=2 * 16 * 8 * 128, k_slot_stride=8 * 128,
                       v_block_stride=2 * 16 * 8 * 128, v_slot_stride=8 * 128)
    parts2 = 128 * 32 * 8
    want2 = -(-parts2 * 128 * 4 // 256) * 256 + -(-parts2 * 2 * 4 // 256) * 256 + -(-(2 * 128 + 2) * 4 // 256) * 256
    assert L.pkv_attn_workspace_size(ctypes.byref(lay2)) == want2
    assert L.pkv_attn_workspace_size(ctypes.byref(good_layout(head_dim=3))) == 0


def test_options_roundtrip_and_errors():
    L = pkv.lib()
    with pkv.options(path=2, split_chunks=3):
        assert pkv.get_option(pkv.PKV_OPT_PATH) == 2
        assert pkv.get_option(pkv.PKV_OPT_SPLIT_CHUNKS) == 3
    assert pkv.get_option(pkv.PKV_OPT_PATH) == 0
    assert L.pkv_set_option(pkv.PKV_OPT_PATH, 5) == -7
    assert L.pkv_set_option(99, 0) == -7
    assert L.pkv_error_string(-4).decode() == "misaligned pointer or stride"


def test_backward_rejects_bad_arguments_before_launch():
    L = pkv.lib()
    lay = good_layout(total_q=2)
    args = dict(q=16, k=16, v=32, bt=64, sk=64, cuq=64, cuk=64, total_k=10, causal=1, scale=0.1,
                out=48, lse=64, dout=80, dq=96, dk=112, dv=128)

    def call(**over):
        a = dict(args, **over)
        return L.pkv_attn_backward(a["q"], a["k"], a["v"], ctypes.byref(lay), a["bt"], a["sk"], a["cuq"], a["cuk"],
                                   a["total_k"], a["causal"], a["scale"], a["out"], a["lse"], a["dout"], a["dq"],
                                   a["dk"], a["dv"], None, 0, None)

    assert call(dout=None) == -1
    assert call(dk=None) == -1
    assert call(cuk=None) == -1
    assert call(dq=8) == -4
    assert call(dout=24) == -4
    assert call(scale=0.0) == -2
    assert call(scale=float("inf")) == -2
    assert call(total_k=-1) == -2
    # a caller workspace that is too small is rejected before any launch
    rc = L.pkv_attn_backward(16, 16, 32, ctypes.byref(lay), 64, 64, 64, 64, 10, 1, 0.1, 48, 64, 80, 96, 112, 128,
                             256, 4, None)
    assert rc == -5


def test_backward_rejects_fp8_and_scaled_caches():
    L = pkv.lib()
    for over, code in (({"dtype": pkv.PKV_FP8_E4M3}, -3), ({"k_scale": 2.0}, -2), ({"v_scale": 0.5}, -2)):
        lay = good_layout(total_q=2, **over)
        rc = L.pkv_attn_backward(16, 16, 32, ctypes.byref(lay), 64, 64, 64, 64, 10, 1, 0.1, 48, 64, 80, 96, 112,
                                 128, None, 0, None)
        assert rc == code, (over, rc)


def test_layout_struct_matches_header():
    """The ctypes mirror has the header's fields, in order, at the C offsets."""
    text = open(HEADER).read()
    body = re.search(r"typedef struct pkv_layout \{(.*?)\} pkv_layout;", text, re.S).group(1)
    names = re.findall(r"(\w+)\s*[,;]", body)
    assert [f[0] for f in pkv.PkvLayout._fields_] == names
    assert ctypes.sizeof(pkv.PkvLayout) == 8 * 4 + 9 * 8 + 2 * 4   # no padding: 112 bytes


def test_backward_workspace_size():
    L = pkv.lib()
    lay = good_layout(total_q=100)
    assert L.pkv_attn_backward_workspace_size(ctypes.byref(lay)) == -(-100 * 16 * 4 // 256) * 256
    assert L.pkv_attn_backward_workspace_size(ctypes.byref(good_layout(head_dim=3))) == 0


def test_chunk_partials_and_merge_reject_bad_arguments():
    L = pkv.lib()
    lay = good_layout(total_q=2)

    def part(c0, c1, mc, po=96, pm=112):
        return L.pkv_attn_chunk_partials(16, 16, 32, ctypes.byref(lay), 64, 64, 64, 1, 0.1, c0, c1, mc, po, pm, None)

    assert part(0, 3, 2) == -2          # chunk_end past max_chunks
    assert part(2, 1, 4) == -2          # empty range reversed
    assert part(-1, 1, 4) == -2
    assert part(0, 1, 0) == -2
    assert part(0, 1, 4, po=None) == -1
    assert part(0, 1, 4, pm=104) == -4  # part_ml must be 16-byte aligned
    assert part(1, 1, 4) == 0           # an idle rank: nothing to do
    assert L.pkv_attn_merge_partials(96, 112, 0, ctypes.byref(lay), 64, 64, 1, 48, 64, None) == -2
    assert L.pkv_attn_merge_partials(None, 112, 4, ctypes.byref(lay), 64, 64, 1, 48, 64, None) == -1
    assert L.pkv_attn_merge_partials(96, 104, 4, ctypes.byref(lay), 64, 64, 1, 48, 64, None) == -4


def test_single_chunk_decode_needs_no_workspace():
    """Sequences within one 1024-key chunk: the split kernels write out / lse themselves (no partials,
    no merge), so the split path asks for no workspace; from 1025 keys on it does."""
    L = pkv.lib()
    one = good_layout(max_blocks_per_seq=64)      # 64 x 16 = 1024 keys
    assert L.pkv_attn_workspace_size(ctypes.byref(one)) == 0
    two = good_layout(max_blocks_per_seq=64, max_seqlen_k=1025, num_blocks=256)
    two.max_blocks_per_seq = 65
    assert L.pkv_attn_workspace_size(ctypes.byref(two)) > 0


def test_noalloc_rejects_a_split_path_beyond_the_scratch_before_any_device_call():
    """The size check of pkv_attn_forward_noalloc runs on the host first: on a
    machine without a GPU it still answers PKV_ERR_WORKSPACE (a device call
    would have failed with PKV_ERR_HIP), and nothing is launched."""
    L = pkv.lib()
    # 4096 decode rows x 64 heads over 2^20 keys: 4096 * 64 * 1024 chunks * 130 fp32 of partials
    lay = good_layout(batch=1, num_heads_q=64, num_heads_k=8, block_size=256, max_blocks_per_seq=4096,
                      total_q=4096, max_seqlen_q=1, k_block_stride=2 * 256 * 8 * 128, k_slot_stride=8 * 128,
                      v_block_stride=2 * 256 * 8 * 128, v_slot_stride=8 * 128)
    assert L.pkv_attn_workspace_size(ctypes.byref(lay)) > pkv.NOALLOC_MAX_BYTES
    rc = L.pkv_attn_forward_noalloc(16, 32, 48, ctypes.byref(lay), 64, 64, 64, 1, 0.1, 80, 96, None)
    assert rc == pkv.PKV_ERR_WORKSPACE
    assert b"scratch" in L.pkv_last_error()
    # a layout that fits passes the size check; a NULL q is then reported, still before any device call
    small = good_layout(max_blocks_per_seq=128)   # 2048 keys: two chunks, partials in the scratch
    assert 0 < L.pkv_attn_workspace_size(ctypes.byref(small)) <= pkv.NOALLOC_MAX_BYTES
    assert L.pkv_attn_forward_noalloc(None, 32, 48, ctypes.byref(small), 64, 64, 64, 1, 0.1, 80, 96,
                                      None) == pkv.PKV_ERR_NULL
