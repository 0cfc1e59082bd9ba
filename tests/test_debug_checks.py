"""The device-data precondition checks of debug mode, run on the host.

pkv_check_inputs evaluates, on host copies of the index data, the same
function (csrc/pkv_checks.h) that debug mode's check kernel runs on the
device before a call's kernels.  The pages' stride bug read memory outside a
sequence's blocks and produced garbage with no error (ROCm/aiter commit
d293d61bbf19, commit message); these checks turn bad index data into an
error.  Each case breaks one precondition and expects its flag, and checks
that entries the call never reads are not flagged.
"""

from __future__ import annotations

import pytest
import torch

import invariant_paged_kv_amd as pkv

BATCH, MBPS, BS, NB = 3, 4, 16, 12


def layout_tensors():
    pool = torch.zeros(NB, 2, BS, 2, 64, dtype=torch.bfloat16)
    return pool[:, 0], pool[:, 1]


def run(bt, sk, cu, total, op=pkv.PKV_CHECK_ATTENTION, max_q=3, max_k=0):
    k, v = layout_tensors()
    pkv.check_inputs(k, v, torch.tensor(bt, dtype=torch.int32), torch.tensor(sk, dtype=torch.int32),
                     torch.tensor(cu, dtype=torch.int32), num_heads_q=4, max_seqlen_q=max_q, total_rows=total, op=op,
                     max_seqlen_k=max_k)


GOOD_BT = [[0, 1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11]]


def expect(flag_text, first, *args, **kw):
    with pytest.raises(pkv.PkvError) as ei:
        run(*args, **kw)
    assert ei.value.code == pkv.PKV_ERR_DEVICE_DATA
    assert flag_text in str(ei.value), str(ei.value)
    assert f"first at sequence {first}" in str(ei.value), str(ei.value)


def test_valid_inputs_pass():
    run(GOOD_BT, [10, 64, 0], [0, 1, 3, 3], 3)
    run(GOOD_BT, [10, 64, 5], [0, 1, 3, 5], 5, op=pkv.PKV_CHECK_APPEND)
    run(GOOD_BT, [10, 60, 0], [0, 2, 6, 9], 9, op=pkv.PKV_CHECK_CACHE_WRITE)


def test_cumulative_counts():
    expect("cu_seqlens", 0, GOOD_BT, [10, 10, 10], [1, 1, 2, 3], 3)    # cu[0] != 0
    expect("cu_seqlens", 1, GOOD_BT, [10, 10, 10], [0, 2, 1, 3], 3)    # decreasing
    expect("cu_seqlens", 2, GOOD_BT, [10, 10, 10], [0, 1, 2, 3], 4)    # cu[batch] != total_q
    expect("cu_seqlens", 1, GOOD_BT, [10, 10, 10], [0, 1, 9, 3], 3)    # beyond total_q


def test_rows_and_key_counts():
    expect("rows>max_seqlen_q", 1, GOOD_BT, [10, 10, 10], [0, 1, 5, 6], 6, max_q=3)
    expect("seqlens_k", 2, GOOD_BT, [10, 10, -1], [0, 1, 2, 3], 3)
    expect("seqlens_k", 1, GOOD_BT, [10, 65, 10], [0, 1, 2, 3], 3)           # > max_blocks_per_seq * bs
    expect("seqlens_k", 0, GOOD_BT, [40, 10, 10], [0, 1, 2, 3], 3, max_k=32)  # > declared max_seqlen_k
    run(GOOD_BT, [32, 10, 10], [0, 1, 2, 3], 3, max_k=32)


def test_block_ids_only_where_read():
    bad = [row[:] for row in GOOD_BT]
    bad[1][1] = NB            # used by 17+ keys
    expect("block_id", 1, bad, [10, 17, 10], [0, 1, 2, 3], 3)
    run(bad, [10, 16, 10], [0, 1, 2, 3], 3)          # 16 keys read entry 0 only
    bad[2][0] = -5
    expect("block_id", 2, bad, [10, 16, 10], [0, 1, 2, 3], 3)
    run(bad, [10, 16, 10], [0, 1, 2, 2], 2)          # sequence 2 has no rows: nothing of it is read


def test_append_rows_within_keys():
    expect("append_rows>keys", 0, GOOD_BT, [1, 10, 10], [0, 2, 3, 4], 4, op=pkv.PKV_CHECK_APPEND)
    run(GOOD_BT, [1, 10, 10], [0, 2, 3, 4], 4)       # fine for a plain forward (row at position < 0)


def test_cache_write_positions():
    # seqlens_k are the counts before the append: sequence 1 writes positions 60..67 of a 64-key table
    expect("write_position", 1, GOOD_BT, [0, 60, 0], [0, 1, 9, 9], 9, op=pkv.PKV_CHECK_CACHE_WRITE)
    bad = [row[:] for row in GOOD_BT]
    bad[0][2] = 99
    expect("block_id", 0, bad, [30, 0, 0], [0, 4, 4, 4], 4, op=pkv.PKV_CHECK_CACHE_WRITE)   # 30..33 -> entries 1, 2
    run(bad, [20, 0, 0], [0, 4, 4, 4], 4, op=pkv.PKV_CHECK_CACHE_WRITE)                     # 20..23 -> entry 1 only


def test_unknown_op_and_null():
    k, v = layout_tensors()
    lay = pkv.make_layout(k, v, torch.zeros(BATCH, MBPS, dtype=torch.int32), 4, 1, 3)
    L = pkv.lib()
    assert L.pkv_check_inputs(lay, None, None, None, 3, 0) == pkv.PKV_ERR_NULL
    sk = torch.zeros(BATCH, dtype=torch.int32)
    assert L.pkv_check_inputs(lay, sk.data_ptr(), sk.data_ptr(), sk.data_ptr(), 3, 7) == pkv.PKV_ERR_OPTION
