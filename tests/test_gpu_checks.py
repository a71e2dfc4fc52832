"""Debug checks of the device-side contract (pa_check_*) and the entry points with the
checks switched on.

The checkers copy the metadata to the host and check it there; no kernel is ever
launched on metadata that breaks the contract (with the checks on, the entry point
returns before its launch).
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_67_amd as pk
from paged_kv_cache_67_amd import harness
from tests.gpu_util import announce
from workloads import make_workload

pytestmark = pytest.mark.gpu

CONTRACT = 8


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def _status(excinfo):
    return excinfo.value.status


def test_check_store_inputs():
    announce("pa_check_store_inputs")
    pk.pa_check_store_inputs(_i32([0, 5, -1, 63, -1]), num_blocks=4, block_size=16)
    pk.pa_check_store_inputs(_i32([]), num_blocks=4, block_size=16)
    with pytest.raises(pk.PAError) as e:
        pk.pa_check_store_inputs(_i32([0, 64]), num_blocks=4, block_size=16)
    assert _status(e) == CONTRACT and "slot_mapping[1] = 64" in str(e.value)
    with pytest.raises(pk.PAError) as e:
        pk.pa_check_store_inputs(_i32([3, -2]), num_blocks=4, block_size=16)
    assert _status(e) == CONTRACT
    with pytest.raises(pk.PAError) as e:
        pk.pa_check_store_inputs(_i32([7, -1, 9, 7]), num_blocks=4, block_size=16)
    assert _status(e) == CONTRACT and "slot 7 appears twice" in str(e.value)


def test_check_decode_inputs():
    announce("pa_check_decode_inputs")
    bt = np.array([[2, 0, -1], [1, -1, -1]])
    # a -1 past a sequence's live blocks is fine
    pk.pa_check_decode_inputs(_i32(bt), _i32([17, 16]), num_blocks=3, block_size=16)
    pk.pa_check_decode_inputs(_i32(bt), _i32([0, 1]), num_blocks=3, block_size=16)
    with pytest.raises(pk.PAError) as e:  # 17 tokens need two blocks, row 1 has one
        pk.pa_check_decode_inputs(_i32(bt), _i32([17, 17]), num_blocks=3, block_size=16)
    assert _status(e) == CONTRACT and "block_table[1][1] = -1" in str(e.value)
    with pytest.raises(pk.PAError) as e:  # block id past the pool
        pk.pa_check_decode_inputs(_i32([[3, 0, 0]]), _i32([5]), num_blocks=3, block_size=16)
    assert _status(e) == CONTRACT
    with pytest.raises(pk.PAError) as e:  # longer than max_context_len
        pk.pa_check_decode_inputs(_i32(bt), _i32([17, 16]), num_blocks=3, block_size=16,
                                  max_context_len=16)
    assert _status(e) == CONTRACT and "context_lens[0] = 17" in str(e.value)
    with pytest.raises(pk.PAError) as e:  # longer than the table rows
        pk.pa_check_decode_inputs(_i32(bt), _i32([49, 1]), num_blocks=3, block_size=16)
    assert _status(e) == CONTRACT
    with pytest.raises(pk.PAError) as e:
        pk.pa_check_decode_inputs(_i32(bt), _i32([-1, 1]), num_blocks=3, block_size=16)
    assert _status(e) == CONTRACT


def test_check_prefill_inputs():
    announce("pa_check_prefill_inputs")
    bt = _i32([[0, 1, -1], [2, -1, -1]])
    ok = dict(total_q=7, max_seqlen_q=5, max_seqlen_k=20, num_blocks=3, block_size=16)
    pk.pa_check_prefill_inputs(bt, _i32([0, 5, 7]), _i32([0, 20, 22]), **ok)

    def bad(cq, ck, needle, **kw):
        args = dict(ok, **kw)
        with pytest.raises(pk.PAError) as e:
            pk.pa_check_prefill_inputs(bt, _i32(cq), _i32(ck), **args)
        assert _status(e) == CONTRACT and needle in str(e.value), str(e.value)

    bad([0, 5, 4], [0, 20, 22], "decrease")
    bad([0, 5, 7], [0, 4, 6], "fewer keys")
    bad([0, 5, 7], [0, 20, 22], "5 queries", max_seqlen_q=4)
    bad([0, 5, 7], [0, 20, 22], "outside [0, 6]", total_q=6)
    bad([0, 5, 7], [0, 20, 40], "block_table[1][1] = -1", max_seqlen_k=40)
    bad([0, 5, 7], [0, 49, 51], "needs 4 blocks", max_seqlen_k=60)  # rows hold 3 blocks
    with pytest.raises(pk.PAError) as e:
        pk.pa_check_prefill_inputs(_i32([[0, 5, -1]]), _i32([0, 5]), _i32([0, 20]), **ok)
    assert _status(e) == CONTRACT and "block_table[0][1] = 5" in str(e.value)


def test_check_store_paged_inputs():
    announce("pa_check_store_paged_inputs")
    bt = _i32([[0, 1, -1], [2, -1, -1]])
    # sequence 0: 2 new tokens at positions 18, 19 (block 1); sequence 1: 1 at position 4
    pk.pa_check_store_paged_inputs(bt, _i32([0, 2, 3]), _i32([20, 5]), num_tokens=3,
                                   num_blocks=3, block_size=16)
    # unmapped tokens (a -1 entry, a position past the row) write nothing and pass
    pk.pa_check_store_paged_inputs(bt, _i32([0, 2, 3]), _i32([20, 60]), num_tokens=3,
                                   num_blocks=3, block_size=16)
    with pytest.raises(pk.PAError) as e:  # both sequences' new tokens land in block 1, row 3
        pk.pa_check_store_paged_inputs(_i32([[0, 1, -1], [1, -1, -1]]), _i32([0, 2, 3]),
                                       _i32([20, 4]), num_tokens=3, num_blocks=3, block_size=16)
    assert _status(e) == CONTRACT and "slot 19 written twice" in str(e.value), str(e.value)
    with pytest.raises(pk.PAError) as e:
        pk.pa_check_store_paged_inputs(bt, _i32([0, 2, 1]), _i32([20, 5]), num_tokens=3,
                                       num_blocks=3, block_size=16)
    assert _status(e) == CONTRACT and "decreases" in str(e.value)
    with pytest.raises(pk.PAError) as e:
        pk.pa_check_store_paged_inputs(bt, _i32([0, 2, 4]), _i32([20, 5]), num_tokens=3,
                                       num_blocks=3, block_size=16)
    assert _status(e) == CONTRACT and "outside [0, 3]" in str(e.value)


@pytest.fixture()
def checks_on():
    prev = pk.pa_set_debug_checks(True)
    try:
        yield
    finally:
        pk.pa_set_debug_checks(prev)


def test_entry_points_check_before_launch(checks_on):
    """With the checks on, the entry points refuse broken metadata before any launch and
    compute the same bits as with them off on good metadata."""
    announce("debug checks on: decode, store and prefill")
    w = make_workload(name="dbg", kind="decode", dtype="bf16", num_q_heads=4, num_kv_heads=2,
                      head_dim=64, block_size=16, seq_lens_k=[40, 1, 17], seed=11)
    dw = harness.DeviceWorkload(w, "cuda")
    dw.load_history()
    dw.slot_mapping()
    dw.store()
    dw.attention()
    torch.cuda.synchronize()
    got = dw.out.clone()
    bad_bt = dw.block_table.clone()
    bad_bt[0, 1] = w.num_blocks  # a live block past the pool
    with pytest.raises(pk.PAError) as e:
        pk.pa_decode(dw.out, dw.q, dw.k_cache, dw.v_cache, bad_bt, dw.seq_lens_k, w.scale,
                     max_context_len=dw.max_context_len, workspace=dw.workspace)
    assert _status(e) == CONTRACT
    bad_slots = dw.slots_new.clone()
    bad_slots[1] = bad_slots[0]
    with pytest.raises(pk.PAError) as e:
        pk.pa_store_kv(dw.k_new, dw.v_new, dw.k_cache, dw.v_cache, bad_slots)
    assert _status(e) == CONTRACT
    twin_bt = dw.block_table.clone()
    twin_bt[2] = twin_bt[0]  # sequences 0 and 2 (40 and 17 tokens) share blocks
    twin_lens = dw.seq_lens_k.clone()
    twin_lens[2] = 40  # so their new tokens map to one slot
    with pytest.raises(pk.PAError) as e:
        pk.pa_store_kv_paged(dw.k_new, dw.v_new, dw.k_cache, dw.v_cache, twin_bt, dw.cu_q,
                             twin_lens, 1, dw.slots_new)
    assert _status(e) == CONTRACT and "written twice" in str(e.value)
    # pa_decode_append: the decode check first, then no two new rows in one slot
    with pytest.raises(pk.PAError) as e:
        pk.pa_decode_append(dw.out, dw.q, dw.k_new, dw.v_new, dw.k_cache, dw.v_cache, bad_bt,
                            dw.seq_lens_k, w.scale, max_context_len=dw.max_context_len,
                            workspace=dw.workspace)
    assert _status(e) == CONTRACT and "block_table[0][1]" in str(e.value), str(e.value)
    with pytest.raises(pk.PAError) as e:
        pk.pa_decode_append(dw.out, dw.q, dw.k_new, dw.v_new, dw.k_cache, dw.v_cache, twin_bt,
                            twin_lens, w.scale, max_context_len=dw.max_context_len,
                            workspace=dw.workspace)
    assert _status(e) == CONTRACT and "share slot" in str(e.value), str(e.value)
    pk.pa_decode_append(dw.out, dw.q, dw.k_new, dw.v_new, dw.k_cache, dw.v_cache, dw.block_table,
                        dw.seq_lens_k, w.scale, max_context_len=dw.max_context_len,
                        workspace=dw.workspace)
    torch.cuda.synchronize()
    assert torch.equal(got, dw.out)

    assert pk.pa_set_debug_checks(False)
    try:
        dw.out.zero_()
        dw.attention()
        torch.cuda.synchronize()
    finally:
        pk.pa_set_debug_checks(True)
    assert torch.equal(got, dw.out)

    wp = make_workload(name="dbgp", kind="prefill", dtype="bf16", num_q_heads=4, num_kv_heads=2,
                       head_dim=64, block_size=16, seq_lens_k=[40, 20], new_lens=[8, 20], seed=12)
    dp = harness.DeviceWorkload(wp, "cuda")
    dp.load_history()
    dp.slot_mapping()
    dp.store()
    bad_cu = dp.cu_k.clone()
    bad_cu[1] = 7  # fewer keys than queries for sequence 0
    with pytest.raises(pk.PAError) as e:
        pk.pa_prefill_paged(dp.out, dp.q, dp.k_cache, dp.v_cache, dp.block_table, dp.cu_q, bad_cu,
                            wp.max_seqlen_q, wp.max_seqlen_k, wp.scale)
    assert _status(e) == CONTRACT
    dp.attention()
    torch.cuda.synchronize()
    assert torch.isfinite(dp.out.float()).all()
