"""pa_decode_noalloc (split-K states in the library's own device array) against pa_decode.

Each call is compared with pa_decode on the same inputs (bitwise: the same kernels run
on the same states, only the scratch memory differs) and with the oracle at the bf16
tolerance.  Two calls in a row share the array, the second with a smaller batch, so
states left by the first cannot leak into the second; a request larger than the array is
refused without disturbing the next call.
"""

import numpy as np
import pytest
import torch

import paged_kv_cache_67_amd as pk
from paged_kv_cache_67_amd import harness
from tests.gpu_util import OracleRun, announce, assert_close, bits_equal, out_f64
from workloads import make_config, make_workload

pytestmark = pytest.mark.gpu


def _both(w, partition):
    dw = harness.DeviceWorkload(w, "cuda", partition_size=partition)
    dw.load_history()
    dw.step()  # slot mapping, store, pa_decode with a caller workspace -> dw.out
    out = torch.full_like(dw.out, float("nan"))
    pk.pa_decode_noalloc(out, dw.q, dw.k_cache, dw.v_cache, dw.block_table, dw.seq_lens_k, w.scale,
                         max_context_len=w.max_seqlen_k, partition_size=partition)
    torch.cuda.synchronize()
    return harness.from_device(dw.out), harness.from_device(out), out_f64(out, w.dtype)


@pytest.mark.parametrize("partition", [0, 1024])
def test_noalloc_equals_pa_decode_on_two_calls(partition):
    first = make_config(2)  # Qwen3-0.6B decode, 256 sequences, contexts up to 4096
    second = make_workload(name="small", kind="decode", dtype="bf16", num_q_heads=16,
                           num_kv_heads=8, head_dim=128, block_size=256,
                           seq_lens_k=[5, 300, 1024, 77], seed=71)
    for i, w in enumerate((first, second)):
        announce(f"pa_decode_noalloc call {i + 1}: {w.name}, {w.num_seqs} sequences, partition {partition}")
        want_bits, got_bits, got = _both(w, partition)
        assert bits_equal(got_bits, want_bits), f"call {i + 1}: differs from pa_decode"
        assert_close(got, OracleRun(w).decode(), w.dtype, f"call {i + 1}")


def test_noalloc_refuses_an_oversized_split_then_runs():
    # the split is sized from the host bound max_context_len: 64 x 16 heads x 256 partitions
    # of 16 tokens x (128 + 2) floats = 136 MB of states, more than the array holds
    w = make_workload(name="big", kind="decode", dtype="bf16", num_q_heads=16, num_kv_heads=8,
                      head_dim=128, block_size=256, seq_lens_k=[16] * 64, seed=72)
    dw = harness.DeviceWorkload(w, "cuda", with_workspace=False)
    assert pk.pa_decode_workspace_size(64, 16, 8, 128, 4096, 16) > 16 << 20
    announce("pa_decode_noalloc refusal (fixed 16-token partitions, max_context_len 4096)")
    with pytest.raises(pk.PAError) as e:
        pk.pa_decode_noalloc(dw.out, dw.q, dw.k_cache, dw.v_cache, dw.block_table, dw.seq_lens_k,
                             w.scale, max_context_len=4096, partition_size=16)
    assert e.value.status == 5
    small = make_workload(name="after", kind="decode", dtype="bf16", num_q_heads=14,
                          num_kv_heads=2, head_dim=64, block_size=16, seq_lens_k=[9, 2048, 700],
                          seed=73)
    announce("pa_decode_noalloc after a refusal")
    want_bits, got_bits, got = _both(small, 0)
    assert bits_equal(got_bits, want_bits)
    assert_close(got, OracleRun(small).decode(), small.dtype, "after refusal")
