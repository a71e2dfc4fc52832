"""pa_decode_append: the decode step's store and attention in one call.

Against the oracle -- outputs to the dtype's tolerance, both pools bit for bit -- on the
decode workloads in every split mode, on the head tiles that store with a launch of their
own (fp16 tiles of 4, 6, 7 or 8 heads), on two head waves per KV head (one of them writes), and
on the edge rows: a key that
is the sequence's only one, empty rows (no row stored), keys on block and chunk boundaries;
and on both sides of the balanced split's 8192-sequence bound.
The pools start NaN-poisoned, so a read of the new row's slot before it is written shows.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_67_amd as pk
from paged_kv_cache_67_amd import harness
from workloads import make_config, make_workload
from tests.gpu_util import announce, assert_close, bits_equal, out_f64
from tests.test_gpu_parity import _random_decode_case

pytestmark = pytest.mark.gpu


def _oracle(w, ctx):
    """Pools after the history and the new rows of the rows with ctx >= 1, and the decode."""
    k_pool, v_pool = w.empty_pool(), w.empty_pool()
    hist = oracle.slot_mapping(w.block_table, w.cu_seqlens_hist, w.hist_lens, w.block_size)
    oracle.store_kv(k_pool, v_pool, w.k_hist, w.v_hist, hist)
    cu = np.arange(w.num_seqs + 1, dtype=np.int32)
    new = oracle.slot_mapping(w.block_table, cu, ctx, w.block_size)
    oracle.store_kv(k_pool, v_pool, w.k_new, w.v_new, new)
    want = oracle.decode(w.q, k_pool, v_pool, w.block_table, ctx, w.scale, w.dtype)
    return k_pool, v_pool, want


def _run(w, ctx, partition, two_pass=False, with_workspace=True):
    dw = harness.DeviceWorkload(w, "cuda", partition_size=partition, with_workspace=False)
    dw.load_history()
    ctx_t = torch.from_numpy(np.asarray(ctx, dtype=np.int32)).cuda()
    out = torch.full_like(dw.out, float("nan"))
    max_ctx = max(1, int(np.max(ctx)))
    nbytes = pk.pa_decode_workspace_size(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                         max_ctx, partition)
    ws = None
    if nbytes and with_workspace:
        ws = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device="cuda")
    args = (out, dw.q, dw.k_new, dw.v_new, dw.k_cache, dw.v_cache, dw.block_table, ctx_t, w.scale)
    if two_pass:
        pk.pa_decode_append_partitions(*args, max_ctx, partition, ws)
        pk.pa_decode_merge(out, ws, ctx_t, w.num_kv_heads, max_ctx, partition)
    else:
        pk.pa_decode_append(*args, max_context_len=max_ctx, partition_size=partition, workspace=ws)
    torch.cuda.synchronize()
    return dw, out


def _two_calls(w, ctx, partition):
    """The same step as pa_store_kv_paged + pa_decode (the results pa_decode_append promises)."""
    dw = harness.DeviceWorkload(w, "cuda", partition_size=partition, with_workspace=False)
    dw.load_history()
    ctx_t = torch.from_numpy(np.asarray(ctx, dtype=np.int32)).cuda()
    cu = torch.arange(w.num_seqs + 1, dtype=torch.int32, device="cuda")
    pk.pa_store_kv_paged(dw.k_new, dw.v_new, dw.k_cache, dw.v_cache, dw.block_table, cu, ctx_t, 1)
    out = torch.full_like(dw.out, float("nan"))
    max_ctx = max(1, int(np.max(ctx)))
    nbytes = pk.pa_decode_workspace_size(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                         max_ctx, partition)
    ws = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device="cuda") if nbytes else None
    pk.pa_decode(out, dw.q, dw.k_cache, dw.v_cache, dw.block_table, ctx_t, w.scale,
                 max_context_len=max_ctx, partition_size=partition, workspace=ws)
    torch.cuda.synchronize()
    return out


def _check(w, ctx, partition, what, two_pass=False, with_workspace=True, bitwise=False):
    dw, out = _run(w, ctx, partition, two_pass, with_workspace)
    k_pool, v_pool, want = _oracle(w, np.asarray(ctx, dtype=np.int32))
    assert bits_equal(harness.from_device(dw.k_cache), k_pool), f"{what}: K pool"
    assert bits_equal(harness.from_device(dw.v_cache), v_pool), f"{what}: V pool"
    assert_close(out_f64(out, w.dtype), want, w.dtype, what)
    if bitwise:  # and the two calls' rows bit for bit
        assert torch.equal(out, _two_calls(w, ctx, partition)), f"{what}: differs from two calls"
    return out


@pytest.mark.parametrize("idx,partition", [(0, 0), (0, -1), (0, 16), (1, 0), (1, -1), (1, 64),
                                           (2, 0), (3, 0), (3, -1), (3, 256)])
def test_append_workloads(idx, partition):
    """The decode workloads (tiny fp32, Qwen2.5-0.5B batch 64 with 7-head tiles, the full
    Qwen3-0.6B batch 256, the skewed batch) in the balanced split, a single pass and fixed
    partitions."""
    w = make_config(idx)
    announce(f"pa_decode_append on {w.name}, partition {partition}")
    _check(w, w.seq_lens_k, partition, f"{w.name} p{partition}")


EDGE_CASES = [
    # dtype, HQ, HKV, D, block_size, context lengths (0 = empty row: nothing stored)
    ("bf16", 16, 8, 128, 256, [0, 1, 2, 15, 16, 17, 0, 300, 4000, 1, 1, 33, 0, 2048, 5, 256, 257]),
    ("bf16", 4, 2, 64, 16, [1, 0, 7, 16, 17, 32, 33, 1000, 0, 64, 65, 1, 2]),
    ("f16", 10, 2, 128, 8, [1, 8, 9, 0, 100, 2, 1, 513]),          # 5-head tiles
    ("bf16", 12, 2, 128, 32, [1, 0, 31, 32, 33, 900]),              # 6-head tiles
    ("f16", 16, 2, 128, 32, [1, 0, 31, 32, 33, 900]),               # fp16 8-head tiles: own store launch
    ("f16", 8, 1, 64, 16, [1, 0, 2, 15, 16, 17, 500]),              # fp16 8-head tiles, d64
    ("f32", 16, 2, 64, 16, [1, 0, 2, 17, 300, 1, 64]),              # 8-head tiles in fp32
    ("f32", 32, 2, 64, 16, [1, 0, 2, 17, 300, 1, 64]),              # two head waves per KV head
    ("bf16", 32, 2, 128, 64, [1, 0, 2, 65, 1200, 1]),               # group 16: two head waves
    ("bf16", 8, 1, 128, 32, [1] * 40 + [3000]),                     # many one-key rows
]


@pytest.mark.parametrize("case", EDGE_CASES,
                         ids=lambda c: f"{c[0]}-{c[1]}q{c[2]}kv-d{c[3]}-bs{c[4]}-n{len(c[5])}")
@pytest.mark.parametrize("partition", [0, -1, 32])
def test_append_edge_rows(case, partition):
    dtype, HQ, HKV, D, bs, lens = case
    lens = np.array(lens, dtype=np.int32)
    w = make_workload(name="append-edges", kind="decode", dtype=dtype, num_q_heads=HQ,
                      num_kv_heads=HKV, head_dim=D, block_size=bs, seq_lens_k=np.maximum(lens, 1),
                      seed=500 + EDGE_CASES.index(case))
    announce(f"pa_decode_append edge rows {case[:5]} partition {partition}")
    _check(w, lens, partition, f"{case[:5]} p{partition}", bitwise=True)


@pytest.mark.parametrize("partition", [0, 64])
def test_append_two_passes_equal_one_call(partition):
    """pa_decode_append_partitions + pa_decode_merge gives pa_decode_append's rows bit for
    bit (and the oracle's within tolerance)."""
    w = make_config(3)
    announce(f"pa_decode_append in two passes, partition {partition}")
    one = _check(w, w.seq_lens_k, partition, "one call")
    two = _check(w, w.seq_lens_k, partition, "two passes", two_pass=True)
    assert torch.equal(one, two)


def test_append_without_workspace_is_a_single_pass():
    w = make_config(1)
    announce("pa_decode_append without a workspace")
    _check(w, w.seq_lens_k, 0, "no workspace", with_workspace=False)


@pytest.mark.parametrize("seed", list(range(16)))
def test_append_random_shapes(seed):
    """The seeded random decode batches of the decode parity suite (GQA 1-8 or 16, d 64 / 128,
    block 8-512, batch 1-300 with short, empty and long rows, three dtypes, every split); the
    rows also equal store + decode bit for bit."""
    c = _random_decode_case(4000 + seed)
    lens = np.array(c["lens"], dtype=np.int32)
    w = make_workload(name="rand-append", kind="decode", dtype=c["dtype"],
                      num_q_heads=c["G"] * c["HKV"], num_kv_heads=c["HKV"], head_dim=c["D"],
                      block_size=c["bs"], seq_lens_k=np.maximum(lens, 1), seed=seed)
    announce(f"random append case {seed}: " + str({k: v for k, v in c.items() if k != "lens"}) +
             f" B={len(lens)} max={int(lens.max())}")
    _check(w, lens, c["P"], str(c), bitwise=True)


@pytest.mark.parametrize("B", [8192, 8193])
def test_append_at_the_balanced_batch_bound(B):
    """Both sides of the balanced split's batch bound: 8192 short sequences take the
    balanced first pass with the store folded in (many sequences per slice, each ending in
    it), 8193 take fixed partitions after a store launch.  Pools bit for bit, rows against
    the oracle and bit for bit against store + pa_decode; empty rows mixed in."""
    rng = np.random.default_rng(B + 1)
    lens = rng.integers(0, 40, size=B, endpoint=True).astype(np.int32)
    w = make_workload(name=f"append-b{B}", kind="decode", dtype="bf16", num_q_heads=14,
                      num_kv_heads=2, head_dim=64, block_size=16, seq_lens_k=np.maximum(lens, 1),
                      seed=B % 991)
    announce(f"pa_decode_append at the balanced batch bound: B={B}")
    _check(w, lens, 0, f"B={B}", bitwise=True)
