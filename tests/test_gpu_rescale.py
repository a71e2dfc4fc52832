"""Parity where the running max of the online softmax grows after the first keys.

The online softmax keeps a running max m, a running sum l and an unnormalised
output o; when a later key scores above m, the method moves m and rescales l and
o by exp(m_old - m_new) ("mini-vLLM v0.4" section 5, the Triton decode kernel's
state update; the nano-vLLM lab manual, appendix B.5, Fig. B-5 rescaling).  With
N(0, 1) inputs at scale 1/sqrt(d) the first keys nearly always hold the row max,
so that update barely runs.  These inputs force it: each test changes the keys so
that later keys score far above every earlier key, checks on the host from its
own inputs that this happens for most rows (a later 64-key block beats the max of
all earlier keys by more than 12 log2 units, well past the prefill kernels'
8-unit lazy-rescale headroom, at block 2 or later so that the part of the key
range it falls in has already accumulated earlier keys), and then compares the
GPU output element by element with the oracle at the stated tolerance.

Three ways of making scores grow, each in bf16 and fp16:

* ``ramp``:  K rows scaled by 1 + 4 * (position // 64), so each 64-key block
  scores higher than the last;
* ``scale``: the softmax scale set to 1 (not 1/sqrt(d)) at d = 128, so scores
  spread over tens of units and later maxima often jump;
* ``low-first``: the first 150 keys scaled by 1/64 (scores near 0) and the rest
  by 5, so the max of the first keys is far below that of the rest.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_67_amd as pk
from paged_kv_cache_67_amd import harness
from tests.gpu_util import OracleRun, announce, assert_close, out_f64
from workloads import make_workload
from workloads.synth import bf16_bits_from_f32

pytestmark = pytest.mark.gpu

GROW_LOG2 = 12.0   # required jump of a later block's max over all earlier keys (log2 units)
BLOCK = 64


def _key_factor(kind, pos):
    pos = np.asarray(pos)
    if kind == "ramp":
        return 1.0 + 4.0 * (pos // BLOCK)
    if kind == "low-first":
        return np.where(pos < 150, 1.0 / 64.0, 5.0)
    return np.ones(pos.shape)


def _scale_rows(rows, factors, dtype):
    """rows [N, HKV, D] in storage bits, times a per-row factor, rounded back to the dtype."""
    x = oracle.to_f64(rows, dtype) * factors[:, None, None]
    if dtype == "bf16":
        return bf16_bits_from_f32(x.astype(np.float32))
    return x.astype(np.float16)


def _positions(w):
    """Logical positions of the history rows and of the new rows, in storage order."""
    hist = np.concatenate([np.arange(h) for h in w.hist_lens]) if w.num_seqs else np.zeros(0)
    new = np.concatenate([np.arange(w.seq_lens_k[b] - w.new_lens[b], w.seq_lens_k[b])
                          for b in range(w.num_seqs)])
    return hist.astype(np.int64), new.astype(np.int64)


def _apply(w, kind):
    if kind == "scale":
        w.scale = 1.0
        return w
    ph, pn = _positions(w)
    w.k_hist = _scale_rows(w.k_hist, _key_factor(kind, ph), w.dtype)
    w.k_new = _scale_rows(w.k_new, _key_factor(kind, pn), w.dtype)
    return w


def _growth(w, ref):
    """(hits, rows): over the (query row, head) pairs that see at least three 64-key
    blocks, how many have some block u >= 2 whose max score (log2 units, scale * q.k *
    log2 e) exceeds the max over all keys before it by more than GROW_LOG2.  Keys a query
    cannot see (causal) are left out."""
    G = w.num_q_heads // w.num_kv_heads
    qf = oracle.to_f64(w.q, w.dtype)
    hits = total = 0
    for b in range(w.num_seqs):
        lq, lk = int(w.new_lens[b]), int(w.seq_lens_k[b])
        if lq == 0:
            continue
        K = oracle.to_f64(oracle.gather_rows(ref.k_pool, w.block_table[b], lk, w.block_size), w.dtype)
        q0 = int(w.cu_seqlens_q[b])
        for h in range(w.num_q_heads):
            s = (qf[q0:q0 + lq, h] @ K[:, h // G].T) * (w.scale * math.log2(math.e))
            for i in range(lq):
                n = lk - lq + i + 1
                nb = -(-n // BLOCK)
                if nb < 3:
                    continue
                blk = np.full(nb * BLOCK, -np.inf)
                blk[:n] = s[i, :n]
                bm = blk.reshape(nb, BLOCK).max(axis=1)
                run = np.maximum.accumulate(bm)
                total += 1
                hits += bool(np.any(bm[2:] > run[1:-1] + GROW_LOG2))
    return hits, total


# (HQ, HKV, D, block_size, seq_lens_k, new_lens)
PREFILL_SHAPES = [
    (16, 8, 128, 256, [1280, 700], [256, 300]),
    (14, 2, 64, 16, [900, 260], [128, 260]),
]
KINDS = ["ramp", "scale", "low-first"]
MIN_FRACTION = {"ramp": 0.7, "scale": 0.1, "low-first": 0.7}
MIN_HITS = 16


def _prefill_workload(shape, dtype, kind, seed):
    HQ, HKV, D, bs, lk, lq = shape
    w = make_workload(name=f"grow-{kind}", kind="prefill", dtype=dtype, num_q_heads=HQ,
                      num_kv_heads=HKV, head_dim=D, block_size=bs, seq_lens_k=lk, new_lens=lq,
                      seed=seed)
    return _apply(w, kind)


# The scale case is defined at d = 128 only.
PREFILL_CASES = [(shape, kind) for shape in PREFILL_SHAPES for kind in KINDS
                 if kind != "scale" or shape[2] == 128]


@pytest.mark.parametrize("shape,kind", PREFILL_CASES,
                         ids=lambda c: c if isinstance(c, str) else f"{c[0]}q{c[1]}kv-d{c[2]}-bs{c[3]}")
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_prefill_and_mixed_with_growing_max(shape, kind, dtype):
    w = _prefill_workload(shape, dtype, kind, seed=300 + KINDS.index(kind))
    ref = OracleRun(w)
    hits, rows = _growth(w, ref)
    frac = hits / rows
    assert frac >= MIN_FRACTION[kind] and hits >= MIN_HITS, f"growth in {hits} of {rows} rows"
    want = ref.prefill(True)
    announce(f"prefill growing max {kind} {dtype} {shape} (growth in {frac:.2f} of rows)")
    dw = harness.DeviceWorkload(w, "cuda")
    dw.load_history()
    dw.slot_mapping()
    dw.store()
    dw.attention()
    torch.cuda.synchronize()
    assert_close(out_f64(dw.out, dtype), want, dtype, f"prefill {kind}")
    announce(f"mixed growing max {kind} {dtype} {shape}")
    dw.out.zero_()
    dw.attention_mixed()
    torch.cuda.synchronize()
    assert_close(out_f64(dw.out, dtype), want, dtype, f"mixed {kind}")


def test_prefill_growing_max_with_decode_rows_in_mixed_batch():
    """Prompt chunks with growing scores next to decode rows (Lq = 1) in one mixed launch."""
    w = make_workload(name="grow-mixed", kind="prefill", dtype="bf16", num_q_heads=16,
                      num_kv_heads=8, head_dim=128, block_size=256,
                      seq_lens_k=[1280, 3000, 1, 700, 2500], new_lens=[256, 1, 1, 200, 1], seed=311)
    w = _apply(w, "ramp")
    ref = OracleRun(w)
    hits, rows = _growth(w, ref)
    assert hits >= 0.9 * rows and hits >= MIN_HITS, (hits, rows)
    announce("mixed growing max with decode rows")
    dw = harness.DeviceWorkload(w, "cuda")
    dw.load_history()
    dw.slot_mapping()
    dw.store()
    dw.attention_mixed()
    torch.cuda.synchronize()
    assert_close(out_f64(dw.out, "bf16"), ref.prefill(True), "bf16", "mixed ramp")


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("partition", [0, 256, -1])
def test_decode_with_growing_max(kind, dtype, partition):
    w = make_workload(name=f"grow-dec-{kind}", kind="decode", dtype=dtype, num_q_heads=16,
                      num_kv_heads=8, head_dim=128, block_size=256,
                      seq_lens_k=[3000, 700, 4096, 129, 2000, 1500, 999, 3500], seed=320 + KINDS.index(kind))
    w = _apply(w, kind)
    ref = OracleRun(w)
    hits, rows = _growth(w, ref)
    frac = hits / rows
    assert frac >= MIN_FRACTION[kind] and hits >= MIN_HITS, (hits, rows)
    announce(f"decode growing max {kind} {dtype} partition {partition} (growth {frac:.2f})")
    dw = harness.DeviceWorkload(w, "cuda", partition_size=partition)
    dw.load_history()
    dw.step()
    torch.cuda.synchronize()
    assert_close(out_f64(dw.out, dtype), ref.decode(), dtype, f"decode {kind}")
