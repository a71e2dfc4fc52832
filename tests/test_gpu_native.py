"""Native C++ callers of the C ABI: tests/native/decode_step and prefill_step, built with g++
from include/pa.h and linked to libpa.so, with no Python in their processes.

decode_step runs a decode step on the GPU -- pa_store_kv_paged then pa_decode, or
pa_decode_append -- and prefill_step a chunked-prefill step (pa_store_kv_paged of the chunk,
then pa_prefill_paged), each from a file of seeded inputs.  Output rows must match the oracle
to the dtype's tolerance, both pools must equal the oracle's bit for bit, and the two decode
forms must give the same rows bit for bit.  The CPU test only checks that the programs link
and start.
"""

import os
import subprocess

import numpy as np
import pytest

import oracle
import paged_kv_cache_67_amd as pk
from tests.gpu_util import OracleRun, announce, assert_close, bits_equal
from tests.native import build as native
from tests.test_gpu_append import _oracle
from workloads import make_config, make_workload

DTYPE_CODE = {"f32": 0, "bf16": 1, "f16": 2}


def _program(name: str = "decode_step") -> str:
    if not os.path.exists(pk.lib_path()):
        from paged_kv_cache_67_amd import build
        build.build()
    exe = os.path.join(native.HERE, name)
    if not os.path.exists(exe) or os.path.getmtime(exe) < os.path.getmtime(exe + ".cpp"):
        native.build()
    return exe


@pytest.mark.parametrize("name", native.PROGRAMS)
def test_native_caller_links_and_starts(name):
    r = subprocess.run([_program(name)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr, (r.returncode, r.stderr)


def _write_input(path, w, ctx, mode):
    k_pool, v_pool = w.empty_pool(), w.empty_pool()
    hist = oracle.slot_mapping(w.block_table, w.cu_seqlens_hist, w.hist_lens, w.block_size)
    oracle.store_kv(k_pool, v_pool, w.k_hist, w.v_hist, hist)
    hdr = np.array([w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                    w.num_blocks, w.max_blocks_per_seq, max(1, int(np.max(ctx))),
                    DTYPE_CODE[w.dtype], mode], dtype=np.int32)
    with open(path, "wb") as f:
        for a in (hdr, np.array([w.scale], dtype=np.float32), w.q, w.k_new, w.v_new, k_pool,
                  v_pool, w.block_table.astype(np.int32), np.asarray(ctx, dtype=np.int32)):
            f.write(np.ascontiguousarray(a).tobytes())


def _run_native(tmp_path, w, ctx, mode):
    src, dst = tmp_path / f"in{mode}.bin", tmp_path / f"out{mode}.bin"
    _write_input(src, w, ctx, mode)
    announce(f"native decode_step mode {mode} on {w.name}")
    r = subprocess.run([_program(), str(src), str(dst)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, f"decode_step exit {r.returncode}: {r.stderr}"
    raw = np.fromfile(dst, dtype=w.q.dtype)
    n_out, n_pool = w.q.size, int(np.prod(w.pool_shape))
    assert raw.size == n_out + 2 * n_pool
    return (raw[:n_out].reshape(w.q.shape), raw[n_out:n_out + n_pool].reshape(w.pool_shape),
            raw[n_out + n_pool:].reshape(w.pool_shape))


def _edge_workload():
    lens = np.array([1, 0, 7, 16, 17, 300, 0, 1, 2049, 33], dtype=np.int32)
    w = make_workload(name="native-edges", kind="decode", dtype="f16", num_q_heads=10,
                      num_kv_heads=2, head_dim=128, block_size=16,
                      seq_lens_k=np.maximum(lens, 1), seed=811)
    return w, lens


@pytest.mark.gpu
@pytest.mark.parametrize("which", ["tiny-f32", "qwen2.5-0.5b-b64", "edges-f16"])
def test_native_decode_step(tmp_path, which):
    if which == "edges-f16":
        w, ctx = _edge_workload()
    else:
        w = make_config(0 if which == "tiny-f32" else 1)
        ctx = w.seq_lens_k
    k_want, v_want, want = _oracle(w, np.asarray(ctx, dtype=np.int32))
    outs = []
    for mode in (0, 1):  # pa_store_kv_paged + pa_decode, then pa_decode_append
        out, k_pool, v_pool = _run_native(tmp_path, w, ctx, mode)
        assert bits_equal(k_pool, k_want), f"{which} mode {mode}: K pool"
        assert bits_equal(v_pool, v_want), f"{which} mode {mode}: V pool"
        assert_close(oracle.to_f64(out, w.dtype), want, w.dtype, f"{which} mode {mode}")
        outs.append(out)
    assert bits_equal(outs[0], outs[1]), f"{which}: pa_decode_append differs from the two calls"


def _history_pools(w):
    k_pool, v_pool = w.empty_pool(), w.empty_pool()
    hist = oracle.slot_mapping(w.block_table, w.cu_seqlens_hist, w.hist_lens, w.block_size)
    oracle.store_kv(k_pool, v_pool, w.k_hist, w.v_hist, hist)
    return k_pool, v_pool


@pytest.mark.gpu
@pytest.mark.parametrize("which", ["qwen3-0.6b-chunked-prefill", "edges-f16"])
@pytest.mark.parametrize("causal", [1, 0])
def test_native_prefill_step(tmp_path, which, causal):
    if which == "edges-f16":  # an empty chunk, a one-token sequence, a prompt with no prefix
        w = make_workload(name="native-prefill-edges", kind="prefill", dtype="f16",
                          num_q_heads=16, num_kv_heads=2, head_dim=128, block_size=32,
                          seq_lens_k=[300, 40, 1, 700, 33], new_lens=[100, 0, 1, 700, 5], seed=812)
    else:
        w = make_config(4)
    ref = OracleRun(w)
    want = ref.prefill(bool(causal))
    k_hist, v_hist = _history_pools(w)
    hdr = np.array([w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                    w.num_blocks, w.max_blocks_per_seq, w.num_new_tokens, w.max_seqlen_q,
                    w.max_seqlen_k, DTYPE_CODE[w.dtype], causal], dtype=np.int32)
    src, dst = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(src, "wb") as f:
        for a in (hdr, np.array([w.scale], dtype=np.float32), w.q, w.k_new, w.v_new, k_hist,
                  v_hist, w.block_table.astype(np.int32), w.cu_seqlens_q, w.cu_seqlens_k,
                  w.seq_lens_k):
            f.write(np.ascontiguousarray(a).tobytes())
    announce(f"native prefill_step on {w.name}, causal {causal}")
    r = subprocess.run([_program("prefill_step"), str(src), str(dst)], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, f"prefill_step exit {r.returncode}: {r.stderr}"
    raw = np.fromfile(dst, dtype=w.q.dtype)
    n_out, n_pool = w.q.size, int(np.prod(w.pool_shape))
    assert raw.size == n_out + 2 * n_pool
    assert bits_equal(raw[n_out:n_out + n_pool].reshape(w.pool_shape), ref.k_pool), "K pool"
    assert bits_equal(raw[n_out + n_pool:].reshape(w.pool_shape), ref.v_pool), "V pool"
    got = oracle.to_f64(raw[:n_out].reshape(w.q.shape), w.dtype)
    assert_close(got, want, w.dtype, f"{w.name} causal {causal}")
