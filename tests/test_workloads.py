"""Properties of the seeded input generator (shapes, determinism, placement)."""

import numpy as np
import pytest
import torch

from workloads import bf16_bits_from_f32, make_config, make_workload


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(1 << 16).astype(np.float32) * 3
    x[:4] = [1.0 + 2**-8, 1.0 + 3 * 2**-8, -1.0 - 2**-8, 65504.0]  # ties and a big value
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits_from_f32(x), want)


@pytest.mark.parametrize("idx", [0, 1, 3, 4])
def test_config_shapes_and_placement(idx):
    w = make_config(idx)
    B, HQ, HKV, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim
    assert w.q.shape == (w.num_new_tokens, HQ, D)
    assert w.k_new.shape == (w.num_new_tokens, HKV, D) == w.v_new.shape
    assert w.k_hist.shape == (int(w.hist_lens.sum()), HKV, D) == w.v_hist.shape
    nblk = -(-w.seq_lens_k // w.block_size)
    used = []
    for b in range(B):
        row = w.block_table[b]
        assert np.all(row[:nblk[b]] >= 0) and np.all(row[nblk[b]:] == -1)
        used.extend(row[:nblk[b]].tolist())
    assert len(set(used)) == len(used), "a physical block is shared"
    assert max(used) < w.num_blocks
    assert w.cu_seqlens_q[-1] == w.new_lens.sum() and w.cu_seqlens_k[-1] == w.seq_lens_k.sum()


def test_named_sizes():
    c0 = make_config(0)
    assert c0.dtype == "f32" and c0.seq_lens_k.tolist() == [17, 33] and c0.num_blocks == 8
    assert c0.block_table.shape == (2, 3) and c0.scale == 1 / 8
    c1 = make_config(1)
    assert c1.block_table.shape == (64, 128) and c1.num_blocks == 10000
    assert c1.seq_lens_k.min() >= 1 and c1.seq_lens_k.max() <= 2048
    c3 = make_config(3)
    assert c3.num_blocks == 178 and c3.seq_lens_k.tolist() == [32768] + [512] * 7
    c4 = make_config(4)
    assert c4.num_blocks == 50 and c4.block_table.shape == (8, 5)
    assert c4.cu_seqlens_q.tolist() == list(range(0, 2049, 256))
    assert c4.cu_seqlens_k.tolist() == list(range(0, 10241, 1280))


def test_deterministic():
    a, b = make_config(1), make_config(1)
    for f in ("seq_lens_k", "block_table", "k_hist", "v_hist", "k_new", "v_new", "q"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c = make_config(1, seed=1)
    assert not np.array_equal(a.q, c.q)


def test_custom_workload_lengths():
    w = make_workload(name="t", kind="prefill", dtype="bf16", num_q_heads=4, num_kv_heads=2,
                      head_dim=64, block_size=16, seq_lens_k=[0, 5, 40], new_lens=[0, 5, 9], seed=3)
    assert w.cu_seqlens_q.tolist() == [0, 0, 5, 14]
    assert w.hist_lens.tolist() == [0, 0, 31]
    assert np.all(w.block_table[0] == -1)
