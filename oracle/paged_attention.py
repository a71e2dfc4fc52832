"""Plain float64 oracle of the paged-attention hot path.  TEST INFRASTRUCTURE ONLY.

Sources (web pages; cited below by the short name in brackets):

* [Lab]      "5. 动手改造：从跑通到可测量的推理服务" -- the nano-vLLM inference lab
             manual (duanmeng.github.io, 实验手册.html), chapter 5 and appendix B.
* [mini]     "mini-vLLM v0.4 -- From-Scratch LLM Inference Serving Runtime"
             (shadowgraph.io/WJX3078/mini-vllm), sections 5 and 9.
* [MinivLLM] "MinivLLM：六步搭出一个 Qwen3 推理引擎，再核清四处文档与代码的分岔"
             (txtmix.com), section "注意力内核的三个分支".
* [KVblog]   "大模型推理引擎学习入门-2：带你理解 nano-vllm 的 KV Cache 以及 Paged
             Attention" (juejin.cn), sections 3.1 and 3.5 and the decode log of 4.4.

What each function is pinned by (tests/test_oracle_pins.py, tests/golden/):

* ``slot_mapping``   -- the worked slot examples of [Lab] B.2.3 and the
                        prefill/decode logs of [KVblog] 3.5 and 4.4; the
                        lifecycle / chunk / prefix metadata of [Lab] B.2.2, B.3,
                        B.6.  Pinned.
* ``store_kv``       -- inverse property (gathering back through the slots
                        returns the rows), -1 rows leave the pool untouched,
                        brute-force comparison with a per-token write.  Pinned.
* ``decode``         -- the hand-computed example of [Lab] B.1.2 (weights
                        [0.24825508, 0.24825508, 0.50348984], output
                        [0.75174492, 1.50348984]); the softmax example of
                        [Lab] B.1.1; torch's float64 scaled_dot_product_attention
                        on the contiguous (un-paged) K/V; block-permutation
                        invariance; GQA == repeated K/V heads; single key
                        returns its V row.  Pinned.
* ``prefill``        -- the causal weight matrix and last output of [Lab] B.1.2;
                        the future-change experiment of [Lab] B.1.2 (earlier rows
                        unchanged with the mask, max change 8.15455 without);
                        torch's float64 SDPA with its lower-right causal bias;
                        prefix/chunk split invariance and decode == last prefill
                        row ([Lab] B.1.4, B.8.1).  Pinned.
* ``decode_partials`` / ``lse_merge`` -- merging any partition of the keys
                        reproduces ``decode`` (the rescaling identity of [Lab]
                        Fig. B-5 and [mini] section 5); one partition is the
                        identity.  Pinned against ``decode``, which is pinned.

Storage dtypes arrive as raw bits (``uint16`` for bfloat16, ``float16`` for
fp16, ``float32`` for fp32) and are widened exactly to float64 by ``to_f64``.
"""

from __future__ import annotations

import numpy as np


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values exactly: bfloat16 bits are the top half of an fp32."""
    if dtype == "bf16":
        u = np.asarray(x, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# a1: physical slot of every new token


def slot_mapping(block_table, cu_seqlens_q, seq_lens_k, block_size) -> np.ndarray:
    """Physical cache row of each new token.

    [KVblog] 3.1/3.5 and [Lab] B.2.3: a token at logical position ``p`` of a
    sequence lives in row ``block_table[p // block_size] * block_size +
    p % block_size``.  The new tokens of sequence ``b`` are the last
    ``Lq = cu_seqlens_q[b+1] - cu_seqlens_q[b]`` of its ``seq_lens_k[b]``
    tokens, so new token ``i`` sits at ``p = seq_lens_k[b] - Lq + i`` (a cached
    prefix shifts the positions, [KVblog] 3.5; a decode token has
    ``p = context_len - 1``, [KVblog] 4.4).

    A position whose logical block has no physical block (index past the table
    or a -1 entry) gets slot -1, the pages' "do not write" marker
    ([MinivLLM] store_kvcache).  So does a negative position (a sequence with
    fewer keys than new tokens, e.g. a decode row of context length 0): it has
    no logical block at all.
    """
    bt = np.asarray(block_table)
    cu = np.asarray(cu_seqlens_q)
    lens = np.asarray(seq_lens_k)
    out = np.empty(int(cu[-1]), dtype=np.int32)
    for b in range(len(lens)):
        lq = int(cu[b + 1] - cu[b])
        for i in range(lq):
            p = int(lens[b]) - lq + i
            j = p // block_size
            blk = int(bt[b, j]) if 0 <= j < bt.shape[1] else -1
            out[int(cu[b]) + i] = blk * block_size + p % block_size if blk >= 0 else -1
    return out


# ---------------------------------------------------------------------------
# a2: scatter of the new K/V rows


def store_kv(k_pool, v_pool, key, value, slots) -> None:
    """Write each new token's K and V row into its slot, in place.

    [MinivLLM] store_kvcache and [KVblog] 3.1: the pool is
    ``[num_blocks, block_size, kv_heads, head_dim]``; token ``t`` goes to
    block ``slot // block_size``, row ``slot % block_size``; slot -1 writes
    nothing.  A pure copy, so the result is bit-exact.
    """
    bs = k_pool.shape[1]
    for t, s in enumerate(np.asarray(slots)):
        s = int(s)
        if s == -1:
            continue
        k_pool[s // bs, s % bs] = key[t]
        v_pool[s // bs, s % bs] = value[t]


def copy_blocks(k_pool, v_pool, pairs) -> None:
    """Copy whole blocks ``src -> dst`` of both pools, in place, for each (src, dst) pair.

    [KVblog] 2.2: sequences that share a physical block write into it only after
    copying it to a block of their own (copy-on-write).  A pair naming a block
    outside the pool, or with src == dst, copies nothing.  Destinations are
    distinct and are not sources of other pairs, so the order of the pairs does
    not matter.  A pure copy, so the result is bit-exact.
    """
    nb = k_pool.shape[0]
    for src, dst in np.asarray(pairs).reshape(-1, 2):
        src, dst = int(src), int(dst)
        if not (0 <= src < nb and 0 <= dst < nb) or src == dst:
            continue
        k_pool[dst] = k_pool[src]
        v_pool[dst] = v_pool[src]


# ---------------------------------------------------------------------------
# reading a sequence back through its block table


def gather_rows(pool, bt_row, n, block_size) -> np.ndarray:
    """The first ``n`` logical rows of one sequence, ``[n, kv_heads, head_dim]``.

    [MinivLLM] paged_attention_decode_kernel: token ``t`` is found in block
    ``block_tables[b, t // block_size]`` at row ``t % block_size``.  A -1 entry
    inside the live range is a caller error.
    """
    t = np.arange(n, dtype=np.int64)
    blk = np.asarray(bt_row, dtype=np.int64)[t // block_size]
    if np.any(blk < 0):
        raise ValueError("block table entry is -1 inside the live range")
    return pool[blk, t % block_size]


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    """Row softmax of float64 scores; -inf entries get weight 0."""
    m = np.max(s, axis=-1, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# a3 + a4: decode attention (q_len = 1)


def decode(q, k_pool, v_pool, block_table, context_lens, scale, dtype) -> np.ndarray:
    """Decode attention output ``[B, q_heads, head_dim]`` in float64.

    For sequence ``b`` with ``L = context_lens[b]`` keys (the count includes the
    token written this step, [KVblog] 4.4) and query head ``h`` served by KV head
    ``g = h // (q_heads // kv_heads)`` ([mini] 5, [MinivLLM]):
    ``out = softmax(scale * K_g q_h) V_g`` over the ``L`` rows read through the
    block table ([Lab] B.1.2 defines the attention step).  ``L == 0`` (a padded
    row) gives an all-zero output.  ``scale`` is applied once, as given.
    """
    B, HQ, D = q.shape
    HKV = k_pool.shape[2]
    bs = k_pool.shape[1]
    G = HQ // HKV
    qf = to_f64(q, dtype)
    out = np.zeros((B, HQ, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        K = to_f64(gather_rows(k_pool, block_table[b], L, bs), dtype)
        V = to_f64(gather_rows(v_pool, block_table[b], L, bs), dtype)
        for h in range(HQ):
            g = h // G
            w = _softmax_rows(scale * (K[:, g, :] @ qf[b, h]))
            out[b, h] = w @ V[:, g, :]
    return out


def decode_partials(q, k_pool, v_pool, block_table, context_lens, scale, dtype,
                    partition_size, num_partitions):
    """Per-partition softmax state of decode, for split-K.

    Partition ``p`` of sequence ``b`` covers keys ``[p*P, min((p+1)*P, L))``.
    For each (b, h, p) with a non-empty range: ``m`` = max of the scaled
    scores, ``l = sum(exp(s - m))`` and ``acc = sum(exp(s - m) * v)`` -- the
    running state ``(m, l, acc)`` of the online softmax ([mini] 5; [Lab]
    Fig. B-5 calls the numerator u).  Empty partitions are NaN.
    Returns ``acc [B, HQ, NP, D], m [B, HQ, NP], l [B, HQ, NP]``.
    """
    B, HQ, D = q.shape
    HKV = k_pool.shape[2]
    bs = k_pool.shape[1]
    G = HQ // HKV
    P = int(partition_size)
    qf = to_f64(q, dtype)
    acc = np.full((B, HQ, num_partitions, D), np.nan)
    m = np.full((B, HQ, num_partitions), np.nan)
    l = np.full((B, HQ, num_partitions), np.nan)
    for b in range(B):
        L = int(context_lens[b])
        if L == 0:
            continue
        K = to_f64(gather_rows(k_pool, block_table[b], L, bs), dtype)
        V = to_f64(gather_rows(v_pool, block_table[b], L, bs), dtype)
        for p in range(-(-L // P)):
            lo, hi = p * P, min((p + 1) * P, L)
            for h in range(HQ):
                g = h // G
                s = scale * (K[lo:hi, g, :] @ qf[b, h])
                mm = np.max(s)
                e = np.exp(s - mm)
                m[b, h, p] = mm
                l[b, h, p] = np.sum(e)
                acc[b, h, p] = e @ V[lo:hi, g, :]
    return acc, m, l


def lse_merge(acc, m, l, num_valid) -> np.ndarray:
    """Combine partition states into the attention output.

    The rescaling of [Lab] Fig. B-5 / [mini] 5 applied across partitions:
    ``M = max_p m_p``, ``out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p``
    over the ``num_valid[b]`` non-empty partitions; zero partitions give 0.
    ``acc [B, HQ, NP, D]``, ``m, l [B, HQ, NP]``, ``num_valid [B]``.
    """
    B, HQ, NP, D = acc.shape
    out = np.zeros((B, HQ, D), dtype=np.float64)
    for b in range(B):
        n = int(num_valid[b])
        if n == 0:
            continue
        for h in range(HQ):
            mm = m[b, h, :n].astype(np.float64)
            M = np.max(mm)
            w = np.exp(mm - M)
            out[b, h] = (w @ acc[b, h, :n].astype(np.float64)) / (w @ l[b, h, :n].astype(np.float64))
    return out


# ---------------------------------------------------------------------------
# a5: varlen chunked prefill over a cached prefix


def prefill(q, k_pool, v_pool, block_table, cu_seqlens_q, cu_seqlens_k, scale, dtype,
            causal=True) -> np.ndarray:
    """Chunked-prefill attention output ``[total_q, q_heads, head_dim]``.

    Sequence ``b`` has ``Lq = cu_q[b+1]-cu_q[b]`` new queries and
    ``Lk = cu_k[b+1]-cu_k[b]`` keys; the first ``Lk - Lq`` keys are the cached
    prefix ([KVblog] 3.5: seqlen_q = seqlen - num_cached_tokens, seqlen_k =
    seqlen) and every key is read from the pool through the block table.
    Query ``i`` sits at position ``Lk - Lq + i`` ([Lab] B.6: the 108 new
    queries of a 620-key request start at position 512), so with ``causal`` it
    sees keys ``j <= Lk - Lq + i`` ([Lab] B.1.2 causal mask); without, all keys.
    """
    T, HQ, D = q.shape
    HKV = k_pool.shape[2]
    bs = k_pool.shape[1]
    G = HQ // HKV
    qf = to_f64(q, dtype)
    out = np.zeros((T, HQ, D), dtype=np.float64)
    for b in range(len(cu_seqlens_q) - 1):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        Lq, Lk = q1 - q0, int(cu_seqlens_k[b + 1] - cu_seqlens_k[b])
        if Lq == 0:
            continue
        K = to_f64(gather_rows(k_pool, block_table[b], Lk, bs), dtype)
        V = to_f64(gather_rows(v_pool, block_table[b], Lk, bs), dtype)
        pos = (Lk - Lq) + np.arange(Lq)[:, None]
        visible = np.arange(Lk)[None, :] <= pos if causal else np.ones((Lq, Lk), dtype=bool)
        for h in range(HQ):
            g = h // G
            s = scale * (qf[q0:q1, h, :] @ K[:, g, :].T)
            s = np.where(visible, s, -np.inf)
            out[q0:q1, h] = _softmax_rows(s) @ V[:, g, :]
    return out
