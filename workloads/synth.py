"""Seeded workload generator (lengths, block placement, random values).

Storage dtypes travel as raw bits so that the oracle and the GPU receive the
very same values: ``f32`` arrays are ``numpy.float32``, ``f16`` arrays are
``numpy.float16`` and ``bf16`` arrays are ``numpy.uint16`` holding bfloat16 bit
patterns (both 16-bit types rounded to nearest-even from an fp32 N(0,1) draw).

Recipe (one ``numpy.random.default_rng(seed)`` per workload, draws in this
order):

1. key lengths (``seq_lens_k``) when the config draws them;
2. ``rng.permutation(num_blocks)``: sequence ``b`` owns the next
   ``ceil(seq_lens_k[b] / block_size)`` entries of the permutation, so every
   physical block belongs to at most one sequence and the rest of the pool is
   unused;
3. history K rows, then history V rows (the ``seq_lens_k - new_lens`` tokens
   that were cached before this step), ``[sum(hist), kv_heads, head_dim]``;
4. new K rows, then new V rows (the tokens this step writes),
   ``[sum(new), kv_heads, head_dim]``;
5. Q, ``[sum(new), q_heads, head_dim]``.

Every N(0,1) draw is made in chunks of ``_CHUNK`` values with
``rng.standard_normal(n, dtype=float32)`` so that the stream does not depend
on available memory.
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

_CHUNK = 1 << 24


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs are finite N(0,1) draws, so no NaN/Inf special-casing is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def nan_bits(dtype: str):
    """A quiet-NaN value in the storage representation of ``dtype``."""
    if dtype == "bf16":
        return np.uint16(0x7FC0)
    if dtype == "f32":
        return np.float32(np.nan)
    if dtype == "f16":
        return np.float16(np.nan)
    raise ValueError(dtype)


def storage_np_dtype(dtype: str):
    return {"bf16": np.uint16, "f32": np.float32, "f16": np.float16}[dtype]


def _normal(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    n = int(np.prod(shape))
    out = np.empty(n, dtype=storage_np_dtype(dtype))
    for s in range(0, n, _CHUNK):
        e = min(n, s + _CHUNK)
        x = rng.standard_normal(e - s, dtype=np.float32)
        out[s:e] = bf16_bits_from_f32(x) if dtype == "bf16" else x  # f16: numpy rounds to nearest even
    return out.reshape(shape)


def normal_values(rng: np.random.Generator, shape, dtype: str) -> np.ndarray:
    """N(0, 1) draws of the given shape in the storage representation of ``dtype``."""
    return _normal(rng, shape, dtype)


@dataclasses.dataclass
class Workload:
    """One batch of synthetic input for a store + attention step.

    ``kind == "decode"``: every sequence adds one token (q_len = 1) and
    ``seq_lens_k`` are the context lengths including that token.
    ``kind == "prefill"``: sequence ``b`` adds ``new_lens[b]`` tokens on top of
    a cached prefix of ``seq_lens_k[b] - new_lens[b]`` tokens.
    """

    name: str
    kind: str
    dtype: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    seq_lens_k: np.ndarray  # int32 [B]
    new_lens: np.ndarray  # int32 [B]
    block_table: np.ndarray  # int32 [B, max_blocks_per_seq], -1 padded
    cu_seqlens_q: np.ndarray  # int32 [B+1] over new tokens
    cu_seqlens_k: np.ndarray  # int32 [B+1] over key tokens
    cu_seqlens_hist: np.ndarray  # int32 [B+1] over cached tokens
    k_hist: np.ndarray
    v_hist: np.ndarray
    k_new: np.ndarray
    v_new: np.ndarray
    q: np.ndarray
    seed: int

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def hist_lens(self) -> np.ndarray:
        return (self.seq_lens_k - self.new_lens).astype(np.int32)

    @property
    def max_seqlen_q(self) -> int:
        return int(self.new_lens.max()) if self.num_seqs else 0

    @property
    def max_seqlen_k(self) -> int:
        return int(self.seq_lens_k.max()) if self.num_seqs else 0

    @property
    def num_new_tokens(self) -> int:
        return int(self.cu_seqlens_q[-1])

    @property
    def pool_shape(self):
        return (self.num_blocks, self.block_size, self.num_kv_heads, self.head_dim)

    def empty_pool(self) -> np.ndarray:
        """A pool with every row poisoned with NaN (nothing is live yet)."""
        return np.full(self.pool_shape, nan_bits(self.dtype), dtype=storage_np_dtype(self.dtype))

    @property
    def kv_bytes_per_token(self) -> int:
        """Bytes of K plus V one token occupies in one layer's pool."""
        elt = 4 if self.dtype == "f32" else 2
        return 2 * self.num_kv_heads * self.head_dim * elt


def _prefix(x: np.ndarray) -> np.ndarray:
    out = np.zeros(len(x) + 1, dtype=np.int64)
    out[1:] = np.cumsum(x, dtype=np.int64)
    return out.astype(np.int32)


def make_workload(
    *,
    name: str,
    kind: str,
    dtype: str,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int,
    seq_lens_k,
    new_lens=None,
    num_blocks: int | None = None,
    pool_factor: float = 1.25,
    max_blocks_per_seq: int | None = None,
    scale: float | None = None,
    seed: int = 0,
    rng: np.random.Generator | None = None,
) -> Workload:
    """Build a workload from explicit lengths (draw steps 2-5 of the recipe)."""
    if rng is None:
        rng = np.random.default_rng(seed)
    seq_lens_k = np.asarray(seq_lens_k, dtype=np.int32).reshape(-1)
    B = len(seq_lens_k)
    if new_lens is None:
        new_lens = np.ones(B, dtype=np.int32) if kind == "decode" else seq_lens_k.copy()
    new_lens = np.asarray(new_lens, dtype=np.int32).reshape(-1)
    assert len(new_lens) == B
    assert np.all(new_lens <= seq_lens_k) and np.all(new_lens >= 0)
    nblk = [-(-int(L) // block_size) for L in seq_lens_k]
    demand = int(sum(nblk))
    if num_blocks is None:
        num_blocks = max(1, math.ceil(pool_factor * demand))
    assert num_blocks >= demand, "pool smaller than demand"
    if max_blocks_per_seq is None:
        max_blocks_per_seq = max([1] + nblk)
    assert max_blocks_per_seq >= max([0] + nblk)
    perm = rng.permutation(num_blocks).astype(np.int32)
    bt = np.full((B, max_blocks_per_seq), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(nblk):
        bt[b, :n] = perm[off:off + n]
        off += n
    hist = seq_lens_k - new_lens
    nh, nn = int(hist.sum()), int(new_lens.sum())
    k_hist = _normal(rng, (nh, num_kv_heads, head_dim), dtype)
    v_hist = _normal(rng, (nh, num_kv_heads, head_dim), dtype)
    k_new = _normal(rng, (nn, num_kv_heads, head_dim), dtype)
    v_new = _normal(rng, (nn, num_kv_heads, head_dim), dtype)
    q = _normal(rng, (nn, num_q_heads, head_dim), dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(head_dim)
    return Workload(
        name=name, kind=kind, dtype=dtype, num_seqs=B, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=block_size,
        num_blocks=int(num_blocks), scale=float(scale), seq_lens_k=seq_lens_k,
        new_lens=new_lens, block_table=bt, cu_seqlens_q=_prefix(new_lens),
        cu_seqlens_k=_prefix(seq_lens_k), cu_seqlens_hist=_prefix(hist),
        k_hist=k_hist, v_hist=v_hist, k_new=k_new, v_new=v_new, q=q, seed=seed)


# ---------------------------------------------------------------------------
# The five named workloads.  Shapes follow the pages: Qwen2.5-0.5B attention is
# 14 Q / 2 KV heads of dim 64 (mini-vLLM, block 16); Qwen3-0.6B is 16 Q / 8 KV
# heads of dim 128 (nano-vllm, block 256).


def _c0(seed):
    return make_workload(
        name="tiny-f32-decode", kind="decode", dtype="f32", num_q_heads=2,
        num_kv_heads=1, head_dim=64, block_size=16, seq_lens_k=[17, 33],
        num_blocks=8, max_blocks_per_seq=3, scale=1.0 / 8.0, seed=seed)


def _c1(seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 2048, size=64, endpoint=True).astype(np.int32)
    return make_workload(
        name="qwen2.5-0.5b-decode-b64", kind="decode", dtype="bf16", num_q_heads=14,
        num_kv_heads=2, head_dim=64, block_size=16, seq_lens_k=lens, num_blocks=10000,
        max_blocks_per_seq=128, scale=1.0 / 8.0, seed=seed, rng=rng)


def _c2(seed):
    rng = np.random.default_rng(seed)
    lens = rng.integers(128, 4096, size=256, endpoint=True).astype(np.int32)
    return make_workload(
        name="qwen3-0.6b-decode-b256", kind="decode", dtype="bf16", num_q_heads=16,
        num_kv_heads=8, head_dim=128, block_size=256, seq_lens_k=lens,
        pool_factor=1.25, max_blocks_per_seq=16, scale=1.0 / math.sqrt(128), seed=seed,
        rng=rng)


def _c3(seed):
    lens = np.array([32768] + [512] * 7, dtype=np.int32)
    return make_workload(
        name="qwen3-0.6b-skewed-decode", kind="decode", dtype="bf16", num_q_heads=16,
        num_kv_heads=8, head_dim=128, block_size=256, seq_lens_k=lens, pool_factor=1.25,
        max_blocks_per_seq=128, scale=1.0 / math.sqrt(128), seed=seed)


def _c4(seed):
    lens = np.full(8, 1024 + 256, dtype=np.int32)
    new = np.full(8, 256, dtype=np.int32)
    return make_workload(
        name="qwen3-0.6b-chunked-prefill", kind="prefill", dtype="bf16", num_q_heads=16,
        num_kv_heads=8, head_dim=128, block_size=256, seq_lens_k=lens, new_lens=new,
        pool_factor=1.25, max_blocks_per_seq=5, scale=1.0 / math.sqrt(128), seed=seed)


CONFIGS = {0: _c0, 1: _c1, 2: _c2, 3: _c3, 4: _c4}


def make_tp_shard(tp: int = 2, seed: int = 67002) -> Workload:
    """One tensor-parallel rank's share of the 256-row Qwen3-0.6B decode batch: the same
    context lengths (seed 67002), with the 16 Q / 8 KV heads split over tp ranks (each rank
    holds whole KV heads and their query groups)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(128, 4096, size=256, endpoint=True).astype(np.int32)
    return make_workload(
        name=f"qwen3-0.6b-decode-b256-tp{tp}-rank", kind="decode", dtype="bf16",
        num_q_heads=16 // tp, num_kv_heads=8 // tp, head_dim=128, block_size=256,
        seq_lens_k=lens, pool_factor=1.25, max_blocks_per_seq=16,
        scale=1.0 / math.sqrt(128), seed=seed, rng=rng)


def make_mixed(seed: int = 67005, num_decode: int = 256, num_prefill: int = 8) -> Workload:
    """A serving step that mixes both kinds of rows (Qwen3-0.6B heads, block 256):
    ``num_decode`` decode rows (one query each, contexts uniform in [128, 4096]) followed
    by ``num_prefill`` chunks of 256 new tokens over 1024 cached ones."""
    rng = np.random.default_rng(seed)
    dec = rng.integers(128, 4096, size=num_decode, endpoint=True).astype(np.int32)
    lens = np.concatenate([dec, np.full(num_prefill, 1024 + 256, dtype=np.int32)])
    new = np.concatenate([np.ones(num_decode, dtype=np.int32),
                          np.full(num_prefill, 256, dtype=np.int32)])
    return make_workload(
        name=f"qwen3-0.6b-mixed-{num_decode}dec-{num_prefill}x1280", kind="prefill",
        dtype="bf16", num_q_heads=16, num_kv_heads=8, head_dim=128, block_size=256,
        seq_lens_k=lens, new_lens=new, pool_factor=1.25, max_blocks_per_seq=16,
        scale=1.0 / math.sqrt(128), seed=seed, rng=rng)


def make_config(index: int, seed: int | None = None) -> Workload:
    """Workload ``index`` (0-4) with its default seed ``67000 + index``."""
    if seed is None:
        seed = 67000 + index
    return CONFIGS[index](seed)
