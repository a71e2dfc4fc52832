"""Host-side harness: put a ``workloads.Workload`` in device memory and run the path.

A step is the whole hot path for one batch: physical slots of the new tokens
(pa_slot_mapping), the scatter of their K/V rows (pa_store_kv), then
attention -- pa_decode (split-K pass + merge) for a decode batch or
pa_prefill_paged for a chunked-prefill batch.  Every step runs in libpa's
kernels; torch only allocates device memory and supplies the stream.
"""

from __future__ import annotations

import numpy as np
import torch

from . import _binding as pa


def to_device(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    """Storage-dtype numpy array (bf16 as uint16 bits, float16 or float32) -> device tensor."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f16":
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float16))
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(device)


def from_device(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy in storage representation (bf16 as uint16 bits)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class DeviceWorkload:
    """Device copies of a workload's inputs plus the pool and outputs."""

    def __init__(self, w, device="cuda", partition_size: int = 0, with_workspace: bool = True):
        self.w = w
        self.device = torch.device(device)
        dev = self.device
        self.tdtype = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[w.dtype]
        i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
        self.block_table = i32(w.block_table)
        self.seq_lens_k = i32(w.seq_lens_k)
        self.hist_lens = i32(w.hist_lens)
        self.cu_q = i32(w.cu_seqlens_q)
        self.cu_k = i32(w.cu_seqlens_k)
        self.cu_hist = i32(w.cu_seqlens_hist)
        self.q = to_device(w.q, w.dtype, dev)
        self.k_new = to_device(w.k_new, w.dtype, dev)
        self.v_new = to_device(w.v_new, w.dtype, dev)
        self.k_hist = to_device(w.k_hist, w.dtype, dev)
        self.v_hist = to_device(w.v_hist, w.dtype, dev)
        # Unused pool rows are poisoned with NaN so a stray read shows in the output.
        self.k_cache = torch.full(w.pool_shape, float("nan"), dtype=self.tdtype, device=dev)
        self.v_cache = torch.full(w.pool_shape, float("nan"), dtype=self.tdtype, device=dev)
        self.slots_new = torch.empty(w.num_new_tokens, dtype=torch.int32, device=dev)
        self.slots_hist = torch.empty(int(w.cu_seqlens_hist[-1]), dtype=torch.int32, device=dev)
        self.out = torch.empty_like(self.q)
        self.max_context_len = w.max_seqlen_k
        self.partition_size = partition_size
        self.workspace = None
        if w.kind == "decode" and with_workspace:
            nbytes = pa.pa_decode_workspace_size(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                                 w.head_dim, max(1, self.max_context_len),
                                                 partition_size)
            if nbytes:
                self.workspace = torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=dev)

    # -- the cached history (not part of a step) ------------------------------------
    def load_history(self, stream=None):
        """Store every sequence's cached tokens (positions 0 .. hist-1) into the pool."""
        w = self.w
        if self.slots_hist.numel() == 0:
            return
        pa.pa_slot_mapping(self.slots_hist, self.block_table, self.cu_hist, self.hist_lens,
                           w.block_size, w.num_blocks, stream)
        pa.pa_store_kv(self.k_hist, self.v_hist, self.k_cache, self.v_cache, self.slots_hist, stream)

    # -- one step of the hot path ---------------------------------------------------
    def slot_mapping(self, stream=None):
        w = self.w
        pa.pa_slot_mapping(self.slots_new, self.block_table, self.cu_q, self.seq_lens_k,
                           w.block_size, w.num_blocks, stream)

    def store(self, stream=None):
        pa.pa_store_kv(self.k_new, self.v_new, self.k_cache, self.v_cache, self.slots_new, stream)

    def store_paged(self, stream=None, write_slots=True):
        """slot_mapping and store in one launch (pa_store_kv_paged)."""
        w = self.w
        pa.pa_store_kv_paged(self.k_new, self.v_new, self.k_cache, self.v_cache, self.block_table,
                             self.cu_q, self.seq_lens_k, max(1, w.max_seqlen_q),
                             self.slots_new if write_slots else None, stream)

    def attention(self, stream=None):
        w = self.w
        if w.kind == "decode":
            pa.pa_decode(self.out, self.q, self.k_cache, self.v_cache, self.block_table,
                         self.seq_lens_k, w.scale, max_context_len=self.max_context_len,
                         partition_size=self.partition_size, workspace=self.workspace,
                         stream=stream)
        else:
            pa.pa_prefill_paged(self.out, self.q, self.k_cache, self.v_cache, self.block_table,
                                self.cu_q, self.cu_k, w.max_seqlen_q, w.max_seqlen_k, w.scale,
                                causal=True, stream=stream)

    def attention_append(self, stream=None):
        """Store of the new rows and decode in one call (pa_decode_append); the cache then
        holds the new rows as after store_paged()."""
        w = self.w
        pa.pa_decode_append(self.out, self.q, self.k_new, self.v_new, self.k_cache, self.v_cache,
                            self.block_table, self.seq_lens_k, w.scale,
                            max_context_len=self.max_context_len,
                            partition_size=self.partition_size, workspace=self.workspace,
                            stream=stream)

    def attention_mixed(self, stream=None):
        """The whole batch in one launch: its one-query sequences take the decode
        path and the others the prefill path (pa_attention_mixed)."""
        w = self.w
        if getattr(self, "mixed_workspace", None) is None:
            nbytes = pa.pa_mixed_workspace_size(w.num_seqs, w.num_q_heads, w.num_kv_heads,
                                                w.head_dim, max(1, w.max_seqlen_k))
            self.mixed_workspace = torch.empty((nbytes + 3) // 4, dtype=torch.float32,
                                               device=self.device)
        pa.pa_attention_mixed(self.out, self.q, self.k_cache, self.v_cache, self.block_table,
                              self.cu_q, self.cu_k, max(1, w.max_seqlen_q), max(1, w.max_seqlen_k),
                              w.scale, self.mixed_workspace, stream=stream)

    def step(self, stream=None):
        self.slot_mapping(stream)
        self.store(stream)
        self.attention(stream)
