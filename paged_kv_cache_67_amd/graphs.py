"""Decode steps replayed from HIP graphs, one per batch-size bucket.

A serving loop runs the same decode step over and over with a batch size that
changes from step to step.  The nano-vLLM lab manual (B.4 and Fig. B-6)
captures the decode step once per batch-size bucket (1, 2, 4, 8, 16, then
steps of 16), copies each step's inputs into the captured fixed buffers and
replays: a batch of 9 replays the 16-row graph, and the 7 padded rows have
slot -1 and context length 0, so they write no cache row.  B.5 adds that a
batch no bucket covers runs eagerly instead of failing.  Both hold here for the
library's kernels: the step is one pa_decode_append call (store of the new rows
and decode; for short slices one first pass and a merge), which stores nothing
for a row with context 0 and gives it zeros without reading the cache, and the
library allocates nothing and never synchronises, so the captured launches are
the eager ones.

    runner = GraphedDecode(k_cache, v_cache, num_q_heads=16, max_blocks_per_seq=16,
                           max_context_len=4096, scale=1 / 128 ** 0.5, max_batch=256)
    out = runner.step(q, k_new, v_new, block_table, context_lens)

``step`` stages the live rows into the graph's buffers with one pa_copy_many
launch (all five inputs and the padding rows' zero lengths) and replays.  A
caller that can produce its inputs in place writes them into the views
``inputs(n)`` returns and calls ``replay(n)``, which copies nothing.
"""

from __future__ import annotations

import bisect

import numpy as np
import torch

from . import _binding as pa


def default_buckets(max_batch):
    """1, 2, 4, 8, 16, then multiples of 16 up to max_batch (which is always a bucket)."""
    out = [b for b in (1, 2, 4, 8, 16) if b < max_batch]
    out += list(range(32, max_batch, 16))
    return tuple(out + [int(max_batch)])


class GraphedDecode:
    """slot addressing + K/V store + decode for one layer, replayed per batch bucket.

    Buffers are sized for the largest bucket.  ``step`` copies the live rows in,
    marks the rows up to the bucket as padding (context 0) and replays that
    bucket's graph (capturing it on first use).  The K/V pools are the caller's
    and are updated in place.
    """

    def __init__(self, k_cache, v_cache, num_q_heads, max_blocks_per_seq, max_context_len, scale,
                 max_batch=256, buckets=None):
        NB, BS, HKV, D = k_cache.shape
        assert v_cache.shape == k_cache.shape and k_cache.is_cuda
        self.k_cache, self.v_cache = k_cache, v_cache
        if buckets is None:
            buckets = default_buckets(max_batch)
        self.buckets = tuple(sorted(set(int(b) for b in buckets)))
        self.max_context_len = int(max_context_len)
        self.scale = float(scale)
        self.block_size, self.num_blocks = BS, NB
        bmax = self.buckets[-1]
        dev, dt = k_cache.device, k_cache.dtype
        self.q = torch.zeros(bmax, num_q_heads, D, dtype=dt, device=dev)
        self.k_new = torch.zeros(bmax, HKV, D, dtype=dt, device=dev)
        self.v_new = torch.zeros(bmax, HKV, D, dtype=dt, device=dev)
        self.out = torch.zeros(bmax, num_q_heads, D, dtype=dt, device=dev)
        self.block_table = torch.full((bmax, max_blocks_per_seq), -1, dtype=torch.int32, device=dev)
        self.context_lens = torch.zeros(bmax, dtype=torch.int32, device=dev)
        nbytes = pa.pa_decode_workspace_size(bmax, num_q_heads, HKV, D, self.max_context_len, 0)
        self.workspace = torch.empty(max(1, (nbytes + 3) // 4), dtype=torch.float32, device=dev)
        self.graphs = {}
        # Staging: one descriptor per input (q, k_new, v_new, block_table, context_lens), then
        # the zero lengths of the padding rows; destinations are the fixed buffers.
        # One descriptor list per batch size, its destinations and sizes filled in advance
        # (the padding rows' lengths are the sixth, a zero fill); a step only writes the five
        # source pointers, through an int64 [6][3] view (src, dst, bytes) of the list.
        bufs = (self.q, self.k_new, self.v_new, self.block_table, self.context_lens)
        dst = [t.data_ptr() for t in bufs]
        row_bytes = [t[0].numel() * t.element_size() for t in bufs]
        self._bucket_of = [self.bucket(n) for n in range(bmax + 1)]
        self._descs, self._desc_rows = [], []
        for n in range(bmax + 1):
            d = pa.copy_descs(6)
            v = np.frombuffer(d, dtype=np.int64).reshape(6, 3)
            b = self._bucket_of[n] or n
            v[:5, 1] = dst
            v[:5, 2] = [n * r for r in row_bytes]
            v[5] = (0, dst[4] + 4 * n, 4 * (b - n))
            self._descs.append(d)
            self._desc_rows.append(v)
        self._copy_many = pa.lib().pa_copy_many
        self._out_rows = [self.out[:n] for n in range(bmax + 1)]
        self._width = max_blocks_per_seq
        # The staging goes to the stream the replay will run on (torch's current stream);
        # torch's raw-stream query is the cheap way to name it.
        self._device = dev.index if dev.index is not None else torch.cuda.current_device()
        self._raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream",
                                   lambda d: torch.cuda.current_stream(d).cuda_stream)
        self._hi = 0  # rows [self._hi, bmax) of context_lens are known to be 0

    def bucket(self, batch):
        """The smallest bucket that holds `batch` rows, or None if none does."""
        i = bisect.bisect_left(self.buckets, batch)
        return self.buckets[i] if i < len(self.buckets) else None

    def _launch(self, b):
        pa.pa_decode_append(self.out[:b], self.q[:b], self.k_new[:b], self.v_new[:b],
                            self.k_cache, self.v_cache, self.block_table[:b],
                            self.context_lens[:b], self.scale,
                            max_context_len=self.max_context_len, partition_size=0,
                            workspace=self.workspace)

    def capture(self, b):
        """Capture bucket b (the buffers' current rows are run once eagerly first)."""
        if b not in self.graphs:
            self._launch(b)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self._launch(b)
            self.graphs[b] = g
        return self.graphs[b]

    def eager(self, q, k_new, v_new, block_table, context_lens):
        """The same step launched directly on the caller's tensors (no graph)."""
        n = q.shape[0]
        dev = q.device
        out = torch.empty_like(q)
        nbytes = pa.pa_decode_workspace_size(n, q.shape[1], self.k_cache.shape[2], q.shape[2],
                                             self.max_context_len, 0)
        ws = torch.empty(max(1, (nbytes + 3) // 4), dtype=torch.float32, device=dev)
        pa.pa_decode_append(out, q, k_new, v_new, self.k_cache, self.v_cache, block_table,
                            context_lens, self.scale, max_context_len=self.max_context_len,
                            partition_size=0, workspace=ws)
        return out

    def inputs(self, n):
        """Views of the fixed buffers for a batch of n rows, to be written in place:
        (q, k_new, v_new, block_table, context_lens); then call replay(n)."""
        return (self.q[:n], self.k_new[:n], self.v_new[:n], self.block_table[:n],
                self.context_lens[:n])

    def replay(self, n):
        """Replays n's bucket over the rows already in the buffers (see inputs); the rows
        between n and the bucket get length 0 (one zero fill, only when fewer rows are
        live than at the bucket's last replay).  Returns a view of the output rows."""
        b = self.bucket(n)
        if b is None:
            raise ValueError(f"batch {n} exceeds the largest bucket {self.buckets[-1]}")
        end = min(self._hi, b)
        if end > n:
            pa.pa_copy_many([(None, self.context_lens[n:end])])
        self._padded(n, b)
        self.capture(b).replay()
        return self.out[:n]

    def _padded(self, n, b):
        """Rows [n, b) were just zeroed and rows [0, n) hold live lengths: rows past the
        bucket may still hold lengths of an earlier, larger batch."""
        self._hi = self._hi if self._hi > b else n

    def step(self, q, k_new, v_new, block_table, context_lens):
        """One decode step for the live rows; returns a view of the output rows (a new
        tensor when the batch is larger than every bucket and runs eagerly).  The inputs
        are staged into the graph's buffers by one pa_copy_many launch."""
        n = q.shape[0]
        b = self._bucket_of[n] if n < len(self._bucket_of) else None
        if b is None:
            return self.eager(q, k_new, v_new, block_table, context_lens)
        srcs = (q, k_new, v_new, block_table, context_lens)
        if block_table.shape[1] != self._width or not all(t.is_contiguous() for t in srcs):
            return self._step_torch(q, k_new, v_new, block_table, context_lens, n, b)
        self._desc_rows[n][:5, 0] = [t.data_ptr() for t in srcs]
        st = self._copy_many(self._descs[n], 6, self._raw_stream(self._device))
        if st:
            pa._check("pa_copy_many", st)
        self._padded(n, b)
        g = self.graphs.get(b)
        (g if g is not None else self.capture(b)).replay()
        return self._out_rows[n]

    def _step_torch(self, q, k_new, v_new, block_table, context_lens, n, b):
        """Staging by separate torch copies (a block table narrower than the buffer's, or
        inputs that are not contiguous)."""
        self.q[:n].copy_(q)
        self.k_new[:n].copy_(k_new)
        self.v_new[:n].copy_(v_new)
        w = block_table.shape[1]
        self.block_table[:n, :w].copy_(block_table)
        if w < self.block_table.shape[1]:
            self.block_table[:n, w:].fill_(-1)
        self.context_lens[:n].copy_(context_lens)
        self.context_lens[n:b].zero_()  # padding rows: no keys, no cache write
        self._padded(n, b)
        self.capture(b).replay()
        return self.out[:n]
