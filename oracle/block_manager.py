"""Plain Python oracle of the block manager and its chain-hash prefix cache.  TEST
INFRASTRUCTURE ONLY: nothing in the product imports it.

Sources (web pages; cited by the short name in brackets):

* [KVblog]   "大模型推理引擎学习入门-2：带你理解 nano-vllm 的 KV Cache 以及 Paged
             Attention" (juejin.cn): 2.2 (sharing of physical blocks through reference
             counts, copy-on-write), 3.3 (allocate / may_append / deallocate and the
             ALLOCATE / REUSE / REACTIVATE paths), 3.4 (chain hash, registration of full
             blocks only, lazy reclamation).
* [Lab]      "5. 动手改造：从跑通到可测量的推理服务" (the nano-vLLM lab manual), B.6 (the
             prompt's last block is not looked up; reallocating a block drops its old
             mapping).
* [MinivLLM] "MinivLLM：六步搭出一个 Qwen3 推理引擎，再核清四处文档与代码的分岔"
             (txtmix.com), "前缀缓存真正生效的条件" (three live sequences sharing two
             blocks).

The pages print the allocate / may_append / deallocate code of nano-vllm; this file is
written from the behaviour they describe instead, in its own structure: admission first
finds the longest run of cached blocks at the front of the prompt, then claims those
(share or take back), then hands out fresh blocks for the rest, then makes every full
block findable.  Only the fingerprint (compute_hash) must match the pages' definition
byte for byte.

Readings where the pages leave a step open:

* The hit test asks that the block the table names still carries this fingerprint and
  these tokens.  ([KVblog] 3.4 compares the tokens; the fingerprint check keeps a block
  that was reallocated and refilled with the same tokens under another prefix from
  matching.)
* A prompt's last block is always computed ([Lab] B.6), even when it is full.
* [MinivLLM]'s copy of the code empties a freed block's tokens, which turns off reuse
  across requests; [KVblog] 3.4 and [Lab] B.6 keep them (REACTIVATE).  The latter is
  followed.
* Copy-on-write ([KVblog] 2.2 describes it, no code is given): a token written into a
  last block that another sequence also references first moves the writer to a fresh
  block; the pair (old, new) is returned so the caller copies the block's K/V rows.
* A sequence handle is an integer counting up from 0; ``fork`` gives the child all of
  the parent's blocks, one more reference each.

Pins (tests/test_block_manager.py, tests/golden/block_manager_examples.json): the logs
of [KVblog] 3.3.3 and 3.3.5 (block tables [0, 1] and [0, 2], 256 cached tokens, free
counts 2232 / 2231 / 2232 / 2233 / 2234), the may_append table of [KVblog] 3.3.4, the
three-sequence table of [MinivLLM], the [Lab] B.6 experiment (cached 512 after the first
request finished; reference counts [0,0] -> [1,1] -> [2,2] -> [1,1] -> [0,0]; 620 tokens
hit 2 blocks, 512 tokens hit 1), the chain-break example of [KVblog] 3.4, XXH64's
published empty-input value, and invariants (reference counts equal table
memberships, free and used blocks partition the pool) over random operation sequences.
"""

from __future__ import annotations

import itertools
from collections import OrderedDict

import numpy as np
import xxhash


class CapacityError(RuntimeError):
    """Not enough free blocks for the request."""


def compute_hash(token_ids, prefix=None) -> int:
    """Chain hash of one full block ([KVblog] 3.4): XXH64 over the previous block's hash
    as 8 little-endian bytes (left out for the first block) followed by the token ids as
    64-bit little-endian integers."""
    h = xxhash.xxh64()
    if prefix is not None:
        h.update(int(prefix).to_bytes(8, "little"))
    h.update(np.asarray(list(token_ids), dtype="<i8").tobytes())
    return h.intdigest()


class _Seq:
    """A live sequence: its token ids, its block table and how many of its prompt tokens
    were found in the cache at admission."""

    def __init__(self, tokens, table, cached):
        self.tokens = tokens
        self.table = table
        self.cached = cached


class BlockManager:
    """The block pool of one KV cache and its prefix index.

    State, per block: a reference count (how many live block tables hold it) and, for a
    full block made findable, what it holds (fingerprint, token ids).  Free blocks (count
    0) wait in an ordered set, least recently freed first; they keep what they hold until
    they are handed out again, so a later prompt with the same prefix can take them back
    (lazy reclamation, [KVblog] 3.4).  The index maps a fingerprint to the block that was
    last made findable under it.
    """

    def __init__(self, num_blocks, block_size):
        assert num_blocks >= 1 and block_size >= 2
        self.num_blocks = num_blocks
        self.block_size = block_size
        self._refs = [0] * num_blocks
        self._holds = [None] * num_blocks           # (fingerprint, tokens) or None
        self._free = OrderedDict.fromkeys(range(num_blocks))
        self._index = {}                            # fingerprint -> block id
        self._seqs = {}
        self._handles = itertools.count()

    # -- helpers on token lists
    def _chunk(self, tokens, i):
        return tuple(tokens[i * self.block_size:(i + 1) * self.block_size])

    def _fingerprints(self, tokens):
        """Chain fingerprints of the full blocks of a token list, first block first."""
        fps, prev = [], None
        for i in range(len(tokens) // self.block_size):
            prev = compute_hash(self._chunk(tokens, i), prev)
            fps.append(prev)
        return fps

    # -- moves of single blocks
    def _fresh(self):
        """The least recently freed block, emptied for new contents: what it held is
        forgotten, and its fingerprint leaves the index if the index still names it
        ([Lab] B.6).  The caller's table is its first reference."""
        b, _ = self._free.popitem(last=False)
        held = self._holds[b]
        if held is not None and self._index.get(held[0]) == b:
            del self._index[held[0]]
        self._holds[b] = None
        self._refs[b] = 1
        return b

    def _findable(self, b, fp, tokens):
        self._holds[b] = (fp, tokens)
        self._index[fp] = b

    def _lookup(self, fp, tokens):
        """The block that still holds exactly these tokens under this fingerprint, if any
        ([KVblog] 3.4: a fingerprint match with other tokens is no match)."""
        b = self._index.get(fp)
        if b is not None and self._holds[b] == (fp, tokens):
            return b
        return None

    def _unref(self, b):
        self._refs[b] -= 1
        if self._refs[b] == 0:
            self._free[b] = None  # joins the back of the free set, contents kept

    # -- operations
    def allocate(self, token_ids):
        """Admit a prompt ([KVblog] 3.3, 3.4; [Lab] B.6): its blocks are matched against
        the cache from the first one on, and the first block without a match ends the
        matching (a fingerprint stands for its whole prefix, so nothing after a miss can
        be a valid hit); the prompt's last block is never matched, so at least its tokens
        are computed.  A matched block in use by another sequence is shared (ALLOCATE's
        REUSE outcome), a matched block that was freed is taken back (REACTIVATE), every
        other block is fresh (ALLOCATE).  All full blocks of the prompt end up findable
        under their fingerprints."""
        tokens = [int(t) for t in token_ids]
        if not tokens:
            raise ValueError("empty prompt")
        need = -(-len(tokens) // self.block_size)
        if len(self._free) < need:
            raise CapacityError(f"{need} blocks needed, {len(self._free)} free")
        fps = self._fingerprints(tokens)
        matched = []
        for i in range(min(len(fps), need - 1)):
            b = self._lookup(fps[i], self._chunk(tokens, i))
            if b is None:
                break
            matched.append(b)
        table = []
        for b in matched:
            if self._refs[b] > 0:
                self._refs[b] += 1  # shared with a live sequence
            else:
                del self._free[b]  # freed but intact: back in use
                self._refs[b] = 1
            table.append(b)
        table += [self._fresh() for _ in range(need - len(matched))]
        for i, fp in enumerate(fps):
            self._findable(table[i], fp, self._chunk(tokens, i))
        handle = next(self._handles)
        self._seqs[handle] = _Seq(tokens, table, len(matched) * self.block_size)
        return handle

    def append(self, handle, token_id):
        """One generated token ([KVblog] 3.3, 2.2).  A token that starts a block gets a
        fresh block; a token written into a last block that other sequences share first
        moves this sequence to a fresh copy of it, and (source, copy) is returned for the
        caller to copy the K/V rows on the device (else None).  A token that completes a
        block makes it findable."""
        s = self._seqs[handle]
        n = len(s.tokens) + 1
        cow = None
        if n % self.block_size == 1:  # the token starts a block
            if not self._free:
                raise CapacityError("no free block")
            s.table.append(self._fresh())
        elif self._refs[s.table[-1]] > 1:  # shared last block: copy on write
            if not self._free:
                raise CapacityError("no free block")
            src = s.table[-1]
            s.table[-1] = self._fresh()
            self._refs[src] -= 1  # others still hold it
            cow = (src, s.table[-1])
        s.tokens.append(int(token_id))
        if n % self.block_size == 0:  # the token completes its block
            i = n // self.block_size - 1
            self._findable(s.table[i], self._fingerprints(s.tokens)[i], self._chunk(s.tokens, i))
        return cow

    def fork(self, handle):
        """A new sequence with the same tokens sharing every block (one more reference
        each); the first token either writes into a shared block copies it."""
        s = self._seqs[handle]
        for b in s.table:
            self._refs[b] += 1
        child = next(self._handles)
        self._seqs[child] = _Seq(list(s.tokens), list(s.table), s.cached)
        return child

    def free(self, handle):
        """A finished sequence gives back one reference per block, its last block first
        ([KVblog] 3.3), so a sequence's blocks join the free set tail first."""
        s = self._seqs.pop(handle)
        for b in reversed(s.table):
            self._unref(b)

    # -- queries
    def block_table(self, handle):
        return list(self._seqs[handle].table)

    def seq_len(self, handle):
        return len(self._seqs[handle].tokens)

    def num_cached_tokens(self, handle):
        return self._seqs[handle].cached

    def ref_count(self, block_id):
        return self._refs[block_id]

    def num_free_blocks(self):
        return len(self._free)

    def snapshot(self):
        """The whole state, for invariant checks: reference counts, the free set in
        order, each block's fingerprint (None if it holds nothing findable), the index,
        and every live sequence's (token ids, block table)."""
        return {"refs": list(self._refs), "free": list(self._free),
                "held": [h[0] if h is not None else None for h in self._holds],
                "index": dict(self._index),
                "seqs": {k: (list(v.tokens), list(v.table)) for k, v in self._seqs.items()}}
