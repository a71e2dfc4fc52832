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

from collections import deque

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


class Block:
    def __init__(self, block_id):
        self.block_id = block_id
        self.ref_count = 0
        self.hash = None  # None: not a registered full block
        self.token_ids = []

    def reset(self):
        """A block handed to a sequence: the allocation is its first reference."""
        self.ref_count = 1
        self.hash = None
        self.token_ids = []

    def update(self, h, token_ids):
        self.hash = h
        self.token_ids = list(token_ids)


class Sequence:
    def __init__(self, token_ids):
        self.token_ids = list(token_ids)
        self.block_table = []
        self.num_cached_tokens = 0


class BlockManager:
    def __init__(self, num_blocks, block_size):
        assert num_blocks >= 1 and block_size >= 2
        self.block_size = block_size
        self.blocks = [Block(i) for i in range(num_blocks)]
        self.hash_to_block_id = {}
        self.free_block_ids = deque(range(num_blocks))
        self.used_block_ids = set()
        self.seqs = {}
        self._next = 0

    # -- the block of logical index i of a sequence
    def _block_tokens(self, seq, i):
        return seq.token_ids[i * self.block_size:(i + 1) * self.block_size]

    def _num_blocks(self, n):
        return (n + self.block_size - 1) // self.block_size

    def _allocate_block(self, block_id):
        block = self.blocks[block_id]
        if block.hash is not None and self.hash_to_block_id.get(block.hash) == block_id:
            del self.hash_to_block_id[block.hash]  # [Lab] B.6: the old mapping goes
        block.reset()
        self.free_block_ids.remove(block_id)
        self.used_block_ids.add(block_id)
        return block

    def _deallocate_block(self, block_id):
        assert self.blocks[block_id].ref_count == 0
        self.used_block_ids.remove(block_id)
        self.free_block_ids.append(block_id)  # keeps hash and tokens (lazy reclamation)

    def can_allocate(self, n):
        return len(self.free_block_ids) >= self._num_blocks(n)

    def allocate(self, token_ids):
        """Admit a prompt: [KVblog] 3.3.3 (three paths, the first miss ends the hits)."""
        if not token_ids:
            raise ValueError("empty prompt")
        if not self.can_allocate(len(token_ids)):
            raise CapacityError(f"{self._num_blocks(len(token_ids))} blocks needed, "
                                f"{len(self.free_block_ids)} free")
        seq = Sequence(token_ids)
        nb = self._num_blocks(len(token_ids))
        h = None
        cache_miss = False
        for i in range(nb):
            tokens = self._block_tokens(seq, i)
            full = len(tokens) == self.block_size
            h = compute_hash(tokens, h) if full else None
            block_id = -1
            if full and i < nb - 1:  # [Lab] B.6: the last block is not looked up
                cand = self.hash_to_block_id.get(h, -1)
                if cand >= 0 and self.blocks[cand].hash == h and \
                        self.blocks[cand].token_ids == tokens:
                    block_id = cand
            if block_id < 0:
                cache_miss = True
            if cache_miss:  # ALLOCATE
                block = self._allocate_block(self.free_block_ids[0])
            else:
                seq.num_cached_tokens += self.block_size
                if block_id in self.used_block_ids:  # REUSE
                    block = self.blocks[block_id]
                    block.ref_count += 1
                else:  # REACTIVATE
                    block = self._allocate_block(block_id)
            if full:
                block.update(h, tokens)
                self.hash_to_block_id[h] = block.block_id
            seq.block_table.append(block.block_id)
        sid = self._next
        self._next += 1
        self.seqs[sid] = seq
        return sid

    def append(self, sid, token_id):
        """One generated token ([KVblog] 3.3.4, with copy-on-write from 2.2).  Returns
        the (src, dst) pair to copy on the device, or None."""
        seq = self.seqs[sid]
        seq.token_ids.append(int(token_id))
        n = len(seq.token_ids)
        cow = None
        if n % self.block_size == 1:  # the token opens a new block
            if not self.free_block_ids:
                seq.token_ids.pop()
                raise CapacityError("no free block")
            block = self._allocate_block(self.free_block_ids[0])
            seq.block_table.append(block.block_id)
        elif self.blocks[seq.block_table[-1]].ref_count > 1:  # shared: copy on write
            if not self.free_block_ids:
                seq.token_ids.pop()
                raise CapacityError("no free block")
            src = seq.block_table[-1]
            block = self._allocate_block(self.free_block_ids[0])
            self.blocks[src].ref_count -= 1
            seq.block_table[-1] = block.block_id
            cow = (src, block.block_id)
        if n % self.block_size == 0:  # the token fills its block: register it
            i = n // self.block_size - 1
            tokens = self._block_tokens(seq, i)
            prefix = self.blocks[seq.block_table[i - 1]].hash if i > 0 else None
            h = compute_hash(tokens, prefix)
            self.blocks[seq.block_table[i]].update(h, tokens)
            self.hash_to_block_id[h] = seq.block_table[i]
        return cow

    def fork(self, sid):
        parent = self.seqs[sid]
        child = Sequence(parent.token_ids)
        child.block_table = list(parent.block_table)
        child.num_cached_tokens = parent.num_cached_tokens
        for b in child.block_table:
            self.blocks[b].ref_count += 1
        cid = self._next
        self._next += 1
        self.seqs[cid] = child
        return cid

    def free(self, sid):
        """[KVblog] 3.3.5: one reference less per block, last block first."""
        seq = self.seqs.pop(sid)
        for b in reversed(seq.block_table):
            self.blocks[b].ref_count -= 1
            if self.blocks[b].ref_count == 0:
                self._deallocate_block(b)

    # -- queries
    def block_table(self, sid):
        return list(self.seqs[sid].block_table)

    def seq_len(self, sid):
        return len(self.seqs[sid].token_ids)

    def num_cached_tokens(self, sid):
        return self.seqs[sid].num_cached_tokens

    def ref_count(self, block_id):
        return self.blocks[block_id].ref_count

    def num_free_blocks(self):
        return len(self.free_block_ids)
