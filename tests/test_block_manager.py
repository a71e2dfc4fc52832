"""Block manager and chain-hash prefix cache: the oracle against the pages' worked
examples, and the library's native block manager (pa_bm_*, host code) against the
oracle, operation by operation.  No GPU is used.
"""

import json
import os
import random

import types

import pytest
import xxhash

import oracle.block_manager as obm
import paged_kv_cache_67_amd as pk

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "block_manager_examples.json")
EX = json.load(open(GOLDEN))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pk.lib_path()):
        from paged_kv_cache_67_amd import build
        build.build()
    return pk.lib()


def check_invariants(m):
    """Reference counts equal table memberships; the free set holds exactly the blocks
    with no reference, each once; every table has ceil(len / block_size) entries; the
    index names blocks that hold the fingerprint it maps."""
    st = m.snapshot()
    refs = [0] * m.num_blocks
    for tokens, table in st["seqs"].values():
        assert len(table) == -(-len(tokens) // m.block_size)
        for b in table:
            refs[b] += 1
    assert refs == st["refs"]
    free = st["free"]
    assert len(free) == len(set(free))
    assert set(free) == {b for b in range(m.num_blocks) if st["refs"][b] == 0}
    for fp, b in st["index"].items():
        assert st["held"][b] == fp


# ---------------------------------------------------------------- oracle pins
#
# Each pin_* takes the oracle module, so that the same pins also run on copies of
# the oracle with a planted mistake (test_planted_mistake_is_caught).

def pin_xxh64_empty_published_value(mod):
    assert mod.compute_hash([]) == int(EX["xxh64_empty"]["digest_hex"], 16)


def pin_chain_hash_example(mod):
    ex = EX["kvblog_chain"]
    a0 = mod.compute_hash(ex["A"][0])
    a1 = mod.compute_hash(ex["A"][1], a0)
    b0 = mod.compute_hash(ex["B"][0])
    b1 = mod.compute_hash(ex["B"][1], b0)
    assert ex["A"][1] == ex["B"][1]
    assert a0 != b0 and a1 != b1
    assert a1 != mod.compute_hash(ex["A"][1])  # the prefix takes part


def pin_chain_break_is_final(mod):
    """[KVblog] 3.3.3: once a block misses, later blocks are allocated even if equal."""
    m = mod.BlockManager(16, 4)
    a = m.allocate([1, 2, 3, 4, 5, 6, 7, 8, 9])
    b = m.allocate([0, 2, 3, 4, 5, 6, 7, 8, 9])  # first block differs, second is equal
    assert m.num_cached_tokens(b) == 0
    assert set(m.block_table(a)).isdisjoint(m.block_table(b))
    check_invariants(m)


def pin_miss_ends_hits_after_remap(mod):
    """[KVblog] 3.3.3: the first miss ends the hits even when a later block's own
    fingerprint is still in the table.  A holds P0 P1 t; E = P0 alone computes its only
    (last) block afresh and takes over P0's table entry; E's block is then reallocated,
    which drops that entry.  B = P0 P1 u misses on P0, so P1 (still mapped to A's block)
    must not be shared either."""
    m = mod.BlockManager(8, 4)
    P0, P1 = [1, 2, 3, 4], [5, 6, 7, 8]
    a = m.allocate(P0 + P1 + [9])          # blocks 0, 1, 2
    e = m.allocate(P0)                     # block 3, registered for P0
    m.free(e)                              # free list 4 5 6 7 3
    f = m.allocate(list(range(100, 117)))  # 5 blocks: 4 5 6 7 3 (P0's entry dropped)
    m.free(f)
    b = m.allocate(P0 + P1 + [10])
    assert m.num_cached_tokens(b) == 0
    assert set(m.block_table(a)).isdisjoint(m.block_table(b))
    check_invariants(m)


def pin_kvblog_allocate_and_free_log(mod):
    ex = EX["kvblog_allocate_log"]
    rng = random.Random(4)
    prompt = [rng.randrange(150000) for _ in range(ex["shared_prefix"])]
    seqs = [prompt + [rng.randrange(150000) for _ in range(n - len(prompt))] for n in ex["lens"]]
    m = mod.BlockManager(ex["num_blocks"], ex["block_size"])
    ids = []
    for toks, want in zip(seqs, ex["after_allocate"]):
        ids.append(m.allocate(toks))
        assert m.block_table(ids[-1]) == want["block_table"]
        assert m.num_cached_tokens(ids[-1]) == want["num_cached_tokens"]
        assert m.num_free_blocks() == want["free_blocks"]
        check_invariants(m)
    assert m.ref_count(0) == ex["ref_count_block0_after_both"]
    m.free(ids[0])
    assert m.num_free_blocks() == ex["free_first"]["free_blocks"]
    assert m.ref_count(0) == ex["free_first"]["ref_count_block0"]
    m.free(ids[1])
    assert m.num_free_blocks() == ex["free_second"]["free_blocks"]
    assert m.ref_count(0) == ex["free_second"]["ref_count_block0"]
    assert m.snapshot()["free"][-3:] == ex["free_second"]["free_list_tail"]
    check_invariants(m)


def pin_kvblog_may_append_table(mod):
    ex = EX["kvblog_may_append"]
    bs = ex["block_size"]
    m = mod.BlockManager(8, bs)
    s = m.allocate(list(range(1, 256)))  # 255 tokens: one partial block
    rows = {r["len"]: r for r in ex["rows"]}
    for n in range(256, 514):
        m.append(s, 1000 + n)
        if n in rows:
            held = m.snapshot()["held"]
            registered = sum(1 for b in m.block_table(s) if held[b] is not None)
            assert len(m.block_table(s)) == rows[n]["blocks"], n
            assert registered == rows[n]["registered"], n
    check_invariants(m)


def pin_lab_b2_step3_boundary(mod):
    """[Lab] B.2 step 3: a 256-token prompt (256 cached after its prefill), one sampled
    token makes length 257 -> 257 % 256 == 1 -> the table grows from one block to two."""
    m = mod.BlockManager(4, 256)
    s = m.allocate(list(range(256)))
    assert len(m.block_table(s)) == 1
    m.append(s, 7)
    assert m.seq_len(s) == 257 and len(m.block_table(s)) == 2


def pin_minivllm_three_sequences(mod):
    ex = EX["minivllm_three_sequences"]
    m = mod.BlockManager(8, ex["block_size"])
    ids = [m.allocate(ex["prefix"] + [x]) for x in ex["suffixes"]]
    assert [m.block_table(i) for i in ids] == ex["block_tables"]
    assert [m.num_cached_tokens(i) for i in ids] == ex["num_cached_tokens"]
    assert {str(b): m.ref_count(b) for b in range(5)} == ex["ref_count"]
    check_invariants(m)


def _b6_prompts(ex, seed=6):
    rng = random.Random(seed)
    shared = [rng.randrange(150000) for _ in range(ex["shared"])]
    tail = lambda: [rng.randrange(150000) for _ in range(ex["len"] - ex["shared"])]  # noqa: E731
    return shared + tail(), shared + tail()


def pin_lab_b6_reactivate_after_finish(mod):
    ex = EX["lab_b6_prefix"]
    a, b = _b6_prompts(ex)
    m = mod.BlockManager(64, ex["block_size"])
    sa = m.allocate(a)
    m.free(sa)  # A finished before B arrives
    sb = m.allocate(b)
    assert m.num_cached_tokens(sb) == ex["cached_after_finished"]
    assert m.seq_len(sb) - m.num_cached_tokens(sb) == ex["scheduled_after_finished"]
    check_invariants(m)


def pin_lab_b6_reference_counts_and_hits(mod):
    ex = EX["lab_b6_prefix"]
    a, b = _b6_prompts(ex)
    m = mod.BlockManager(64, ex["block_size"])
    shared_blocks = [0, 1]
    seen = [[m.ref_count(x) for x in shared_blocks]]
    sa = m.allocate(a)
    seen.append([m.ref_count(x) for x in shared_blocks])
    sb = m.allocate(b)
    seen.append([m.ref_count(x) for x in shared_blocks])
    assert m.block_table(sb)[:2] == shared_blocks
    assert m.num_cached_tokens(sb) // ex["block_size"] == ex["hits_620"]
    m.free(sa)
    seen.append([m.ref_count(x) for x in shared_blocks])
    m.free(sb)
    seen.append([m.ref_count(x) for x in shared_blocks])
    assert seen == ex["ref_counts"]
    # exactly 512 tokens: the last block is not looked up, so one block hits
    m2 = mod.BlockManager(64, ex["block_size"])
    m2.allocate(a[:ex["shared"]])
    s = m2.allocate(b[:ex["shared"]])
    assert m2.num_cached_tokens(s) // ex["block_size"] == ex["hits_512"]
    check_invariants(m2)


def pin_collision_guard(mod):
    """[KVblog] 3.4: a fingerprint hit with other tokens is a miss.  Every block is
    given the same fingerprint; no block with different tokens may be shared."""
    real = mod.compute_hash
    mod.compute_hash = lambda tokens, prefix=None: 12345
    try:
        m = mod.BlockManager(32, 4)
        a = m.allocate([1, 2, 3, 4, 5, 6, 7, 8, 9])
        b = m.allocate([9, 9, 9, 9, 5, 6, 7, 8, 9])
        assert m.num_cached_tokens(b) == 0
        assert set(m.block_table(a)).isdisjoint(m.block_table(b))
        c = m.allocate([1, 2, 3, 4, 1])  # the table holds b's last full block: a miss
        assert m.num_cached_tokens(c) == 0
        check_invariants(m)
    finally:
        mod.compute_hash = real


def pin_copy_on_write_after_fork(mod):
    m = mod.BlockManager(16, 4)
    p = m.allocate([1, 2, 3, 4, 5, 6])  # blocks: full, partial (2 tokens)
    c = m.fork(p)
    assert m.block_table(c) == m.block_table(p)
    assert all(m.ref_count(b) == 2 for b in m.block_table(p))
    cow = m.append(c, 70)  # writes into the shared partial block
    assert cow is not None and cow[0] == m.block_table(p)[1]
    assert m.block_table(c) == [m.block_table(p)[0], cow[1]]
    assert m.ref_count(cow[0]) == 1 and m.ref_count(cow[1]) == 1
    assert m.append(p, 71) is None  # the parent now owns its block alone
    assert m.append(c, 72) is None and m.append(c, 73) is None  # fills c's block (8 tokens)
    cow2 = m.append(c, 74)  # opens a new block: nothing to copy
    assert cow2 is None and len(m.block_table(c)) == 3
    check_invariants(m)
    m.free(p)
    m.free(c)
    assert m.num_free_blocks() == 16
    check_invariants(m)


def pin_capacity(mod):
    m = mod.BlockManager(2, 4)
    try:
        m.allocate(list(range(9)))
        raise AssertionError("admitted a prompt larger than the pool")
    except mod.CapacityError:
        pass
    s = m.allocate(list(range(8)))
    try:
        m.append(s, 1)
        raise AssertionError("appended past the pool")
    except mod.CapacityError:
        pass
    assert m.seq_len(s) == 8
    check_invariants(m)


def random_operations(mod, seed, steps=400, each=None):
    """Random allocate / append / fork / free over prompts drawn from a few shared stems
    (prefix hits, reactivation, copy-on-write and capacity failures all occur)."""
    rng = random.Random(seed)
    bs = rng.choice([2, 4, 8, 16])
    m = mod.BlockManager(rng.choice([12, 24, 64]), bs)
    stems = [[rng.randrange(50) for _ in range(rng.randrange(1, 6 * bs))] for _ in range(4)]
    live = []
    for _ in range(steps):
        r = rng.random()
        try:
            if r < 0.3 or not live:
                stem = rng.choice(stems)
                toks = stem[:rng.randrange(1, len(stem) + 1)] + \
                    [rng.randrange(50) for _ in range(rng.randrange(0, 2 * bs))]
                live.append(m.allocate(toks))
            elif r < 0.75:
                m.append(rng.choice(live), rng.randrange(50))
            elif r < 0.85:
                live.append(m.fork(rng.choice(live)))
            else:
                s = rng.choice(live)
                live.remove(s)
                m.free(s)
        except mod.CapacityError:
            pass
        check_invariants(m)
    for s in live:
        m.free(s)
    assert m.num_free_blocks() == m.num_blocks
    check_invariants(m)


def pin_random_invariants(mod):
    for seed in range(3):
        random_operations(mod, seed, steps=200)


PINS = [pin_xxh64_empty_published_value, pin_chain_hash_example, pin_chain_break_is_final,
        pin_miss_ends_hits_after_remap,
        pin_kvblog_allocate_and_free_log, pin_kvblog_may_append_table, pin_lab_b2_step3_boundary,
        pin_minivllm_three_sequences, pin_lab_b6_reactivate_after_finish,
        pin_lab_b6_reference_counts_and_hits, pin_collision_guard, pin_copy_on_write_after_fork,
        pin_capacity, pin_random_invariants]


@pytest.mark.parametrize("pin", PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(_fresh_oracle())


def _fresh_oracle(old=None, new=None):
    """A private copy of the oracle module, optionally with one planted mistake."""
    src = open(obm.__file__).read()
    if old is not None:
        assert src.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("block_manager_copy")
    exec(compile(src, obm.__file__, "exec"), mod.__dict__)
    return mod


MUTANTS = [
    ("hash ignores the prefix", 'h.update(int(prefix).to_bytes(8, "little"))', "pass"),
    ("sharing forgets the reference", "self._refs[b] += 1  # shared with a live sequence",
     "pass  # shared with a live sequence"),
    ("a miss does not end the matching", "            if b is None:\n                break",
     "            if b is None:\n                continue"),
    ("the last block is matched", "for i in range(min(len(fps), need - 1)):", "for i in range(len(fps)):"),
    ("no token comparison", "self._holds[b] == (fp, tokens)", "self._holds[b] is not None"),
    ("cached tokens not counted", "len(matched) * self.block_size)", "0)"),
    ("a freed block shared instead of taken back", "            if self._refs[b] > 0:\n",
     "            if True:\n"),
    ("free walks first block first", "for b in reversed(s.table):", "for b in s.table:"),
    ("freed block to the front", "self._free[b] = None  # joins the back",
     "self._free[b] = None; self._free.move_to_end(b, last=False)  # joins the back"),
    ("new block on % == 0", "if n % self.block_size == 1:  # the token starts",
     "if n % self.block_size == 0:  # the token starts"),
    ("findable on % == 1", "if n % self.block_size == 0:  # the token completes",
     "if n % self.block_size == 1:  # the token completes"),
    ("no copy-on-write", "elif self._refs[s.table[-1]] > 1:", "elif False:"),
    ("fork adds no references", "        for b in s.table:\n            self._refs[b] += 1\n",
     "        for b in s.table:\n            pass\n"),
    ("stale index entry kept", "            del self._index[held[0]]", "            pass"),
    ("capacity off by one", "if len(self._free) < need:", "if len(self._free) < need - 1:"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new):
    mod = _fresh_oracle(old, new)
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except Exception:
            failed.append(pin.__name__)
    assert failed, f"no pin catches mutant: {name}"


# ---------------------------------------------------------------- native vs oracle

def test_native_chain_hash_matches(lib):
    rng = random.Random(11)
    for n in list(range(0, 70)) + [255, 256, 1024]:
        toks = [rng.randrange(-2**31, 2**31) for _ in range(n)]
        assert pk.pa_chain_hash(toks) == obm.compute_hash(toks), n
        pre = rng.randrange(2**64)
        assert pk.pa_chain_hash(toks, pre) == obm.compute_hash(toks, pre), n
    assert pk.pa_chain_hash([]) == xxhash.xxh64(b"").intdigest()


class Both:
    """The oracle and the native manager driven by the same operations."""

    def __init__(self, num_blocks, block_size):
        self.o = obm.BlockManager(num_blocks, block_size)
        self.n = pk.BlockManager(num_blocks, block_size)
        self.ids = {}  # oracle id -> native id

    def same(self):
        o, n = self.o, self.n
        assert o.num_free_blocks() == n.num_free_blocks()
        for b in range(o.num_blocks):
            assert o.ref_count(b) == n.ref_count(b), b
        for so, sn in self.ids.items():
            assert o.block_table(so) == n.block_table(sn)
            assert o.seq_len(so) == n.seq_len(sn)
            assert o.num_cached_tokens(so) == n.num_cached_tokens(sn)
        check_invariants(o)

    def allocate(self, toks):
        try:
            so = self.o.allocate(toks)
        except obm.CapacityError:
            with pytest.raises(pk.PAError) as e:
                self.n.allocate(toks)
            assert e.value.status == 7
            return None
        self.ids[so] = self.n.allocate(toks)
        return so

    def append(self, so, tok):
        try:
            want = self.o.append(so, tok)
        except obm.CapacityError:
            with pytest.raises(pk.PAError) as e:
                self.n.append(self.ids[so], tok)
            assert e.value.status == 7
            return
        assert self.n.append(self.ids[so], tok) == want

    def fork(self, so):
        c = self.o.fork(so)
        self.ids[c] = self.n.fork(self.ids[so])
        return c

    def free(self, so):
        self.o.free(so)
        self.n.free(self.ids.pop(so))


def test_native_worked_examples(lib):
    ex = EX["kvblog_allocate_log"]
    rng = random.Random(4)
    prompt = [rng.randrange(150000) for _ in range(ex["shared_prefix"])]
    bm = Both(ex["num_blocks"], ex["block_size"])
    ids = [bm.allocate(prompt + [rng.randrange(150000) for _ in range(n - len(prompt))])
           for n in ex["lens"]]
    bm.same()
    for s in ids:
        bm.free(s)
        bm.same()
    ex = EX["minivllm_three_sequences"]
    bm = Both(8, ex["block_size"])
    for x in ex["suffixes"]:
        bm.allocate(ex["prefix"] + [x])
    bm.same()
    assert [bm.n.block_table(i) for i in bm.ids.values()] == ex["block_tables"]
    # the first miss ends the hits, also after a table entry was dropped
    bm = Both(8, 4)
    P0, P1 = [1, 2, 3, 4], [5, 6, 7, 8]
    bm.allocate(P0 + P1 + [9])
    e = bm.allocate(P0)
    bm.free(e)
    bm.free(bm.allocate(list(range(100, 117))))
    b = bm.allocate(P0 + P1 + [10])
    bm.same()
    assert bm.n.num_cached_tokens(bm.ids[b]) == 0


@pytest.mark.parametrize("seed", range(6))
def test_native_random_operations(lib, seed):
    """The oracle and the native manager under the same random operations."""
    rng = random.Random(seed)
    bs = rng.choice([2, 4, 8, 16])
    bm = Both(rng.choice([12, 24, 64]), bs)
    stems = [[rng.randrange(50) for _ in range(rng.randrange(1, 6 * bs))] for _ in range(4)]
    live = []
    for _ in range(400):
        r = rng.random()
        if r < 0.3 or not live:
            stem = rng.choice(stems)
            toks = stem[:rng.randrange(1, len(stem) + 1)] + \
                [rng.randrange(50) for _ in range(rng.randrange(0, 2 * bs))]
            s = bm.allocate(toks)
            if s is not None:
                live.append(s)
        elif r < 0.75:
            bm.append(rng.choice(live), rng.randrange(50))
        elif r < 0.85:
            live.append(bm.fork(rng.choice(live)))
        else:
            s = rng.choice(live)
            live.remove(s)
            bm.free(s)
        bm.same()
    for s in live:
        bm.free(s)
    bm.same()
    assert bm.o.num_free_blocks() == bm.o.num_blocks


def test_native_errors(lib):
    assert lib.pa_bm_create(0, 16) is None
    assert lib.pa_bm_create(4, 1) is None
    m = pk.BlockManager(4, 4)
    with pytest.raises(pk.PAError):
        m.allocate([])
    with pytest.raises(pk.PAError):
        m.free(99)
    with pytest.raises(pk.PAError):
        m.block_table(99)
    with pytest.raises(pk.PAError):
        m.ref_count(4)
    assert pk.pa_status_string(7) == "not enough free blocks"
