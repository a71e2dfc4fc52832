"""A continuous-batching loop end to end: block manager -> slots -> store -> attention.

Requests arrive over the steps; each step admits new prompts (allocate, whole prompt as
one chunk), extends the running sequences by one token (append, with a block taken at each
block boundary and a copy-on-write after a fork), stores the step's K/V rows through
pa_slot_mapping + pa_store_kv, and runs the whole varlen batch (prompt chunks and decode
rows) through pa_attention_mixed.  Every step is mirrored on the CPU with the oracle's
block manager, slot mapping, store and attention, and compared: block tables exactly, the
pools bit for bit, the attention output within the bf16 tolerance.
"""

import random

import numpy as np
import pytest
import torch

import oracle
import oracle.block_manager as obm
import paged_kv_cache_67_amd as pk
from paged_kv_cache_67_amd import harness
from tests.gpu_util import announce, assert_close, bits_equal, out_f64
from workloads import normal_values

pytestmark = pytest.mark.gpu

DTYPE, NB, BS, HQ, HKV, D = "bf16", 96, 16, 8, 2, 64
SCALE = 1.0 / 8.0


def _dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def test_continuous_batching_loop():
    rng = np.random.default_rng(91)
    rt = random.Random(91)
    # (arrival step, prompt length, new tokens); request 0 is forked after its prompt
    requests = [(0, 37, 12), (0, 16, 20), (2, 70, 8), (5, 5, 16), (7, 33, 6)]
    bm, om = pk.BlockManager(NB, BS), obm.BlockManager(NB, BS)
    dk = harness.to_device(np.zeros((NB, BS, HKV, D), np.uint16), DTYPE, "cuda")
    dv = harness.to_device(np.zeros((NB, BS, HKV, D), np.uint16), DTYPE, "cuda")
    k_host = np.zeros((NB, BS, HKV, D), np.uint16)
    v_host = np.zeros_like(k_host)
    running = {}  # native seq id -> [oracle seq id, tokens left]
    forked = False
    copies = grown = freed = 0
    for step in range(24):
        batch = []  # (native id, oracle id, new tokens this step)
        for (arrive, plen, gen) in requests:
            if arrive != step:
                continue
            toks = [rt.randrange(50000) for _ in range(plen)]
            s, o = bm.allocate(toks), om.allocate(toks)
            running[s] = [o, gen]
            batch.append((s, o, plen))
        pairs = []
        for s, (o, left) in list(running.items()):
            if any(b[0] == s for b in batch):
                continue
            if left == 0:
                bm.free(s)
                om.free(o)
                del running[s]
                freed += 1
                continue
            tok = rt.randrange(50000)
            nblk = len(bm.block_table(s))
            cow, ocow = bm.append(s, tok), om.append(o, tok)
            grown += len(bm.block_table(s)) > nblk
            assert cow == ocow
            if cow is not None:
                pairs.append(cow)
            running[s][1] -= 1
            batch.append((s, o, 1))
        if not forked and step == 1:  # a sibling of request 0 shares its blocks
            s0 = min(running)
            f, fo = bm.fork(s0), om.fork(running[s0][0])
            running[f] = [fo, 4]
            forked = True
        if not batch:
            continue
        tables = [bm.block_table(s) for s, _, _ in batch]
        assert tables == [om.block_table(o) for _, o, _ in batch]
        lens_k = np.array([bm.seq_len(s) for s, _, _ in batch], np.int32)
        lens_q = np.array([n for _, _, n in batch], np.int32)
        cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
        cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
        width = max(len(t) for t in tables)
        bt = np.full((len(batch), width), -1, np.int32)
        for i, t in enumerate(tables):
            bt[i, :len(t)] = t
        T = int(cu_q[-1])
        announce(f"serving loop step {step}: {len(batch)} sequences, {T} new tokens, "
                 f"{len(pairs)} copies")

        copies += len(pairs)
        if pairs:
            pk.pa_copy_blocks(dk, dv, _dev_i32(np.array(pairs)))
            oracle.copy_blocks(k_host, v_host, np.array(pairs))
        knew, vnew = (normal_values(rng, (T, HKV, D), DTYPE) for _ in range(2))
        q = normal_values(rng, (T, HQ, D), DTYPE)
        slots = torch.empty(T, dtype=torch.int32, device="cuda")
        d_bt, d_cuq, d_lens = _dev_i32(bt), _dev_i32(cu_q), _dev_i32(lens_k)
        pk.pa_slot_mapping(slots, d_bt, d_cuq, d_lens, BS, NB)
        pk.pa_store_kv(harness.to_device(knew, DTYPE, "cuda"),
                       harness.to_device(vnew, DTYPE, "cuda"), dk, dv, slots)
        want_slots = oracle.slot_mapping(bt, cu_q, lens_k, BS)
        oracle.store_kv(k_host, v_host, knew, vnew, want_slots)

        out = torch.empty(T, HQ, D, dtype=torch.bfloat16, device="cuda")
        ws_bytes = pk.pa_mixed_workspace_size(len(batch), HQ, HKV, D, int(lens_k.max()))
        ws = torch.empty(ws_bytes // 4 + 1, dtype=torch.float32, device="cuda")
        pk.pa_attention_mixed(out, harness.to_device(q, DTYPE, "cuda"), dk, dv, d_bt, d_cuq,
                              _dev_i32(cu_k), int(lens_q.max()), int(lens_k.max()), SCALE, ws)
        torch.cuda.synchronize()
        assert np.array_equal(slots.cpu().numpy(), want_slots)
        assert bits_equal(harness.from_device(dk), k_host)
        assert bits_equal(harness.from_device(dv), v_host)
        want = oracle.prefill(q, k_host, v_host, bt, cu_q, cu_k, SCALE, DTYPE)
        assert_close(out_f64(out, DTYPE), want, DTYPE, f"serving loop step {step}")
    assert bm.num_free_blocks() == om.num_free_blocks()
    # the loop went through a copy-on-write, block-boundary allocations and frees
    assert copies >= 1 and grown >= 3 and freed >= 3, (copies, grown, freed)
