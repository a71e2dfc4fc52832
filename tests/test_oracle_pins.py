"""The CPU oracle against what the pages and the mathematics fix.

``test_pin`` runs every check of ``oracle_checks`` on the oracle.
``test_planted_mistake_is_caught`` plants one plausible mistake at a time in a
copy of the oracle's source (a dropped term, a wrong sign or index, a swapped
operand) and requires that at least one check fails for it.
"""

import types

import pytest

import oracle.paged_attention as pa_mod
from tests import oracle_checks as oc


@pytest.mark.parametrize("check", oc.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(oc.real_oracle())


MUTANTS = [
    ("slot offset uses // instead of %", "blk * block_size + p % block_size", "blk * block_size + p // block_size"),
    ("slot ignores cached prefix", "p = int(lens[b]) - lq + i", "p = i"),
    ("slot position off by one", "p = int(lens[b]) - lq + i", "p = int(lens[b]) - lq + i + 1"),
    ("store writes V into K pool", "k_pool[s // bs, s % bs] = key[t]", "k_pool[s // bs, s % bs] = value[t]"),
    ("store does not skip -1", "if s == -1:\n            continue", "pass"),
    ("gather row off by one", "return pool[blk, t % block_size]", "return pool[blk, (t + 1) % block_size]"),
    ("decode GQA maps h % HKV", "            g = h // G\n            w = _softmax_rows(scale", "            g = h % HKV\n            w = _softmax_rows(scale"),
    ("decode drops scale", "_softmax_rows(scale * (K[:, g, :] @ qf[b, h]))", "_softmax_rows(K[:, g, :] @ qf[b, h])"),
    ("decode weights K not V", "out[b, h] = w @ V[:, g, :]", "out[b, h] = w @ K[:, g, :]"),
    ("softmax not normalised", "return e / np.sum(e, axis=-1, keepdims=True)", "return e"),
    ("softmax exponent sign", "e = np.exp(s - m)\n    return", "e = np.exp(m - s)\n    return"),
    ("prefill mask off by one", "np.arange(Lk)[None, :] <= pos", "np.arange(Lk)[None, :] < pos"),
    ("prefill mask top-left aligned", "pos = (Lk - Lq) + np.arange(Lq)[:, None]", "pos = np.arange(Lq)[:, None]"),
    ("prefill softmax over the query axis", "out[q0:q1, h] = _softmax_rows(s) @ V[:, g, :]", "out[q0:q1, h] = _softmax_rows(s.T).T @ V[:, g, :]"),
    ("prefill scores against V", "s = scale * (qf[q0:q1, h, :] @ K[:, g, :].T)", "s = scale * (qf[q0:q1, h, :] @ V[:, g, :].T)"),
    ("prefill GQA maps h % HKV", "            g = h // G\n            s = scale", "            g = h % HKV\n            s = scale"),
    ("merge weight sign", "w = np.exp(mm - M)", "w = np.exp(M - mm)"),
    ("partial drops last key", "lo, hi = p * P, min((p + 1) * P, L)", "lo, hi = p * P, min((p + 1) * P, L - 1)"),
    ("merge forgets l", "/ (w @ l[b, h, :n].astype(np.float64))", "/ np.sum(w)"),
    ("bf16 widening shift", "<< np.uint32(16)", "<< np.uint32(15)"),
    ("copy_blocks copies K only", "        v_pool[dst] = v_pool[src]\n", "\n"),
    ("copy_blocks direction swapped", "k_pool[dst] = k_pool[src]", "k_pool[src] = k_pool[dst]"),
    ("negative positions wrap to the table's end", "if 0 <= j < bt.shape[1] else -1", "if j < bt.shape[1] else -1"),
    ("copy_blocks keeps out-of-range pairs", "if not (0 <= src < nb and 0 <= dst < nb) or src == dst:", "if src == dst:"),
]


def _mutant_namespace(old, new):
    src = open(pa_mod.__file__).read()
    assert src.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return types.SimpleNamespace(
        decode=mod.decode, prefill=mod.prefill, slot_mapping=mod.slot_mapping,
        store_kv=mod.store_kv, decode_partials=mod.decode_partials, lse_merge=mod.lse_merge,
        gather_rows=mod.gather_rows, to_f64=mod.to_f64, copy_blocks=mod.copy_blocks)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new):
    ns = _mutant_namespace(old, new)
    failed = []
    for check in oc.ALL_CHECKS:
        try:
            check(ns)
        except Exception:  # AssertionError, or the mutant crashing outright
            failed.append(check.__name__)
    assert failed, f"no pin catches mutant: {name}"
