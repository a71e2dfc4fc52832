"""The worked attention examples of the nano-vLLM lab manual ([Lab] appendix B.1.1-B.1.2),
run through the HIP kernels and held to the values the page prints.

The fixtures are tests/golden/lab_b1_attention.json.  The examples use 2-d vectors; here they
sit in the first dimensions of 64, the rest zero, which changes no dot product.  Each value row
also carries a one-hot code of its key position in spare dimensions, so one call returns the
output row and the attention weights that produced it.  The scale is the example's own
(1/sqrt(2), or 1 for the hand-given scores), passed as given.

Decode runs in fp32 and is held to the page's printed precision, except for the 8-digit
hand example: the page's 5e-9 is below fp32 resolution, so the fp32 tolerance (1e-5) applies
there.  The prefill kernels are bf16/fp16 only; the prefill examples run in fp16 at the fp16
tolerance (max 1e-2).  The pools are written by pa_store_kv_paged through a block table, and
start NaN-poisoned.
"""

import json
import os

import numpy as np
import pytest
import torch

import paged_kv_cache_67_amd as pk
from tests.gpu_util import TOL, announce

pytestmark = pytest.mark.gpu

D = 64
BS = 8
OH = 8  # first dimension of the one-hot position code in a value row
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "lab_b1_attention.json")


def _g():
    with open(GOLDEN) as f:
        return json.load(f)


def _rows(vectors, dtype, onehot=False):
    """[n, 1, D] device rows: vector i in the first dimensions, and with onehot the code of
    position i at dimension OH + i."""
    a = torch.zeros(len(vectors), 1, D, dtype=torch.float64)
    for i, v in enumerate(vectors):
        a[i, 0, :len(v)] = torch.tensor(v, dtype=torch.float64)
        if onehot:
            a[i, 0, OH + i] = 1.0
    return a.to(dtype).cuda()


def _pool(keys, values, dtype):
    """One sequence's keys and values at positions 0..n-1 of block 3 of a poisoned 4-block pool,
    stored by pa_store_kv_paged."""
    n = len(keys)
    kc = torch.full((4, BS, 1, D), float("nan"), dtype=dtype, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    bt = torch.tensor([[3]], dtype=torch.int32, device="cuda")
    cu = torch.tensor([0, n], dtype=torch.int32, device="cuda")
    lens = torch.tensor([n], dtype=torch.int32, device="cuda")
    pk.pa_store_kv_paged(_rows(keys, dtype), values, kc, vc, bt, cu, lens, n)
    return kc, vc, bt


def _decode(queries, lens, kc, vc, bt, scale):
    """fp32 decode of len(queries) sequences that share the pool's block table row; sequence i
    sees the first lens[i] keys."""
    B = len(queries)
    q = _rows(queries, torch.float32)
    out = torch.full_like(q, float("nan"))
    ctx = torch.tensor(lens, dtype=torch.int32, device="cuda")
    pk.pa_decode(out, q, kc, vc, bt.expand(B, -1).contiguous(), ctx, scale)
    torch.cuda.synchronize()
    return out[:, 0].double().cpu().numpy()


def _prefill(x, causal, scale):
    """fp16 prefill of one sequence with Q = K = V = x (value rows with their position code)."""
    n = len(x)
    kc, vc, bt = _pool(x, _rows(x, torch.float16, onehot=True), torch.float16)
    q = _rows(x, torch.float16)
    out = torch.full_like(q, float("nan"))
    cu = torch.tensor([0, n], dtype=torch.int32, device="cuda")
    pk.pa_prefill_paged(out, q, kc, vc, bt, cu, cu, n, n, scale, causal=causal)
    torch.cuda.synchronize()
    return out[:, 0].double().cpu().numpy()


def test_softmax_of_the_hand_given_scores():
    """B.1.1: scores [2, 1, 0] give probabilities of about [0.66524, 0.24473, 0.09003].  The
    keys are the scores along dimension 0 and the query is e0 (scale 1), so the weights are
    the softmax of the scores; the value rows are the position codes."""
    g = _g()["softmax_example"]
    announce("page example: softmax of [2, 1, 0] through pa_decode (fp32)")
    keys = [[s] for s in g["scores"]]
    kc, vc, bt = _pool(keys, _rows([[]] * 3, torch.float32, onehot=True), torch.float32)
    out = _decode([[1.0]], [3], kc, vc, bt, 1.0)
    np.testing.assert_allclose(out[0, OH:OH + 3], g["probabilities"], atol=g["abs_tol"], rtol=0)
    assert np.all(out[0, :OH] == 0) and np.all(out[0, OH + 3:] == 0)


def test_causal_self_attention_rows_by_decode():
    """B.1.2 step 2: X = [[1,0],[0,1],[1,1]], Q = K = V = X, causal, scale 1/sqrt(2): weight rows
    [1,0,0], [0.3302,0.6698,0], [0.2483,0.2483,0.5035], last output [0.7517, 0.7517].  Row i is
    a decode of query x_i over the first i + 1 keys."""
    g = _g()["causal_qkv_equal"]
    x = g["x"]
    announce("page example: causal rows of X through pa_decode (fp32)")
    kc, vc, bt = _pool(x, _rows(x, torch.float32, onehot=True), torch.float32)
    out = _decode(x, [1, 2, 3], kc, vc, bt, g["scale"])
    np.testing.assert_allclose(out[:, OH:OH + 3], g["weights"], atol=g["abs_tol"], rtol=0)
    np.testing.assert_allclose(out[2, :2], g["last_output"], atol=g["abs_tol"], rtol=0)
    want = np.array(g["weights"]) @ np.array(x)  # earlier rows from the printed weights
    np.testing.assert_allclose(out[:, :2], want, atol=2 * g["abs_tol"], rtol=0)


def test_causal_self_attention_rows_by_prefill():
    """The same three rows from one causal fp16 prefill of the whole sequence."""
    g = _g()["causal_qkv_equal"]
    announce("page example: causal rows of X through pa_prefill_paged (fp16)")
    out = _prefill(g["x"], True, g["scale"])
    tol = TOL["f16"][0]
    np.testing.assert_allclose(out[:, OH:OH + 3], g["weights"], atol=tol, rtol=0)
    np.testing.assert_allclose(out[2, :2], g["last_output"], atol=tol, rtol=0)


def test_hand_calculation_with_distinct_values():
    """B.1.2 supplementary hand calculation: Q = K = X, V = [[1,0],[0,2],[1,2]], q3 = [1,1]:
    weights [0.24825508, 0.24825508, 0.50348984], output [0.75174492, 1.50348984]."""
    g = _g()["hand_example_v_differs"]
    announce("page example: hand calculation through pa_decode (fp32)")
    kc, vc, bt = _pool(g["k"], _rows(g["v"], torch.float32, onehot=True), torch.float32)
    out = _decode([g["q"][-1]], [3], kc, vc, bt, g["scale"])
    tol = TOL["f32"][0]
    np.testing.assert_allclose(out[0, :2], g["last_output"], atol=tol, rtol=0)
    np.testing.assert_allclose(out[0, OH:OH + 3], g["last_weights"], atol=tol, rtol=0)


def test_future_change_moves_only_unmasked_rows():
    """B.1.2 step 3: the last position changed to [9, -5].  Causal: the two earlier output rows
    do not change (bit for bit).  Without the mask they change by about 8.15455 (largest
    absolute change over the two rows' value dimensions)."""
    g = _g()
    x = g["causal_qkv_equal"]["x"]
    fc = g["future_change"]
    y = [list(r) for r in x]
    y[-1] = fc["changed_last"]
    sc = g["causal_qkv_equal"]["scale"]
    announce("page example: a changed last position through pa_prefill_paged (fp16)")
    a, b = _prefill(x, True, sc), _prefill(y, True, sc)
    assert np.array_equal(a[:2], b[:2])
    a, b = _prefill(x, False, sc), _prefill(y, False, sc)
    delta = np.abs(a[:2, :2] - b[:2, :2]).max()
    assert abs(delta - fc["unmasked_earlier_delta"]) <= TOL["f16"][0], delta


def test_cached_append_equals_full_recomputation():
    """B.1.2 printed run: after one vector is appended, the new query reading the cached K/V
    matches a full recomputation over the four positions.  Here the cache holds X, and
    pa_decode_append stores the appended row and attends in one call (fp32); it must match the
    last row of a causal fp16 prefill of all four positions to the fp16 tolerance, for the
    appended vector [0.5, 1.0] (which reproduces the printed last output [0.6304, 0.8374]) and
    four random ones."""
    g = _g()
    x = g["causal_qkv_equal"]["x"]
    sc = g["causal_qkv_equal"]["scale"]
    c = g["cached_append"]
    rng = np.random.default_rng(3)
    appended = [c["appended_reading"]] + [list(rng.normal(0.0, 2.0, 2)) for _ in range(4)]
    for a in appended:
        announce(f"page example: pa_decode_append of {np.round(a, 3).tolist()} (fp32)")
        y = [list(r) for r in x] + [list(a)]
        kc, vc, bt = _pool(x, _rows(x, torch.float32, onehot=True), torch.float32)
        q = _rows([a], torch.float32)
        new_v = _rows(y, torch.float32, onehot=True)[3:]
        out = torch.full_like(q, float("nan"))
        ctx = torch.tensor([4], dtype=torch.int32, device="cuda")
        pk.pa_decode_append(out, q, _rows([a], torch.float32), new_v, kc, vc, bt, ctx, sc)
        torch.cuda.synchronize()
        cached = out[0, 0].double().cpu().numpy()
        assert torch.equal(kc[3, 3, 0].cpu(), _rows([a], torch.float32)[0, 0].cpu())  # stored
        full = _prefill(y, True, sc)[3]
        np.testing.assert_allclose(cached[:OH + 4], full[:OH + 4], atol=TOL["f16"][0], rtol=0)
        if a is c["appended_reading"]:
            np.testing.assert_allclose(cached[:2], c["last_output"], atol=c["abs_tol"], rtol=0)
