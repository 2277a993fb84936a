"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test checks one part of the oracle against a closed form, a special case that
reduces to a library routine, a brute-force computation on tiny inputs, an invariance,
or a hand-derived fixture under tests/golden/.  A plausible mistake (dropped bias,
wrong summation order, gate/up swapped, transposed weight, unstable grouping, missing
combine weight, wrong tie-break) fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from moe_inputs import bf16_bits_to_f32, small_case, to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(v: float) -> int:
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])


# ----------------------------------------------------------------------------- router

def test_router_summation_order_fixture():
    g = json.load(open(os.path.join(GOLDEN, "router_order.json")))
    d, E = g["d"], g["E"]
    Wr = np.full((d, E), g["wr_value"], dtype=np.float32)
    for case in g["cases"]:
        x = np.zeros((1, d), dtype=np.float32)
        for j, v in case["x_nonzero"].items():
            x[0, int(j)] = v
        xb = to_bf16_bits(x)
        assert np.array_equal(bf16_bits_to_f32(xb), x), "fixture values must be exact in bf16"
        logit = oracle.router_logits(xb, Wr)[0, 0]
        assert _bits(logit) == int(case["expected_hex"], 16), case["name"]


@pytest.mark.parametrize("B,d,E,zipf", [(16, 256, 8, None), (9, 2048, 64, None), (5, 7168, 256, 1.2)])
def test_router_within_higham_bound_of_fp64(B, d, E, zipf):
    cfg, x, Wr, bias, *_ = small_case(B, d, 128, E, 2, seed=7 + d, zipf_s=zipf) if d <= 256 else (None,) * 7
    if cfg is None:  # avoid drawing large expert weights for router-only checks
        from moe_inputs import Config, make_bias, make_wr, normal_bf16, T_X
        cfg = Config("r", d=d, f=128, E=E, k=2, batches=(B,), seed=7 + d, zipf_s=zipf)
        x = normal_bf16((B, d), 1.0, cfg.seed, T_X, 0)
        Wr, bias = make_wr(cfg), make_bias(cfg)
    logits = oracle.router_logits(x, Wr, bias).astype(np.float64)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    exact = xf @ Wr.astype(np.float64) + (0.0 if bias is None else bias.astype(np.float64))
    n = d // 64 + 7
    u = 2.0 ** -24
    gamma = n * u / (1 - n * u)
    bound = gamma * (np.abs(xf) @ np.abs(Wr.astype(np.float64)) + (0 if bias is None else np.abs(bias)))
    assert np.all(np.abs(logits - exact) <= bound + 1e-30)
    if bias is not None:  # a dropped bias would be far outside the bound
        assert np.max(np.abs(bias)) > 100 * np.max(bound)


def test_router_one_hot_rows_are_exact():
    d, E = 192, 16
    rng = np.random.default_rng(3)
    Wr = rng.standard_normal((d, E)).astype(np.float32)
    js = [0, 1, 63, 64, 100, 191]
    x = np.zeros((len(js), d), dtype=np.float32)
    for r, j in enumerate(js):
        x[r, j] = 1.0
    logits = oracle.router_logits(to_bf16_bits(x), Wr)
    assert np.array_equal(logits, Wr[js])
    idx = oracle.topk(logits, 3)
    for r, j in enumerate(js):
        ref = np.lexsort((np.arange(E), -Wr[j].astype(np.float64)))[:3]
        assert list(idx[r]) == list(ref)


def test_router_zero_input_ties_go_to_lowest_index():
    B, d, E, k = 4, 128, 8, 2
    x = np.zeros((B, d), dtype=np.uint16)
    Wr = np.random.default_rng(0).standard_normal((d, E)).astype(np.float32)
    r = oracle.routing(x, Wr, None, k)
    assert np.all(r["logits"] == 0.0) and not np.any(np.signbit(r["logits"]))
    assert np.all(r["topk_idx"] == np.arange(k))
    assert np.all(r["topk_w"] == 0.5)


def test_router_bias_is_added_after_the_sum():
    cfg, x, Wr, _, *_ = small_case(6, 256, 128, 16, 2, seed=11)
    bias = np.linspace(-1, 1, 16).astype(np.float32)
    a = oracle.router_logits(x, Wr, None)
    b = oracle.router_logits(x, Wr, bias)
    assert np.array_equal(b, (a + bias).astype(np.float32))


# ----------------------------------------------------------------------------- top-k

def _brute_topk(row, k):
    order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))
    return order[:k]


def test_topk_matches_brute_force_with_ties():
    rng = np.random.default_rng(5)
    B, E = 40, 12
    logits = rng.integers(-3, 4, size=(B, E)).astype(np.float32)  # many exact ties
    for k in (1, 3, E):
        idx = oracle.topk(logits, k)
        for b in range(B):
            assert list(idx[b]) == _brute_topk(logits[b], k)


def test_topk_k1_is_first_argmax_and_signed_zero_ties():
    logits = np.array([[-0.0, 0.0, -1.0], [0.0, -0.0, -1.0], [-5.0, 2.0, 2.0]], dtype=np.float32)
    idx = oracle.topk(logits, 1)
    assert list(idx[:, 0]) == [0, 0, 1]
    assert list(idx[:, 0]) == list(np.argmax(logits, axis=1))


def test_topk_rejects_nan():
    with pytest.raises(ValueError):
        oracle.topk(np.array([[0.0, np.nan]], dtype=np.float32), 1)


# ----------------------------------------------------------------------------- softmax

def test_softmax_closed_forms():
    rng = np.random.default_rng(9)
    B, E = 30, 16
    logits = rng.standard_normal((B, E)).astype(np.float32)
    for k in (1, 2, 6, E):
        idx = oracle.topk(logits, k)
        w = oracle.softmax_topk(logits, idx)
        assert np.all(np.abs(w.sum(1) - 1.0) <= k * 2.0 ** -52 * 4)
        if k == 1:
            assert np.all(w == 1.0)
        sel = np.take_along_axis(logits, idx, 1).astype(np.float64)
        full = np.exp(logits.astype(np.float64))  # full softmax, renormalised over the selection
        ren = np.take_along_axis(full, idx, 1)
        ren = ren / ren.sum(1, keepdims=True)
        assert np.allclose(w, ren, rtol=1e-13, atol=0)
        for i, j in itertools.combinations(range(k), 2):
            assert np.allclose(w[:, i] / w[:, j], np.exp(sel[:, i] - sel[:, j]), rtol=1e-13)
        assert np.all(np.diff(w, axis=1) <= 0)  # slot order is descending logit
    eq = np.zeros((1, E), dtype=np.float32)
    w = oracle.softmax_topk(eq, oracle.topk(eq, 4))
    assert np.all(w == 0.25)


# ----------------------------------------------------------------------------- histogram / scan / permutation

@pytest.mark.parametrize("B,E,k", [(1, 8, 2), (37, 16, 4), (128, 256, 8), (0, 8, 2)])
def test_histogram_and_permutation_invariants(B, E, k):
    rng = np.random.default_rng(B + E)
    logits = rng.standard_normal((B, E)).astype(np.float32)
    idx = oracle.topk(logits, k) if B else np.zeros((0, k), np.int32)
    hist, indptr = oracle.histogram(idx, E)
    assert hist.sum() == B * k and indptr[E] == B * k and indptr[0] == 0
    assert np.array_equal(hist, np.bincount(idx.ravel(), minlength=E))
    assert np.all(hist <= B)
    assert np.array_equal(np.diff(indptr), hist)
    perm, inv = oracle.permutation(idx, indptr, E)
    if B == 0:
        return
    assert np.array_equal(np.sort(perm), np.arange(B * k))
    assert np.array_equal(inv[perm], np.arange(B * k))
    for e in range(E):
        seg = perm[indptr[e]:indptr[e + 1]]
        assert np.all(idx.ravel()[seg] == e)
        assert np.all(np.diff(seg // k) > 0)  # tokens strictly ascending


def test_routing_is_permutation_invariant():
    cfg, x, Wr, bias, W1, W3, W2 = small_case(24, 128, 128, 8, 3, seed=21, zipf_s=1.2)
    P = np.random.default_rng(1).permutation(24)
    a = oracle.forward(x, Wr, bias, W1, W3, W2, 3)
    b = oracle.forward(x[P], Wr, bias, W1, W3, W2, 3)
    assert np.array_equal(b["topk_idx"], a["topk_idx"][P])
    assert np.array_equal(b["topk_w"], a["topk_w"][P])
    assert np.array_equal(b["hist"], a["hist"]) and np.array_equal(b["exp_indptr"], a["exp_indptr"])
    assert np.array_equal(b["out"], a["out"][P])  # bitwise: tokens are independent


# ----------------------------------------------------------------------------- experts / combine

def _torch_ffn(xf, W1, W3, W2):
    g = xf @ W1
    return (g * torch.sigmoid(g) * (xf @ W3)) @ W2


def test_single_expert_is_dense_swiglu_ffn():
    cfg, x, Wr, bias, W1, W3, W2 = small_case(7, 128, 96, 1, 1, seed=31)
    r = oracle.forward(x, Wr, bias, W1, W3, W2, 1)
    t = lambda a: torch.from_numpy(bf16_bits_to_f32(a).astype(np.float64))
    ref = _torch_ffn(t(x), t(W1[0]), t(W3[0]), t(W2[0])).numpy()
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_identical_experts_give_the_dense_ffn_for_any_routing():
    cfg, x, Wr, bias, W1, W3, W2 = small_case(10, 128, 64, 6, 3, seed=41)
    W1[:] = W1[0]
    W3[:] = W3[0]
    W2[:] = W2[0]
    r = oracle.forward(x, Wr, bias, W1, W3, W2, 3)
    t = lambda a: torch.from_numpy(bf16_bits_to_f32(a).astype(np.float64))
    ref = _torch_ffn(t(x), t(W1[0]), t(W3[0]), t(W2[0])).numpy()
    assert np.allclose(r["out"], ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())


def test_expert_arithmetic_equals_brute_force_dense_loop():
    # pins the per-token expert arithmetic (gate/up, SwiGLU, down, combine weights) and the
    # top-k decision against plain fp64 loops; grouping is pinned by the bijection, stable
    # segment and permutation-invariance tests
    B, d, f, E, k = 3, 4, 3, 3, 2
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, f, E, k, seed=51)
    r = oracle.forward(x, Wr, bias, W1, W3, W2, k)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    w1, w3, w2 = (bf16_bits_to_f32(a).astype(np.float64) for a in (W1, W3, W2))
    for b in range(B):
        # brute force: score every expert in fp64 (decisions cross-checked against the fp32 ones)
        out = [0.0] * d
        for i in range(k):
            e = int(r["topk_idx"][b, i])
            h = []
            for n in range(f):
                g = sum(xf[b, c] * w1[e, c, n] for c in range(d))
                u = sum(xf[b, c] * w3[e, c, n] for c in range(d))
                h.append(g / (1.0 + math.exp(-g)) * u)
            for j in range(d):
                out[j] += r["topk_w"][b, i] * sum(h[n] * w2[e, n, j] for n in range(f))
        assert np.allclose(r["out"][b], out, rtol=1e-13, atol=1e-15)
        sc = xf[b] @ Wr.astype(np.float64)
        assert list(r["topk_idx"][b]) == _brute_topk(sc, k)


def test_worked_example_fixture():
    g = json.load(open(os.path.join(GOLDEN, "worked_example.json")))
    ev = lambda s: eval(s, {"exp": math.exp, "e": math.e})  # closed forms written in the fixture
    x = to_bf16_bits(np.array([g["x"]], dtype=np.float32))
    Wr = np.array(g["Wr"], dtype=np.float32)
    W1, W3, W2 = (to_bf16_bits(np.array(g[n], dtype=np.float32)) for n in ("W1", "W3", "W2"))
    for case in g["cases"]:
        r = oracle.forward(x, Wr, None, W1, W3, W2, case["k"])
        assert list(r["topk_idx"][0]) == case["topk_idx"]
        assert np.allclose(r["topk_w"][0], [ev(s) for s in case["topk_w"]], rtol=1e-15, atol=0)
        assert np.allclose(r["out"][0], [ev(s) for s in case["out"]], rtol=1e-15, atol=1e-300)
        if "out_if_gate_up_swapped" in case:
            assert not np.allclose(r["out"][0], [ev(s) for s in case["out_if_gate_up_swapped"]])


def test_combine_scaling_and_single_slot():
    cfg, x, Wr, bias, W1, W3, W2 = small_case(8, 128, 64, 4, 2, seed=61)
    a = oracle.forward(x, Wr, bias, W1, W3, W2, 2)
    W2x2 = to_bf16_bits(bf16_bits_to_f32(W2) * 2)  # exact in bf16
    b = oracle.forward(x, Wr, bias, W1, W3, W2x2, 2)
    assert np.array_equal(b["out"], 2 * a["out"])
    one = oracle.forward(x, Wr, bias, W1, W3, W2, 1)
    for t in range(8):
        e = int(one["topk_idx"][t, 0])
        assert one["topk_w"][t, 0] == 1.0
        y = oracle.expert_row(x[t], W1[e], W3[e], W2[e])
        assert np.array_equal(one["out"][t], y)


def test_batch_prefix_invariance():
    cfg, x, Wr, bias, W1, W3, W2 = small_case(20, 128, 64, 8, 3, seed=71)
    full = oracle.forward(x, Wr, bias, W1, W3, W2, 3)
    for B in (1, 3, 11):
        part = oracle.forward(x[:B], Wr, bias, W1, W3, W2, 3)
        assert np.array_equal(part["topk_idx"], full["topk_idx"][:B])
        assert np.array_equal(part["out"], full["out"][:B])


def test_empty_batch():
    cfg, x, Wr, bias, W1, W3, W2 = small_case(1, 128, 64, 4, 2, seed=81)
    r = oracle.forward(x[:0], Wr, bias, W1, W3, W2, 2)
    assert r["out"].shape == (0, 128) and r["hist"].sum() == 0 and r["exp_indptr"][-1] == 0


def test_oracle_thread_count_does_not_change_results():
    cfg, x, Wr, bias, W1, W3, W2 = small_case(12, 256, 512, 8, 2, seed=91)
    n = oracle.num_threads()
    oracle.set_threads(1)
    a = oracle.forward(x, Wr, bias, W1, W3, W2, 2)
    oracle.set_threads(max(2, n))
    b = oracle.forward(x, Wr, bias, W1, W3, W2, 2)
    oracle.set_threads(n)
    assert np.array_equal(a["logits"], b["logits"]) and np.array_equal(a["out"], b["out"])


def test_token_parallel_batch_equals_single_token_calls():
    # the token-parallel call and the column-parallel single-token call give the same bits,
    # at one thread and at several, for any order of the listed tokens
    cfg, x, Wr, bias, W1, W3, W2 = small_case(9, 256, 384, 6, 3, seed=93)
    r = oracle.routing(x, Wr, bias, 3)
    toks = [8, 0, 3, 3, 5]
    n = oracle.num_threads()
    outs = []
    for th in (1, max(3, n)):
        oracle.set_threads(th)
        outs.append(oracle.moe_tokens(x, toks, r["topk_idx"], r["topk_w"], (W1, W3, W2), 256, 384))
    oracle.set_threads(n)
    assert np.array_equal(outs[0], outs[1])
    for row, t in zip(outs[0], toks):
        single = oracle.moe_token(x[t], r["topk_idx"][t], r["topk_w"][t], (W1, W3, W2), 256, 384)
        assert np.array_equal(row, single)
