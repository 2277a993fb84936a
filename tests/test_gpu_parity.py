"""GPU parity of the HIP megakernel against the CPU oracle, through the C ABI.

Routing (logits, top-k indices, histogram, exp_indptr, perm, inv) must match bit for bit;
topk_w within 1e-6; the layer output within 2e-2 * max|ref| (bf16 operands, fp32
accumulation).  Every case compares routing and output on every token, except the
four-times-prefill batch, whose output is compared on a token of every row tile of every
expert.
"""
import gc

import numpy as np
import pytest
import torch

import moe_groupgemm_amd as mk
import oracle
from gpu_cases import (check_out, check_routing, check_row_tiles, ctl_words, dev_inputs, expected_task_counts, log,
                       routing_numpy, row_tiles)
from moe_inputs import CONFIGS, Config, device_weights, make_bias, make_wr, make_x, small_case, to_torch_bf16

pytestmark = pytest.mark.gpu

SCHEDS = [mk.MOE_MK_SCHED_STATIC, mk.MOE_MK_SCHED_DYNAMIC]
SNAME = {0: "static", 1: "dynamic"}


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


def _info(E, k, d, f, B, key):
    """The library's per-batch choice `key` (moe_mk_forward_info) for a plan of this shape."""
    plan = mk.moe_mk_plan(E, k, d, f, mk.MOE_MK_SCHED_STATIC)
    try:
        return mk.moe_mk_forward_info(plan, B, key)
    finally:
        mk.moe_mk_plan_destroy(plan)


def run_small(x, Wr, bias, W1, W3, W2, k, sched, max_batch=None):
    B, d = x.shape
    E, _, f = W1.shape
    tx, tWr, tb, t1, t3, t2 = dev_inputs(x, Wr, bias, W1, W3, W2)
    layer = mk.MoELayer(E, k, d, f, tWr, t1, t3, t2, router_bias=tb, sched=sched,
                        max_batch=max(1, max_batch or B))
    out = layer(tx)
    torch.cuda.synchronize()
    assert layer.error() == 0
    got = routing_numpy(layer, B)
    res = out.float().cpu().numpy()
    return layer, res, got


def full_check(x, Wr, bias, W1, W3, W2, k, sched, what, debug=0):
    """Routing and output of one forward against the oracle, and the row tiles against the
    histogram; returns the output and the number of wide row tiles."""
    B = x.shape[0]
    E, d, f = W1.shape
    ref = oracle.forward(x, Wr, bias, W1, W3, W2, k)
    tx, tWr, tb, t1, t3, t2 = dev_inputs(x, Wr, bias, W1, W3, W2)
    layer = mk.MoELayer(E, k, d, f, tWr, t1, t3, t2, router_bias=tb, sched=sched, max_batch=B)
    mk.moe_mk_plan_set_debug(layer.plan, 0, debug)
    out = layer(tx).float().cpu().numpy()
    torch.cuda.synchronize()
    assert layer.error() == 0
    check_routing(routing_numpy(layer, B), ref, B, E)
    check_out(out, ref["out"], what)
    tiles, mw = row_tiles(layer, B)
    wide_min = mk.moe_mk_plan_info(layer.plan, "wide_min_rows")
    if debug & mk.MOE_MK_DEBUG_NARROW_ONLY or not mk.moe_mk_forward_info(layer.plan, B, "wide_ok") or \
            (debug & mk.MOE_MK_DEBUG_BATCH_RULE and B * k < 128 * E):
        wide_min = 1 << 30
    all_token = bool(mk.moe_mk_forward_info(layer.plan, B, "all_token_gate_up")) and \
        not debug & mk.MOE_MK_DEBUG_GROUPED_GATE_UP
    check_row_tiles(tiles, mw, ref["hist"], ref["exp_indptr"], wide_min, all_token=all_token)
    layer.close()
    return out, mw


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
@pytest.mark.parametrize("B", list(range(1, 10)))
def test_tiny_shapes(B, sched):
    log(f"tiny shape B={B} sched={SNAME[sched]}")
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, 128, 128, 4, 2, seed=1000 + B)
    full_check(x, Wr, bias, W1, W3, W2, 2, sched, f"tiny B={B}")


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_tiny_config(sched):
    cfg = CONFIGS["tiny"]
    log(f"config tiny sched={SNAME[sched]}")
    cfg2, x, Wr, bias, W1, W3, W2 = small_case(cfg.B, cfg.d, cfg.f, cfg.E, cfg.k, seed=cfg.seed)
    full_check(x, Wr, bias, W1, W3, W2, cfg.k, sched, "tiny config")


# Batches of one routing tile in which nearly every expert has tokens run the all-token gate/up
# (forward_info "all_token_gate_up"): each expert's gate/up tiles take every token of the batch,
# started before the routing, and the down projection gathers its rows from them.  Per output
# element that is the same MFMA sequence as over the grouped rows, so the result equals the
# grouped gate/up (MOE_MK_DEBUG_GROUPED_GATE_UP) bit for bit.  Cases: 16, 32 and 64 staged A rows,
# a four-way split down projection, k = E, and Zipf routing that leaves experts without tokens.
@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
@pytest.mark.parametrize("B,d,f,E,k,zipf", [(16, 256, 512, 8, 2, None), (24, 256, 384, 8, 2, None),
                                           (64, 256, 256, 16, 4, None), (32, 256, 8192, 8, 2, None),
                                           (5, 128, 256, 4, 4, None), (57, 256, 384, 64, 6, None),
                                           (48, 256, 384, 16, 6, 2.0)],
                         ids=["a16", "a32", "a64", "split4", "k_eq_E", "sweep_shape", "zipf_idle_experts"])
def test_all_token_gate_up(B, d, f, E, k, zipf, sched):
    log(f"all-token gate/up B={B} d={d} f={f} E={E} k={k} zipf={zipf} sched={SNAME[sched]}")
    assert _info(E, k, d, f, B, "all_token_gate_up") == 1
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, f, E, k, seed=4000 + B, zipf_s=zipf)
    ref = oracle.forward(x, Wr, bias, W1, W3, W2, k)
    if zipf:
        assert np.count_nonzero(ref["hist"] == 0) >= 1  # experts that get no token
    dense, _ = full_check(x, Wr, bias, W1, W3, W2, k, sched, "all-token gate/up")
    grouped, _ = full_check(x, Wr, bias, W1, W3, W2, k, sched, "grouped gate/up",
                            debug=mk.MOE_MK_DEBUG_GROUPED_GATE_UP)
    assert np.array_equal(dense.view(np.uint32), grouped.view(np.uint32))


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_ragged_multi_tile(sched):
    # several row tiles per expert, ragged row/column tails, several K steps, 4 routing tiles
    log(f"ragged multi-tile sched={SNAME[sched]}")
    cfg, x, Wr, bias, W1, W3, W2 = small_case(203, 256, 384, 16, 4, seed=77)
    full_check(x, Wr, bias, W1, W3, W2, 4, sched, "ragged B=203")


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_zero_input_all_ties(sched):
    cfg, x, Wr, bias, W1, W3, W2 = small_case(37, 128, 128, 8, 2, seed=5)
    x[:] = 0
    out, _ = full_check(x, Wr, bias, W1, W3, W2, 2, sched, "zero input")
    assert np.all(out == 0)


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_constant_input_one_expert_set(sched):
    # every token identical: the same k experts receive all 150 rows (3 row tiles each)
    cfg, x, Wr, bias, W1, W3, W2 = small_case(150, 128, 256, 8, 2, seed=6)
    x[:] = x[0]
    full_check(x, Wr, bias, W1, W3, W2, 2, sched, "constant input")


@pytest.mark.parametrize("k,E", [(1, 8), (8, 8), (1, 1), (16, 16), (3, 5)])
def test_k_and_e_edges(k, E):
    cfg, x, Wr, bias, W1, W3, W2 = small_case(70, 128, 128, E, k, seed=10 + k * 31 + E)
    full_check(x, Wr, bias, W1, W3, W2, k, mk.MOE_MK_SCHED_STATIC, f"k={k} E={E}")


@pytest.mark.parametrize("B,d,E", [(13, 512, 20), (70, 1024, 8), (512, 4096, 16), (600, 512, 12), (2048, 256, 256),
                                   (2100, 384, 252)],
                         ids=["four_experts_ragged", "four_experts_two_groups", "deep_stages", "four_tokens_per_wave",
                              "eight_tokens_per_wave", "eight_tokens_ragged"])
def test_router_stage_depths(B, d, E):
    # one token per wave: router tasks of 4 experts when 16-expert ones would be fewer than
    # 64 (d a multiple of 512; E = 20 leaves five blocks), else 16 experts with stages of
    # 512 values when d > 2048; more than 512 tokens: four tokens per wave, eight once that
    # leaves 512 router tasks (the last case also has a ragged token group and d not a
    # multiple of 256); E not a multiple of 16 leaves a ragged expert block
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, 128, E, 2, seed=900 + B)
    for sched in SCHEDS:
        full_check(x, Wr, bias, W1, W3, W2, 2, sched, f"router B={B} d={d} E={E} {SNAME[sched]}")


def test_zipf_bias_small():
    cfg, x, Wr, bias, W1, W3, W2 = small_case(100, 256, 128, 32, 4, seed=404, zipf_s=1.2)
    for sched in SCHEDS:
        full_check(x, Wr, bias, W1, W3, W2, 4, sched, f"zipf small {SNAME[sched]}")


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
@pytest.mark.parametrize("f,S", [(4096, 2), (8192, 4), (12288, 4)])
def test_down_projection_k_splits(f, S, sched):
    # small batches with a long f split the down projection's reduction into S ranges
    B, d, E, k = 21, 128, 4, 2
    assert _info(E, k, d, f, B, "S") == S
    log(f"down-projection splits S={S} f={f} sched={SNAME[sched]}")
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, f, E, k, seed=900 + S)
    full_check(x, Wr, bias, W1, W3, W2, k, sched, f"S={S}")


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
@pytest.mark.parametrize("B,d,f,E,k", [(300, 256, 384, 4, 2), (517, 256, 256, 16, 4), (129, 512, 128, 1, 1),
                                       (700, 256, 256, 2, 1)])
def test_wide_tiles(B, d, f, E, k, sched):
    # an expert averages >= 128 rows: 256-row tiles, ragged last tiles (some with rows for
    # one of the two 128-row halves only; experts of more than 256 rows with a second
    # tile), several K steps of 32
    log(f"wide tiles B={B} d={d} f={f} E={E} k={k} sched={SNAME[sched]}")
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, f, E, k, seed=1300 + B)
    _, mw = full_check(x, Wr, bias, W1, W3, W2, k, sched, f"wide B={B}")
    assert mw > 0


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_wide_tiles_constant_input(sched):
    # every token identical: k experts take all 324 rows each (tiles of 256 and 68 rows)
    cfg, x, Wr, bias, W1, W3, W2 = small_case(324, 256, 256, 4, 2, seed=61)
    x[:] = x[0]
    _, mw = full_check(x, Wr, bias, W1, W3, W2, 2, sched, "wide constant input")
    assert mw == 4  # two experts of 324 rows: a wide tile of 256 and one of 68 rows each


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_wide_forward_thin_row_tiles(sched):
    # Routing set by the input: logit e of token b is x[b, e] (Wr is the identity on the
    # first E values of j), so each expert receives an exact row count.  Experts of more than
    # 64 rows take wide row tiles (68 rows: one wide tile); their remainders of at most 64 rows
    # past a multiple of 256 (1, 16, 17, 64 rows) are narrow row tiles, as is the expert of 11
    # rows; the remainder of 65 rows is a wide row tile.
    counts = [257, 272, 273, 320, 11, 68, 321]
    E, k, d, f = len(counts), 2, 512, 256
    slots = np.repeat(np.arange(E), counts)
    B = len(slots) // k
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, f, E, k, seed=1700)
    x[:, :E] = 0
    x[np.arange(B), slots[:B]] = 0x4040       # bf16 3.0: slot 0
    x[np.arange(B), slots[B:]] = 0x3FC0       # bf16 1.5: slot 1 (a different expert)
    assert np.all(slots[:B] != slots[B:])
    Wr[:] = 0
    Wr[np.arange(E), np.arange(E)] = 1.0
    log(f"wide forward with thin row tiles B={B} counts={counts} sched={SNAME[sched]}")
    ref = oracle.forward(x, Wr, bias, W1, W3, W2, k)
    assert np.array_equal(ref["hist"], counts)
    layer, out, got = run_small(x, Wr, bias, W1, W3, W2, k, sched)
    check_routing(got, ref, B, E)
    check_out(out, ref["out"], "wide forward, thin row tiles")
    tiles, mw = row_tiles(layer, B)
    check_row_tiles(tiles, mw, ref["hist"], ref["exp_indptr"], 65)
    assert mw == 7 and len(tiles) - mw == 5
    layer.close()


def test_wide_tiles_static_dynamic_identical():
    cfg, x, Wr, bias, W1, W3, W2 = small_case(300, 256, 384, 4, 2, seed=1600)
    outs = []
    for sched in SCHEDS:
        layer, out, got = run_small(x, Wr, bias, W1, W3, W2, 2, sched)
        outs.append(out)
        layer.close()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
@pytest.mark.parametrize("d,f,S,dc", [(256, 4096, 2, 128), (384, 512, 1, 128)], ids=["split", "no_split"])
def test_exact_row_counts_narrow_forward(d, f, S, dc, sched):
    # A narrow forward whose routing is set by the input (token b's logit e is x[b, e]), so
    # the experts receive exactly 1, 16, 17, 40, 3, 0, 5 and 2 rows: row tiles at both sides of
    # the 16-row tile variant.  With d = 256 the down projection is split in two f ranges, each
    # split's partials added by the last one; with d = 384 it is not split.  Either way its
    # tasks are 128-column tiles (forward_info "down_cols": 256-column tasks would not fill a
    # round of the grid here); the two-weight split tiles run in the Mixtral-shaped test.
    counts = [1, 16, 17, 40, 3, 0, 5, 2]
    E, k = len(counts), 1
    B = sum(counts)
    assert _info(E, k, d, f, B, "S") == S and _info(E, k, d, f, B, "down_cols") == dc
    slots = np.repeat(np.arange(E), counts)
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, f, E, k, seed=1800 + d)
    x[:, :E] = 0
    x[np.arange(B), slots] = 0x4040  # bf16 3.0
    Wr[:] = 0
    Wr[np.arange(E), np.arange(E)] = 1.0
    log(f"exact row counts d={d} f={f} counts={counts} sched={SNAME[sched]}")
    ref = oracle.forward(x, Wr, bias, W1, W3, W2, k)
    assert np.array_equal(ref["hist"], counts)
    layer, out, got = run_small(x, Wr, bias, W1, W3, W2, k, sched)
    check_routing(got, ref, B, E)
    check_out(out, ref["out"], f"exact row counts d={d}")
    tiles, mw = row_tiles(layer, B)
    check_row_tiles(tiles, mw, ref["hist"], ref["exp_indptr"], 1 << 30)
    assert mw == 0 and len(tiles) == 7
    layer.close()


def test_down_projection_splits_static_dynamic_identical():
    cfg, x, Wr, bias, W1, W3, W2 = small_case(13, 128, 12288, 4, 2, seed=901)
    outs = []
    for sched in SCHEDS:
        layer, out, got = run_small(x, Wr, bias, W1, W3, W2, 2, sched)
        outs.append(out)
        layer.close()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


def test_zero_batch_enqueues_nothing():
    cfg, x, Wr, bias, W1, W3, W2 = small_case(4, 128, 128, 4, 2, seed=3)
    tx, tWr, tb, t1, t3, t2 = dev_inputs(x, Wr, bias, W1, W3, W2)
    layer = mk.MoELayer(4, 2, 128, 128, tWr, t1, t3, t2, max_batch=4)
    out = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    mk.moe_mk_forward(layer.plan, tx[:0], tWr, None, t1, t3, t2, out, 0, layer.ws)
    torch.cuda.synchronize()
    assert layer.error() == 0
    layer.close()


def test_static_and_dynamic_are_bitwise_identical():
    cfg, x, Wr, bias, W1, W3, W2 = small_case(131, 256, 256, 16, 3, seed=88)
    outs = []
    for sched in SCHEDS:
        layer, out, got = run_small(x, Wr, bias, W1, W3, W2, 3, sched)
        outs.append((out, got))
        layer.close()
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32))
    for key in ("topk_idx", "perm", "inv", "hist", "exp_indptr"):
        assert np.array_equal(outs[0][1][key], outs[1][1][key])


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
@pytest.mark.parametrize("B,E,d,f", [(40, 8, 256, 384), (90, 8, 256, 384), (300, 4, 256, 384), (2048, 256, 256, 384),
                                     (40, 12, 512, 384), (256, 64, 512, 1024), (4096, 32, 1024, 2048)],
                         ids=["one_tile", "narrow", "wide", "router_eight_tokens", "router_four_experts",
                              "static_takes_other_xcds", "wide_static_takes_other_xcds"])
def test_rest_state_and_task_counts(B, E, d, f, sched):
    # the last two cases have more than two GroupGEMM positions per workgroup (static:
    # workgroups take other XCDs' positions, in the wide forward down-projection ones only, and
    # combine tasks from one counter); every task runs once
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, f, E, 2, seed=12)
    tx, tWr, tb, t1, t3, t2 = dev_inputs(x, Wr, bias, W1, W3, W2)
    layer = mk.MoELayer(E, 2, d, f, tWr, t1, t3, t2, sched=sched, max_batch=B)
    before = ctl_words(layer, B).copy()
    outs = [layer(tx) for _ in range(3)]
    torch.cuda.synchronize()
    assert layer.error() == 0
    ref = oracle.forward(x, Wr, bias, W1, W3, W2, 2)
    check_routing(routing_numpy(layer, B), ref, B, E)
    check_out(outs[0].float().cpu().numpy(), ref["out"], f"rest state B={B} E={E}")
    for o in outs[1:]:  # every forward from the rest state gives the same bits
        assert torch.equal(o.view(torch.int16), outs[0].view(torch.int16))
    c = ctl_words(layer, B)
    C = mk.CTL
    assert c[C["epoch"]] == before[C["epoch"]] + 3    # epoch advanced once per forward
    assert c[C["exit"]] == 0                           # exit counter at rest
    assert c[C["qhead"]] == c[C["qtail"]] == 0        # queue at rest
    assert c[C["pf"]] == 0                             # weight-prefetch claims at rest
    assert all(c[C["xq"] + 32 * x] == 0 for x in range(8))  # static per-XCD claim counters at rest
    assert c[C["cq"]] == 0                             # static combine claim counter at rest
    assert c[C["ev_topk"]] == 0 and c[C["ev_scan"]] == 1 and c[C["ev_g1"]] == 0  # events at rest
    hist = routing_numpy(layer, B)["hist"]
    exp = expected_task_counts(layer, B)
    delta = c[C["dbg"]:C["dbg"] + 7] - before[C["dbg"]:C["dbg"] + 7]
    names = ["route", "topk", "scan", "group", "gemm1", "gemm2", "combine"]
    for i, n in enumerate(names):
        assert delta[i] == 3 * exp[n], (n, delta[i], exp[n])
    layer.close()


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_watchdog_turns_a_lost_notify_into_an_error(sched):
    cfg, x, Wr, bias, W1, W3, W2 = small_case(40, 128, 128, 4, 2, seed=21)
    tx, tWr, tb, t1, t3, t2 = dev_inputs(x, Wr, bias, W1, W3, W2)
    layer = mk.MoELayer(4, 2, 128, 128, tWr, t1, t3, t2, sched=sched, max_batch=40)
    mk.moe_mk_plan_set_debug(layer.plan, 2_000_000, mk.MOE_MK_DEBUG_DROP_NOTIFY)  # 20 ms watchdog
    layer(tx)
    torch.cuda.synchronize()
    assert layer.error() & mk.MOE_MK_ERR_WATCHDOG
    mk.moe_mk_plan_set_debug(layer.plan, 0, 0)
    layer.reinit()
    out = layer(tx)
    torch.cuda.synchronize()
    assert layer.error() == 0
    ref = oracle.forward(x, Wr, bias, W1, W3, W2, 2)
    check_out(out.float().cpu().numpy(), ref["out"], "after re-init")
    layer.close()


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
@pytest.mark.parametrize("B", [90, 40], ids=["two_tiles", "one_tile_all_token"])
def test_nonfinite_input_is_reported(B, sched):
    # a NaN and an infinity in x make router logits non-finite: the forward ends with
    # MOE_MK_ERR_NONFINITE in the error word, and after re-initialising the workspace a
    # clean input runs exactly as usual (B = 40: gate/up tiles that started before the routing
    # wait for it at their end and leave on the error)
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, 256, 256, 8, 2, seed=23)
    bad = x.copy()
    bad[5, 17] = 0x7FC0   # bf16 quiet NaN
    bad[B - 20, 3] = 0x7F80   # bf16 +infinity
    tx, tWr, tb, t1, t3, t2 = dev_inputs(bad, Wr, bias, W1, W3, W2)
    layer = mk.MoELayer(8, 2, 256, 256, tWr, t1, t3, t2, sched=sched, max_batch=B)
    layer(tx)
    torch.cuda.synchronize()
    assert layer.error() & mk.MOE_MK_ERR_NONFINITE
    layer.reinit()
    clean = to_torch_bf16(x).cuda()
    out = layer(clean)
    torch.cuda.synchronize()
    assert layer.error() == 0
    ref = oracle.forward(x, Wr, bias, W1, W3, W2, 2)
    check_routing(routing_numpy(layer, B), ref, B, 8)
    check_out(out.float().cpu().numpy(), ref["out"], "after a non-finite input")
    layer.close()


def test_two_layers_interleaved_on_a_side_stream():
    # two plans of different shapes and schedules, each with its own workspace, run
    # alternately on a non-default stream into preallocated outputs: neither disturbs the
    # other, and every output matches the oracle
    cases = [(70, 256, 384, 8, 2, mk.MOE_MK_SCHED_STATIC, 2000), (33, 128, 256, 16, 4, mk.MOE_MK_SCHED_DYNAMIC, 2001)]
    layers = []
    for B, d, f, E, k, sched, seed in cases:
        cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, f, E, k, seed=seed)
        tx, tWr, tb, t1, t3, t2 = dev_inputs(x, Wr, bias, W1, W3, W2)
        layer = mk.MoELayer(E, k, d, f, tWr, t1, t3, t2, router_bias=tb, sched=sched, max_batch=B)
        out = torch.empty((B, d), dtype=torch.bfloat16, device="cuda")
        ref = oracle.forward(x, Wr, bias, W1, W3, W2, k)
        layers.append((layer, tx, out, ref, B, E))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        for layer, tx, out, ref, B, E in layers:
            layer(tx, out=out, stream=side)
        side.synchronize()
        for layer, tx, out, ref, B, E in layers:
            assert layer.error(stream=side) == 0
            check_routing(routing_numpy(layer, B), ref, B, E)
            check_out(out.float().cpu().numpy(), ref["out"], f"interleaved B={B} pass {rep}")
    for layer, *_ in layers:
        layer.close()


def test_uninitialised_workspace_is_reported():
    cfg, x, Wr, bias, W1, W3, W2 = small_case(8, 128, 128, 4, 2, seed=22)
    tx, tWr, tb, t1, t3, t2 = dev_inputs(x, Wr, bias, W1, W3, W2)
    plan = mk.moe_mk_plan(4, 2, 128, 128, 0)
    n = mk.moe_mk_workspace_bytes(plan, 8)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    out = torch.empty((8, 128), dtype=torch.bfloat16, device="cuda")
    mk.moe_mk_forward(plan, tx, tWr, None, t1, t3, t2, out, 8, ws)
    torch.cuda.synchronize()
    assert mk.moe_mk_workspace_error(plan, ws) & mk.MOE_MK_ERR_UNINIT
    mk.moe_mk_plan_destroy(plan)


# ------------------------------------------------------------------------------ full-size configurations
# Each full configuration runs at its real size and is compared with the oracle on EVERY
# token (the oracle's token-parallel call), except the four-times-prefill batch, which is
# compared on a few hundred tokens chosen so that every row tile of every expert holds at
# least one of them.  Inputs and oracle results are computed once per configuration and
# shared by both schedules.

_FULL = {"key": None, "val": None}


class _FullCase:
    """Host inputs, device weights and (lazily) oracle results of one configuration."""

    def __init__(self, cfg):
        log(f"config {cfg.name}: generating inputs, routing on the oracle")
        self.cfg = cfg
        self.x_all = make_x(cfg)
        self.Wr, self.bias = make_wr(cfg), make_bias(cfg)
        self.routing = {B: oracle.routing(self.x_all[:B], self.Wr, self.bias, cfg.k) for B in cfg.batches}
        used = set()
        for r in self.routing.values():
            used |= {int(e) for e in np.unique(r["topk_idx"])}
        tWr, tb, t1, t3, t2, self.host = device_weights(cfg, keep=used)
        self.dev = (tWr, tb, t1, t3, t2)
        self.tx_all = to_torch_bf16(self.x_all).cuda()
        self.outs = {}

    def ref_out(self, B, toks):
        key = (B, tuple(toks))
        if key not in self.outs:
            r = self.routing[B]
            log(f"  oracle: {len(toks)} tokens of B={B}")
            self.outs[key] = oracle.moe_tokens(self.x_all[:B], toks, r["topk_idx"], r["topk_w"],
                                               lambda e: self.host[e], self.cfg.d, self.cfg.f)
        return self.outs[key]


def _case(cfg):
    if _FULL["key"] != cfg:
        _FULL["key"], _FULL["val"] = None, None
        gc.collect()
        torch.cuda.empty_cache()
        _FULL["val"] = _FullCase(cfg)
        _FULL["key"] = cfg
    return _FULL["val"]


def _tokens_of_every_row_tile(r, k, BM):
    """One token from the first row, every BM-th row and the last row of each expert's segment
    (with BM = 64 this hits every row tile of either shape)."""
    toks = set()
    ip = r["exp_indptr"]
    for e in range(len(ip) - 1):
        lo, hi = int(ip[e]), int(ip[e + 1])
        for p in list(range(lo, hi, BM)) + ([hi - 1] if hi > lo else []):
            toks.add(int(r["perm"][p]) // k)
    return sorted(toks)


def _full_config_of(cfg, sched, tokens="all"):
    c = _case(cfg)
    tWr, tb, t1, t3, t2 = c.dev
    log(f"config {cfg.name} sched={SNAME[sched]}")
    layer = mk.MoELayer(cfg.E, cfg.k, cfg.d, cfg.f, tWr, t1, t3, t2, router_bias=tb, sched=sched,
                        max_batch=max(cfg.batches))
    results = []
    for B in cfg.batches:
        out = layer(c.tx_all[:B])
        torch.cuda.synchronize()
        assert layer.error() == 0
        ref = c.routing[B]
        check_routing(routing_numpy(layer, B), ref, B, cfg.E)
        if tokens == "all":
            toks = list(range(B))
        else:
            toks = _tokens_of_every_row_tile(ref, cfg.k, 64)
            assert len(toks) >= tokens, len(toks)
        ref_out = c.ref_out(B, toks)
        got = out.float().cpu().numpy()
        check_out(got[toks], ref_out, f"{cfg.name} B={B} ({len(toks)} of {B} tokens)")
        results.append((B, out.clone()))
        log(f"  B={B}: routing exact, output within tolerance on {len(toks)} tokens")
    layer.close()
    return results, c


def _full_config(name, sched):
    return _full_config_of(CONFIGS[name], sched)


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_threshold_batches_one_plan(sched):
    # one plan and one workspace, batch sizes on both sides of every batch-size switch:
    # one routing tile or several (64/65), tokens per router wave (512/513), narrow or wide
    # tiles (B*k = 1022/1024 rows for 8 experts: 511/512), tokens per combine task
    # (1023/1024), then back to the smallest; every output is compared in full
    E, k, d, f = 8, 2, 256, 256
    Bmax = 1025
    cfg, x, Wr, bias, W1, W3, W2 = small_case(Bmax, d, f, E, k, seed=1900)
    tx, tWr, tb, t1, t3, t2 = dev_inputs(x, Wr, bias, W1, W3, W2)
    layer = mk.MoELayer(E, k, d, f, tWr, t1, t3, t2, router_bias=tb, sched=sched, max_batch=Bmax)
    for B in (64, 65, 511, 512, 513, 1023, 1024, 1025, 1):
        log(f"threshold batch B={B} sched={SNAME[sched]}")
        out = layer(tx[:B])
        torch.cuda.synchronize()
        assert layer.error() == 0
        ref = oracle.forward(x[:B], Wr, bias, W1, W3, W2, k)
        check_routing(routing_numpy(layer, B), ref, B, E)
        check_out(out.float().cpu().numpy(), ref["out"], f"threshold B={B}")
    layer.close()


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_config_mixtral_decode(sched):
    _full_config("mixtral_decode", sched)


def test_config_sweep_one_plan_no_recompile():
    cfg = CONFIGS["sweep"]
    results, c = _full_config("sweep", mk.MOE_MK_SCHED_STATIC)
    tWr, tb, t1, t3, t2 = c.dev
    # the same batches run on fresh workspaces in isolation give bitwise the same output,
    # and the leading tokens of a larger batch equal a smaller batch (batch-prefix invariance)
    full = dict(results)
    for B in (3, 57):
        layer = mk.MoELayer(cfg.E, cfg.k, cfg.d, cfg.f, tWr, t1, t3, t2, max_batch=B)
        out = layer(c.tx_all[:B])
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), full[B].view(torch.int16))
        assert torch.equal(full[512][:B].view(torch.int16), out.view(torch.int16))
        layer.close()


def test_config_sweep_dynamic():
    _full_config("sweep", mk.MOE_MK_SCHED_DYNAMIC)


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_config_deepseek_zipf(sched):
    _full_config("deepseek_zipf", sched)


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_config_prefill(sched):
    _full_config("prefill", sched)


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_large_batch_prefill_shape(sched):
    # four times the prefill batch (131072 routed rows): queue capacity, the per-XCD lists,
    # eight-token router tasks and wide tiles at a size well past the benchmark's; the output
    # is compared on a token of every row tile of every expert (first rows and last rows)
    cfg = Config("prefill_x4", d=2048, f=768, E=128, k=8, batches=(16384,), seed=606)
    _full_config_of(cfg, sched, tokens=256)


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_wide_long_k_every_token(sched):
    # wide tiles with the prefill's long reduction (d = 2048: 64 stages of the gate/up ring,
    # f = 768 for the down projection), about 256 rows per expert so experts take one full
    # tile and some a second, thin one; every token compared
    cfg = Config("wide_long_k", d=2048, f=768, E=8, k=2, batches=(1024,), seed=808)
    _full_config_of(cfg, sched)


def test_max_experts_and_top_k_wide():
    # the largest E and k the plan accepts, at a batch whose 128 rows per expert take wide tiles
    cfg, x, Wr, bias, W1, W3, W2 = small_case(2048, 256, 128, 256, 16, seed=707)
    for sched in SCHEDS:
        full_check(x, Wr, bias, W1, W3, W2, 16, sched, f"E=256 k=16 B=2048 {SNAME[sched]}")


@pytest.mark.parametrize("shape", [
    (1, 2048, 1408, 64, 6),   # the sweep's B = 1: six 1-row tiles, half-width gate/up and down tiles
    (40, 1024, 256, 4, 1),    # up to 40 rows per expert: the 64-row staging of the half-width tile
    (3, 1024, 4096, 4, 1),    # half width with the down projection split in two f ranges
    (2, 1024, 8192, 4, 1),    # ... and in four
], ids=["sweep_b1", "rows_40", "split_2", "split_4"])
def test_half_width_tiles(shape):
    # The smallest batches take narrow tiles of half the columns (forward_info "BN"), whose
    # eight waves split each K step in two halves and add them through LDS: every token
    # against the oracle on both schedules, and the two schedules bitwise equal.
    B, d, f, E, k = shape
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, f, E, k, seed=1900 + B)
    outs = []
    for sched in SCHEDS:
        plan = mk.moe_mk_plan(E, k, d, f, sched)
        assert mk.moe_mk_forward_info(plan, B, "BN") == mk.moe_mk_plan_info(plan, "BN1") // 2
        mk.moe_mk_plan_destroy(plan)
        out, _ = full_check(x, Wr, bias, W1, W3, W2, k, sched, f"half width B={B} d={d} f={f} {SNAME[sched]}")
        outs.append(out)
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
@pytest.mark.parametrize("B", [600, 200], ids=["batch_600", "batch_200"])
@pytest.mark.parametrize("policy", [0, mk.MOE_MK_DEBUG_NARROW_ONLY, mk.MOE_MK_DEBUG_BATCH_RULE],
                         ids=["by_rows", "narrow_only", "batch_rule"])
def test_tile_shape_per_expert(policy, sched, B):
    # Skewed routing (Zipf bias): a few experts receive hundreds of rows, most a few dozen.
    # The scan chooses each expert's row-tile shape from its own row count (default: wide
    # above 64 rows), or the debug policy forces all narrow or decides from the batch size
    # alone (B = 600 averages 150 rows per expert: wide; B = 200 averages 50: narrow); every
    # choice gives the oracle's result.
    d, f, E, k = 256, 256, 16, 4
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, f, E, k, seed=1800, zipf_s=1.2)
    ref = oracle.routing(x, Wr, bias, k)
    assert ref["hist"].max() > 64 and np.count_nonzero(ref["hist"] <= 64) >= 4
    log(f"tile shape per expert B={B} policy={policy} sched={SNAME[sched]} hist={ref['hist'].tolist()}")
    _, mw = full_check(x, Wr, bias, W1, W3, W2, k, sched, f"per-expert tiles policy={policy}", debug=policy)
    narrow = policy == mk.MOE_MK_DEBUG_NARROW_ONLY or (policy == mk.MOE_MK_DEBUG_BATCH_RULE and B * k < 128 * E)
    assert (mw == 0) == narrow


@pytest.mark.parametrize("B,d,f,E,k", [(16, 256, 512, 8, 2), (203, 256, 384, 16, 4), (300, 256, 384, 4, 2)],
                         ids=["one_tile", "ragged_multi_tile", "wide"])
def test_static_cooperative_launch(B, d, f, E, k):
    # the static schedule launched as a cooperative kernel (co-residency guaranteed by the
    # runtime) gives the plain static launch's output bit for bit
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, f, E, k, seed=2100 + B)
    out_c, _ = full_check(x, Wr, bias, W1, W3, W2, k, mk.MOE_MK_SCHED_STATIC_COOPERATIVE, f"cooperative B={B}")
    out_s, _ = full_check(x, Wr, bias, W1, W3, W2, k, mk.MOE_MK_SCHED_STATIC, f"static B={B}")
    assert np.array_equal(out_c.view(np.uint32), out_s.view(np.uint32))


# ------------------------------------------------------------------------------ unfused pipeline

@pytest.mark.parametrize("B,d,f,E,k,zipf", [(16, 256, 512, 8, 2, None), (203, 256, 384, 16, 4, None),
                                            (300, 256, 384, 4, 2, None), (21, 128, 8192, 4, 2, None),
                                            (600, 256, 256, 16, 4, 1.2), (1, 256, 256, 8, 2, None)],
                         ids=["one_tile", "ragged_multi_tile", "wide", "down_splits", "zipf_mixed_tiles", "B1"])
def test_unfused_pipeline_matches_megakernel(B, d, f, E, k, zipf):
    # seven kernels, one per phase, with the megakernel's task code: routing exact, output
    # within tolerance of the oracle and bitwise the megakernel's; the workspace stays at rest
    # (a megakernel forward on it afterwards is unaffected)
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, f, E, k, seed=2300 + B, zipf_s=zipf)
    ref = oracle.forward(x, Wr, bias, W1, W3, W2, k)
    tx, tWr, tb, t1, t3, t2 = dev_inputs(x, Wr, bias, W1, W3, W2)
    layer = mk.MoELayer(E, k, d, f, tWr, t1, t3, t2, router_bias=tb, sched=mk.MOE_MK_SCHED_STATIC, max_batch=B)
    log(f"unfused pipeline B={B} d={d} f={f} E={E} k={k}")
    out_u = layer.forward_unfused(tx)
    torch.cuda.synchronize()
    check_routing(routing_numpy(layer, B), ref, B, E)
    check_out(out_u.float().cpu().numpy(), ref["out"], f"unfused B={B}")
    out_m = layer(tx)
    torch.cuda.synchronize()
    assert layer.error() == 0
    assert torch.equal(out_u.view(torch.int16), out_m.view(torch.int16))
    layer.close()


@pytest.mark.parametrize("path", ["unfused", "megakernel"])
def test_graph_replays_match_eager(path):
    # the forward captured in a HIP graph (no memset nodes: the unfused pipeline arms no
    # events, the megakernel restores its control block itself), replayed several times with
    # eager forwards and synchronisations in between; every replay equals the eager result
    B, d, f, E, k = 90, 256, 384, 8, 2
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, f, E, k, seed=2400)
    tx, tWr, tb, t1, t3, t2 = dev_inputs(x, Wr, bias, W1, W3, W2)
    layer = mk.MoELayer(E, k, d, f, tWr, t1, t3, t2, sched=mk.MOE_MK_SCHED_DYNAMIC, max_batch=B)
    run = layer.forward_unfused if path == "unfused" else layer.forward
    out = torch.empty((B, d), dtype=torch.bfloat16, device="cuda")
    ref = run(tx).clone()
    torch.cuda.synchronize()
    run(tx, out)  # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(tx, out)
    for rep in range(4):
        out.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        eager = layer(tx)  # eager work between the replays
        torch.cuda.synchronize()
        assert torch.equal(eager.view(torch.int16), ref.view(torch.int16))
    assert layer.error() == 0
    del g
    layer.close()


def _random_shapes(n, seed):
    """Seeded layer shapes within what the plan accepts, sized so that the oracle finishes
    each in about a second (B*k*d*f below 2e9): every tile shape and both task loops are met
    (one and several routing tiles, half-width, narrow and wide row tiles, splits)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        E = int(rng.choice([4, 8, 12, 16, 32, 64]))
        k = int(rng.integers(1, min(E, 8) + 1))
        d = int(rng.choice([256, 512, 1024, 2048]))
        f = int(rng.choice([128, 256, 384, 512, 768, 1024, 4096]))
        B = int(rng.choice([1, 2, 5, 17, 64, 65, 130, 257, 700, 1500, 3000]))
        zipf = float(rng.choice([0.0, 1.2]))
        if B * k * d * f > 2e9:
            continue
        out.append((B, d, f, E, k, zipf))
    return out


@pytest.mark.parametrize("shape", _random_shapes(10, 2024), ids=lambda s: "B%d_d%d_f%d_E%d_k%d_z%g" % s)
def test_random_shapes(shape):
    # Every token against the oracle on both schedules, the two bitwise equal, and the row
    # tiles against the histogram.
    B, d, f, E, k, zipf = shape
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, f, E, k, seed=3000 + B + E, zipf_s=zipf or None)
    outs = [full_check(x, Wr, bias, W1, W3, W2, k, sched, f"random B={B} d={d} f={f} E={E} k={k} {SNAME[sched]}")[0]
            for sched in SCHEDS]
    assert np.array_equal(outs[0], outs[1])
