"""GPU parity of the HIP megakernel against the CPU oracle, through the C ABI.

Routing (logits, top-k indices, histogram, exp_indptr, perm, inv) must match bit for bit;
topk_w within 1e-6; the layer output within 2e-2 * max|ref| (bf16 operands, fp32
accumulation).  Small cases compare every token; the full-size configurations compare
routing for every token and the output on sampled tokens the oracle computes one by one.
"""
import gc

import numpy as np
import pytest
import torch

import moe_groupgemm_amd as mk
import oracle
from gpu_cases import (check_out, check_routing, ctl_words, dev_inputs, down_splits, expected_task_counts, log,
                       routing_numpy, tile_config)
from moe_inputs import (CONFIGS, Config, bf16_bits_to_f32, device_weights, device_x, expert_weights, make_bias,
                        make_wr, make_x, small_case, to_torch_bf16)

pytestmark = pytest.mark.gpu

SCHEDS = [mk.MOE_MK_SCHED_STATIC, mk.MOE_MK_SCHED_DYNAMIC]
SNAME = {0: "static", 1: "dynamic"}


@pytest.fixture(autouse=True)
def _free_memory():
    yield
    gc.collect()
    torch.cuda.empty_cache()


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


def full_check(x, Wr, bias, W1, W3, W2, k, sched, what):
    B = x.shape[0]
    ref = oracle.forward(x, Wr, bias, W1, W3, W2, k)
    layer, out, got = run_small(x, Wr, bias, W1, W3, W2, k, sched)
    check_routing(got, ref, B, W1.shape[0])
    check_out(out, ref["out"], what)
    layer.close()
    return out


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
    out = full_check(x, Wr, bias, W1, W3, W2, 2, sched, "zero input")
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
    assert down_splits(B, k, f) == S
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
    assert tile_config(B, k, E, d, f)[0] == 256
    log(f"wide tiles B={B} d={d} f={f} E={E} k={k} sched={SNAME[sched]}")
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, f, E, k, seed=1300 + B)
    full_check(x, Wr, bias, W1, W3, W2, k, sched, f"wide B={B}")


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_wide_tiles_constant_input(sched):
    # every token identical: k experts take all 324 rows each (tiles of 256 and 68 rows)
    cfg, x, Wr, bias, W1, W3, W2 = small_case(324, 256, 256, 4, 2, seed=61)
    x[:] = x[0]
    assert tile_config(324, 2, 4, 256, 256)[0] == 256
    full_check(x, Wr, bias, W1, W3, W2, 2, sched, "wide constant input")


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_wide_forward_thin_row_tiles(sched):
    # Routing set by the input: logit e of token b is x[b, e] (Wr is the identity on the
    # first E values of j), so each expert receives an exact row count.  In this wide-tile
    # forward the row tiles of at most 64 rows (1, 16, 17, 64 rows past 256; experts of 11
    # and 68 rows) run as narrow tiles, the others (65 past 256, 68 alone) as wide tiles.
    counts = [257, 272, 273, 320, 11, 68, 321]
    E, k, d, f = len(counts), 2, 512, 256
    slots = np.repeat(np.arange(E), counts)
    B = len(slots) // k
    assert tile_config(B, k, E, d, f)[0] == 256
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
    layer.close()


def test_wide_tiles_static_dynamic_identical():
    cfg, x, Wr, bias, W1, W3, W2 = small_case(300, 256, 384, 4, 2, seed=1600)
    outs = []
    for sched in SCHEDS:
        layer, out, got = run_small(x, Wr, bias, W1, W3, W2, 2, sched)
        outs.append(out)
        layer.close()
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


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
                                     (40, 12, 512, 384), (256, 64, 512, 1024)],
                         ids=["one_tile", "narrow", "wide", "router_eight_tokens", "router_four_experts",
                              "static_takes_other_xcds"])
def test_rest_state_and_task_counts(B, E, d, f, sched):
    # the last case has more than two GroupGEMM positions per workgroup (static: workgroups
    # take other XCDs' positions, combine tasks from one counter); every task runs once
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, f, E, 2, seed=12)
    tx, tWr, tb, t1, t3, t2 = dev_inputs(x, Wr, bias, W1, W3, W2)
    layer = mk.MoELayer(E, 2, d, f, tWr, t1, t3, t2, sched=sched, max_batch=B)
    before = ctl_words(layer, B).copy()
    for _ in range(3):
        layer(tx)
    torch.cuda.synchronize()
    assert layer.error() == 0
    c = ctl_words(layer, B)
    C = mk.CTL
    assert c[C["epoch"]] == before[C["epoch"]] + 3    # epoch advanced once per forward
    assert c[C["exit"]] == 0                           # exit counter at rest
    assert c[C["qhead"]] == c[C["qtail"]] == 0        # queue at rest
    assert c[C["pf"]] == 0                             # weight-prefetch claims at rest
    assert all(c[C["xq"] + 32 * x] == 0 for x in range(8))  # static per-XCD claim counters at rest
    assert c[C["cq"]] == 0                             # static combine claim counter at rest
    assert c[C["ev_topk"]] == 0 and c[C["ev_scan"]] == 1 and c[C["ev_y"]] == 0  # events at rest
    hist = routing_numpy(layer, B)["hist"]
    exp = expected_task_counts(hist, B, E, d, f, 2)
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
def test_nonfinite_input_is_reported(sched):
    # a NaN and an infinity in x make router logits non-finite: the forward ends with
    # MOE_MK_ERR_NONFINITE in the error word, and after re-initialising the workspace a
    # clean input runs exactly as usual
    B = 90
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, 256, 256, 8, 2, seed=23)
    bad = x.copy()
    bad[5, 17] = 0x7FC0   # bf16 quiet NaN
    bad[70, 3] = 0x7F80   # bf16 +infinity
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

def _full_config(name, sched, sample):
    return _full_config_of(CONFIGS[name], sched, sample)


def _full_config_of(cfg, sched, sample):
    name = cfg.name
    log(f"config {name} sched={SNAME[sched]}: generating inputs")
    tWr, tb, t1, t3, t2 = device_weights(cfg)
    Wr, bias = make_wr(cfg), make_bias(cfg)
    results = []
    layer = mk.MoELayer(cfg.E, cfg.k, cfg.d, cfg.f, tWr, t1, t3, t2, router_bias=tb, sched=sched,
                        max_batch=max(cfg.batches))
    x_all = make_x(cfg)
    tx_all = to_torch_bf16(x_all).cuda()
    for B in cfg.batches:
        x = x_all[:B]
        out = layer(tx_all[:B])
        torch.cuda.synchronize()
        assert layer.error() == 0
        got = routing_numpy(layer, B)
        ref = oracle.routing(x, Wr, bias, cfg.k)
        check_routing(got, ref, B, cfg.E)
        toks = sorted(set(np.linspace(0, B - 1, min(B, sample)).astype(int).tolist()))
        ref_out = oracle.moe_tokens(x, toks, ref["topk_idx"], ref["topk_w"], lambda e: expert_weights(cfg, e),
                                    cfg.d, cfg.f)
        check_out(out.float().cpu().numpy()[toks], ref_out, f"{name} B={B} ({len(toks)} tokens)")
        results.append((B, out.clone()))
        log(f"  B={B}: routing exact, output within tolerance")
    layer.close()
    return results, (tWr, tb, t1, t3, t2, tx_all)


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
        log(f"threshold batch B={B} tiles={'wide' if tile_config(B, k, E, d, f)[0] == 256 else 'narrow'} "
            f"sched={SNAME[sched]}")
        out = layer(tx[:B])
        torch.cuda.synchronize()
        assert layer.error() == 0
        ref = oracle.forward(x[:B], Wr, bias, W1, W3, W2, k)
        check_routing(routing_numpy(layer, B), ref, B, E)
        check_out(out.float().cpu().numpy(), ref["out"], f"threshold B={B}")
    layer.close()


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_config_mixtral_decode(sched):
    _full_config("mixtral_decode", sched, sample=8)


def test_config_sweep_one_plan_no_recompile():
    cfg = CONFIGS["sweep"]
    results, (tWr, tb, t1, t3, t2, tx_all) = _full_config("sweep", mk.MOE_MK_SCHED_STATIC, sample=12)
    # the same batches run on fresh workspaces in isolation give bitwise the same output,
    # and the leading tokens of a larger batch equal a smaller batch (batch-prefix invariance)
    full = dict(results)
    for B in (3, 57):
        layer = mk.MoELayer(cfg.E, cfg.k, cfg.d, cfg.f, tWr, t1, t3, t2, max_batch=B)
        out = layer(tx_all[:B])
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), full[B].view(torch.int16))
        assert torch.equal(full[512][:B].view(torch.int16), out.view(torch.int16))
        layer.close()


def test_config_sweep_dynamic():
    _full_config("sweep", mk.MOE_MK_SCHED_DYNAMIC, sample=6)


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_config_deepseek_zipf(sched):
    _full_config("deepseek_zipf", sched, sample=4)


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_config_prefill(sched):
    _full_config("prefill", sched, sample=8)


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_large_batch_prefill_shape(sched):
    # four times the prefill batch (131072 routed rows): queue capacity, the per-XCD lists,
    # eight-token router tasks and wide tiles at a size well past the benchmark's
    cfg = Config("prefill_x4", d=2048, f=768, E=128, k=8, batches=(16384,), seed=606)
    _full_config_of(cfg, sched, sample=6)


def test_max_experts_and_top_k_wide():
    # the largest E and k the plan accepts, at a batch whose 128 rows per expert take wide tiles
    cfg, x, Wr, bias, W1, W3, W2 = small_case(2048, 256, 128, 256, 16, seed=707)
    for sched in SCHEDS:
        full_check(x, Wr, bias, W1, W3, W2, 16, sched, f"E=256 k=16 B=2048 {SNAME[sched]}")
