"""GPU test of the allocation-free entry point moe_mk_forward_noalloc (static per-GPU
scratch instead of a caller workspace), through the C ABI: its output equals
moe_mk_forward's on a caller workspace, bit for bit, on two calls in a row (the second
with a smaller batch), in both schedules, across plans sharing the scratch, and after a
forward that reported a device error."""
import numpy as np
import pytest
import torch

import moe_groupgemm_amd as mk
import oracle
from gpu_cases import check_out, dev_inputs, log
from moe_inputs import small_case, to_torch_bf16

pytestmark = pytest.mark.gpu

SCHEDS = [mk.MOE_MK_SCHED_STATIC, mk.MOE_MK_SCHED_DYNAMIC]


def _layer(B, d, f, E, k, sched, seed):
    cfg, x, Wr, bias, W1, W3, W2 = small_case(B, d, f, E, k, seed=seed)
    tx, tWr, tb, t1, t3, t2 = dev_inputs(x, Wr, bias, W1, W3, W2)
    layer = mk.MoELayer(E, k, d, f, tWr, t1, t3, t2, router_bias=tb, sched=sched, max_batch=B)
    return layer, tx, (x, Wr, bias, W1, W3, W2)


def _noalloc(layer, tx, B):
    out = torch.empty((B, layer.d), dtype=torch.bfloat16, device="cuda")
    err = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    mk.moe_mk_forward_noalloc(layer.plan, tx[:B], layer.Wr, layer.bias, layer.W1, layer.W3, layer.W2, out, B, err)
    return out, err


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
@pytest.mark.parametrize("B1,B2,d,f,E,k", [(40, 13, 256, 512, 8, 2), (300, 90, 256, 384, 4, 2),
                                            (203, 64, 256, 384, 16, 4)],
                         ids=["one_tile", "wide_then_narrow", "ragged_multi_tile"])
def test_noalloc_equals_workspace_forward(B1, B2, d, f, E, k, sched):
    layer, tx, host = _layer(B1, d, f, E, k, sched, seed=3100 + B1)
    for B in (B1, B2):  # two calls in a row, the second smaller
        log(f"no-alloc forward B={B} d={d} f={f} E={E} k={k} sched={sched}")
        out_na, err = _noalloc(layer, tx, B)
        out_ws = layer(tx[:B])
        torch.cuda.synchronize()
        assert int(err.item()) == 0
        assert layer.error() == 0
        assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16)), f"B={B}: outputs differ"
        x, Wr, bias, W1, W3, W2 = host
        ref = oracle.forward(x[:B], Wr, bias, W1, W3, W2, k)
        check_out(out_na.float().cpu().numpy(), ref["out"], f"no-alloc B={B}")
    layer.close()


def test_noalloc_plans_share_the_scratch():
    # two plans of different shapes alternate on the one scratch: each switch prepares it
    # again, and every output equals the workspace forward's
    a = _layer(70, 256, 384, 8, 2, mk.MOE_MK_SCHED_STATIC, seed=3201)
    b = _layer(33, 128, 256, 16, 4, mk.MOE_MK_SCHED_DYNAMIC, seed=3202)
    for rep in range(2):
        for layer, tx, _ in (a, b):
            B = tx.shape[0] - rep
            out_na, err = _noalloc(layer, tx, B)
            out_ws = layer(tx[:B])
            torch.cuda.synchronize()
            assert int(err.item()) == 0
            assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16))
    a[0].close()
    b[0].close()


def test_noalloc_batch_beyond_the_scratch_is_rejected():
    # Mixtral-shaped plan: the 64 MiB scratch holds a few hundred tokens, not 4096
    E, k, d, f = 8, 2, 4096, 14336
    plan = mk.moe_mk_plan(E, k, d, f, mk.MOE_MK_SCHED_DYNAMIC)
    B = 4096
    assert mk.moe_mk_workspace_bytes(plan, B) > 64 << 20
    x = torch.zeros((B, d), dtype=torch.bfloat16, device="cuda")
    Wr = torch.zeros((d, E), dtype=torch.float32, device="cuda")
    W = torch.zeros((E, d, f), dtype=torch.bfloat16, device="cuda")
    W2 = torch.zeros((E, f, d), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((B, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mk.MoeMkError) as ei:
        mk.moe_mk_forward_noalloc(plan, x, Wr, None, W, W, W2, out, B)
    assert ei.value.code == -3  # MOE_MK_EWORKSPACE
    mk.moe_mk_plan_destroy(plan)


@pytest.mark.parametrize("sched", SCHEDS, ids=["static", "dynamic"])
def test_noalloc_recovers_after_a_device_error(sched):
    # a NaN in x makes a router logit non-finite: the forward reports MOE_MK_ERR_NONFINITE
    # through err, puts the scratch back to rest itself, and the next call is clean
    B = 90
    layer, tx, host = _layer(B, 256, 256, 8, 2, sched, seed=3300)
    x = host[0]
    bad = x.copy()
    bad[5, 17] = 0x7FC0  # bf16 quiet NaN
    tbad = to_torch_bf16(bad).cuda()
    _, err = _noalloc(layer, tbad, B)
    torch.cuda.synchronize()
    assert int(err.item()) & mk.MOE_MK_ERR_NONFINITE
    out_na, err = _noalloc(layer, tx, B)
    out_ws = layer(tx)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16))
    layer.close()
