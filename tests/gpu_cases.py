"""Helpers shared by the GPU parity tests: run the HIP layer through the C ABI and compare
with the CPU oracle on the same seeded inputs."""
import sys

import numpy as np
import torch

import moe_groupgemm_amd as mk
import oracle
from moe_inputs import to_torch_bf16

TOL = 2e-2  # max |out - ref| <= TOL * max |ref|, bf16 operands with fp32 accumulation


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_inputs(x, Wr, bias, W1, W3, W2, device="cuda"):
    t = lambda a: to_torch_bf16(a).to(device)
    return (t(x), torch.from_numpy(np.ascontiguousarray(Wr)).to(device),
            None if bias is None else torch.from_numpy(np.ascontiguousarray(bias)).to(device),
            t(W1), t(W3), t(W2))


def routing_numpy(layer, B):
    r = layer.routing(B)
    return {k: v.cpu().numpy() for k, v in r.items()}


def check_routing(got, ref, B, E):
    assert np.array_equal(got["logits"].view(np.uint32), ref["logits"].view(np.uint32)), "logits differ bitwise"
    assert np.array_equal(got["topk_idx"], ref["topk_idx"]), "top-k indices differ"
    assert np.array_equal(got["hist"], ref["hist"]), "histogram differs"
    assert np.array_equal(got["exp_indptr"], ref["exp_indptr"]), "exp_indptr differs"
    assert np.array_equal(got["perm"], ref["perm"]), "permutation differs"
    assert np.array_equal(got["inv"], ref["inv"]), "inverse permutation differs"
    assert np.max(np.abs(got["topk_w"].astype(np.float64) - ref["topk_w"]), initial=0.0) <= 1e-6


def check_out(got, ref_out, what=""):
    got = np.asarray(got, dtype=np.float64)
    scale = np.abs(ref_out).max()
    err = np.abs(got - ref_out).max() if ref_out.size else 0.0
    log(f"  {what} max|err| = {err:.3e}, max|ref| = {scale:.3e}, ratio = {err / max(scale, 1e-300):.2e}")
    assert err <= TOL * scale, f"{what}: max|err| {err:.3e} > {TOL} * {scale:.3e}"


def ctl_words(layer, B):
    return layer.routing(B)["ctl"].cpu().numpy()


def expected_task_counts(plan, hist, B):
    """Tasks of each kind one forward runs, from the library's own per-batch choices
    (moe_mk_forward_info) and the routing histogram."""
    info = lambda key: mk.moe_mk_forward_info(plan, B, key)
    BM, NB1, NB2, S = info("BM"), info("NB1"), info("NB2"), info("S")
    mt = int(sum((int(h) + BM - 1) // BM for h in hist))
    return {"route": info("route_tasks"), "topk": info("T"), "scan": 1, "group": info("T"),
            "gemm1": mt * NB1, "gemm2": mt * S * NB2, "combine": info("combine_tasks")}
