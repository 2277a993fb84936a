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


WAVES = 8           # waves per workgroup
NARROW_BN = 128     # narrow GroupGEMM tile columns
COMBINE_COLS = 2048


def down_splits(B, k, f):
    """K splits of the down projection the library uses at this batch size (narrow tiles)."""
    a, nb1 = B * k, f // NARROW_BN
    if a <= 1024 and f >= 8192 and nb1 % 4 == 0:
        return 4
    if a <= 1024 and f >= 4096 and nb1 % 2 == 0:
        return 2
    return 1


def tile_config(B, k, E, d, f, wide_bn1=128, wide_bn2=256, wide_bm=256):
    """(rows per tile, gate/up tiles per row tile, down tiles per row tile and split, splits):
    wide tiles once an expert averages 128 rows (d, f multiples of the wide widths), else
    64-row narrow tiles."""
    if B * k >= 128 * E and d % wide_bn2 == 0 and f % wide_bn1 == 0:
        return wide_bm, f // wide_bn1, d // wide_bn2, 1
    return 64, f // NARROW_BN, d // NARROW_BN, down_splits(B, k, f)


def expected_task_counts(hist, B, E, d, f, k):
    BM, NB1, NB2, S = tile_config(B, k, E, d, f)
    mt = int(sum((int(h) + BM - 1) // BM for h in hist))
    # router tokens per wave, and experts per router task
    tpw = 1 if B <= 512 else 8 if E % 4 == 0 and d % 128 == 0 and -(-B // 64) * -(-E // 16) >= 512 else 4
    reb = 4 if tpw == 1 and E % 4 == 0 and d % 512 == 0 and -(-B // WAVES) * -(-E // 16) < 64 else 16
    return {"route": -(-B // (WAVES * tpw)) * -(-E // reb), "topk": -(-B // 64), "scan": 1, "group": -(-B // 64),
            "gemm1": mt * NB1, "gemm2": mt * S * NB2, "combine": -(-B // (8 if B >= 1024 and k <= 8 else 1 if B <= 64 else 4)) * -(-d // COMBINE_COLS)}
