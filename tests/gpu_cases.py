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


def row_tiles(layer, B):
    """The forward's row tiles as the scan task published them: (expert, row0, rows) per row
    tile in expert order, and how many are wide (more than 64 rows)."""
    r = layer.routing(B)
    ctl = r["ctl"].cpu().numpy()
    mt, mw = int(ctl[mk.CTL["mt_total"]]), int(ctl[mk.CTL["mw"]])
    tiles = np.stack([r[key][:mt].cpu().numpy() for key in ("mt_expert", "mt_row0", "mt_rows")], axis=1)
    return tiles, mw


def check_row_tiles(tiles, mw, hist, indptr, wide_min, BM=64, wide_BM=256, all_token=False):
    """The row tiles partition every expert's grouped rows, in expert order and in row order
    within an expert: a wide tile holds more than BM and at most wide_BM rows and goes to an
    expert with at least wide_min rows, a narrow one at most BM; mw counts the wide ones.
    all_token (a forward with the all-token gate/up): row tile e holds exactly expert e's rows,
    none for an expert without tokens."""
    if all_token:
        E = len(hist)
        assert mw == 0 and len(tiles) == E
        assert np.array_equal(tiles[:, 0], np.arange(E))
        assert np.array_equal(tiles[:, 1], indptr[:E]) and np.array_equal(tiles[:, 2], hist)
        assert np.all(hist <= BM)
        return
    assert np.all(tiles[:, 2] >= 1) and np.all(tiles[:, 2] <= wide_BM)
    assert np.count_nonzero(tiles[:, 2] > BM) == mw
    assert np.all(np.diff(tiles[:, 0]) >= 0) and np.all(np.diff(tiles[:, 1]) > 0)
    for e in range(len(hist)):
        mine = tiles[tiles[:, 0] == e]
        assert int(mine[:, 2].sum()) == int(hist[e])
        if len(mine):
            starts = mine[:, 1]
            ends = starts + mine[:, 2]
            assert starts[0] == indptr[e] and np.all(starts[1:] == ends[:-1]) and ends[-1] == indptr[e + 1]
        wide = np.count_nonzero(mine[:, 2] > BM)
        if hist[e] >= wide_min:
            assert wide == hist[e] // wide_BM + (1 if hist[e] % wide_BM > BM else 0), (e, hist[e], wide)
        else:
            assert wide == 0, (e, hist[e])


def expected_task_counts(layer, B):
    """Tasks of each kind one forward runs, from the library's per-batch choices
    (moe_mk_forward_info) and the row tiles the scan task chose."""
    info = lambda key: mk.moe_mk_forward_info(layer.plan, B, key)
    tiles, mw = row_tiles(layer, B)
    mt = len(tiles)
    if info("all_token_gate_up"):
        # gate/up tiles of every expert over all tokens; down-projection tiles only for the
        # experts that received tokens
        gemm1, mt = mt * info("NB1"), int(np.count_nonzero(tiles[:, 2]))
    else:
        gemm1 = mt * info("NB1")
    S = info("S")
    # a down-projection tile of a forward without wide row tiles spans one narrow column block
    # or, with full-width tiles, two (forward_info "down_cols"); they tile d exactly
    dc = info("down_cols")
    assert dc * info("NB2") == layer.d, (dc, info("NB2"), layer.d)
    assert dc == info("BN") or (dc == 2 * info("BN") == 2 * mk.moe_mk_plan_info(layer.plan, "BN1")), (dc, S)
    return {"route": info("route_tasks"), "topk": info("T"), "scan": 1, "group": info("T"),
            "gemm1": gemm1, "gemm2": S * mt * (info("NB2_wide") if mw else info("NB2")),
            "combine": info("combine_tasks")}
