"""Seeded synthetic inputs for the MoE layer, shared by the tests, the benchmark and the oracle checks.

This module holds no arithmetic of the layer itself: it only draws the inputs (token
activations, router weights, router bias and expert weights) with fixed seeds, so the
GPU path and the CPU oracle see the same values.

Draws use numpy's PCG64 seeded with ``SeedSequence([config_seed, tensor_id, expert])``,
so any single expert can be regenerated on its own.  Distributions:

* x: N(0, 1) in fp32, rounded to bf16 (round to nearest even);
* Wr: N(0, 1/d) (standard deviation 1/sqrt(d)), fp32, layout [d, E];
* W1, W3: standard deviation 1/sqrt(d), bf16, layout [E, d, f];
* W2: standard deviation 1/sqrt(f), bf16, layout [E, f, d];
* router bias (skewed configuration only): bias[e] = -s * ln(1 + pi(e)) with pi a seeded
  permutation of the experts, i.e. the log of Zipf(s) weights by rank.

bf16 arrays are numpy.uint16 bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

T_X, T_WR, T_W1, T_W3, T_W2, T_BIAS = 0, 1, 2, 3, 4, 5


@dataclass(frozen=True)
class Config:
    name: str
    d: int
    f: int
    E: int
    k: int
    batches: tuple
    seed: int
    zipf_s: float | None = None
    x_rows: int = 0            # rows drawn for x; every batch uses the leading rows
    note: str = field(default="", compare=False)

    @property
    def B(self) -> int:
        return self.batches[0]

    @property
    def rows(self) -> int:
        return self.x_rows or max(self.batches)


CONFIGS = {
    "tiny": Config("tiny", d=256, f=512, E=8, k=2, batches=(16,), seed=101,
                   note="tiny MoE layer, B=16 d=256 f=512 E=8 k=2"),
    "mixtral_decode": Config("mixtral_decode", d=4096, f=14336, E=8, k=2, batches=(32,), seed=202,
                             note="Mixtral-shaped decode, B=32 d=4096 f=14336 E=8 k=2"),
    "sweep": Config("sweep", d=2048, f=1408, E=64, k=6, batches=(1, 3, 16, 57, 128, 512), seed=303,
                    x_rows=512, note="dynamic-shape sweep, d=2048 f=1408 E=64 k=6"),
    "deepseek_zipf": Config("deepseek_zipf", d=7168, f=2048, E=256, k=8, batches=(128,), seed=404,
                            zipf_s=1.2, note="DeepSeek-V3-shaped skewed routing, B=128 d=7168 f=2048 E=256 k=8"),
    "prefill": Config("prefill", d=2048, f=768, E=128, k=8, batches=(4096,), seed=505,
                      note="prefill-sized, B=4096 d=2048 f=768 E=128 k=8"),
}


def _rng(*key) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(v) for v in key])))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + (((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(shape, std: float, *key) -> np.ndarray:
    g = _rng(*key).standard_normal(int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        g *= np.float32(std)
    return to_bf16_bits(g).reshape(shape)


def make_x(cfg: Config, rows: int | None = None) -> np.ndarray:
    rows = cfg.rows if rows is None else rows
    full = normal_bf16((cfg.rows, cfg.d), 1.0, cfg.seed, T_X, 0)
    return np.ascontiguousarray(full[:rows])


def make_wr(cfg: Config) -> np.ndarray:
    g = _rng(cfg.seed, T_WR, 0).standard_normal(cfg.d * cfg.E, dtype=np.float32)
    return (g * np.float32(1.0 / np.sqrt(cfg.d))).reshape(cfg.d, cfg.E)


def make_bias(cfg: Config) -> np.ndarray | None:
    if cfg.zipf_s is None:
        return None
    pi = _rng(cfg.seed, T_BIAS, 0).permutation(cfg.E)
    return (-cfg.zipf_s * np.log1p(pi.astype(np.float64))).astype(np.float32)


def expert_weights(cfg: Config, e: int):
    """(W1[e] [d,f], W3[e] [d,f], W2[e] [f,d]) as bf16 bit patterns."""
    sd, sf = 1.0 / np.sqrt(cfg.d), 1.0 / np.sqrt(cfg.f)
    return (normal_bf16((cfg.d, cfg.f), sd, cfg.seed, T_W1, e),
            normal_bf16((cfg.d, cfg.f), sd, cfg.seed, T_W3, e),
            normal_bf16((cfg.f, cfg.d), sf, cfg.seed, T_W2, e))


def _threads() -> int:
    env = os.environ.get("MOE_INPUT_THREADS")
    if env:
        return max(1, int(env))
    return max(1, min(16, os.cpu_count() or 1))


def for_each_expert(cfg: Config, fn, experts=None) -> None:
    """Call ``fn(e, W1e, W3e, W2e)`` for every expert, generating them on a thread pool.

    ``fn`` is called from the caller's thread in expert order, so it may copy to a device.
    """
    experts = list(range(cfg.E)) if experts is None else list(experts)
    nthreads = _threads()
    with ThreadPoolExecutor(nthreads) as ex:
        window = []
        it = iter(experts)
        for e in it:
            window.append((e, ex.submit(expert_weights, cfg, e)))
            if len(window) >= 2 * nthreads:
                e0, fut = window.pop(0)
                fn(e0, *fut.result())
        for e0, fut in window:
            fn(e0, *fut.result())


def all_expert_weights(cfg: Config):
    """Full host arrays W1 [E,d,f], W3 [E,d,f], W2 [E,f,d] (bf16 bits); only for modest sizes."""
    W1 = np.empty((cfg.E, cfg.d, cfg.f), dtype=np.uint16)
    W3 = np.empty_like(W1)
    W2 = np.empty((cfg.E, cfg.f, cfg.d), dtype=np.uint16)

    def put(e, a, b, c):
        W1[e], W3[e], W2[e] = a, b, c

    for_each_expert(cfg, put)
    return W1, W3, W2


def small_case(B: int, d: int, f: int, E: int, k: int, seed: int, zipf_s: float | None = None,
               x_std: float = 1.0):
    """A complete small input set drawn with the same recipe (for parity tests at small sizes)."""
    cfg = Config(f"small_{seed}", d=d, f=f, E=E, k=k, batches=(B,), seed=seed, zipf_s=zipf_s)
    x = normal_bf16((B, d), x_std, seed, T_X, 0)
    Wr = make_wr(cfg)
    bias = make_bias(cfg)
    W1, W3, W2 = all_expert_weights(cfg)
    return cfg, x, Wr, bias, W1, W3, W2


# ----------------------------------------------------------------------------- device copies (torch)

def to_torch_bf16(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)


def device_weights(cfg: Config, device="cuda", keep=None):
    """Wr, bias and the expert weights of ``cfg`` as device tensors (generated expert by expert).

    With ``keep`` (a set of expert indices) the host arrays of those experts are also
    returned, as a sixth item ``{e: (W1e, W3e, W2e)}``, so the same draws can serve a
    host-side computation without being generated twice.
    """
    import torch
    Wr = torch.from_numpy(make_wr(cfg)).to(device)
    b = make_bias(cfg)
    bias = None if b is None else torch.from_numpy(b).to(device)
    W1 = torch.empty((cfg.E, cfg.d, cfg.f), dtype=torch.bfloat16, device=device)
    W3 = torch.empty_like(W1)
    W2 = torch.empty((cfg.E, cfg.f, cfg.d), dtype=torch.bfloat16, device=device)
    kept = {}

    def put(e, a1, a3, a2):
        W1[e].copy_(to_torch_bf16(a1))
        W3[e].copy_(to_torch_bf16(a3))
        W2[e].copy_(to_torch_bf16(a2))
        if keep is not None and e in keep:
            kept[e] = (a1, a3, a2)

    for_each_expert(cfg, put)
    if keep is not None:
        return Wr, bias, W1, W3, W2, kept
    return Wr, bias, W1, W3, W2


def device_x(cfg: Config, rows: int | None = None, device="cuda"):
    return to_torch_bf16(make_x(cfg, rows)).to(device)
