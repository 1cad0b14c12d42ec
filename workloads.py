"""Seeded synthetic workloads for ring-attention forward.

This module is shared by the tests, the benchmark and the smoke check. It
holds shapes, seeds and the random-number recipe only: no attention
arithmetic, no sequence layouts and no positions. Both the CPU oracle and the
HIP path receive the tensors it makes, and neither imports the other.

Input recipe (the pages fix no data, so inputs are synthetic): a
``torch.Generator`` on the CPU seeded with the workload's seed draws float32
standard normals for q [B,Hq,S,D], then k [B,Hkv,S,D], then v [B,Hkv,S,D], one
``randn`` call each. k is multiplied by ``k_scale`` (a power of two, so the
scaling commutes with rounding), then all three are rounded to the workload's
dtype (round-to-nearest-even for bfloat16). The shapes follow the long-context
GQA setting the pages discuss: 128k to 1M tokens with 8 KV heads or fewer.
"""
from __future__ import annotations

import dataclasses

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    S: int
    dtype: str          # "bf16" or "f32"
    seed: int
    causal: bool
    N: int              # virtual ring size
    layout: str         # "contiguous", "zigzag", "striped", "ulysses" or "usp"
    k_scale: float = 1.0
    note: str = ""
    P_u: int = 1                # "usp": devices per node (Ulysses degree); N / P_u nodes
    ring_layout: str = "zigzag"  # "usp": the ring's layout over the nodes

    @property
    def torch_dtype(self) -> torch.dtype:
        return {"bf16": torch.bfloat16, "f32": torch.float32}[self.dtype]

    @property
    def C(self) -> int:
        """Tokens held by one virtual rank."""
        return self.S // self.N


# The five benchmark configurations, in order. The first is the small case the
# oracle finishes in seconds; the fourth is the headline workload.
WORKLOADS = (
    Workload("tiny_f32_causal_contig_s512", B=1, Hq=2, Hkv=2, D=64, S=512,
             dtype="f32", seed=0, causal=True, N=4, layout="contiguous",
             note="4-step ring of 128-token KV blocks"),
    Workload("noncausal_mha_s8k", B=1, Hq=8, Hkv=8, D=128, S=8192,
             dtype="bf16", seed=1, causal=False, N=4, layout="contiguous",
             note="every rank's queries against all 4 KV blocks"),
    Workload("causal_zigzag_mha_s32k", B=1, Hq=32, Hkv=32, D=128, S=32768,
             dtype="bf16", seed=2, causal=True, N=8, layout="zigzag",
             note="16 chunks of 2048"),
    Workload("gqa_causal_zigzag_s128k", B=1, Hq=64, Hkv=8, D=128, S=131072,
             dtype="bf16", seed=3, causal=True, N=8, layout="zigzag",
             k_scale=0.5, note="16 chunks of 8192, 8 q heads per KV head"),
    Workload("mqa_causal_zigzag_s1m", B=1, Hq=8, Hkv=1, D=128, S=1048576,
             dtype="bf16", seed=4, causal=True, N=16, layout="zigzag",
             note="32 chunks of 32768"),
)

# The same 128k GQA inputs on the striped split (token t on rank t mod N): a
# parity case and a measurement of that layout, not one of the five configs.
STRIPED_128K = Workload("gqa_causal_striped_s128k", B=1, Hq=64, Hkv=8, D=128, S=131072,
                        dtype="bf16", seed=3, causal=True, N=8, layout="striped",
                        k_scale=0.5, note="rank r holds tokens r, r+8, ...")

# The same inputs under DeepSpeed-Ulysses with 8 ranks: each rank starts with
# a contiguous eighth of the sequence for all heads; the all-to-all gives it 8
# query heads and 1 KV head over the whole sequence.
ULYSSES_128K = Workload("gqa_causal_ulysses_s128k", B=1, Hq=64, Hkv=8, D=128, S=131072,
                        dtype="bf16", seed=3, causal=True, N=8, layout="ulysses",
                        k_scale=0.5, note="8 ranks: 8 query heads and 1 KV head each")

# The same inputs on the 2D grid of unified sequence parallelism: 4 nodes of 8
# devices (Ulysses inside a node, the zigzag ring across nodes).
USP_128K = Workload("gqa_causal_usp_s128k", B=1, Hq=64, Hkv=8, D=128, S=131072,
                    dtype="bf16", seed=3, causal=True, N=32, layout="usp", k_scale=0.5,
                    P_u=8, ring_layout="zigzag",
                    note="4 nodes x 8 devices: 8 query heads / 1 KV head per device")

BY_NAME = {w.name: w for w in WORKLOADS + (STRIPED_128K, ULYSSES_128K, USP_128K)}
HEADLINE = WORKLOADS[3]


def make_inputs(w: Workload, device: str | torch.device = "cpu"):
    """Return (q, k, v) for workload ``w`` in its dtype, contiguous, on ``device``.

    The values are always drawn on the CPU so they do not depend on the device.
    """
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    q = torch.randn((w.B, w.Hq, w.S, w.D), generator=g, dtype=torch.float32)
    k = torch.randn((w.B, w.Hkv, w.S, w.D), generator=g, dtype=torch.float32)
    v = torch.randn((w.B, w.Hkv, w.S, w.D), generator=g, dtype=torch.float32)
    if w.k_scale != 1.0:
        k.mul_(w.k_scale)
    dt = w.torch_dtype
    q, k, v = (t.to(dt) for t in (q, k, v))
    if str(device) != "cpu":
        q, k, v = (t.to(device) for t in (q, k, v))
    return q, k, v


def make_random(shape, seed: int, dtype=torch.float32, scale: float = 1.0):
    """One seeded standard-normal tensor (CPU), times ``scale``, cast to dtype."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t.to(dtype)


def sample_rows(S: int, n: int, seed: int, head: int):
    """Seeded choice of ``n`` distinct query rows out of ``S`` for one head."""
    import numpy as np
    rng = np.random.default_rng([seed, head])
    if n >= S:
        return np.arange(S, dtype=np.int64)
    return np.sort(rng.choice(S, size=n, replace=False)).astype(np.int64)
