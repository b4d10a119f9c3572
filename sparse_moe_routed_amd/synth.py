"""Seeded synthetic inputs for the routed MoE layer.

This module only draws random numbers and stores them in the layer's input
dtypes (bf16 activations and expert weights, fp32 router).  It holds none of
the layer's arithmetic: no routing, no quantisation, no GEMM.  Both the CPU
oracle (tests) and the GPU path (bench, tests) take their inputs from here.

Shapes follow the Nemotron 3.5 Transcribe checkpoint facts (bloomery issue
#967, section 2 "Checkpoint facts"): width 2688, 128 experts, top-6 routing,
ungated ReLU^2 experts of width 1856.

Recipe (all PCG64 `numpy.random.default_rng`):
  router W_r      rng(1000+l).normal(0, 0.02, (E, H)) as fp32
  router bias     perm = rng(2000+l).permutation(E); b_e = -0.5*ln(perm[e]+1)
                  (b_e = 0.5*log(1/rank_e): skewed expert use, "experts
                  ordered by use" in the cortiq CMF model card, "Files")
  experts         SeedSequence(3000+l).spawn(E); expert e draws
                  W_up  = bf16(std_normal((F, H), f32) / sqrt(H))
                  W_down = bf16(std_normal((H, F), f32) / sqrt(F))
  tokens x        bf16(rng(4000+T).standard_normal((T, H), f32))
  outlier rows    rng(5000+T).choice(T, round(0.1*T), replace=False), x4
                  (exact in bf16: a power-of-two scale)
  shared expert   rng(3500+l): W_up = bf16(std_normal((F_s, H)) / sqrt(H)),
                  W_down = bf16(std_normal((H, F_s)) / sqrt(F_s)), F_s = 3712
                  (assumed: the pages give no shared-expert width)
bf16 conversion is round-to-nearest-even (torch's `.to(torch.bfloat16)`).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np
import torch

HIDDEN = 2688
FFN = 1856
N_EXPERTS = 128
TOP_K = 6
N_MOE_LAYERS = 23
# Width of the shared expert beside the routed ones.  The pages keep shared
# experts on the card but give no width; two routed-expert widths is an
# assumption of this build, not a fact from them.
SHARED_FFN = 2 * FFN


@dataclass(frozen=True)
class Dims:
    hidden: int = HIDDEN
    ffn: int = FFN
    n_experts: int = N_EXPERTS
    top_k: int = TOP_K


def _to_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(torch.bfloat16)


def make_router(layer: int = 0, dims: Dims = Dims()):
    """Router weight fp32 [E, H] and bias fp32 [E] (torch CPU tensors)."""
    w = np.random.default_rng(1000 + layer).normal(0.0, 0.02, (dims.n_experts, dims.hidden)).astype(np.float32)
    perm = np.random.default_rng(2000 + layer).permutation(dims.n_experts)
    b = (-0.5 * np.log(perm.astype(np.float64) + 1.0)).astype(np.float32)
    return torch.from_numpy(w), torch.from_numpy(b)


def _expert_pair(ss: np.random.SeedSequence, dims: Dims):
    rng = np.random.default_rng(ss)
    up = rng.standard_normal((dims.ffn, dims.hidden), dtype=np.float32)
    up /= np.float32(math.sqrt(dims.hidden))
    down = rng.standard_normal((dims.hidden, dims.ffn), dtype=np.float32)
    down /= np.float32(math.sqrt(dims.ffn))
    return _to_bf16(up), _to_bf16(down)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_experts(layer: int = 0, dims: Dims = Dims(), experts=None):
    """bf16 expert banks W_up [E, F, H] and W_down [E, H, F] (torch CPU).

    `experts` optionally selects a subset of expert ids; the returned banks
    then hold only those experts, in the order given, each drawn from its own
    stream so any subset equals the matching slice of the full bank.
    """
    seqs = np.random.SeedSequence(3000 + layer).spawn(dims.n_experts)
    ids = list(range(dims.n_experts)) if experts is None else [int(e) for e in experts]
    up = torch.empty((len(ids), dims.ffn, dims.hidden), dtype=torch.bfloat16)
    down = torch.empty((len(ids), dims.hidden, dims.ffn), dtype=torch.bfloat16)

    def fill(j):
        u, d = _expert_pair(seqs[ids[j]], dims)
        up[j].copy_(u)
        down[j].copy_(d)

    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(fill, range(len(ids))))
    return up, down


def make_shared_expert(layer: int = 0, hidden: int = HIDDEN, ffn: int = SHARED_FFN):
    """bf16 shared expert W_up [F_s, H] and W_down [H, F_s] (torch CPU), drawn
    like a routed expert from rng(3500 + layer)."""
    rng = np.random.default_rng(3500 + layer)
    up = rng.standard_normal((ffn, hidden), dtype=np.float32) / np.float32(math.sqrt(hidden))
    down = rng.standard_normal((hidden, ffn), dtype=np.float32) / np.float32(math.sqrt(ffn))
    return _to_bf16(up), _to_bf16(down)


def outlier_rows(T: int) -> np.ndarray:
    n = int(round(0.1 * T))
    return np.sort(np.random.default_rng(5000 + T).choice(T, n, replace=False))


def make_tokens(T: int, dims: Dims = Dims(), outliers: bool = False) -> torch.Tensor:
    """bf16 activations x [T, H]; with `outliers`, 10% of rows are scaled x4."""
    x = np.random.default_rng(4000 + T).standard_normal((T, dims.hidden), dtype=np.float32)
    if outliers and T > 0:
        x[outlier_rows(T)] *= np.float32(4.0)
    return _to_bf16(x)


def make_tokens_device(T: int, dims: Dims = Dims(), seed: int = 6000,
                       device: str = "cuda") -> torch.Tensor:
    """bf16 activations x [T, H] drawn on the device (torch generator seeded
    with `seed`): for batches too large to generate on the host.  Callers that
    need host copies of some rows copy them back."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn((T, dims.hidden), generator=g, device=device, dtype=torch.float32)
    return x.to(torch.bfloat16)


def make_f32(shape, seed: int) -> torch.Tensor:
    """Standard-normal fp32 tensor from rng(seed) (generic test rows)."""
    return torch.from_numpy(np.random.default_rng(seed).standard_normal(shape, dtype=np.float32))


# Workloads: the single-layer decode/prefill shapes and the stacked 4-bit path.
WORKLOADS = {
    "decode_t4_bf16": dict(T=4, fmt="bf16", outliers=False, layers=1),
    "decode_t64_bf16": dict(T=64, fmt="bf16", outliers=False, layers=1),
    "prefill_t4096_bf16": dict(T=4096, fmt="bf16", outliers=True, layers=1),
    "decode_t64_fp8": dict(T=64, fmt="fp8", outliers=False, layers=1),
    "decode_t4_fp8": dict(T=4, fmt="fp8", outliers=False, layers=1),
    "decode_t64_nvfp4": dict(T=64, fmt="nvfp4", outliers=False, layers=1),
    "decode_t4_nvfp4": dict(T=4, fmt="nvfp4", outliers=False, layers=1),
    "prefill_t4096_fp8": dict(T=4096, fmt="fp8", outliers=True, layers=1),
    "prefill_t4096_nvfp4": dict(T=4096, fmt="nvfp4", outliers=False, layers=1),
    "stack23_t4096_nvfp4": dict(T=4096, fmt="nvfp4", outliers=False, layers=N_MOE_LAYERS),
}
