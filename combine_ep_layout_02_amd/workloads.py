"""Seeded synthetic workloads for MoE dispatch / combine.

This module only draws inputs: token activations ``x``, router outputs
(``topk_idx``, ``topk_weights``) and expert outputs ``y``.  It contains none of
the layout, dispatch or combine arithmetic, so the CPU oracle and the HIP
library can both be fed from it without sharing any of the method's code.

Workload shapes follow the pages' own benchmark setting (8K tokens per batch,
hidden 7168, top-8 experts, FP8 dispatch and BF16 combine: GeekNews "DeepSeek
publica DeepEP ...", section "Resultados de medición de rendimiento") and the
group-limited gating the kernels are said to be aligned with (downcodes.com
DeepEP launch news, third paragraph).  Nothing here is read from a dataset:
activations, router logits and expert outputs are normal draws of the stated
shapes, and router decisions are computed from those logits on the host.

Random streams: ``numpy.random.default_rng([seed, stream])`` (PCG64) with
stream 0 = x, 1 = router logits, 2 = y, 3 = the Zipf popularity permutation.
Normals are drawn as float32 and rounded to BF16 with round-to-nearest-even
(torch's CPU cast).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

import numpy as np
import torch

STREAM_X, STREAM_LOGITS, STREAM_Y, STREAM_PERM = 0, 1, 2, 3
_CHUNK_ELEMS = 1 << 25  # draw big tensors in 32M-element pieces to bound host memory


@dataclass(frozen=True)
class Workload:
    """One synthetic configuration.

    ``routing`` is one of ``"softmax_pair"`` (top-2 by logit, softmax over the
    pair), ``"softmax_renorm"`` (softmax over all experts, top-k, renormalise)
    and ``"group_limited"`` (sigmoid scores, group-limited top-k, normalised
    weights).  ``zipf_alpha`` > 0 adds a Zipf(``zipf_s``) per-expert popularity
    bias to the logits before the sigmoid.
    """

    name: str
    num_tokens: int
    hidden: int
    num_experts: int
    num_ranks: int
    num_topk: int
    routing: str
    dispatch_dtypes: Tuple[str, ...]
    seed: int
    capacity: int = 0
    expert_alignment: int = 1
    num_groups: int = 1
    topk_groups: int = 1
    zipf_s: float = 0.0
    zipf_alpha: float = 0.0
    note: str = ""

    @property
    def recv_rows(self) -> int:
        """Worst-case receive rows: T*k + E*(A-1) (flat) or E*C (padded)."""
        if self.capacity > 0:
            return self.num_experts * self.capacity
        return self.num_tokens * self.num_topk + self.num_experts * (self.expert_alignment - 1)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in (
        Workload("tiny", 128, 256, 8, 2, 2, "softmax_pair", ("bf16", "fp8"), seed=1,
                 note="T=128, H=256, E=8 in 2 ranks, top-2, BF16 and FP8 dispatch"),
        Workload("mid", 4096, 4096, 64, 8, 6, "softmax_renorm", ("bf16",), seed=2,
                 note="T=4096, H=4096, E=64 in 8 ranks, top-6, BF16 dispatch"),
        Workload("v3", 8192, 7168, 256, 8, 8, "group_limited", ("fp8",), seed=3,
                 num_groups=8, topk_groups=4,
                 note="8K tokens, hidden 7168, 256 experts top-8 group-limited, FP8 dispatch"),
        Workload("decode", 128, 7168, 256, 8, 8, "group_limited", ("fp8",), seed=4,
                 capacity=128, num_groups=8, topk_groups=4,
                 note="128 decode tokens into a padded [256, 128, 7168] per-expert layout"),
        Workload("skew", 16384, 7168, 256, 8, 8, "group_limited", ("fp8",), seed=5,
                 num_groups=8, topk_groups=4, zipf_s=1.2, zipf_alpha=0.2,
                 note="16K tokens with a Zipf(1.2) expert popularity bias"),
    )
}


def rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to BF16 (nearest-even, torch CPU cast); return uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of BF16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(seed: int, stream: int, rows: int, cols: int) -> np.ndarray:
    """[rows, cols] BF16 bit patterns of N(0,1) float32 draws, drawn in row chunks."""
    g = rng(seed, stream)
    out = np.empty((rows, cols), dtype=np.uint16)
    step = max(1, _CHUNK_ELEMS // max(cols, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        out[r0:r1] = f32_to_bf16_bits(g.standard_normal((r1 - r0, cols), dtype=np.float32))
    return out


def _stable_topk(score: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest entries per row, larger first, ties to lower index."""
    return np.argsort(-score, axis=1, kind="stable")[:, :k]


def _softmax(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z, dtype=np.float32)
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def _sigmoid(z: np.ndarray) -> np.ndarray:
    return (np.float32(1.0) / (np.float32(1.0) + np.exp(-z, dtype=np.float32))).astype(np.float32)


def zipf_bias(w: Workload) -> np.ndarray:
    """Per-expert logit bias alpha * ln p_pi(e) with p_r proportional to r^-s."""
    E = w.num_experts
    p = np.arange(1, E + 1, dtype=np.float64) ** (-w.zipf_s)
    p /= p.sum()
    perm = rng(w.seed, STREAM_PERM).permutation(E)
    return (w.zipf_alpha * np.log(p[perm])).astype(np.float32)


def route(w: Workload, logits: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Router decisions from logits: (topk_idx int32 [T,k], topk_weights fp32 [T,k])."""
    k = w.num_topk
    if w.routing == "softmax_pair":
        idx = _stable_topk(logits, k)
        wts = _softmax(np.take_along_axis(logits, idx, axis=1))
    elif w.routing == "softmax_renorm":
        p = _softmax(logits)
        idx = _stable_topk(p, k)
        sel = np.take_along_axis(p, idx, axis=1)
        wts = sel / sel.sum(axis=1, keepdims=True)
    elif w.routing == "group_limited":
        z = logits
        if w.zipf_alpha > 0:
            z = z + zipf_bias(w)[None, :]
        s = _sigmoid(z.astype(np.float32))
        T, E = s.shape
        G = w.num_groups
        gs = s.reshape(T, G, E // G)
        top2 = -np.sort(-gs, axis=2)[:, :, :2]
        gscore = top2.sum(axis=2)
        gsel = _stable_topk(gscore, w.topk_groups)
        keep = np.zeros((T, G), dtype=bool)
        np.put_along_axis(keep, gsel, True, axis=1)
        masked = np.where(np.repeat(keep, E // G, axis=1), s, -np.inf).astype(np.float32)
        idx = _stable_topk(masked, k)
        sel = np.take_along_axis(s, idx, axis=1)
        wts = sel / sel.sum(axis=1, keepdims=True)
    else:
        raise ValueError(f"unknown routing {w.routing!r}")
    return idx.astype(np.int32), wts.astype(np.float32)


@dataclass
class Inputs:
    workload: Workload
    x: np.ndarray             # uint16 BF16 bits [T, H]
    topk_idx: np.ndarray      # int32 [T, k]
    topk_weights: np.ndarray  # float32 [T, k]
    y: Optional[np.ndarray] = field(default=None)  # uint16 BF16 bits [recv_rows, H]


def make_routing(w: Workload) -> Tuple[np.ndarray, np.ndarray]:
    logits = rng(w.seed, STREAM_LOGITS).standard_normal((w.num_tokens, w.num_experts), dtype=np.float32)
    return route(w, logits)


def make_inputs(w: Workload, with_y: bool = True) -> Inputs:
    x = normal_bf16(w.seed, STREAM_X, w.num_tokens, w.hidden)
    idx, wts = make_routing(w)
    y = normal_bf16(w.seed, STREAM_Y, w.recv_rows, w.hidden) if with_y else None
    return Inputs(w, x, idx, wts, y)


def custom(name: str, T: int, H: int, E: int, R: int, k: int, seed: int, *,
           capacity: int = 0, expert_alignment: int = 1, routing: str = "softmax_renorm",
           dispatch_dtypes: Tuple[str, ...] = ("bf16", "fp8")) -> Workload:
    """A small ad-hoc workload for edge cases (same generators, other sizes)."""
    return Workload(name, T, H, E, R, k, routing, dispatch_dtypes, seed,
                    capacity=capacity, expert_alignment=expert_alignment)
