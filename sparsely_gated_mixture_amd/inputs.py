"""Seeded synthetic inputs for the sparsely-gated MoE layer.

This module only draws numbers. It holds none of the layer's arithmetic, so
both the HIP path and the CPU oracle can take their inputs from here without
sharing any of the method.

Workloads (shapes follow the pages' own workloads; none of their datasets is
used or needed, random draws stand in for them):

  switch_toy     T=8 D=4 E=3 k=1 H=8, fp32, Switch top-1, capacity factor 1.0
                 (Switch Transformer explainer, "Implementation": eight tokens,
                 width 4, three experts, FFN width 8)
  noisy_fp32     T=4096 D=512 E=64 k=4 H=1024, fp32, noisy top-k, no capacity
                 (Outrageously Large Neural Networks summary, "Network Bandwidth
                 and Expert Sizing": d=512, h=1024 experts, k=4)
  shrinking_bf16 T=1024 D=512 E=1024 k=4 H=1024, bf16, noisy top-k, no capacity
                 (Sparsely-Gated MoE knowledge-base page, section 1: E=1024, K=4,
                 B=1024 gives about four tokens per expert)
  switch_bf16    T=16384 D=768 E=128 k=1 H=3072, bf16, Switch top-1, capacity
                 factor 1.25, router bias skewed by a Zipf(1.1) pmf
  top2_bf16      T=65536 D=1024 E=256 k=2 H=4096, bf16, noisy top-2, capacity
                 factor 1.0, 10% of the token rows duplicated
  hier_bf16      T=16384 D=512 H=1024, bf16, hierarchical: 16 groups of 64
                 experts (E=1024), k_p=2 groups then k_s=2 experts (k=4), no
                 capacity (Outrageously Large Neural Networks summary,
                 "Hierarchical Mixture-of-Experts", with the first-level
                 branching factor 16 and two choices per level of the paper's
                 1024-expert hierarchical model)
  flat1024_bf16  the same shapes with one flat noisy top-4 gate over the 1024
                 experts (routing-cost comparison)
  batchwise_bf16 T=16384 D=512 E=256 k=2 H=2048, bf16, batchwise (strictly
                 balanced) mask: every expert keeps m = kT/E = 128 tokens
                 (Outrageously Large Neural Networks summary, "Strictly Balanced
                 Gating"; the translation experts' widths s=512, h=2048 of the
                 Mixture-of-Experts lesson, chapter 4)

Recipe. Every tensor comes from its own numpy PCG64 stream keyed by
SeedSequence([seed, tag]) (expert weights: [seed, tag, expert]; token rows in
chunks of 4096: [seed, tag, chunk]), so any part can be regenerated alone and
the draws can run in parallel threads.
  X        ~ N(0, 1)
  Wg, Wnoise ~ N(0, 1/D)            (router weights stay fp32)
  W1[e]    ~ N(0, 1/D)  as [D, H]   (fan-in D)
  W2[e]    ~ N(0, 1/H)  as [H, D]   (fan-in H)
  bias[e]  = (e+1)^-1.1 / sum_j j^-1.1   (switch_bf16 only)
  hierarchical gates: Wpg, Wpn ~ N(0, 1/D) as [D, a]; Wsg[i], Wsn[i] ~ N(0, 1/D)
  as [D, b] from streams [seed, tag, i]
  duplicates: floor(0.1 T) token rows, chosen without replacement, copy the row
  of a source token drawn uniformly from the remaining rows (top2_bf16 only).
bf16 tensors are produced by rounding the fp32 draw to nearest-even and are
returned as their raw uint16 bit patterns.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os

import numpy as np

TAG_X, TAG_WG, TAG_WNOISE, TAG_W1, TAG_W2, TAG_DUP = 1, 2, 3, 4, 5, 6
TAG_WPG, TAG_WPN, TAG_WSG, TAG_WSN = 7, 8, 9, 10
TAG_DY = 11


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    D: int
    E: int
    k: int
    H: int
    act: str              # "f32" or "bf16": X, expert weights and activations
    gating: str           # "noisy", "switch" or "batchwise"
    noise: bool
    capacity_factor: float  # <= 0: no capacity limit
    seed: int
    min_capacity: int = 1
    zipf_bias: float = 0.0  # > 0: router bias = Zipf(s) pmf over experts
    dup_frac: float = 0.0   # fraction of token rows that duplicate another row
    groups: int = 0         # > 0: hierarchical gate over `groups` groups of E/groups experts
    k_primary: int = 0      # hierarchical: groups kept per token (k / k_primary experts each)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "switch_toy": Workload("switch_toy", T=8, D=4, E=3, k=1, H=8, act="f32",
                           gating="switch", noise=False, capacity_factor=1.0, seed=0),
    "noisy_fp32": Workload("noisy_fp32", T=4096, D=512, E=64, k=4, H=1024, act="f32",
                           gating="noisy", noise=True, capacity_factor=0.0, seed=1),
    "shrinking_bf16": Workload("shrinking_bf16", T=1024, D=512, E=1024, k=4, H=1024,
                               act="bf16", gating="noisy", noise=True,
                               capacity_factor=0.0, seed=1),
    "switch_bf16": Workload("switch_bf16", T=16384, D=768, E=128, k=1, H=3072, act="bf16",
                            gating="switch", noise=False, capacity_factor=1.25, seed=4,
                            zipf_bias=1.1),
    "top2_bf16": Workload("top2_bf16", T=65536, D=1024, E=256, k=2, H=4096, act="bf16",
                          gating="noisy", noise=True, capacity_factor=1.0, seed=1,
                          dup_frac=0.1),
}
WORKLOAD_ORDER = ["switch_toy", "noisy_fp32", "shrinking_bf16", "switch_bf16", "top2_bf16"]

HIER_WORKLOADS = {
    "hier_bf16": Workload("hier_bf16", T=16384, D=512, E=1024, k=4, H=1024, act="bf16",
                          gating="noisy", noise=True, capacity_factor=0.0, seed=2,
                          groups=16, k_primary=2),
}
WORKLOADS.update(HIER_WORKLOADS)
WORKLOADS["batchwise_bf16"] = Workload("batchwise_bf16", T=16384, D=512, E=256, k=2, H=2048,
                                       act="bf16", gating="batchwise", noise=False,
                                       capacity_factor=0.0, seed=3)
# the hierarchical layer's shape with one flat gate over all 1024 experts (k = 4), for
# comparing the routing cost of the two gates
WORKLOADS["flat1024_bf16"] = Workload("flat1024_bf16", T=16384, D=512, E=1024, k=4, H=1024,
                                      act="bf16", gating="noisy", noise=True,
                                      capacity_factor=0.0, seed=2)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def as_f32(a: np.ndarray) -> np.ndarray:
    """Values of an input tensor as fp32 (bf16 bit patterns are widened exactly)."""
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a.astype(np.float32, copy=False)


def _normal(rng: np.random.Generator, shape, scale: float) -> np.ndarray:
    out = rng.standard_normal(shape, dtype=np.float32)
    if scale != 1.0:
        out *= np.float32(scale)
    return out


def _run(fn, items, threads):
    items = list(items)
    threads = threads or min(16, os.cpu_count() or 1)
    if threads <= 1 or len(items) <= 1:
        for i in items:
            fn(i)
    else:
        with _cf.ThreadPoolExecutor(threads) as ex:
            list(ex.map(fn, items))


def _cast(a: np.ndarray, act: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if act == "bf16" else a


ROW_CHUNK = 4096


def make_tokens(w: Workload, threads: int | None = None) -> np.ndarray:
    """X [T,D]; rows are drawn in chunks of ROW_CHUNK, chunk c from stream [seed, TAG_X, c]."""
    X = np.empty((w.T, w.D), dtype=np.float32)

    def one(c):
        r0, r1 = c * ROW_CHUNK, min(w.T, (c + 1) * ROW_CHUNK)
        X[r0:r1] = _normal(_rng(w.seed, TAG_X, c), (r1 - r0, w.D), 1.0)

    _run(one, range((w.T + ROW_CHUNK - 1) // ROW_CHUNK), threads)
    if w.dup_frac > 0:
        src, dst = duplicate_map(w)
        X[dst] = X[src]
    return _cast(X, w.act)


def duplicate_map(w: Workload):
    """(src, dst) token indices: row dst is a copy of row src."""
    n = int(np.floor(w.dup_frac * w.T))
    rng = _rng(w.seed, TAG_DUP)
    dst = np.sort(rng.choice(w.T, size=n, replace=False))
    keep = np.setdiff1d(np.arange(w.T), dst)
    src = rng.choice(keep, size=n, replace=True)
    return src.astype(np.int64), dst.astype(np.int64)


def make_router(w: Workload):
    Wg = _normal(_rng(w.seed, TAG_WG), (w.D, w.E), 1.0 / np.sqrt(w.D))
    Wn = _normal(_rng(w.seed, TAG_WNOISE), (w.D, w.E), 1.0 / np.sqrt(w.D)) if w.noise else None
    bias = None
    if w.zipf_bias > 0:
        j = np.arange(1, w.E + 1, dtype=np.float64)
        pmf = j ** (-w.zipf_bias)
        bias = (pmf / pmf.sum()).astype(np.float32)
    return Wg, Wn, bias


def make_hier_router(w: Workload):
    """Primary gate weights [D, a] and per-group secondary weights [a, D, b] (fp32)."""
    a, b = w.groups, w.E // w.groups
    sc = 1.0 / np.sqrt(w.D)
    Wpg = _normal(_rng(w.seed, TAG_WPG), (w.D, a), sc)
    Wpn = _normal(_rng(w.seed, TAG_WPN), (w.D, a), sc) if w.noise else None
    Wsg = np.stack([_normal(_rng(w.seed, TAG_WSG, i), (w.D, b), sc) for i in range(a)])
    Wsn = (np.stack([_normal(_rng(w.seed, TAG_WSN, i), (w.D, b), sc) for i in range(a)])
           if w.noise else None)
    return Wpg, Wpn, Wsg, Wsn


def make_expert(w: Workload, e: int):
    """(W1[e] as [D,H], W2[e] as [H,D]) for one expert."""
    W1 = _normal(_rng(w.seed, TAG_W1, e), (w.D, w.H), 1.0 / np.sqrt(w.D))
    W2 = _normal(_rng(w.seed, TAG_W2, e), (w.H, w.D), 1.0 / np.sqrt(w.H))
    return _cast(W1, w.act), _cast(W2, w.act)


def make_experts(w: Workload, threads: int | None = None):
    """All expert weights: W1 [E,D,H], W2 [E,H,D] (uint16 bf16 bits or fp32)."""
    dt = np.uint16 if w.act == "bf16" else np.float32
    W1 = np.empty((w.E, w.D, w.H), dtype=dt)
    W2 = np.empty((w.E, w.H, w.D), dtype=dt)

    def one(e):
        a, b = make_expert(w, e)
        W1[e] = a
        W2[e] = b

    _run(one, range(w.E), threads)
    return W1, W2


def make_inputs(w: Workload, experts: bool = True, threads: int | None = None) -> dict:
    X = make_tokens(w, threads)
    if w.groups > 0:
        Wpg, Wpn, Wsg, Wsn = make_hier_router(w)
        out = dict(X=X, Wpg=Wpg, Wpn=Wpn, Wsg=Wsg, Wsn=Wsn)
    else:
        Wg, Wn, bias = make_router(w)
        out = dict(X=X, Wg=Wg, Wnoise=Wn, bias=bias)
    if experts:
        out["W1"], out["W2"] = make_experts(w, threads)
    return out


def make_output_grad(w: Workload, threads: int | None = None) -> np.ndarray:
    """dY [T, D]: an incoming gradient for the layer output, N(0, 1/D), in the activation
    dtype (bf16 as uint16 bits); chunk c of ROW_CHUNK rows from stream [seed, TAG_DY, c]."""
    dY = np.empty((w.T, w.D), dtype=np.float32)

    def one(c):
        r0, r1 = c * ROW_CHUNK, min(w.T, (c + 1) * ROW_CHUNK)
        dY[r0:r1] = _normal(_rng(w.seed, TAG_DY, c), (r1 - r0, w.D), 1.0 / np.sqrt(w.D))

    _run(one, range((w.T + ROW_CHUNK - 1) // ROW_CHUNK), threads)
    return _cast(dY, w.act)
