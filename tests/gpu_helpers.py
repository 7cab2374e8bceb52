"""Shared helpers for the GPU parity tests (imported by test_gpu_*.py only).

Inputs come from the seeded generator; expected values come from the CPU
oracle. Nothing computed by the HIP path is ever fed back into the oracle: the
stage tests hand the oracle's intermediate results to the GPU stage, never the
other way round.
"""
from __future__ import annotations

import functools
import sys

import numpy as np
import torch

from oracle import moe as O
from sparsely_gated_mixture_amd import inputs as I

# float tolerances: max|got - ref| / max|ref| per output tensor
TOL = {"f32": 1e-4, "bf16": 2e-2}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a):
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(a).to("cuda")


def host(t):
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def f64(a):
    return O.widen(a)


def rel_err(got, ref) -> float:
    got = f64(got)
    ref = f64(ref)
    den = np.abs(ref).max()
    if den == 0:
        return float(np.abs(got - ref).max())
    return float(np.abs(got - ref).max() / den)


def problem_for(moe, w: I.Workload, **kw):
    return moe.problem(T=w.T, D=w.D, E=w.E, H=w.H, k=w.k, dtype=w.act, gating=w.gating,
                       noise=w.noise, capacity_factor=w.capacity_factor,
                       min_capacity=w.min_capacity, seed=w.seed, **kw)


@functools.lru_cache(maxsize=2)
def workload_inputs(name: str):
    w = I.WORKLOADS[name]
    return w, I.make_inputs(w)


@functools.lru_cache(maxsize=2)
def oracle_routing(name: str):
    w, inp = workload_inputs(name)
    r = O.route(inp["X"], inp["Wg"], inp["Wnoise"], inp["bias"], w.k, w.gating, w.noise,
                seed=w.seed)
    C = O.capacity(w.T, w.k, w.capacity_factor, w.E, w.min_capacity)
    d = O.dispatch(r.ids, w.E, C)
    return r, d


def sample_tokens(w: I.Workload, d: O.Dispatch, n: int = 48, seed: int = 0):
    """A seeded spread of tokens: first / last rows, random rows, dropped rows."""
    rng = np.random.default_rng(seed)
    picks = {0, 1, w.T - 1, w.T // 2}
    picks.update(rng.choice(w.T, size=min(n, w.T), replace=False).tolist())
    dropped = np.nonzero(~d.accepted.all(axis=1))[0]
    if dropped.size:
        picks.update(rng.choice(dropped, size=min(8, dropped.size), replace=False).tolist())
    return np.array(sorted(picks), dtype=np.int64)


def set_mismatch(ids_gpu, ids_ref):
    a = np.sort(ids_gpu, axis=1)
    b = np.sort(ids_ref, axis=1)
    return np.nonzero((a != b).any(axis=1))[0]


def gates_by_id(ids_gpu, gates_gpu, ids_ref, rows):
    """GPU gates re-ordered to the oracle's id order on `rows` (ids equal as sets)."""
    out = np.zeros((rows.size, ids_ref.shape[1]))
    for n, t in enumerate(rows):
        m = {int(e): g for e, g in zip(ids_gpu[t], gates_gpu[t])}
        out[n] = [m[int(e)] for e in ids_ref[t]]
    return out


def max_abs(got, ref) -> float:
    return float(np.abs(f64(got) - f64(ref)).max()) if np.size(ref) else 0.0


_Z_CACHE: dict = {}


def oracle_expert_outputs(key, w: I.Workload, inp: dict, d: O.Dispatch, on_expert=None):
    """The oracle's expert output Z [A, D] (fp64) for every accepted row of its dispatch, one
    expert's rows at a time ([LESSON] ch. 1's gathered form, pinned equal to the per-token loop);
    on_expert(e, r0, r1, h, z) also sees each expert's hidden rows h as they are made. The
    result for one key (a workload name) is kept for the next caller."""
    if key is not None and key in _Z_CACHE and on_expert is None:
        return _Z_CACHE[key]
    A = int(d.offsets[-1])
    Z = np.zeros((A, w.D))
    bank = O.ExpertBank(inp["W1"], inp["W2"], keep=2)
    for e in range(w.E):
        r0, r1 = int(d.offsets[e]), int(d.offsets[e + 1])
        if r1 == r0:
            continue
        h, z = O.expert_rows(inp["X"], d, None, bank, np.arange(r0, r1), hidden=True)
        Z[r0:r1] = z
        if on_expert is not None:
            on_expert(e, r0, r1, h, z)
    _Z_CACHE.clear()
    if key is not None:
        _Z_CACHE[key] = Z
    return Z
