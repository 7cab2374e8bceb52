"""Plain fp64 definition of the MoE forward with the batchwise (strictly
balanced) mask (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages cited:
  [OLNN]   "Outrageously Large Neural Networks" summary, section 3.4, "Strictly
           Balanced Gating (Batchwise Mask, Used in Some MT Experiments)": for
           each expert, keep the m examples of the batch with the highest dense
           gate scores, m = k |X| / n; the threshold mask and the batchwise
           loss used to distil it for inference.
  [LESSON] "Mixture-of-Experts: Sparse Computation", chapter 4, "A stricter
           alternative: forcing exactly equal batches" (the mask multiplied into
           the plain softmax gate and renormalised; every expert gets exactly m
           examples), and chapter 2 for that mask-and-renormalise form.

Readings (listed in the design notes as well):
  * The scores the mask ranks are the dense softmax gate G_sigma(x) =
    Softmax(x . Wg (+ bias)) (the summary names G_sigma(x)_i; the mask-and-
    renormalise form of [LESSON] ch. 2 / ch. 4 multiplies the mask into it).
    No noise.
  * m = floor(k * T / E), required to be at least 1.
  * Ranking along the batch: (score descending, token index ascending), decided
    on the fp32 rounding of the fp64 score; every expert keeps exactly m tokens,
    listed in ascending token order.
  * A token kept by the experts S(x) gets G(x)_i = G_sigma(x)_i / sum over S(x)
    of G_sigma(x)_j for i in S(x), else 0; a token no expert kept keeps only the
    residual (0/0 read as 0). A token may be kept by any number of experts.
  * Near-tie: an expert whose m-th and (m+1)-th scores differ by less than
    2e-6 of the m-th (relative) decides inside fp32 resolution; reported, not
    counted. When the two are exactly equal (identical token rows) the token
    index decides on any hardware, and the expert is a near-tie only if a
    distinct score lies within that margin of the tied value.
  * L_batchwise(X, T, m) = sum_j sum_i (1[s_ji > T_i] - M_ji) (s_ji - T_i), with
    s the same dense scores and T the caller's per-expert thresholds.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import moe as O

NEAR_TIE_REL = 2e-6


@dataclass
class BatchwiseRouting:
    m: int
    clean: np.ndarray      # [T,E] fp64 x . Wg (+ bias)
    probs: np.ndarray      # [T,E] fp64 dense softmax scores
    sel: np.ndarray        # [E,m] int32 tokens kept by each expert, ascending
    mask: np.ndarray       # [T,E] bool
    gates: np.ndarray      # [T,E] fp64 G(x), zero outside the mask
    near_tie: np.ndarray   # [E] bool


def batch_m(T: int, k: int, E: int) -> int:
    return (k * T) // E


def route_batchwise(X, Wg, bias, k: int) -> BatchwiseRouting:
    X64 = O.widen(X)
    clean = X64 @ O.widen(Wg)
    if bias is not None:
        clean = clean + O.widen(bias)[None, :]
    T, E = clean.shape
    m = batch_m(T, k, E)
    if m < 1:
        raise ValueError("batchwise mask needs k * T >= E")
    z = np.exp(clean - clean.max(axis=1, keepdims=True))
    probs = z / z.sum(axis=1, keepdims=True)
    key = probs.astype(np.float32)
    sel = np.zeros((E, m), dtype=np.int32)
    mask = np.zeros((T, E), dtype=bool)
    near = np.zeros(E, dtype=bool)
    for i in range(E):
        order = np.argsort(-key[:, i], kind="stable")  # score desc, token asc
        kept = np.sort(order[:m])
        sel[i] = kept
        mask[kept, i] = True
        if m < T:
            a, b = probs[order[m - 1], i], probs[order[m], i]
            if a != b:
                near[i] = abs(a - b) < NEAR_TIE_REL * abs(a)
            else:
                # an exact tie (identical rows) is decided by the token index on any
                # hardware; only distinct scores close to it could round into it
                u = np.unique(probs[:, i])
                k_ = np.searchsorted(u, a)
                gaps = [u[k_ + 1] - a] if k_ + 1 < u.size else []
                gaps += [a - u[k_ - 1]] if k_ > 0 else []
                near[i] = bool(gaps) and min(gaps) < NEAR_TIE_REL * abs(a)
    num = np.where(mask, probs, 0.0)
    den = num.sum(axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        gates = np.where(den > 0, num / den, 0.0)
    return BatchwiseRouting(m=m, clean=clean, probs=probs, sel=sel, mask=mask, gates=gates,
                            near_tie=near)


def rows(r: BatchwiseRouting) -> np.ndarray:
    """Expert-major row r = i*m + s holds token sel[i, s]."""
    return r.sel.reshape(-1)


def combine_tokens(X, r: BatchwiseRouting, bank: O.ExpertBank, tokens, residual=True):
    """Y[t] = X[t] + sum over the experts i that kept t (ascending i) of G(t)_i E_i(X[t])."""
    tokens = np.asarray(tokens, dtype=np.int64)
    D = X.shape[1]
    out = np.zeros((tokens.size, D))
    for n, t in enumerate(tokens):
        x = O.widen(X[t])
        y = x.copy() if residual else np.zeros(D)
        for i in np.nonzero(r.mask[t])[0]:
            W1e, W2e = bank(int(i))
            y = y + r.gates[t, i] * O.expert(x, W1e, W2e)
        out[n] = y
    return out


def batchwise_loss(r: BatchwiseRouting, thresholds) -> float:
    thr = O.widen(thresholds)[None, :]
    s = r.probs
    return float((((s > thr).astype(np.float64) - r.mask) * (s - thr)).sum())


def aux_batchwise(r: BatchwiseRouting, thresholds=None) -> dict:
    """Importance (sum of gates per expert), its CV^2, the batchwise loss for the given
    thresholds, and how many experts kept each token."""
    imp = r.gates.sum(axis=0)
    per_tok = r.mask.sum(axis=1)
    out = np.array([
        O.cv2(imp),
        batchwise_loss(r, thresholds) if thresholds is not None else 0.0,
        per_tok.mean(),
        float(per_tok.max()),
        float((per_tok == 0).sum()),
        imp.sum(),
        float(r.m),
        0.0,
    ])
    return dict(importance=imp, out=out)


def forward_batchwise(inp: dict, w, tokens=None, thresholds=None) -> dict:
    r = route_batchwise(inp["X"], inp["Wg"], inp.get("bias"), w.k)
    if tokens is None:
        tokens = np.arange(w.T)
    bank = O.ExpertBank(inp["W1"], inp["W2"])
    Y = combine_tokens(inp["X"], r, bank, tokens)
    return dict(routing=r, Y=Y, tokens=np.asarray(tokens), aux=aux_batchwise(r, thresholds),
                bank=bank)
