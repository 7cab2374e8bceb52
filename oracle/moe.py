"""Plain fp64 definition of the sparsely-gated MoE layer forward pass (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages cited (by title; sections as the pages name them):
  [OLNN]   "Outrageously Large Neural Networks: The Sparsely-Gated
           Mixture-of-Experts Layer" -- paper summary page, section 3.4.
  [SWITCH] "Switch Transformer" explainer page, "Implementation", steps 1-8.
  [KB]     "Sparsely-Gated MoE" knowledge-base page, sections 2-3.
  [LESSON] "Mixture-of-Experts: Sparse Computation" lesson page, chapters 1-5.

Readings where the pages are silent or disagree (each one is listed in the
design notes as well):
  * The top-k decision is taken on the fp32 rounding of the fp64 score (the
    precision the routing kernel decides in; [SWITCH] step 1 routes in fp32),
    ordering by (score descending, expert index ascending): ties go to the
    lower index ([SWITCH] step 2). Gates use the fp64 scores.
  * Switch top-1 decides on the fp32 logit. Softmax is monotone, so this is the
    page's argmax over probabilities except inside fp32 resolution, where the
    token is a near-tie and is reported, not counted.
  * Capacity for k > 1: C = max(min_cap, min(T, floor(k*T*cf/E))), which is
    [SWITCH] step 3 at k = 1. cf <= 0 means no limit, i.e. C = T (a token's k
    experts are distinct, so no expert can receive more than T rows).
  * Slots are token-major: an assignment's slot counts the earlier
    assignments (lower t, then lower j) to the same expert ([SWITCH] step 3).
  * Gates are not renormalised after drops ([SWITCH] step 4: capacity removes
    an expert contribution, not a token); the residual is the input X.
  * CV uses the population variance (ddof 0), which the [LESSON] chapter 5
    example (0.68 for [25, 10, 1]) fixes.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
from scipy.special import ndtr

from .philox import gaussian_noise

NEAR_TIE = 1e-6


# --------------------------------------------------------------------------- helpers

def widen(a) -> np.ndarray:
    """Exact fp64 values of an fp32 array or of bf16 bit patterns (uint16)."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def softplus(z: np.ndarray) -> np.ndarray:
    """ln(1 + e^z), written in a form that cannot overflow ([OLNN] 3.4, Step 1)."""
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def cv2(v: np.ndarray) -> float:
    """Squared coefficient of variation, population variance ([OLNN] 3.4, importance loss)."""
    v = np.asarray(v, dtype=np.float64)
    m = v.mean()
    if m == 0.0:
        return 0.0
    return float(((v - m) ** 2).mean() / (m * m))


def capacity(T: int, k: int, cf: float, E: int, min_cap: int = 1) -> int:
    """Per-expert slot count ([SWITCH] step 3, generalised to k as above)."""
    if not cf > 0.0:
        return T
    return max(min_cap, min(T, int(math.floor(float(k) * float(T) * float(cf) / float(E)))))


# --------------------------------------------------------------------------- router

@dataclass
class Routing:
    ids: np.ndarray        # [T,k] int32, by (score desc, index asc)
    gates: np.ndarray      # [T,k] fp64
    clean: np.ndarray      # [T,E] fp64 = X.Wg (+ bias)
    std: np.ndarray | None  # [T,E] fp64 = softplus(X.Wnoise) (noisy gate only)
    score: np.ndarray      # [T,E] fp64 selection score: H (noisy) or clean (Switch / no noise)
    row_stats: np.ndarray  # [T,2] fp64: k-th and (k+1)-th largest score (-inf if k = E)
    gap: np.ndarray        # [T] fp64 margin that decides the selected set
    near_tie: np.ndarray   # [T] bool: gap < NEAR_TIE


def _order(score: np.ndarray) -> np.ndarray:
    """Experts of each row by (fp32 score descending, index ascending)."""
    key = score.astype(np.float32)
    return np.argsort(-key, axis=1, kind="stable")


def route(X, Wg, Wnoise, bias, k: int, gating: str, noise: bool, seed: int = 0,
          eps: np.ndarray | None = None, t0: int = 0) -> Routing:
    """Router for tokens t0 .. t0+T-1.

    Noisy top-k ([OLNN] 3.4, "Noisy Top-K Gating", Steps 1-3; [KB] section 2):
      clean = X.Wg, std = Softplus(X.Wnoise), H = clean + eps * std,
      keep the k largest H, G = softmax over the kept values (others exactly 0).
    Switch top-1 ([SWITCH] steps 1-2): p = softmax(X.Wr (+ bias)) in full,
      expert = argmax (first on ties), gate = p[expert], not renormalised.
    """
    X64 = widen(X)
    T = X64.shape[0]
    clean = X64 @ widen(Wg)
    if bias is not None:
        clean = clean + widen(bias)[None, :]
    E = clean.shape[1]
    std = None
    if gating == "switch":
        score = clean
    elif noise:
        std = softplus(X64 @ widen(Wnoise))
        if eps is None:
            eps = gaussian_noise(seed, T, E, t0)
        score = clean + widen(eps) * std
    else:
        score = clean
    order = _order(score)
    ids = order[:, :k].astype(np.int32)
    rows = np.arange(T)[:, None]
    kept = score[rows, ids]
    if gating == "switch":
        m = clean.max(axis=1, keepdims=True)
        p = np.exp(clean - m)
        p /= p.sum(axis=1, keepdims=True)
        gates = p[rows, ids]
    else:
        z = np.exp(kept - kept.max(axis=1, keepdims=True))
        gates = z / z.sum(axis=1, keepdims=True)
    vk = kept[:, k - 1]
    vk1 = score[np.arange(T), order[:, k]] if k < E else np.full(T, -np.inf)
    s64 = -np.sort(-score, axis=1)
    gap = (s64[:, k - 1] - s64[:, k]) if k < E else np.full(T, np.inf)
    return Routing(ids=ids, gates=gates, clean=clean, std=std, score=score,
                   row_stats=np.stack([vk, vk1], axis=1), gap=gap, near_tie=gap < NEAR_TIE)


def kth_excluding(h_row: np.ndarray, k: int, i: int) -> float:
    """k-th largest entry of h_row among all entries except i ([OLNN] 3.4, load estimator)."""
    others = np.delete(np.asarray(h_row, dtype=np.float64), i)
    if k > others.size:
        return -np.inf
    return float(np.sort(others)[::-1][k - 1])


# --------------------------------------------------------------------------- dispatch

@dataclass
class Dispatch:
    C: int
    pos: np.ndarray        # [T,k] int32 slot of each assignment
    accepted: np.ndarray   # [T,k] bool: pos < C
    counts: np.ndarray     # [E] int32 assignments per expert, before capacity
    offsets: np.ndarray    # [E+1] int32 exclusive scan of min(count, C)
    row_token: np.ndarray  # [offsets[E]] int32: token held by each expert-major row


def dispatch(ids: np.ndarray, E: int, C: int) -> Dispatch:
    """Stable slots and the capacity mask ([SWITCH] steps 3-5).

    Walks the assignments in token order; an assignment's slot is the number of
    earlier assignments to the same expert, and it is kept if the slot is
    below C. Expert-major rows: expert e owns rows offsets[e] .. offsets[e+1]-1
    in slot order.
    """
    T, k = ids.shape
    cnt = np.zeros(E, dtype=np.int64)
    pos = np.zeros((T, k), dtype=np.int32)
    for t in range(T):
        for j in range(k):
            e = int(ids[t, j])
            pos[t, j] = cnt[e]
            cnt[e] += 1
    accepted = pos < C
    kept = np.minimum(cnt, C)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    row_token = np.full(int(offsets[E]), -1, dtype=np.int32)
    tt, jj = np.nonzero(accepted)
    row_token[offsets[ids[tt, jj]] + pos[tt, jj]] = tt
    return Dispatch(C=C, pos=pos, accepted=accepted, counts=cnt.astype(np.int32),
                    offsets=offsets.astype(np.int32), row_token=row_token)


# --------------------------------------------------------------------------- experts + combine

def expert(x64: np.ndarray, W1e64: np.ndarray, W2e64: np.ndarray, hidden: bool = False):
    """One expert on one token (or on a batch of rows): ReLU(x.W1) . W2, no biases
    ([SWITCH] step 6). hidden: return (ReLU(x.W1), output)."""
    h = np.maximum(x64 @ W1e64, 0.0)
    z = h @ W2e64
    return (h, z) if hidden else z


class ExpertBank:
    """fp64 copies of expert weights, widened on first use (the last `keep` kept)."""

    def __init__(self, W1, W2, keep: int = 64):
        self.W1, self.W2 = W1, W2
        self.keep = keep
        self._cache = {}

    def __call__(self, e: int):
        if e in self._cache:
            v = self._cache.pop(e)
        else:
            v = (widen(self.W1[e]), widen(self.W2[e]))
            while len(self._cache) >= self.keep:
                self._cache.pop(next(iter(self._cache)))
        self._cache[e] = v
        return v


def expert_rows(X, d: Dispatch, ids: np.ndarray, bank: ExpertBank, rows, hidden: bool = False):
    """Expert outputs for expert-major rows: row r holds token row_token[r] of
    the expert whose range contains r ([SWITCH] steps 5-6). Rows of one expert
    go through that expert together, as one gathered batch ([LESSON] ch. 1,
    forward_batched). hidden: return (hidden activations, outputs)."""
    rows = np.asarray(rows, dtype=np.int64)
    experts = np.searchsorted(d.offsets, rows, side="right") - 1
    out = np.zeros((rows.size, X.shape[1]))
    hid = None
    for e in np.unique(experts):
        sel = np.nonzero(experts == e)[0]
        W1e, W2e = bank(int(e))
        h, out[sel] = expert(widen(X[d.row_token[rows[sel]]]), W1e, W2e, hidden=True)
        if hidden:
            if hid is None:
                hid = np.zeros((rows.size, W1e.shape[1]))
            hid[sel] = h
    if hidden:
        return (np.zeros((rows.size, 0)) if hid is None else hid), out
    return out


def combine_rows(Z, r: Routing, d: Dispatch, R=None, tokens=None) -> np.ndarray:
    """Y[t] = R[t] + sum over accepted j (ascending) of gate_tj * Z[offsets[e] + pos]
    given expert-major outputs Z ([SWITCH] step 7; R = None means no residual)."""
    T, k = r.ids.shape
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    Z64 = widen(Z)
    D = Z64.shape[1]
    out = np.zeros((tokens.size, D))
    for n, t in enumerate(tokens):
        y = widen(R[t]).copy() if R is not None else np.zeros(D)
        for j in range(k):
            if d.accepted[t, j]:
                y = y + r.gates[t, j] * Z64[d.offsets[r.ids[t, j]] + d.pos[t, j]]
        out[n] = y
    return out


def combine_tokens(X, r: Routing, d: Dispatch, bank: ExpertBank, tokens, residual: bool = True):
    """Y[t] = X[t] + sum over accepted j (ascending) of gate_tj * E_{e_tj}(X[t]).

    A per-token loop over the chosen experts only ([OLNN] 3.4, the MoE output;
    [LESSON] chapter 1; [SWITCH] step 7). Returns fp64 rows for `tokens`.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    D = X.shape[1]
    out = np.zeros((tokens.size, D), dtype=np.float64)
    for n, t in enumerate(tokens):
        x = widen(X[t])
        y = x.copy() if residual else np.zeros(D)
        for j in range(r.ids.shape[1]):
            if d.accepted[t, j]:
                W1e, W2e = bank(int(r.ids[t, j]))
                y = y + r.gates[t, j] * expert(x, W1e, W2e)
        out[n] = y
    return out


# --------------------------------------------------------------------------- aux losses

def load_probs(r: Routing, k: int) -> np.ndarray:
    """P(x, i) = Phi((clean_i - kth_excluding(H, k, i)) / std_i)  ([OLNN] 3.4, load).

    kth_excluding is read off the sorted row: for an expert inside the top k it
    is the (k+1)-th largest score, otherwise the k-th (pinned against the
    brute-force definition in the tests). A zero std leaves a step function.
    """
    T, E = r.clean.shape
    thr = np.repeat(r.row_stats[:, :1], E, axis=1)
    inside = np.zeros((T, E), dtype=bool)
    inside[np.arange(T)[:, None], r.ids] = True
    thr = np.where(inside, r.row_stats[:, 1:2], thr)
    diff = r.clean - thr
    with np.errstate(divide="ignore", invalid="ignore"):
        z = diff / r.std
        P = ndtr(z)
    step = np.where(diff > 0, 1.0, np.where(diff == 0, 0.5, 0.0))
    return np.where(r.std > 0, P, step)


def aux(r: Routing, d: Dispatch, k: int) -> dict:
    """Importance, Load and the Switch term, unweighted.

    importance_e = sum of gates to e (before capacity)     [OLNN] 3.4, importance
    load_e       = sum_t P(t, e)   (noisy gate only)      [OLNN] 3.4, load
    switch_fP    = E * sum_e f_e * Pbar_e, f_e = count_e / T before capacity,
                   Pbar_e = mean_t softmax(clean)_e       [SWITCH] step 8
    """
    T, E = r.clean.shape
    imp = np.zeros(E)
    np.add.at(imp, r.ids.ravel(), r.gates.ravel())
    if r.std is not None:
        load = load_probs(r, k).sum(axis=0)
    else:
        load = np.zeros(E)
    m = r.clean.max(axis=1, keepdims=True)
    p = np.exp(r.clean - m)
    p /= p.sum(axis=1, keepdims=True)
    f = d.counts.astype(np.float64) / T
    switch_fP = E * float((f * p.mean(axis=0)).sum())
    lm = load.mean()
    cm = d.counts.mean()
    out = np.array([
        cv2(imp),
        cv2(load),
        switch_fP,
        load.max() / lm if lm > 0 else 0.0,
        d.counts.max() / cm if cm > 0 else 0.0,
        float((~d.accepted).sum()),
        imp.sum(),
        0.0,
    ])
    return dict(importance=imp, load=load, out=out)


# --------------------------------------------------------------------------- whole layer

def forward(inp: dict, w, tokens=None, t_count: int | None = None, eps=None) -> dict:
    """Whole forward pass for workload `w` on the first t_count tokens (default all).

    Routing and slots cover tokens 0 .. t_count-1 (a prefix keeps every slot
    exact); capacity always uses the workload's full T. Outputs Y only for
    `tokens` (default: all routed tokens).
    """
    T = w.T if t_count is None else t_count
    X = inp["X"][:T]
    r = route(X, inp["Wg"], inp.get("Wnoise"), inp.get("bias"), w.k, w.gating, w.noise,
              seed=w.seed, eps=eps)
    C = capacity(w.T, w.k, w.capacity_factor, w.E, w.min_capacity)
    d = dispatch(r.ids, w.E, C)
    if tokens is None:
        tokens = np.arange(T)
    bank = ExpertBank(inp["W1"], inp["W2"])
    Y = combine_tokens(X, r, d, bank, tokens)
    a = aux(r, d, w.k)
    return dict(routing=r, dispatch=d, Y=Y, tokens=np.asarray(tokens), aux=a, bank=bank)
