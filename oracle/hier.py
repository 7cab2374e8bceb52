"""Plain fp64 definition of the hierarchical (two-level) MoE forward (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages cited:
  [OLNN]   "Outrageously Large Neural Networks" summary, section 3.4,
           "Hierarchical Mixture-of-Experts": a groups of b experts; a primary
           gate picks groups, group i's secondary gate picks experts inside it;
           y_H = sum_i sum_j Gp(x)_i * G_i(x)_j * E_ij(x); Importance_H and
           Load_H as defined there.
  [LESSON] "Mixture-of-Experts: Sparse Computation", chapter 1 ("When n gets
           too large to gate directly") and chapter 5 ("Balancing at every
           level, once the gate is hierarchical"): the same equations, X^(i) =
           the examples routed to group i, and the division by |X^(i)|.

Readings (listed in the design notes as well):
  * Both levels are noisy top-k gates of the flat kind (same steps, same
    tie rule); the primary keeps k_p of a groups, each secondary keeps k_s of
    its b experts, so every token uses k = k_p * k_s experts.
  * Expert (i, j) is global expert i*b + j; a token's k assignments are listed
    primary slot first (in the primary's order), then the secondary's order.
  * Noise: the primary gate draws as the flat gate does (key (seed, 0)); the
    secondary gate of group i draws from key (seed, 1 + i), counter (t, j/4),
    so every (token, group, expert) has its own sample.
  * Capacity, dispatch, experts and combine are the flat layer's, applied to
    the k final assignments and the product gates over the a*b experts.
  * Load_i(X^(i)) is the flat load estimator of gate i over the tokens of
    X^(i) (its own k_s, noise scale and thresholds). A group that received no
    token has Load_H = 0 for all its experts (0/0 read as 0).
  * The balancing terms are CV^2 of the a*b-vectors Importance_H and Load_H;
    the primary gate's own CV^2 terms are returned beside them.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import moe as O
from .philox import gaussian_noise


@dataclass
class HierRouting:
    primary: O.Routing          # over the a groups, k_p kept
    members: list               # members[i]: ascending token indices of X^(i)
    secondary: list             # secondary[i]: O.Routing over the b experts for X^(i)
    ids: np.ndarray             # [T, k_p*k_s] global expert ids
    gates: np.ndarray           # [T, k_p*k_s] Gp * G_i
    near_tie: np.ndarray        # [T] primary or any secondary decision inside the margin


def route_hier(X, Wpg, Wpn, Wsg, Wsn, kp: int, ks: int, noise: bool, seed: int = 0,
               eps_primary=None, eps_secondary=None) -> HierRouting:
    """Primary gate over groups, then group i's gate over its experts for X^(i).

    eps_primary [T, a] and eps_secondary (a list of [|X^(i)|, b]) replace the
    generated noise when given."""
    T = X.shape[0]
    a = Wpg.shape[1]
    b = Wsg.shape[2]
    p = O.route(X, Wpg, Wpn, None, kp, "noisy", noise, seed=seed, eps=eps_primary)
    members, sec = [], []
    ids = np.zeros((T, kp * ks), dtype=np.int32)
    gates = np.zeros((T, kp * ks))
    near = p.near_tie.copy()
    for i in range(a):
        tok = np.nonzero((p.ids == i).any(axis=1))[0]
        members.append(tok)
        if tok.size == 0:
            sec.append(None)
            continue
        eps = None
        if noise:
            eps = (gaussian_noise(seed, 0, b, key1=1 + i, tokens=tok) if eps_secondary is None
                   else eps_secondary[i])
        r = O.route(X[tok], Wsg[i], Wsn[i] if Wsn is not None else None, None, ks, "noisy",
                    noise, eps=eps)
        sec.append(r)
        near[tok] |= r.near_tie
        slot = np.argmax(p.ids[tok] == i, axis=1)  # where group i sits in each token's list
        for j in range(ks):
            ids[tok, slot * ks + j] = i * b + r.ids[:, j]
            gates[tok, slot * ks + j] = p.gates[tok, slot] * r.gates[:, j]
    return HierRouting(primary=p, members=members, secondary=sec, ids=ids, gates=gates,
                       near_tie=near)


def as_routing(h: HierRouting) -> O.Routing:
    """The final assignments in the flat layer's form (ids and gates only)."""
    T = h.ids.shape[0]
    return O.Routing(ids=h.ids, gates=h.gates, clean=None, std=None, score=None,
                     row_stats=None, gap=np.full(T, np.inf), near_tie=h.near_tie)


def aux_hier(h: HierRouting, a: int, b: int, kp: int, ks: int) -> dict:
    """Importance_H, Load_H and their CV^2 ([OLNN] 3.4, hierarchical metrics).

    Importance_H(i, j) = sum over x of Gp(x)_i * G_i(x)_j
    Load_H(i, j)       = Load_p(X)_i * Load_i(X^(i))_j / |X^(i)|
    """
    imp = np.zeros(a * b)
    np.add.at(imp, h.ids.ravel(), h.gates.ravel())
    noisy = h.primary.std is not None
    load = np.zeros(a * b)
    lp = np.zeros(a)
    if noisy:
        lp = O.load_probs(h.primary, kp).sum(axis=0)
        for i in range(a):
            n = h.members[i].size
            if n == 0:
                continue
            ls = O.load_probs(h.secondary[i], ks).sum(axis=0)
            load[i * b:(i + 1) * b] = lp[i] * ls / n
    ip = np.zeros(a)
    np.add.at(ip, h.primary.ids.ravel(), h.primary.gates.ravel())
    lm = load.mean()
    out = np.array([
        O.cv2(imp),
        O.cv2(load),
        O.cv2(ip),
        O.cv2(lp),
        load.max() / lm if lm > 0 else 0.0,
        float(sum(m.size == 0 for m in h.members)),
        imp.sum(),
        0.0,
    ])
    return dict(importance=imp, load=load, importance_primary=ip, load_primary=lp, out=out)


def forward_hier(inp: dict, w, tokens=None) -> dict:
    """Whole hierarchical forward for workload `w` (w.groups = a, w.k_primary = k_p)."""
    a, kp = w.groups, w.k_primary
    b, ks = w.E // a, w.k // kp
    h = route_hier(inp["X"], inp["Wpg"], inp["Wpn"], inp["Wsg"], inp["Wsn"], kp, ks, w.noise,
                   seed=w.seed)
    r = as_routing(h)
    C = O.capacity(w.T, w.k, w.capacity_factor, w.E, w.min_capacity)
    d = O.dispatch(h.ids, w.E, C)
    if tokens is None:
        tokens = np.arange(w.T)
    bank = O.ExpertBank(inp["W1"], inp["W2"])
    Y = O.combine_tokens(inp["X"], r, d, bank, tokens)
    return dict(hier=h, routing=r, dispatch=d, Y=Y, tokens=np.asarray(tokens),
                aux=aux_hier(h, a, b, kp, ks), bank=bank)
