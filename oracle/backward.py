"""Gradients of the sparsely-gated MoE layer (oracle): reverse mode through the
plain definition, in fp64 on the CPU (torch autograd as the differentiation
primitive).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages cited:
  [OLNN]   "Outrageously Large Neural Networks" summary, section 3.4 (the MoE
           output, Noisy Top-K Gating steps 1-3, the importance and load
           losses); the paper's purpose is training, and k > 1 is chosen so the
           gate receives gradient through the softmax over the kept experts.
  [LESSON] "Mixture-of-Experts: Sparse Computation", chapter 2 ("trace it
           forward, then backward": the kept experts share an incoming gradient
           in proportion to their gates; masked experts are absent from the
           backward pass) and chapter 5 (the losses).

Readings (listed in the design notes as well):
  * The selection (which experts are kept, and which assignments the capacity
    drops) is piecewise constant: it is held fixed, so gradients flow through
    the kept scores H, the softmax over them, the experts and the residual.
    The noise sample eps is held fixed (H = clean + eps * Softplus(raw)).
  * The load estimator's threshold is the score of a specific other expert
    (the k-th or (k+1)-th of the row); its gradient goes to that expert's H.
  * The objective whose gradient is taken is
        <Y, dY> + w_imp * CV^2(Importance) + w_load * CV^2(Load)
    for a given upstream gradient dY and loss weights (0 turns a term off).
  * Noisy top-k gating only (the Switch gate's full softmax is not covered).
"""
from __future__ import annotations

import numpy as np
import torch

from . import moe as O


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(O.widen(a))).requires_grad_(True)


def _cv2(v):
    m = v.mean()
    return ((v - m) ** 2).mean() / (m * m)


def layer_grads(inp: dict, w, r: O.Routing, d: O.Dispatch, eps, dY, w_imp=0.0, w_load=0.0,
                residual=True, experts=None) -> dict:
    """Gradients of <Y, dY> + w_imp CV^2(Imp) + w_load CV^2(Load) w.r.t. X, Wg, Wnoise,
    bias, W1 and W2 (expert weights only for `experts`, default all), with the routing
    r / d and the noise eps held fixed."""
    X = _t(inp["X"])
    Wg = _t(inp["Wg"])
    noisy = w.noise and inp.get("Wnoise") is not None
    Wn = _t(inp["Wnoise"]) if noisy else None
    bias = _t(inp["bias"]) if inp.get("bias") is not None else None
    T, E, k = w.T, w.E, w.k
    ids = torch.from_numpy(r.ids.astype(np.int64))
    clean = X @ Wg
    if bias is not None:
        clean = clean + bias[None, :]
    if noisy:
        std = torch.nn.functional.softplus(X @ Wn)
        H = clean + torch.from_numpy(O.widen(eps)) * std
    else:
        std, H = None, clean
    Hk = torch.gather(H, 1, ids)
    G = torch.softmax(Hk, dim=1)
    ex = sorted(set(np.unique(r.ids).tolist())) if experts is None else list(experts)
    W1 = {e: _t(inp["W1"][e]) for e in ex}
    W2 = {e: _t(inp["W2"][e]) for e in ex}
    Y = X * 1.0 if residual else torch.zeros_like(X)
    acc = torch.from_numpy(d.accepted)
    contrib = []
    for e in np.unique(r.ids):
        tt, jj = np.nonzero((r.ids == e) & d.accepted)
        if tt.size == 0:
            continue
        if e in W1:
            z = torch.relu(X[tt] @ W1[e]) @ W2[e]
        else:
            W1e = torch.from_numpy(O.widen(inp["W1"][e]))
            W2e = torch.from_numpy(O.widen(inp["W2"][e]))
            z = torch.relu(X[tt] @ W1e) @ W2e
        contrib.append((torch.from_numpy(tt), G[tt, jj][:, None] * z))
    for tt, c in contrib:
        Y = Y.index_add(0, tt, c)
    obj = (Y * torch.from_numpy(O.widen(dY))).sum()
    if w_imp:
        imp = torch.zeros(E, dtype=torch.float64).index_add(0, ids.reshape(-1), G.reshape(-1))
        obj = obj + w_imp * _cv2(imp)
    if w_load and noisy:
        # thresholds: the k-th and (k+1)-th scores of the row, by index (the forward's order)
        order = np.argsort(-r.score.astype(np.float32), axis=1, kind="stable")
        ik = torch.from_numpy(order[:, k - 1].astype(np.int64))
        vk = H[torch.arange(T), ik]
        inside = torch.zeros(T, E, dtype=torch.bool)
        inside[torch.arange(T)[:, None], ids] = True
        if k < E:
            ik1 = torch.from_numpy(order[:, k].astype(np.int64))
            vk1 = H[torch.arange(T), ik1]
            thr = torch.where(inside, vk1[:, None], vk[:, None])
            P = torch.special.ndtr((clean - thr) / std)
        else:
            # k = E: every expert is kept and no (k+1)-th score exists, so each expert is kept
            # under every noise draw; P = 1 is a constant and the term has no gradient
            P = torch.ones(T, E, dtype=torch.float64)
        obj = obj + w_load * _cv2(P.sum(dim=0))
    obj.backward()
    out = dict(dX=X.grad.numpy(), dWg=Wg.grad.numpy(),
               dWnoise=Wn.grad.numpy() if noisy else None,
               dW1={e: W1[e].grad.numpy() if W1[e].grad is not None else np.zeros(W1[e].shape)
                    for e in ex},
               dW2={e: W2[e].grad.numpy() if W2[e].grad is not None else np.zeros(W2[e].shape)
                    for e in ex},
               objective=float(obj.detach()))
    if bias is not None:
        out["dbias"] = bias.grad.numpy()
    return out
