"""Gradients of the sparsely-gated MoE layer (oracle): reverse mode through the
plain definition, in fp64 on the CPU (torch autograd as the differentiation
primitive).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Pages cited:
  [OLNN]   "Outrageously Large Neural Networks" summary, section 3.4 (the MoE
           output, Noisy Top-K Gating steps 1-3, the importance and load
           losses); the paper's purpose is training, and k > 1 is chosen so the
           gate receives gradient through the softmax over the kept experts.
  [LESSON] "Mixture-of-Experts: Sparse Computation", chapter 3 ("trace it
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
                residual=True, experts=None, w_switch=0.0) -> dict:
    """Gradients of <Y, dY> + w_imp CV^2(Imp) + w_load CV^2(Load) w.r.t. X, Wg, Wnoise,
    bias, W1 and W2 (expert weights only for `experts`, default all), with the routing
    r / d and the noise eps held fixed.

    Switch gate ([SWITCH] steps 2 and 8): the gate is the selected expert's probability
    under the full softmax of the clean logits (not renormalised); the balancing term
    w_switch * E * sum_e f_e * Pbar_e adds its gradient through the mean probabilities
    Pbar, the hard fractions f = count / T (before capacity) held fixed."""
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
    if w.gating == "switch":
        probs = torch.softmax(clean, dim=1)
        G = torch.gather(probs, 1, ids)
    else:
        G = torch.softmax(torch.gather(H, 1, ids), dim=1)
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
    if w_switch and w.gating == "switch":
        f = torch.from_numpy(d.counts.astype(np.float64) / T)
        obj = obj + w_switch * E * (f * probs.mean(dim=0)).sum()
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


# --------------------------------------------------------------------------- sampled, closed form
#
# The same gradients written out by hand in numpy fp64, for a chosen subset of
# outputs (token rows of dX, whole experts of dW1 / dW2, expert columns of dWg /
# dWnoise / dbias), so that a full-size layer can be checked where the autograd
# graph above would not fit. Agreement with layer_grads is pinned in the tests.

def cv2_grad(v: np.ndarray) -> np.ndarray:
    """d CV^2 / d v with CV^2 = var / mean^2 (population variance, [OLNN] 3.4):
    2 / (E mean^2) * ((v_e - mean) - var / mean); zero for a zero mean."""
    v = np.asarray(v, dtype=np.float64)
    E, m = v.size, v.mean()
    if m == 0:
        return np.zeros(E)
    var = ((v - m) ** 2).mean()
    return 2.0 / (E * m * m) * ((v - m) - var / m)


def _phi(z):
    return np.exp(-0.5 * z * z) / np.sqrt(2.0 * np.pi)


class SampledGrads:
    """Closed-form gradients of <Y, dY> + w_imp CV^2(Imp) + w_load CV^2(Load) for
    sampled outputs, routing r / d and noise eps fixed (the readings of the module
    docstring). Terms, for token t with kept experts e_j, gates G_j, accepted a_j:

      z_j      = ReLU(x W1_ej) W2_ej                     (expert output)
      dG_j     = a_j <dY_t, z_j> + dImp[e_j]              (output + importance term)
      dH_j     = G_j (dG_j - sum_l G_l dG_l)              (softmax over the kept scores)
      load:    P(t,e) = Phi((clean - thr) / std), thr = H of the (k+1)-th expert for
               kept e, of the k-th otherwise; dP = dLoad[e]:
               dclean += dP phi / std, dstd -= dP phi z / std, and the threshold's
               expert receives minus the sum of dP phi / std over the experts using it
      dH on expert e splits into dclean += dH, dstd += dH eps (H = clean + eps std)
      draw     = dstd * sigmoid(x Wnoise)                 (d Softplus)
      dX_t     = dY_t + sum_j a_j ((G_j dY_t W2^T) * 1[x W1 > 0]) W1^T
                 + dclean_t Wg^T + draw_t Wnoise^T
      dW2_e    = sum over rows of e of ReLU(x W1_e)^T (G dY_t),
      dW1_e    = sum over rows of e of x^T ((G dY_t W2_e^T) * 1[x W1_e > 0])
      dWg[:,e] = X^T dclean[:, e], dWnoise[:, e] = X^T draw[:, e], dbias[e] = sum dclean[:, e]
    """

    def __init__(self, inp: dict, w, r: O.Routing, d: O.Dispatch, eps, dY, w_imp=0.0,
                 w_load=0.0, residual=True, bank: O.ExpertBank | None = None, w_switch=0.0):
        self.inp, self.w, self.r, self.d = inp, w, r, d
        self.switch = w.gating == "switch"
        # Switch: dPbar_e = w_switch * E * f_e, so every probability p[t, e] gets that / T
        self.dprob = (w_switch * w.E * d.counts.astype(np.float64) / w.T / w.T
                      if (self.switch and w_switch) else None)
        self.noisy = w.noise and inp.get("Wnoise") is not None and not self.switch
        self.eps = O.widen(eps) if self.noisy else None
        self.dY = dY
        self.residual = residual
        self.bank = bank if bank is not None else O.ExpertBank(inp["W1"], inp["W2"], keep=16)
        T, E, k = w.T, w.E, w.k
        a = O.aux(r, d, k)
        self.dimp = w_imp * cv2_grad(a["importance"]) if w_imp else np.zeros(E)
        self.dload = w_load * cv2_grad(a["load"]) if (w_load and self.noisy) else None
        self.order = O._order(r.score)
        self._dg = {}

    def _z(self, t: int, j: int) -> np.ndarray:
        W1e, W2e = self.bank(int(self.r.ids[t, j]))
        return O.expert(O.widen(self.inp["X"][t]), W1e, W2e)

    def _dgates(self, tokens) -> np.ndarray:
        """a_j <dY_t, z_j> for the given tokens, experts visited in index order."""
        tokens = np.asarray(tokens, dtype=np.int64)
        need = [(t, j) for t in tokens.tolist() for j in range(self.w.k)
                if self.d.accepted[t, j] and (t, j) not in self._dg]
        for e in sorted({int(self.r.ids[t, j]) for t, j in need}):
            W1e, W2e = self.bank(e)
            tj = [(t, j) for t, j in need if self.r.ids[t, j] == e]
            xs = O.widen(self.inp["X"][[t for t, _ in tj]])
            zs = O.expert(xs, W1e, W2e)
            for (t, j), z in zip(tj, zs):
                self._dg[(t, j)] = float(O.widen(self.dY[t]) @ z)
        out = np.zeros((tokens.size, self.w.k))
        for n, t in enumerate(tokens.tolist()):
            for j in range(self.w.k):
                out[n, j] = self._dg.get((t, j), 0.0)
        return out

    def row_grads(self, tokens):
        """dclean, dstd [len(tokens), E] for the given token rows."""
        r, k, E = self.r, self.w.k, self.w.E
        tokens = np.asarray(tokens, dtype=np.int64)
        n = tokens.size
        dcl = np.zeros((n, E))
        dsd = np.zeros((n, E))
        ids = r.ids[tokens]
        G = r.gates[tokens]
        dG = self._dgates(tokens) + self.dimp[ids]
        rows = np.arange(n)[:, None]
        if self.switch:
            # p = softmax(clean) over all E; G = p[e*]: dclean = p * (dp - <p, dp>)
            z = r.clean[tokens] - r.clean[tokens].max(axis=1, keepdims=True)
            p = np.exp(z)
            p /= p.sum(axis=1, keepdims=True)
            dp = np.zeros((n, E)) if self.dprob is None else np.repeat(self.dprob[None, :], n, 0)
            dp[rows, ids] += dG
            return p * (dp - (p * dp).sum(axis=1, keepdims=True)), np.zeros((n, E))
        dH = G * (dG - (G * dG).sum(axis=1, keepdims=True))
        dcl[rows, ids] += dH
        if self.noisy:
            dsd[rows, ids] += dH * self.eps[tokens[:, None], ids]
        if self.dload is not None:
            clean, std = r.clean[tokens], r.std[tokens]
            inside = np.zeros((n, E), dtype=bool)
            inside[rows, ids] = True
            thr = np.where(inside, r.row_stats[tokens, 1:2], r.row_stats[tokens, 0:1])
            ok = (std > 0) & np.isfinite(thr)
            with np.errstate(invalid="ignore", divide="ignore"):
                z = np.where(ok, (clean - thr) / std, 0.0)
                c = np.where(ok, self.dload[None, :] * _phi(z) / std, 0.0)
            dcl += c
            dsd -= c * z
            s_in = np.where(inside, c, 0.0).sum(axis=1)
            s_out = np.where(inside, 0.0, c).sum(axis=1)
            ik = ids[:, k - 1]
            dcl[np.arange(n), ik] -= s_out
            dsd[np.arange(n), ik] -= s_out * self.eps[tokens, ik]
            if k < E:
                ik1 = self.order[tokens, k]
                dcl[np.arange(n), ik1] -= s_in
                dsd[np.arange(n), ik1] -= s_in * self.eps[tokens, ik1]
        return dcl, dsd

    def _sigmoid_raw(self, tokens):
        raw = O.widen(self.inp["X"][tokens]) @ O.widen(self.inp["Wnoise"])
        return 1.0 / (1.0 + np.exp(-raw))

    def dX(self, tokens) -> np.ndarray:
        """Rows of dX for the given tokens."""
        tokens = np.asarray(tokens, dtype=np.int64)
        inp, r, d = self.inp, self.r, self.d
        dcl, dsd = self.row_grads(tokens)
        out = dcl @ O.widen(inp["Wg"]).T
        if self.noisy:
            out += (dsd * self._sigmoid_raw(tokens)) @ O.widen(inp["Wnoise"]).T
        for n, t in enumerate(tokens.tolist()):
            x = O.widen(inp["X"][t])
            dy = O.widen(self.dY[t])
            if self.residual:
                out[n] += dy
            for j in range(self.w.k):
                if d.accepted[t, j]:
                    W1e, W2e = self.bank(int(r.ids[t, j]))
                    dpre = (r.gates[t, j] * dy @ W2e.T) * (x @ W1e > 0)
                    out[n] += dpre @ W1e.T
        return out

    def expert_grads(self, e: int):
        """dW1_e [D, H], dW2_e [H, D] over the expert's accepted rows."""
        r, d = self.r, self.d
        tt, jj = np.nonzero((r.ids == e) & d.accepted)
        W1e, W2e = self.bank(int(e))
        if tt.size == 0:
            return np.zeros(W1e.shape), np.zeros(W2e.shape)
        x = O.widen(self.inp["X"][tt])
        dz = r.gates[tt, jj][:, None] * O.widen(self.dY[tt])
        pre = x @ W1e
        dpre = (dz @ W2e.T) * (pre > 0)
        return x.T @ dpre, np.maximum(pre, 0.0).T @ dz

    def router_columns(self, cols):
        """dWg[:, cols], dWnoise[:, cols] (None without noise) and dbias[cols]: every
        token's dclean / draw at those experts (full rows only where needed)."""
        r, k, E, T = self.r, self.w.k, self.w.E, self.w.T
        cols = [int(c) for c in cols]
        X64 = O.widen(self.inp["X"])
        gw, nw, bw = [], [], []
        for e in cols:
            # tokens whose row reaches e beyond its own load term: e kept, or e a threshold
            # (Switch: every row, through the full softmax)
            touch = (r.ids == e).any(axis=1) | self.switch
            if self.dload is not None:
                touch |= self.order[:, k - 1] == e
                if k < E:
                    touch |= self.order[:, k] == e
            rows = np.nonzero(touch)[0]
            dcl = np.zeros(T)
            dsd = np.zeros(T)
            if rows.size:
                c, s = self.row_grads(rows)
                dcl[rows], dsd[rows] = c[:, e], s[:, e]
            if self.dload is not None:  # the load term of e on every other row
                rest = np.setdiff1d(np.arange(T), rows)  # e is not kept there: thr = v_k
                thr = r.row_stats[rest, 0]
                clean, std = r.clean[rest, e], r.std[rest, e]
                ok = (std > 0) & np.isfinite(thr)
                with np.errstate(invalid="ignore", divide="ignore"):
                    z = np.where(ok, (clean - thr) / std, 0.0)
                    cc = np.where(ok, self.dload[e] * _phi(z) / std, 0.0)
                dcl[rest] += cc
                dsd[rest] -= cc * z
            gw.append(X64.T @ dcl)
            bw.append(dcl.sum())
            if self.noisy:
                raw = X64 @ O.widen(self.inp["Wnoise"][:, e])
                nw.append(X64.T @ (dsd / (1.0 + np.exp(-raw))))
        return (np.stack(gw, axis=1), np.stack(nw, axis=1) if self.noisy else None,
                np.array(bw))
