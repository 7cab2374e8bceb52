"""Pins for the batchwise-mask oracle (CPU only): the defining property of the
mask (every expert keeps exactly m tokens, none outscored by a token it left
out, ties to the lower token), the renormalised gate, hand-computed masks and
batchwise-loss values, a token no expert kept, the one-expert case and a case
where the mask equals the per-token top-1.

Passages: "Outrageously Large Neural Networks" summary, section 3.4, "Strictly
Balanced Gating"; the "Mixture-of-Experts: Sparse Computation" lesson, chapter 4,
"A stricter alternative", and chapter 2's mask-and-renormalise form.
"""
import numpy as np
import pytest
import torch

from oracle import batchwise as BO
from oracle import moe as O
from sparsely_gated_mixture_amd import inputs as I


def _wl(T=64, D=8, E=8, k=2, H=6, seed=4, dup=0.0):
    return I.Workload("bw_pin", T=T, D=D, E=E, k=k, H=H, act="f32", gating="batchwise",
                      noise=False, capacity_factor=0.0, seed=seed, dup_frac=dup)


def _route_logits(L, k):
    """Route with the given logits as X . Wg (Wg = identity)."""
    L = np.asarray(L, dtype=np.float64)
    return BO.route_batchwise(L, np.eye(L.shape[1]), None, k)


def test_every_expert_keeps_m_and_none_is_outscored():
    w = _wl(T=96, E=12, k=3)
    inp = I.make_inputs(w, experts=False)
    r = BO.route_batchwise(inp["X"], inp["Wg"], None, w.k)
    assert r.m == 96 * 3 // 12
    assert (r.mask.sum(axis=0) == r.m).all() and r.mask.sum() == 12 * r.m
    key = r.probs.astype(np.float32)
    for i in range(12):
        kept = np.nonzero(r.mask[:, i])[0]
        np.testing.assert_array_equal(r.sel[i], kept)  # ascending token order
        out = np.nonzero(~r.mask[:, i])[0]
        assert key[kept, i].min() >= key[out, i].max()


def test_ties_go_to_the_lower_token():
    """Three identical rows (1, 0) and one (0, 1), m = 2: expert 0 keeps tokens 0 and 1 of
    the three tied ones; expert 1 keeps token 3 and the lowest of the tied tokens, 0."""
    r = _route_logits([[1.0, 0.0], [1.0, 0.0], [1.0, 0.0], [0.0, 1.0]], k=1)
    assert r.m == 2
    assert r.sel.tolist() == [[0, 1], [0, 3]]


def test_gate_is_the_renormalised_dense_softmax():
    w = _wl()
    inp = I.make_inputs(w, experts=False)
    r = BO.route_batchwise(inp["X"], inp["Wg"], None, w.k)
    P = torch.softmax(torch.from_numpy(inp["X"].astype(np.float64) @ inp["Wg"].astype(np.float64)),
                      dim=1).numpy()
    for t in range(w.T):
        S = np.nonzero(r.mask[t])[0]
        if S.size == 0:
            assert (r.gates[t] == 0).all()
            continue
        np.testing.assert_allclose(r.gates[t, S], P[t, S] / P[t, S].sum(), rtol=1e-12)
        assert (r.gates[t, ~r.mask[t]] == 0).all()


def test_ranks_by_the_softmax_score_not_the_logit():
    """Token 0 has logits (2, 0) -> p = (0.881, 0.119); token 1 has (3, 3) -> (0.5, 0.5).
    Ranked by the dense softmax, expert 0 keeps token 0 and expert 1 keeps token 1 (ranked
    by logits, expert 0 would keep token 1 and token 0 would get nothing)."""
    r = _route_logits([[2.0, 0.0], [3.0, 3.0]], k=1)
    assert r.m == 1
    assert r.sel.tolist() == [[0], [1]]
    np.testing.assert_allclose(r.gates, [[1.0, 0.0], [0.0, 1.0]])


def test_hand_computed_mask_and_batchwise_loss():
    """Scores [[0.7, 0.3], [0.4, 0.6]], m = 1: expert 0 keeps token 0, expert 1 keeps
    token 1. Thresholds (0.35, 0.5): only (token 1, expert 0) disagrees, loss
    (1 - 0)(0.4 - 0.35) = 0.05. Thresholds (0.8, 0.2): (0,0) gives (0 - 1)(0.7 - 0.8) = 0.1
    and (0,1) gives (1 - 0)(0.3 - 0.2) = 0.1, loss 0.2."""
    r = _route_logits(np.log([[0.7, 0.3], [0.4, 0.6]]), k=1)
    assert r.mask.tolist() == [[True, False], [False, True]]
    assert BO.batchwise_loss(r, [0.35, 0.5]) == pytest.approx(0.05, abs=1e-12)
    assert BO.batchwise_loss(r, [0.8, 0.2]) == pytest.approx(0.2, abs=1e-12)
    assert BO.batchwise_loss(r, [0.65, 0.45]) == pytest.approx(0.0, abs=1e-12)


def test_token_kept_by_no_expert_and_one_kept_twice():
    """m = 1 over three tokens: expert 0 and expert 1 both keep token 0, expert 2 keeps
    token 2; token 1 gets no expert (gate 0, output = residual) and token 0's gates are
    0.5 / 0.95 and 0.45 / 0.95."""
    P = np.array([[0.5, 0.45, 0.05], [0.3, 0.3, 0.4], [0.2, 0.25, 0.55]])
    r = _route_logits(np.log(P), k=1)
    assert r.sel.tolist() == [[0], [0], [2]]
    np.testing.assert_allclose(r.gates[0], [0.5 / 0.95, 0.45 / 0.95, 0.0], rtol=1e-12)
    assert (r.gates[1] == 0).all()
    np.testing.assert_allclose(r.gates[2], [0.0, 0.0, 1.0])
    rng = np.random.default_rng(0)
    X = rng.standard_normal((3, 3)).astype(np.float32)
    W1 = rng.standard_normal((3, 3, 4)).astype(np.float32)
    W2 = rng.standard_normal((3, 4, 3)).astype(np.float32)
    Y = BO.combine_tokens(X, r, O.ExpertBank(W1, W2), [0, 1, 2])
    np.testing.assert_array_equal(Y[1], X[1].astype(np.float64))
    out = BO.aux_batchwise(r)["out"]
    assert out[3] == 2 and out[4] == 1 and out[2] == pytest.approx(1.0)


def test_one_expert_keeps_every_token():
    """E = 1, k = 1: m = T, every token kept with gate 1, Y = X + ReLU(X W1) W2 (torch fp64)."""
    w = _wl(T=20, D=5, E=1, k=1, H=7)
    inp = I.make_inputs(w)
    f = BO.forward_batchwise(inp, w)
    r = f["routing"]
    assert r.m == 20 and r.mask.all()
    np.testing.assert_allclose(r.gates, 1.0)
    X = torch.from_numpy(inp["X"].astype(np.float64))
    ref = X + torch.relu(X @ torch.from_numpy(inp["W1"][0].astype(np.float64))) @ \
        torch.from_numpy(inp["W2"][0].astype(np.float64))
    np.testing.assert_allclose(f["Y"], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_clustered_scores_give_the_top1_layer():
    """Tokens in E clusters of m, each cluster strongly preferring its own expert: the
    batchwise mask is then the per-token top-1 mask, so the layer equals the flat top-1
    layer without capacity."""
    E, m, D, H = 4, 5, 4, 6
    T = E * m
    rng = np.random.default_rng(3)
    X = (6.0 * np.repeat(np.eye(E), m, axis=0) + 0.1 * rng.standard_normal((T, D))).astype(np.float32)
    Wg = np.eye(E, dtype=np.float32)
    W1 = rng.standard_normal((E, D, H)).astype(np.float32)
    W2 = rng.standard_normal((E, H, D)).astype(np.float32)
    r = BO.route_batchwise(X, Wg, None, 1)
    flat = O.route(X, Wg, None, None, 1, "noisy", False)
    dense = np.zeros((T, E), dtype=bool)
    dense[np.arange(T), flat.ids[:, 0]] = True
    np.testing.assert_array_equal(r.mask, dense)
    d = O.dispatch(flat.ids, E, T)
    bank = O.ExpertBank(W1, W2)
    np.testing.assert_allclose(BO.combine_tokens(X, r, bank, np.arange(T)),
                               O.combine_tokens(X, flat, d, bank, np.arange(T)), rtol=1e-12)


def test_importance_sums_to_tokens_with_an_expert():
    w = _wl(T=80, E=10, k=2)
    inp = I.make_inputs(w, experts=False)
    r = BO.route_batchwise(inp["X"], inp["Wg"], None, w.k)
    a = BO.aux_batchwise(r)
    n_with = (r.mask.sum(axis=1) > 0).sum()
    assert a["importance"].sum() == pytest.approx(n_with, rel=1e-12)
    assert a["out"][2] == pytest.approx(10 * r.m / 80)


def test_m_is_rounded_down():
    """k T / E = 2.5 keeps m = 2 tokens per expert (8 of the 10 token slots)."""
    w = _wl(T=10, E=4, k=1)
    inp = I.make_inputs(w, experts=False)
    r = BO.route_batchwise(inp["X"], inp["Wg"], None, 1)
    assert r.m == 2 and r.mask.sum() == 8
    with pytest.raises(ValueError):
        BO.route_batchwise(inp["X"][:3], inp["Wg"], None, 1)  # k T < E: no token per expert


def _route_two_experts(a, k=1):
    """Two experts with logits (a_t, 0): expert 0 scores sigmoid(a_t), expert 1 sigmoid(-a_t)."""
    X = np.asarray(a, dtype=np.float64)[:, None]
    return BO.route_batchwise(X, np.array([[1.0, 0.0]]), None, k)


def test_near_tie_margin_is_relative_to_the_mth_score():
    """Near-tie reading: the m-th and (m+1)-th scores of an expert closer than 2e-6 of the m-th
    score (relative). Four tokens, k = 1, E = 2, so m = 2."""
    r = _route_two_experts([1.0, 0.5, 0.5 - 2e-6, -1.0])  # 4.7e-7 apart at 0.62 and 0.38
    assert r.m == 2 and r.near_tie.tolist() == [True, True]
    r = _route_two_experts([1.0, 0.5, 0.4, -1.0])
    assert r.near_tie.tolist() == [False, False]
    # 5e-7 apart at scores near 0.05 (relative 1e-5: not near) and near 0.95 (5e-7: near)
    r = _route_two_experts([-2.0, -2.944, -2.944 - 1.05e-5, -4.0])
    assert r.near_tie.tolist() == [False, True]


def test_exact_tie_is_decided_by_the_token_index():
    """Identical rows tie exactly: the lower token is kept and the expert is no near-tie, unless a
    distinct score lies within the margin of the tied value."""
    r = _route_two_experts([1.0, 0.5, 0.5, -1.0])
    assert r.sel.tolist() == [[0, 1], [1, 3]]
    assert r.near_tie.tolist() == [False, False]
    r = _route_two_experts([0.5 + 2e-6, 0.5, 0.5, -1.0])
    assert r.sel.tolist() == [[0, 1], [1, 3]]
    assert r.near_tie.tolist() == [True, True]
