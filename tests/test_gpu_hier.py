"""GPU parity of the hierarchical MoE (two-level gating) against the CPU oracle:
both gate levels, the grouping of the secondary rows, the final assignments and
product gates, the whole forward (flat dispatch / FFN / combine on the final
assignments) and Importance_H / Load_H.

Decisions inside the 1e-6 near-tie margin (at either level) are reported, not
counted, as for the flat layer.
"""
import numpy as np
import pytest

from gpu_helpers import TOL, dev, host, log, problem_for, rel_err, set_mismatch
from oracle import hier as HO
from oracle import moe as O
from sparsely_gated_mixture_amd import inputs as I
from test_gpu_forward import _check_forward

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def moe():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    from sparsely_gated_mixture_amd import moe as m
    return m


def _w(name, T, D, a, b, kp, ks, H, act, noise, cf, seed):
    return I.Workload(name, T=T, D=D, E=a * b, k=kp * ks, H=H, act=act, gating="noisy",
                      noise=noise, capacity_factor=cf, seed=seed, groups=a, k_primary=kp)


SMALL = [
    _w("h_f32", 300, 40, 4, 6, 2, 2, 32, "f32", True, 0.0, 21),
    _w("h_bf16_cap", 257, 72, 5, 12, 1, 2, 48, "bf16", True, 1.0, 22),
    _w("h_nonoise", 128, 32, 4, 4, 2, 2, 16, "f32", False, 0.0, 23),
    _w("h_kp_eq_a", 100, 24, 3, 3, 3, 1, 16, "bf16", True, 0.0, 24),
    _w("h_wide", 160, 64, 8, 40, 2, 3, 32, "bf16", True, 0.0, 25),
]


def _layer(moe, w, inp):
    p = problem_for(moe, w)
    h = moe.hier(w.groups, w.k_primary)
    return moe.HierLayer(p, h, dev(inp["Wpg"]), dev(inp["Wpn"]) if w.noise else None,
                         dev(inp["Wsg"]), dev(inp["Wsn"]) if w.noise else None,
                         dev(inp["W1"]), dev(inp["W2"]))


def _check_levels(w, hr, st):
    """Primary gate, grouping and secondary gate rows against the oracle."""
    p = hr.primary
    a, kp = w.groups, w.k_primary
    b, ks = w.E // a, w.k // kp
    assert rel_err(host(st["clean_p"]), p.clean) < 1e-5
    if w.noise:
        assert rel_err(host(st["std_p"]), p.std) < 1e-5
    bad_p = set_mismatch(host(st["ids_p"]), p.ids)
    log(f"  primary near-ties {int(p.near_tie.sum())}, flipped {bad_p.size}")
    assert p.near_tie[bad_p].all()
    if bad_p.size:
        return bad_p  # the grouping differs from the oracle's; the final check still runs
    counts = np.array([m.size for m in hr.members])
    np.testing.assert_array_equal(host(st["counts_p"]), counts)
    offs = np.concatenate([[0], np.cumsum(counts)])
    np.testing.assert_array_equal(host(st["offsets_p"]), offs)
    np.testing.assert_array_equal(host(st["row_token_p"]), np.concatenate(hr.members))
    np.testing.assert_array_equal(host(st["accepted_p"]), 1)
    cs, ss, ids_s = host(st["clean_s"]), host(st["std_s"]) if w.noise else None, host(st["ids_s"])
    for i in range(a):
        r = hr.secondary[i]
        if r is None:
            continue
        rows = slice(offs[i], offs[i + 1])
        assert rel_err(cs[rows], r.clean) < 1e-5
        if w.noise:
            assert rel_err(ss[rows], r.std) < 1e-5
        flipped = set_mismatch(ids_s[rows], r.ids)
        assert r.near_tie[flipped].all()
    return bad_p


def _check_aux(w, f, Lb, hr_bad):
    if hr_bad.size:
        return
    ax = f["aux"]
    assert rel_err(host(Lb.importance), ax["importance"]) < TOL["f32"]
    if w.noise:
        assert rel_err(host(Lb.load), ax["load"]) < TOL["f32"]
    o = host(Lb.aux_out).astype(np.float64)
    for i in range(8):
        assert abs(o[i] - ax["out"][i]) <= 1e-4 * max(abs(ax["out"][i]), 1e-2), (i, o[i], ax["out"][i])


def _run(moe, w, inp, full_y):
    import torch
    f = HO.forward_hier(inp, w, tokens=np.arange(0))  # Y: _check_forward, expert by expert
    hr, r, d = f["hier"], f["routing"], f["dispatch"]
    L = _layer(moe, w, inp)
    Lb = L.forward(dev(inp["X"]))
    torch.cuda.synchronize()
    bad_p = _check_levels(w, hr, L.st)
    _check_forward(moe, w, inp, r, d, Lb, full_y=full_y, flat_aux=False)
    bad = set_mismatch(host(Lb.ids), hr.ids)
    _check_aux(w, f, Lb, np.union1d(bad_p, bad))


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_hier_small(moe, w):
    log(f"[hier] {w}")
    _run(moe, w, I.make_inputs(w), full_y=True)


def test_hier_bf16_full_size(moe):
    """The measured hierarchical workload (16 groups of 64 experts, 2 + 2 choices) at full
    size: both levels, grouping, final assignments, aux; Y on every token."""
    w = I.WORKLOADS["hier_bf16"]
    log(f"[hier full] {w}")
    _run(moe, w, I.make_inputs(w), full_y=True)


def test_hier_empty_group(moe):
    """Many groups, few tokens, k_p = 1: some groups receive no token (|X^(i)| = 0); their
    Load_H is 0 and they are counted in out[5]."""
    import torch
    w = _w("h_empty", 6, 16, 16, 4, 1, 2, 8, "f32", True, 0.0, 26)
    inp = I.make_inputs(w)
    f = HO.forward_hier(inp, w)
    assert f["aux"]["out"][5] > 0
    L = _layer(moe, w, inp)
    Lb = L.forward(dev(inp["X"]))
    torch.cuda.synchronize()
    bad = set_mismatch(host(Lb.ids), f["hier"].ids)
    assert f["hier"].near_tie[bad].all()
    _check_aux(w, f, Lb, bad)
    assert host(Lb.aux_out)[5] == f["aux"]["out"][5]
