"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of the oracle's source (a
dropped term, a wrong sign or index, a swapped operand, an off-by-one) and
requires that at least one pin in test_oracle_pins fails on the mutant. The
real oracle is untouched: the mutant is a separate module object and the pins
see it only through a monkeypatched attribute table for the duration of one
case.
"""
import os
import sys
import types

import pytest

import oracle.moe as O
import oracle.philox as PH
import test_oracle_pins as pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    ("moe", "softplus -> relu",
     "np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))", "np.maximum(z, 0.0)"),
    ("moe", "noise not scaled by std",
     "score = clean + widen(eps) * std", "score = clean + widen(eps)"),
    ("moe", "ties to the higher index",
     'return np.argsort(-key, axis=1, kind="stable")',
     'return np.argsort(key, axis=1, kind="stable")[:, ::-1]'),
    ("moe", "gate softmax over all experts",
     "gates = z / z.sum(axis=1, keepdims=True)",
     "gates = z / np.exp(score - kept.max(axis=1, keepdims=True)).sum(axis=1, keepdims=True)"),
    ("moe", "Switch gate renormalised to one",
     "gates = p[rows, ids]", "gates = p[rows, ids] / p[rows, ids]"),
    ("moe", "rank-major slot order",
     "    for t in range(T):\n        for j in range(k):\n            e = int(ids[t, j])",
     "    for j in range(k):\n        for t in range(T):\n            e = int(ids[t, j])"),
    ("moe", "capacity test off by one", "accepted = pos < C", "accepted = pos <= C"),
    ("moe", "capacity ignores k", "float(k) * float(T)", "float(T)"),
    ("moe", "CV with ddof 1",
     "((v - m) ** 2).mean() / (m * m)", "((v - m) ** 2).sum() / (v.size - 1) / (m * m)"),
    ("moe", "load threshold swapped",
     "thr = np.where(inside, r.row_stats[:, 1:2], thr)",
     "thr = np.where(inside, r.row_stats[:, :1], thr)"),
    ("moe", "residual dropped",
     "y = x.copy() if residual else np.zeros(D)", "y = np.zeros(D)"),
    ("moe", "expert ReLU dropped",
     "h = np.maximum(x64 @ W1e64, 0.0)", "h = x64 @ W1e64"),
    ("moe", "dropped assignments combined", "if d.accepted[t, j]:", "if True:"),
    ("moe", "importance counts instead of gates",
     "np.add.at(imp, r.ids.ravel(), r.gates.ravel())", "np.add.at(imp, r.ids.ravel(), 1.0)"),
    ("moe", "Switch f after capacity",
     "f = d.counts.astype(np.float64) / T",
     "f = np.minimum(d.counts, d.C).astype(np.float64) / T"),
    ("moe", "load uses H instead of clean",
     "diff = r.clean - thr", "diff = r.score - thr"),
    ("moe", "bf16 widened with a 15-bit shift", "<< np.uint32(16)", "<< np.uint32(15)"),
    ("moe", "bf16 patterns read as IEEE half",
     "return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)",
     "return a.view(np.float16).astype(np.float64)"),
    ("moe", "near-tie always flagged", "near_tie=gap < NEAR_TIE", "near_tie=gap == gap"),
    ("moe", "near-tie never flagged", "near_tie=gap < NEAR_TIE", "near_tie=gap < 0"),
    ("moe", "near-tie gap one place early", "gap = (s64[:, k - 1] - s64[:, k])",
     "gap = (s64[:, k - 2] - s64[:, k - 1])"),
    ("moe", "near-tie gap one place late", "gap = (s64[:, k - 1] - s64[:, k])",
     "gap = (s64[:, k] - s64[:, k + 1 if k + 1 < E else k])"),
    ("moe", "near-tie gap on the clean logits", "s64 = -np.sort(-score, axis=1)",
     "s64 = -np.sort(-clean, axis=1)"),
    ("moe", "near-tie flagged at k = E", "np.full(T, np.inf)", "np.zeros(T)"),
    ("philox", "wrong multiplier",
     "0xD2E7470EE14C6C93", "0xD2E7470EE14C6C95"),
    ("philox", "key not bumped", "k0 = k0 + _W0", "k0 = k0"),
    ("philox", "Box-Muller without sqrt",
     "rho = np.sqrt(-2.0 * np.log(u1))", "rho = -2.0 * np.log(u1)"),
    ("philox", "sine branch reused as cosine",
     "return rho * np.cos(theta), rho * np.sin(theta)",
     "return rho * np.cos(theta), rho * np.cos(theta)"),
]


def _mutant(modname, old, new):
    path = os.path.join(ROOT, "oracle", modname + ".py")
    src = open(path).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new)
    mod = types.ModuleType("oracle." + modname + "_mutant")
    mod.__package__ = "oracle"
    mod.__file__ = path
    sys.modules[mod.__name__] = mod  # dataclasses look their module up here
    try:
        exec(compile(src, path, "exec"), mod.__dict__)
    finally:
        sys.modules.pop(mod.__name__, None)
    return mod


# the whole-workload check takes tens of seconds; every mutation it could catch is caught by
# the near-tie pins first
PIN_TESTS = [getattr(pins, n) for n in dir(pins)
             if n.startswith("test_") and n != "test_fp32_decision_equals_fp64_order_outside_the_margin"]


def _run_pins():
    failed = []
    for fn in PIN_TESTS:
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        cases = [()]
        if params:
            names, values = params[0].args
            cases = [v if isinstance(v, tuple) else (v,) for v in values]
        for c in cases:
            try:
                fn(*c)
            except Exception:
                failed.append(fn.__name__)
                return failed
    return failed


@pytest.mark.parametrize("modname,label,old,new", MUTATIONS, ids=[m[1] for m in MUTATIONS])
def test_pins_catch_mutation(monkeypatch, modname, label, old, new):
    mut = _mutant(modname, old, new)
    if modname == "philox":
        for name in ("philox4x64_10", "gaussian_noise", "_box_muller", "_mulhilo"):
            monkeypatch.setattr(PH, name, getattr(mut, name))
        monkeypatch.setattr(O, "gaussian_noise", mut.gaussian_noise)
    else:
        for name, val in vars(mut).items():
            if callable(val) and getattr(val, "__module__", None) == mut.__name__ or \
                    isinstance(val, types.FunctionType):
                if hasattr(O, name):
                    monkeypatch.setattr(O, name, val)
    assert _run_pins(), f"no pin failed for mutation: {label}"


# ------------------------------------------------------------ hierarchical oracle

import oracle.hier as HO  # noqa: E402
import test_oracle_hier as hier_pins  # noqa: E402

HIER_MUTATIONS = [
    ("slot ignored in the final layout", "ids[tok, slot * ks + j] = i * b + r.ids[:, j]",
     "ids[tok, j] = i * b + r.ids[:, j]"),
    ("final gate without the primary factor",
     "gates[tok, slot * ks + j] = p.gates[tok, slot] * r.gates[:, j]",
     "gates[tok, slot * ks + j] = r.gates[:, j]"),
    ("secondary noise on the primary key", "key1=1 + i, tokens=tok", "key1=0, tokens=tok"),
    ("secondary noise key off by one", "key1=1 + i, tokens=tok", "key1=i, tokens=tok"),
    ("Load_H without the primary load", "load[i * b:(i + 1) * b] = lp[i] * ls / n",
     "load[i * b:(i + 1) * b] = ls / n"),
    ("Load_H not divided by |X^(i)|", "load[i * b:(i + 1) * b] = lp[i] * ls / n",
     "load[i * b:(i + 1) * b] = lp[i] * ls"),
    ("X^(i) from the first primary slot only", "tok = np.nonzero((p.ids == i).any(axis=1))[0]",
     "tok = np.nonzero((p.ids[:, :1] == i).any(axis=1))[0]"),
    ("expert id group-minor", "i * b + r.ids[:, j]", "r.ids[:, j] * a + i"),
    ("secondary keeps k_p experts", "None, None, ks, \"noisy\"", "None, None, kp, \"noisy\""),
]

HIER_PIN_TESTS = [getattr(hier_pins, n) for n in dir(hier_pins) if n.startswith("test_")]


@pytest.mark.parametrize("label,old,new", HIER_MUTATIONS, ids=[m[0] for m in HIER_MUTATIONS])
def test_hier_pins_catch_mutation(monkeypatch, label, old, new):
    mut = _mutant("hier", old, new)
    for name, val in vars(mut).items():
        if isinstance(val, types.FunctionType) and hasattr(HO, name):
            monkeypatch.setattr(HO, name, val)
    failed = []
    for fn in HIER_PIN_TESTS:
        try:
            fn()
        except Exception:
            failed.append(fn.__name__)
            break
    assert failed, f"no hierarchical pin failed for mutation: {label}"


# ------------------------------------------------------------ batchwise-mask oracle

import oracle.batchwise as BWO  # noqa: E402
import test_oracle_batchwise as bw_pins  # noqa: E402

BW_MUTATIONS = [
    ("ties to the higher token", 'order = np.argsort(-key[:, i], kind="stable")',
     'order = np.argsort(key[:, i], kind="stable")[::-1]'),
    ("gate not renormalised", "gates = np.where(den > 0, num / den, 0.0)",
     "gates = np.where(den > 0, num, 0.0)"),
    ("mask ranks the logits", "key = probs.astype(np.float32)", "key = clean.astype(np.float32)"),
    ("m rounded up", "return (k * T) // E", "return -(-k * T // E)"),
    ("loss sign swapped", "(((s > thr).astype(np.float64) - r.mask) * (s - thr))",
     "((r.mask - (s > thr).astype(np.float64)) * (s - thr))"),
    ("residual dropped", "y = x.copy() if residual else np.zeros(D)", "y = np.zeros(D)"),
    ("softmax over kept only", "probs = z / z.sum(axis=1, keepdims=True)", "probs = z"),
    ("near-tie margin never flagged", "near[i] = abs(a - b) < NEAR_TIE_REL * abs(a)",
     "near[i] = False"),
    ("near-tie margin absolute", "near[i] = abs(a - b) < NEAR_TIE_REL * abs(a)",
     "near[i] = abs(a - b) < NEAR_TIE_REL"),
    ("exact tie always a near-tie",
     "near[i] = bool(gaps) and min(gaps) < NEAR_TIE_REL * abs(a)", "near[i] = True"),
    ("exact tie never a near-tie",
     "near[i] = bool(gaps) and min(gaps) < NEAR_TIE_REL * abs(a)", "near[i] = False"),
]

BW_PIN_TESTS = [getattr(bw_pins, n) for n in dir(bw_pins) if n.startswith("test_")]


@pytest.mark.parametrize("label,old,new", BW_MUTATIONS, ids=[m[0] for m in BW_MUTATIONS])
def test_batchwise_pins_catch_mutation(monkeypatch, label, old, new):
    mut = _mutant("batchwise", old, new)
    for name, val in vars(mut).items():
        if isinstance(val, types.FunctionType) and hasattr(BWO, name):
            monkeypatch.setattr(BWO, name, val)
    failed = []
    for fn in BW_PIN_TESTS:
        try:
            fn()
        except Exception:
            failed.append(fn.__name__)
            break
    assert failed, f"no batchwise pin failed for mutation: {label}"


# ------------------------------------------------------------ backward oracle

import oracle.backward as OBW  # noqa: E402
import test_oracle_backward as bwd_pins  # noqa: E402

BWD_MUTATIONS = [
    ("load threshold detached", "thr = torch.where(inside, vk1[:, None], vk[:, None])",
     "thr = torch.where(inside, vk1[:, None], vk[:, None]).detach()"),
    ("noise scale detached", "H = clean + torch.from_numpy(O.widen(eps)) * std",
     "H = clean + torch.from_numpy(O.widen(eps)) * std.detach()"),
    ("dropped assignments contribute", "tt, jj = np.nonzero((r.ids == e) & d.accepted)",
     "tt, jj = np.nonzero(r.ids == e)"),
    ("gate detached", "G = torch.softmax(torch.gather(H, 1, ids), dim=1)",
     "G = torch.softmax(torch.gather(H, 1, ids).detach(), dim=1)"),
    ("Switch gate renormalised over the kept expert", "G = torch.gather(probs, 1, ids)",
     "G = torch.softmax(torch.gather(clean, 1, ids), dim=1)"),
    ("Switch fractions differentiable", "f = torch.from_numpy(d.counts.astype(np.float64) / T)",
     "f = probs.mean(dim=0)"),
    ("sampled Switch Jacobian sign", "return p * (dp - (p * dp).sum(axis=1, keepdims=True)), np.zeros((n, E))",
     "return p * (dp + (p * dp).sum(axis=1, keepdims=True)), np.zeros((n, E))"),
    ("sampled threshold share to the wrong expert", "dcl[np.arange(n), ik] -= s_out",
     "dcl[np.arange(n), ik] -= s_in"),
    ("sampled d softplus", "return 1.0 / (1.0 + np.exp(-raw))", "return 1.0 / (1.0 + np.exp(raw))"),
    ("residual dropped", "Y = X * 1.0 if residual else torch.zeros_like(X)",
     "Y = torch.zeros_like(X)"),
    ("CV with ddof 1", "return ((v - m) ** 2).mean() / (m * m)",
     "return ((v - m) ** 2).sum() / (v.numel() - 1) / (m * m)"),
]

BWD_PIN_TESTS = [getattr(bwd_pins, n) for n in dir(bwd_pins) if n.startswith("test_")]


@pytest.mark.parametrize("label,old,new", BWD_MUTATIONS, ids=[m[0] for m in BWD_MUTATIONS])
def test_backward_pins_catch_mutation(monkeypatch, label, old, new):
    mut = _mutant("backward", old, new)
    for name, val in vars(mut).items():
        if isinstance(val, (types.FunctionType, type)) and hasattr(OBW, name) and \
                getattr(val, "__module__", None) == mut.__name__:
            monkeypatch.setattr(OBW, name, val)
    failed = []
    for fn in BWD_PIN_TESTS:
        marks = getattr(fn, "pytestmark", [])
        params = [m_ for m_ in marks if m_.name == "parametrize"]
        cases = [()]
        if params:
            cases = [v if isinstance(v, tuple) else (v,) for v in params[0].args[1]]
        try:
            for c in cases:
                fn(*c)
        except Exception:
            failed.append(fn.__name__)
            break
    assert failed, f"no backward pin failed for mutation: {label}"
