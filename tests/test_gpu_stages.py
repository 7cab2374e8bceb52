"""GPU parity of each C-ABI stage against the CPU oracle, at every workload's
full size. Each stage gets the oracle's inputs (never GPU results fed to the
oracle), so a stage is judged alone:

  route     X, weights            -> ids (bit-exact as sets outside 1e-6 near-ties), gates,
                                     clean, std, row_stats (fp32 tolerance)
  dispatch  oracle ids            -> pos, accepted, counts, offsets, row_token, Xd (bit-exact)
  ffn       oracle rows / offsets -> Z (dtype tolerance; sampled rows at the large sizes)
  combine   oracle routing + Z    -> Y (dtype tolerance), dropped tokens Y == X bit-exact
  aux       oracle routing        -> importance, load, scalars (fp32 tolerance)
"""
import math

import numpy as np
import pytest

from gpu_helpers import (TOL, dev, f64, gates_by_id, host, log, max_abs, oracle_expert_outputs,
                         oracle_routing, problem_for, rel_err, sample_tokens, set_mismatch,
                         workload_inputs)
from oracle import moe as O
from sparsely_gated_mixture_amd import inputs as I

pytestmark = pytest.mark.gpu

ALL = I.WORKLOAD_ORDER


@pytest.fixture(scope="module")
def moe():
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    from sparsely_gated_mixture_amd import moe as m
    return m


def _route_gpu(moe, w, inp, eps=None):
    import torch
    p = problem_for(moe, w)
    noisy = w.gating == "noisy" and w.noise
    ids = torch.empty(w.T, w.k, dtype=torch.int32, device="cuda")
    gates = torch.empty(w.T, w.k, device="cuda")
    clean = torch.empty(w.T, w.E, device="cuda")
    std = torch.empty(w.T, w.E, device="cuda") if noisy else None
    rs = torch.empty(w.T, 2, device="cuda")
    ws = torch.empty(moe.moe_workspace_size(p, moe.MOE_WS_ROUTE), dtype=torch.uint8, device="cuda")
    moe.moe_route(p, dev(inp["X"]), dev(inp["Wg"]), dev(inp["Wnoise"]) if noisy else None,
                  dev(inp["bias"]), dev(eps), ids, gates, clean, std, rs, ws)
    return dict(ids=host(ids), gates=host(gates), clean=host(clean),
                std=host(std) if noisy else None, row_stats=host(rs))


@pytest.mark.parametrize("name", ALL)
def test_route(moe, name):
    log(f"[route] {name}")
    w, inp = workload_inputs(name)
    r, _ = oracle_routing(name)
    _check_route(w, r, _route_gpu(moe, w, inp))


# token counts that select the router's 64-row tiles (T = 40000, 96 experts) and its widest
# selection rows (E = 300 with few tokens: 16 lanes per row)
ROUTE_SHAPES = [
    I.Workload("bm64", T=40000, D=64, E=96, k=2, H=16, act="bf16", gating="noisy", noise=True,
               capacity_factor=0.0, seed=14),
    I.Workload("lpr16", T=96, D=48, E=300, k=3, H=16, act="f32", gating="noisy", noise=True,
               capacity_factor=0.0, seed=15),
    I.Workload("sw64", T=40000, D=40, E=24, k=1, H=16, act="bf16", gating="switch", noise=False,
               capacity_factor=1.0, seed=16),
    # 128-row tiles (at least 512 blocks: the router's 8-wave form, noise waves beside the
    # MFMA waves): 128 experts with a router bias and a ragged last tile (512 tiles + 77 rows);
    # 202 experts (a partial 4-expert group and a partial 32-expert block, k = 3, half a last
    # tile); fp32 X over 64 experts; 256 experts without noise (the 4-wave form); 256 experts
    # with noise, k = 1 and D = 128 (two k-stages: the noise waves draw several groups a stage);
    # 256 experts with noise at D = 96 (the 8-wave form with a k tail: no whole 64-deep stages)
    I.Workload("lists_e128", T=65613, D=512, E=128, k=3, H=16, act="bf16", gating="noisy",
               noise=True, capacity_factor=0.0, seed=17, zipf_bias=1.1),
    I.Workload("lists_e202", T=65600, D=64, E=202, k=3, H=16, act="bf16", gating="noisy",
               noise=True, capacity_factor=0.0, seed=20),
    I.Workload("lists_f32", T=65536, D=96, E=64, k=2, H=16, act="f32", gating="noisy",
               noise=True, capacity_factor=0.0, seed=21),
    I.Workload("fused_clean", T=32768, D=192, E=256, k=2, H=16, act="bf16", gating="noisy",
               noise=False, capacity_factor=0.0, seed=18),
    I.Workload("fused_top1", T=33000, D=128, E=256, k=1, H=16, act="bf16", gating="noisy",
               noise=True, capacity_factor=0.0, seed=19),
    I.Workload("tail_d96", T=65536, D=96, E=256, k=2, H=16, act="bf16", gating="noisy",
               noise=True, capacity_factor=0.0, seed=22),
]


@pytest.mark.parametrize("w", ROUTE_SHAPES, ids=[w.name for w in ROUTE_SHAPES])
def test_route_tile_shapes(moe, w):
    log(f"[route shape] {w}")
    inp = I.make_inputs(w, experts=False)
    r = O.route(inp["X"], inp["Wg"], inp["Wnoise"], inp["bias"], w.k, w.gating, w.noise,
                seed=w.seed)
    _check_route(w, r, _route_gpu(moe, w, inp))


def test_route_external_noise_full_size(moe):
    """top2_bf16's shape with the noise given by the caller: the scores use it exactly (the
    oracle given the same noise)."""
    w, inp = workload_inputs("top2_bf16")
    eps = np.random.default_rng(5).standard_normal((w.T, w.E)).astype(np.float32)
    r = O.route(inp["X"], inp["Wg"], inp["Wnoise"], inp["bias"], w.k, w.gating, w.noise,
                seed=w.seed, eps=eps)
    _check_route(w, r, _route_gpu(moe, w, inp, eps=eps))


def _check_route(w, r, g):
    assert rel_err(g["clean"], r.clean) < 1e-5
    if r.std is not None:
        assert rel_err(g["std"], r.std) < 1e-5
    bad = set_mismatch(g["ids"], r.ids)
    log(f"  near-ties {int(r.near_tie.sum())}, id-set mismatches {bad.size}")
    assert r.near_tie[bad].all(), f"id mismatch outside the near-tie margin: tokens {bad[:10]}"
    ok = np.setdiff1d(np.arange(w.T), bad)
    gg = gates_by_id(g["ids"], g["gates"], r.ids, ok)
    assert rel_err(gg, r.gates[ok]) < TOL["f32"]
    # the output order is (score desc, index asc); with no near-tie inside the kept set the
    # order matches exactly
    order_ok = ok[np.all(np.diff(-r.score[ok[:, None], r.ids[ok]], axis=1) > 1e-6, axis=1)] \
        if w.k > 1 else ok
    assert (g["ids"][order_ok] == r.ids[order_ok]).all()
    fin = np.isfinite(r.row_stats[ok])
    assert (np.isfinite(g["row_stats"][ok]) == fin).all()
    assert rel_err(g["row_stats"][ok][fin], r.row_stats[ok][fin]) < TOL["f32"]


def test_route_worked_example(moe):
    """Lesson ch. 2 worked example through the C ABI: D = 1, X = 1, Wg = clean logits,
    Softplus(Wnoise) = 1, external noise [0.3, -0.2, 0.1, -1.5]."""
    from conftest import golden
    gld = golden("lesson_worked_example.json")
    clean = np.array(gld["clean_logits"], np.float32)
    eps = (np.array(gld["noisy_scores"]) - np.array(gld["clean_logits"])).astype(np.float32)
    for case, k in (("k1", 1), ("k2", 2), ("k3", 3)):
        w = I.Workload("lesson", T=1, D=1, E=4, k=k, H=8, act="f32", gating="noisy", noise=True,
                       capacity_factor=0.0, seed=0)
        inp = dict(X=np.ones((1, 1), np.float32), Wg=clean[None, :],
                   Wnoise=np.full((1, 4), math.log(math.e - 1), np.float32), bias=None)
        g = _route_gpu(moe, w, inp, eps=eps[None, :])
        G = np.zeros(4)
        G[g["ids"][0]] = g["gates"][0]
        want = gld["gates"][case]
        np.testing.assert_array_equal(np.round(G, want["decimals"]), want["G"])


def test_route_exact_ties(moe):
    """Duplicated router columns, no noise: exact ties go to the lower index (Switch step 2)."""
    rng = np.random.default_rng(4)
    for gating, k, act in (("switch", 1, "f32"), ("noisy", 2, "bf16"), ("noisy", 3, "f32")):
        w = I.Workload("ties", T=300, D=64, E=40, k=k, H=8, act=act, gating=gating, noise=False,
                       capacity_factor=0.0, seed=0)
        X = rng.standard_normal((w.T, w.D)).astype(np.float32)
        X = I.f32_to_bf16_bits(X) if act == "bf16" else X
        Wg = (rng.standard_normal((w.D, w.E)) / 8).astype(np.float32)
        Wg[:, 7] = Wg[:, 3]
        Wg[:, 30] = Wg[:, 3]
        Wg[:, 12] = Wg[:, 5]
        g = _route_gpu(moe, w, dict(X=X, Wg=Wg, Wnoise=None, bias=None))
        r = O.route(X, Wg, None, None, k, gating, False)
        np.testing.assert_array_equal(np.sort(g["ids"], 1), np.sort(r.ids, 1))
        c = g["clean"]
        assert (c[:, 7] == c[:, 3]).all() and (c[:, 30] == c[:, 3]).all()
        for t in range(w.T):
            s = set(g["ids"][t].tolist())
            if 7 in s or 30 in s:
                assert 3 in s
            if 12 in s:
                assert 5 in s


def test_route_duplicate_rows_identical(moe):
    """top2_bf16: duplicated token rows give bit-identical clean logits and noise scales."""
    w, inp = workload_inputs("top2_bf16")
    g = _route_gpu(moe, w, inp)
    src, dst = I.duplicate_map(w)
    assert (g["clean"][dst] == g["clean"][src]).all()
    assert (g["std"][dst] == g["std"][src]).all()


def test_route_noise_stream(moe):
    """Wg = 0, Softplus(Wnoise) = 1: the scores are the noise itself, so the kept experts and
    gates test the in-kernel Philox / Box-Muller stream against the oracle's."""
    for act in ("f32", "bf16"):
        w = I.Workload("noise", T=2048, D=8, E=64, k=4, H=8, act=act, gating="noisy", noise=True,
                       capacity_factor=0.0, seed=987654321)
        X = np.zeros((w.T, w.D), np.float32)
        X[:, 0] = 1.0
        X = I.f32_to_bf16_bits(X) if act == "bf16" else X
        Wn = np.zeros((w.D, w.E), np.float32)
        Wn[0, :] = math.log(math.e - 1)
        inp = dict(X=X, Wg=np.zeros((w.D, w.E), np.float32), Wnoise=Wn, bias=None)
        g = _route_gpu(moe, w, inp)
        r = O.route(X, inp["Wg"], Wn, None, w.k, "noisy", True, seed=w.seed)
        bad = set_mismatch(g["ids"], r.ids)
        assert r.near_tie[bad].all()
        ok = np.setdiff1d(np.arange(w.T), bad)
        assert rel_err(gates_by_id(g["ids"], g["gates"], r.ids, ok), r.gates[ok]) < 1e-5


@pytest.mark.parametrize("name", ALL)
def test_dispatch(moe, name):
    import torch
    log(f"[dispatch] {name}")
    w, inp = workload_inputs(name)
    r, d = oracle_routing(name)
    p = problem_for(moe, w)
    rows = moe.moe_max_rows(p)
    dt = torch.bfloat16 if w.act == "bf16" else torch.float32
    X = dev(inp["X"])
    pos = torch.full((w.T, w.k), -7, dtype=torch.int32, device="cuda")
    acc = torch.full((w.T, w.k), 9, dtype=torch.uint8, device="cuda")
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(w.E + 1, dtype=torch.int32, device="cuda")
    row_token = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    Xd = torch.zeros(rows, w.D, dtype=dt, device="cuda")
    ws = torch.empty(moe.moe_workspace_size(p, moe.MOE_WS_DISPATCH), dtype=torch.uint8, device="cuda")
    moe.moe_dispatch(p, X, dev(r.ids), pos, acc, counts, offsets, row_token, Xd, ws)
    np.testing.assert_array_equal(host(counts), d.counts)
    np.testing.assert_array_equal(host(offsets), d.offsets)
    np.testing.assert_array_equal(host(pos), d.pos)
    np.testing.assert_array_equal(host(acc).astype(bool), d.accepted)
    A = int(d.offsets[-1])
    np.testing.assert_array_equal(host(row_token)[:A], d.row_token)
    np.testing.assert_array_equal(host(Xd)[:A], inp["X"][d.row_token])
    log(f"  C={d.C} rows={A} dropped={int((~d.accepted).sum())}")


def _ffn_inputs(moe, w, inp, d):
    import torch
    p = problem_for(moe, w)
    rows = moe.moe_max_rows(p)
    dt = torch.bfloat16 if w.act == "bf16" else torch.float32
    A = int(d.offsets[-1])
    Xd_host = np.zeros((rows, w.D), dtype=inp["X"].dtype)
    Xd_host[:A] = inp["X"][d.row_token]
    W1p = torch.empty(moe.moe_packed_weight_bytes(p, 1), dtype=torch.uint8, device="cuda")
    W2p = torch.empty(moe.moe_packed_weight_bytes(p, 2), dtype=torch.uint8, device="cuda")
    moe.moe_pack_expert_weights(p, dev(inp["W1"]), dev(inp["W2"]), W1p, W2p)
    return p, dev(Xd_host), W1p, W2p, dev(d.offsets), rows, dt


@pytest.mark.parametrize("name", ALL)
def test_expert_ffn(moe, name):
    import torch
    log(f"[ffn] {name}")
    w, inp = workload_inputs(name)
    r, d = oracle_routing(name)
    p, Xd, W1p, W2p, offsets, rows, dt = _ffn_inputs(moe, w, inp, d)
    Hd = torch.empty(rows, w.H, dtype=dt, device="cuda")
    Z = torch.full((rows, w.D), float("nan"), dtype=dt, device="cuda")
    moe.moe_expert_ffn(p, Xd, W1p, W2p, offsets, Hd, Z)
    A = int(d.offsets[-1])
    # every accepted row of both layers against the oracle, expert by expert
    Hh, Zh = host(Hd), host(Z)
    st = dict(dh=0.0, rh=0.0, dz=0.0, rz=0.0, n=0)

    def one(e, r0, r1, h, z):
        st["n"] += r1 - r0
        st["dh"] = max(st["dh"], max_abs(Hh[r0:r1], h))
        st["rh"] = max(st["rh"], float(np.abs(h).max()))
        st["dz"] = max(st["dz"], max_abs(Zh[r0:r1], z))
        st["rz"] = max(st["rz"], float(np.abs(z).max()))

    oracle_expert_outputs(name, w, inp, d, on_expert=one)
    eh, ez = st["dh"] / st["rh"], st["dz"] / st["rz"]
    log(f"  all {A} rows: Hd rel err {eh:.2e} (max abs {st['dh']:.2e}), "
        f"Z rel err {ez:.2e} (max abs {st['dz']:.2e})")
    assert st["n"] == A  # every accepted row was compared
    assert eh < TOL[w.act] and ez < TOL[w.act]
    # rows past the accepted ones are untouched
    if A < rows:
        assert np.isnan(f64(Zh[A:])).all()


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_grouped_gemm_ragged(moe, act):
    """Ragged groups (empty experts, groups of 1 row, groups longer than a tile), widths that
    are not multiples of the tile or vector sizes; each layer against numpy fp64."""
    import torch
    rng = np.random.default_rng(11 if act == "f32" else 12)
    for (D, H) in ((40, 72), (37, 100), (256, 520)):
        E = 7
        sizes = np.array([0, 1, 130, 0, 257, 5, 64])
        T = int(sizes.sum())
        w = I.Workload("rag", T=T, D=D, E=E, k=1, H=H, act=act, gating="noisy", noise=False,
                       capacity_factor=0.0, seed=0)
        p = problem_for(moe, w)
        rows = moe.moe_max_rows(p)
        offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
        cast = (lambda a: I.f32_to_bf16_bits(a)) if act == "bf16" else (lambda a: a)
        A = cast(rng.standard_normal((rows, D)).astype(np.float32))
        W1 = cast((rng.standard_normal((E, D, H)) / math.sqrt(D)).astype(np.float32))
        W2 = cast((rng.standard_normal((E, H, D)) / math.sqrt(H)).astype(np.float32))
        W1p = torch.empty(moe.moe_packed_weight_bytes(p, 1), dtype=torch.uint8, device="cuda")
        W2p = torch.empty(moe.moe_packed_weight_bytes(p, 2), dtype=torch.uint8, device="cuda")
        moe.moe_pack_expert_weights(p, dev(W1), dev(W2), W1p, W2p)
        dt = torch.bfloat16 if act == "bf16" else torch.float32
        Hd = torch.empty(rows, H, dtype=dt, device="cuda")
        Z = torch.empty(rows, D, dtype=dt, device="cuda")
        moe.moe_grouped_gemm(p, 1, dev(A), W1p, dev(offs), Hd)
        moe.moe_grouped_gemm(p, 2, Hd, W2p, dev(offs), Z)
        Hh = f64(host(Hd))
        ref1 = np.zeros((T, H))
        ref2 = np.zeros((T, D))
        for e in range(E):
            s = slice(offs[e], offs[e + 1])
            ref1[s] = np.maximum(f64(A[s]) @ f64(W1[e]), 0.0)
            ref2[s] = Hh[s] @ f64(W2[e])  # layer 2 checked on the GPU's own layer-1 output
        assert rel_err(Hh[:T], ref1) < TOL[act]
        assert rel_err(host(Z)[:T], ref2) < TOL[act]


@pytest.mark.parametrize("D,H", [(1024, 1024), (256, 1024), (448, 1280)])
def test_grouped_gemm_large_ragged(moe, D, H):
    """The 256 x 256 kernel (bf16, at least 192 rows an expert on average, one tile per CU)
    on ragged groups: empty experts, 1-row groups, 255 / 256 / 257 rows, long groups, a
    short last tile; both layers (ReLU, then plain) against numpy fp64 on every row. With
    D = 256 and 448, layer 1's tiles are 4 and 7 k-stages of 64 long: shorter than the 8
    stages over which a tile's output leaves during the next tile, so the rest is stored
    before the next epilogue (layer 2 then runs on the 128 x 256 kernel where D is not a
    multiple of 256)."""
    import torch
    rng = np.random.default_rng(23)
    E = 64  # with D = H = 1024: 484 tiles of 256 x 256 in either layer
    sizes = rng.integers(300, 520, E)
    sizes[[3, 17, 40]] = 0
    sizes[[5, 33]] = 1
    sizes[[8, 9, 10]] = (255, 256, 257)
    sizes[20] = 1100
    T = int(sizes.sum())
    w = I.Workload("bigrag", T=T, D=D, E=E, k=1, H=H, act="bf16", gating="noisy", noise=False,
                   capacity_factor=0.0, seed=0)
    p = problem_for(moe, w)
    rows = moe.moe_max_rows(p)
    assert rows >= 192 * E
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    A = I.f32_to_bf16_bits(rng.standard_normal((rows, D)).astype(np.float32))
    W1 = I.f32_to_bf16_bits((rng.standard_normal((E, D, H)) / math.sqrt(D)).astype(np.float32))
    W2 = I.f32_to_bf16_bits((rng.standard_normal((E, H, D)) / math.sqrt(H)).astype(np.float32))
    W1p = torch.empty(moe.moe_packed_weight_bytes(p, 1), dtype=torch.uint8, device="cuda")
    W2p = torch.empty(moe.moe_packed_weight_bytes(p, 2), dtype=torch.uint8, device="cuda")
    moe.moe_pack_expert_weights(p, dev(W1), dev(W2), W1p, W2p)
    Hd = torch.empty(rows, H, dtype=torch.bfloat16, device="cuda")
    Z = torch.empty(rows, D, dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(p, 1, dev(A), W1p, dev(offs), Hd)
    moe.moe_grouped_gemm(p, 2, Hd, W2p, dev(offs), Z)
    Hh, Zh = f64(host(Hd)), f64(host(Z))
    e1 = e2 = 0.0
    for e in range(E):
        s_ = slice(offs[e], offs[e + 1])
        if offs[e + 1] == offs[e]:
            continue
        r1 = np.maximum(f64(A[s_]) @ f64(W1[e]), 0.0)
        r2 = Hh[s_] @ f64(W2[e])  # layer 2 on the GPU's own layer-1 output
        e1 = max(e1, np.abs(Hh[s_] - r1).max() / max(np.abs(r1).max(), 1e-30))
        e2 = max(e2, np.abs(Zh[s_] - r2).max() / max(np.abs(r2).max(), 1e-30))
    log(f"[gemm large ragged] {T} rows over {E} experts, D {D} H {H}: layer 1 {e1:.2e}, "
        f"layer 2 {e2:.2e}")
    assert e1 < TOL["bf16"] and e2 < TOL["bf16"]


def test_grouped_gemm_long_k_half_tiles(moe):
    """The 256 x 256 kernel where K >= 2048 lets it take groups of 96-191 rows an expert (its
    row tiles then about half empty): 128 experts of about 130 rows, D = 512, H = 2048, with
    empty experts, 1-row groups, 255 / 256 / 257 rows and a long group. Layer 2 (K = 2048)
    runs on that kernel, layer 1 (K = 512) on the 128-row one; both against numpy fp64 on
    every row (layer 2 on the GPU's own layer-1 output)."""
    import torch
    rng = np.random.default_rng(29)
    E, D, H = 128, 512, 2048
    sizes = rng.integers(100, 160, E)
    sizes[[7, 70, 127]] = 0
    sizes[[11, 90]] = 1
    sizes[[30, 31, 32]] = (255, 256, 257)
    sizes[64] = 600
    T = int(sizes.sum())
    w = I.Workload("longk", T=T, D=D, E=E, k=1, H=H, act="bf16", gating="noisy", noise=False,
                   capacity_factor=0.0, seed=0)
    p = problem_for(moe, w)
    rows = moe.moe_max_rows(p)
    assert 96 * E <= rows < 192 * E
    offs = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    A = I.f32_to_bf16_bits(rng.standard_normal((rows, D)).astype(np.float32))
    W1 = I.f32_to_bf16_bits((rng.standard_normal((E, D, H)) / math.sqrt(D)).astype(np.float32))
    W2 = I.f32_to_bf16_bits((rng.standard_normal((E, H, D)) / math.sqrt(H)).astype(np.float32))
    W1p = torch.empty(moe.moe_packed_weight_bytes(p, 1), dtype=torch.uint8, device="cuda")
    W2p = torch.empty(moe.moe_packed_weight_bytes(p, 2), dtype=torch.uint8, device="cuda")
    moe.moe_pack_expert_weights(p, dev(W1), dev(W2), W1p, W2p)
    Hd = torch.empty(rows, H, dtype=torch.bfloat16, device="cuda")
    Z = torch.full((rows, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(p, 1, dev(A), W1p, dev(offs), Hd)
    moe.moe_grouped_gemm(p, 2, Hd, W2p, dev(offs), Z)
    Hh, Zh = f64(host(Hd)), f64(host(Z))
    e1 = e2 = 0.0
    for e in range(E):
        s_ = slice(offs[e], offs[e + 1])
        if offs[e + 1] == offs[e]:
            continue
        r1 = np.maximum(f64(A[s_]) @ f64(W1[e]), 0.0)
        r2 = Hh[s_] @ f64(W2[e])
        e1 = max(e1, np.abs(Hh[s_] - r1).max() / max(np.abs(r1).max(), 1e-30))
        e2 = max(e2, np.abs(Zh[s_] - r2).max() / max(np.abs(r2).max(), 1e-30))
    assert np.isfinite(Zh[:T]).all(), "a row of Z was not written"
    log(f"[gemm long K half tiles] {T} rows over {E} experts: layer 1 {e1:.2e}, layer 2 {e2:.2e}")
    assert e1 < TOL["bf16"] and e2 < TOL["bf16"]


def test_grouped_gemm_check_finite_large(moe):
    """The non-finite check of the 256 x 256 kernel (top2_bf16's layer-2 shapes, 512 rows an
    expert): clean rows raise nothing, one NaN in one expert's rows raises MOE_ERR_NONFINITE
    at the next check, and the record is cleared after it is reported."""
    import torch
    w = I.Workload("chk", T=65536, D=1024, E=256, k=2, H=4096, act="bf16", gating="noisy",
                   noise=True, capacity_factor=1.0, seed=22)
    p = problem_for(moe, w, check_finite=True)
    rows = moe.moe_max_rows(p)
    assert rows == 256 * 512
    torch.manual_seed(22)
    W2 = (torch.randn(w.E, w.H, w.D, device="cuda") / 64).to(torch.bfloat16)
    W2p = torch.empty(moe.moe_packed_weight_bytes(p, 2), dtype=torch.uint8, device="cuda")
    moe.moe_pack_expert_weights(p, None, W2, None, W2p)
    offs = dev((np.arange(w.E + 1) * 512).astype(np.int32))
    Hd = (torch.randn(rows, w.H, device="cuda") / 8).to(torch.bfloat16)
    Z = torch.empty(rows, w.D, dtype=torch.bfloat16, device="cuda")
    moe.moe_grouped_gemm(p, 2, Hd, W2p, offs, Z)
    moe.moe_check_finite()  # clean: no error
    Hd[77 * 512 + 300, 1234] = float("nan")
    moe.moe_grouped_gemm(p, 2, Hd, W2p, offs, Z)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_check_finite()
    assert ei.value.status == -3
    z = Z.float()
    assert torch.isnan(z[77 * 512 + 300]).all() and not torch.isnan(z[77 * 512 + 299]).any()
    moe.moe_check_finite()  # the record was cleared



def _fragment_layout(B, V, KS, stage_order):
    """The packed operand layout moe.h states, from B [E, K, N]: fragment (e, nb, ks) holds,
    for lane l, column nb*32 + l%32, rows ks*2V + (l//32)*V .. +V-1, zeros past K or N; the
    fragments are ordered [e][ks // 4][nb][ks % 4] in k-stage order, else [e][nb][ks]."""
    E, K, N = B.shape
    NB = -(-N // 32)
    Q = KS // 4
    Bp = np.zeros((E, KS * 2 * V, NB * 32), dtype=B.dtype)
    Bp[:, :K, :N] = B
    # [E, q, r, half, i, nb, col] (ks = 4q + r)
    t = Bp.reshape(E, Q, 4, 2, V, NB, 32)
    if stage_order:  # -> [E, q, nb, r, half, col, i]
        t = t.transpose(0, 1, 5, 2, 3, 6, 4)
    else:  # -> [E, nb, q, r, half, col, i]
        t = t.transpose(0, 5, 1, 2, 3, 6, 4)
    return np.ascontiguousarray(t).reshape(-1, 64, V)


@pytest.mark.parametrize("act", ["f32", "bf16"])
def test_weight_pack_layouts(moe, act):
    """moe_pack_expert_weights (layers 1, 2) and moe_pack_expert_weights_t (layers 3, 4: the
    transposes W2^T and W1^T for the backward) against the fragment layout built on the host,
    bit-exact, with widths that are not multiples of the fragment (zero padding) and, for
    D = 37, rows that are not whole 16-byte vectors; in column-block order (few rows an
    expert) and in k-stage order (at least 128 rows an expert: T = 256, 512 below)."""
    import torch
    rng = np.random.default_rng(21)
    for (E, D, H, T) in ((3, 40, 72, 8), (2, 37, 100, 8), (2, 256, 520, 8), (2, 256, 520, 256),
                         (3, 40, 72, 512), (2, 37, 100, 300)):
        w = I.Workload("pk", T=T, D=D, E=E, k=1, H=H, act=act, gating="noisy", noise=False,
                       capacity_factor=0.0, seed=0)
        p = problem_for(moe, w)
        stage_order = moe.moe_max_rows(p) >= 128 * E
        cast = (lambda a: I.f32_to_bf16_bits(a)) if act == "bf16" else (lambda a: a)
        W1 = cast(rng.standard_normal((E, D, H)).astype(np.float32))
        W2 = cast(rng.standard_normal((E, H, D)).astype(np.float32))
        V = 8 if act == "bf16" else 4
        bufs = [torch.zeros(moe.moe_packed_weight_bytes(p, layer), dtype=torch.uint8,
                            device="cuda") for layer in (1, 2, 3, 4)]
        moe.moe_pack_expert_weights(p, dev(W1), dev(W2), bufs[0], bufs[1])
        moe.moe_pack_expert_weights_t(p, dev(W1), dev(W2), bufs[3], bufs[2])  # W1t, W2t
        # B of each layer as [E, K, N]: W1, W2, W2^T, W1^T
        Bs = [W1, W2, W2.transpose(0, 2, 1), W1.transpose(0, 2, 1)]
        for layer, (buf, B) in enumerate(zip(bufs, Bs), start=1):
            K = B.shape[1]
            KS = -(-K // (16 * V // 2)) * 4  # k stages of 128 bytes, 4 k-steps each
            want = _fragment_layout(B, V, KS, stage_order)
            got = host(buf).view(B.dtype)
            assert got.size == want.size, (layer, got.size, want.size)
            assert (got.reshape(want.shape).view(np.uint8) == want.view(np.uint8)).all(), \
                (layer, D, H, T)

@pytest.mark.parametrize("name", ALL)
def test_combine(moe, name):
    import torch
    log(f"[combine] {name}")
    w, inp = workload_inputs(name)
    r, d = oracle_routing(name)
    p = problem_for(moe, w)
    rows = moe.moe_max_rows(p)
    rng = np.random.default_rng(3)
    Zh = rng.standard_normal((rows, w.D)).astype(np.float32)
    Zh = I.f32_to_bf16_bits(Zh) if w.act == "bf16" else Zh
    dt = torch.bfloat16 if w.act == "bf16" else torch.float32
    Y = torch.empty(w.T, w.D, dtype=dt, device="cuda")
    moe.moe_combine(p, dev(Zh), dev(r.ids), dev(r.gates.astype(np.float32)),
                    dev(d.pos), dev(d.accepted.astype(np.uint8)), dev(d.offsets), dev(inp["X"]), Y)
    Yh = host(Y)
    toks = np.arange(w.T)  # every token
    ref = O.combine_rows(Zh, r, d, inp["X"], tokens=toks)
    err = rel_err(Yh[toks], ref)
    log(f"  Y on all {w.T} tokens: rel err {err:.2e}, max abs {max_abs(Yh[toks], ref):.2e}")
    assert err < TOL[w.act]
    dropped = np.nonzero(~d.accepted.any(axis=1))[0]
    log(f"  fully dropped tokens {dropped.size}")
    np.testing.assert_array_equal(Yh[dropped], inp["X"][dropped])
    # no residual
    Y0 = torch.empty(w.T, w.D, dtype=dt, device="cuda")
    moe.moe_combine(p, dev(Zh), dev(r.ids), dev(r.gates.astype(np.float32)),
                    dev(d.pos), dev(d.accepted.astype(np.uint8)), dev(d.offsets), None, Y0)
    ref0 = O.combine_rows(Zh, r, d, None, tokens=toks)
    err0 = rel_err(host(Y0)[toks], ref0)
    log(f"  no residual (the branch alone): rel err {err0:.2e}, max abs {max_abs(host(Y0)[toks], ref0):.2e}")
    assert err0 < TOL[w.act]


# Shapes that reach every instance of the aux row pass: E in (256, 512] (two 16-byte
# vectors a lane), E not a multiple of 4 (the column pass), a small T (4 rows a block, fewer
# blocks than slices), Switch gating over 96 experts, and a ragged last block.
AUX_SHAPES = [
    I.Workload("aux_e512", T=4100, D=64, E=512, k=2, H=16, act="bf16", gating="noisy",
               noise=True, capacity_factor=1.0, seed=31),
    I.Workload("aux_e202", T=3001, D=48, E=202, k=3, H=16, act="f32", gating="noisy",
               noise=True, capacity_factor=0.0, seed=32),
    I.Workload("aux_t60", T=60, D=32, E=40, k=2, H=16, act="f32", gating="noisy", noise=True,
               capacity_factor=1.25, seed=33),
    I.Workload("aux_sw96", T=5000, D=40, E=96, k=1, H=16, act="bf16", gating="switch",
               noise=False, capacity_factor=1.0, seed=34),
]


@pytest.mark.parametrize("w", AUX_SHAPES, ids=[w.name for w in AUX_SHAPES])
def test_aux_shapes(moe, w):
    log(f"[aux shape] {w}")
    inp = I.make_inputs(w, experts=False)
    r = O.route(inp["X"], inp["Wg"], inp["Wnoise"], inp["bias"], w.k, w.gating, w.noise,
                seed=w.seed)
    d = O.dispatch(r.ids, w.E, O.capacity(w.T, w.k, w.capacity_factor, w.E, w.min_capacity))
    _check_aux(moe, w, r, d)


@pytest.mark.parametrize("name", ALL)
def test_aux(moe, name):
    log(f"[aux] {name}")
    w, inp = workload_inputs(name)
    r, d = oracle_routing(name)
    _check_aux(moe, w, r, d)


def _check_aux(moe, w, r, d):
    import torch
    a = O.aux(r, d, w.k)
    p = problem_for(moe, w)
    noisy = r.std is not None
    f32 = lambda x: dev(np.ascontiguousarray(x, dtype=np.float32))
    imp = torch.empty(w.E, device="cuda")
    load = torch.empty(w.E, device="cuda")
    out = torch.empty(8, device="cuda")
    ws = torch.empty(moe.moe_workspace_size(p, moe.MOE_WS_AUX), dtype=torch.uint8, device="cuda")
    moe.moe_aux_loss(p, dev(r.ids), f32(r.gates), f32(r.clean), f32(r.std) if noisy else None,
                     f32(r.row_stats) if noisy else None, dev(d.counts), imp, load, out, ws)
    e_imp = rel_err(host(imp), a["importance"])
    e_load = rel_err(host(load), a["load"]) if noisy else 0.0
    log(f"  importance rel err {e_imp:.2e}, load rel err {e_load:.2e}")
    assert e_imp < TOL["f32"] and e_load < TOL["f32"]
    o = host(out).astype(np.float64)
    ref = a["out"]
    log(f"  out gpu {np.round(o, 6).tolist()}\n      ref {np.round(ref, 6).tolist()}")
    for i in range(8):
        assert abs(o[i] - ref[i]) <= TOL["f32"] * max(abs(ref[i]), 1e-2), (i, o[i], ref[i])
