"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/moe.h, and rejects bad arguments on the host before any
HIP call (so these run on a machine without a GPU)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "sparsely_gated_mixture_amd", "libmoe.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libmoe.so not built")


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def m():
    from sparsely_gated_mixture_amd import moe
    return moe


def test_exports_every_declared_symbol(m):
    names = _declared()
    assert len(names) >= 12
    lib = ctypes.CDLL(LIB)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(m.ENTRY_POINTS) == names


def test_problem_struct_layout(m):
    assert ctypes.sizeof(m.Problem) == 56
    assert m.Problem.seed.offset == 40


def _p(m, **kw):
    base = dict(T=64, D=32, E=8, H=48, k=2, dtype="bf16", gating="noisy", noise=True,
                capacity_factor=1.0, seed=3)
    base.update(kw)
    return m.problem(**base)


def test_capacity_formula(m):
    # Switch explainer step 3 (floor, clamp to T, minimum), scaled by k
    assert m.moe_capacity(_p(m, T=8, E=3, k=1, gating="switch", noise=False)) == 2
    assert m.moe_capacity(_p(m, T=16384, E=128, k=1, capacity_factor=1.25)) == 160
    assert m.moe_capacity(_p(m, T=65536, E=256, k=2, capacity_factor=1.0)) == 512
    assert m.moe_capacity(_p(m, T=100, E=8, k=2, capacity_factor=0.0)) == 100
    assert m.moe_capacity(_p(m, T=8, E=8, k=1, capacity_factor=0.01, min_capacity=3)) == 3
    assert m.moe_max_rows(_p(m, T=65536, E=256, k=2, capacity_factor=1.0)) == 131072
    assert m.moe_max_rows(_p(m, T=64, E=8, k=2, capacity_factor=0.5)) == 8 * 8


@pytest.mark.parametrize("kw", [
    dict(T=0), dict(D=0), dict(E=0), dict(H=0), dict(k=0), dict(k=9, E=4),
    dict(gating="switch", k=2), dict(capacity_factor=math.nan), dict(capacity_factor=math.inf),
    dict(min_capacity=0),
])
def test_invalid_problem(m, kw):
    p = _p(m, **kw)
    assert m._lib.moe_capacity(ctypes.byref(p)) == -1
    assert m.moe_workspace_size(p, m.MOE_WS_ROUTE) == 0
    st = m._lib.moe_route(ctypes.byref(p), *([None] * 10), None, 0, None)
    assert st == -1


def test_unsupported_problem(m):
    p = _p(m, E=16, k=9)  # k above MOE_MAX_K
    st = m._lib.moe_route(ctypes.byref(p), *([None] * 10), None, 0, None)
    assert st == -2
    p = _p(m, E=5000, k=2)
    assert m._lib.moe_dispatch(ctypes.byref(p), *([None] * 8), None, 0, None) == -2


def test_null_pointers_and_workspace(m):
    p = _p(m)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: rejected on the host
    # required pointer missing
    st = m._lib.moe_route(ctypes.byref(p), fake, None, fake, None, None, fake, fake, fake, fake,
                          None, fake, 1 << 20, None)
    assert st == -1
    # noisy gate without Wnoise
    st = m._lib.moe_route(ctypes.byref(p), fake, fake, None, None, None, fake, fake, fake, fake,
                          None, fake, 1 << 20, None)
    assert st == -1
    # workspace too small
    need = m.moe_workspace_size(p, m.MOE_WS_ROUTE)
    assert need > 0
    st = m._lib.moe_route(ctypes.byref(p), fake, fake, fake, None, None, fake, fake, fake, fake,
                          None, fake, need - 1, None)
    assert st == -5
    st = m._lib.moe_dispatch(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake, fake,
                             None, 0, None)
    assert st == -5
    st = m._lib.moe_aux_loss(ctypes.byref(p), fake, fake, fake, None, fake, fake, None, None, fake,
                             fake, 1 << 30, None)
    assert st == -1  # noise on but no noise_std
    assert m._lib.moe_grouped_gemm(ctypes.byref(p), 3, fake, fake, fake, fake, None) == -1
    assert m._lib.moe_pack_expert_weights(ctypes.byref(p), None, None, None, None, None) == -1


def test_status_strings(m):
    for s in (0, -1, -2, -3, -4, -5):
        assert m._lib.moe_status_string(s).decode() != "unknown status"
    assert m._lib.moe_status_string(7).decode() == "unknown status"


def test_sizes_scale(m):
    p = _p(m, T=65536, D=1024, E=256, H=4096, k=2)
    # packed expert weights: zero padding only to 32 columns / 64-deep k stages
    assert m.moe_packed_weight_bytes(p, 1) == 256 * 1024 * 4096 * 2
    assert m.moe_packed_weight_bytes(p, 2) == 256 * 4096 * 1024 * 2
    # transposed layers for the backward pass: W2^T (3) and W1^T (4)
    assert m.moe_packed_weight_bytes(p, 3) == 256 * 1024 * 4096 * 2
    assert m.moe_packed_weight_bytes(p, 4) == 256 * 4096 * 1024 * 2
    assert m.moe_packed_weight_bytes(p, 5) == 0
    # router: three bf16 pieces of [Wg | Wnoise] plus the fp32 noisy scores [T,E]
    assert m.moe_workspace_size(p, m.MOE_WS_ROUTE) == 3 * 1024 * 512 * 2 + 65536 * 256 * 4


def test_hier_validation(m):
    p = _p(m, T=64, E=12, k=4, noise=True)
    assert m.moe_hier_workspace_size(p, m.hier(4, 2), m.MOE_WS_ROUTE) > 0
    assert m.moe_hier_workspace_size(p, m.hier(4, 2), m.MOE_WS_AUX) > 0
    for h in (m.hier(5, 2), m.hier(4, 3), m.hier(4, 5), m.hier(0, 1), m.hier(12, 1)):
        # 12 not divisible by 5; 4 % 3 != 0; k_primary > groups; no groups; k_s = 4 > b = 1
        assert m.moe_hier_workspace_size(p, h, m.MOE_WS_ROUTE) == 0
    h = m.hier(4, 2)
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: rejected on the host
    st = m.HierState(**{n: 0x1000 for n in m.HIER_STATE_FIELDS})
    args = [fake] * 7
    sw = _p(m, T=64, E=12, k=1, gating="switch", noise=False)
    assert m._lib.moe_route_hier(ctypes.byref(sw), ctypes.byref(m.hier(4, 1)), *args,
                                 ctypes.byref(st), fake, 1 << 30, None) == -1
    assert m._lib.moe_route_hier(ctypes.byref(p), ctypes.byref(h), *args, None, fake, 1 << 30,
                                 None) == -1
    need = m.moe_hier_workspace_size(p, h, m.MOE_WS_ROUTE)
    assert m._lib.moe_route_hier(ctypes.byref(p), ctypes.byref(h), *args, ctypes.byref(st), fake,
                                 need - 1, None) == -5
    st_nostd = m.HierState(**{n: (None if n in ("std_p", "std_s") else 0x1000)
                              for n in m.HIER_STATE_FIELDS})
    assert m._lib.moe_aux_loss_hier(ctypes.byref(p), ctypes.byref(h), ctypes.byref(st_nostd),
                                    fake, fake, fake, fake, 1 << 30, None) == -1



def test_unaligned_pointers_rejected(m):
    """A tensor pointer that is not 16-byte aligned is an argument error, returned before
    anything is enqueued (each call below is otherwise complete; the fake addresses are never
    dereferenced)."""
    p = _p(m)
    ok, bad = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1004)
    big = 1 << 30

    def route(i):  # X, Wg, Wnoise, bias, eps, ids, gates, clean, noise_std, row_stats, ws
        a = [ok] * 11
        a[i] = bad
        return m._lib.moe_route(ctypes.byref(p), *a[:10], a[10], big, None)
    for i in range(11):
        assert route(i) == -1, i
    a = [ok] * 9
    a[7] = bad  # Xd
    assert m._lib.moe_dispatch(ctypes.byref(p), *a, big, None) == -1
    assert m._lib.moe_grouped_gemm(ctypes.byref(p), 1, ok, ok, ok, bad, None) == -1
    assert m._lib.moe_expert_ffn(ctypes.byref(p), ok, ok, ok, ok, ok, bad, None) == -1
    for i in range(5):  # X, row_token, W1p, offsets, Hd
        a = [ok] * 5
        a[i] = bad
        assert m._lib.moe_grouped_gemm_gather(ctypes.byref(p), *a, None) == -1, i
    for i in range(7):  # X, row_token, W1p, W2p, offsets, Hd, Z
        a = [ok] * 7
        a[i] = bad
        assert m._lib.moe_expert_ffn_gather(ctypes.byref(p), *a, None) == -1, i
    # residual (optional) misaligned
    assert m._lib.moe_combine(ctypes.byref(p), ok, ok, ok, ok, ok, ok, bad, ok, None) == -1
    assert m._lib.moe_pack_expert_weights(ctypes.byref(p), bad, None, ok, None, None) == -1
    assert m._lib.moe_expert_weight_grad(ctypes.byref(p), 1, ok, ok, ok, bad, None) == -1
    assert m._lib.moe_expert_weight_grad(ctypes.byref(p), 2, bad, ok, ok, ok, None) == -1
    pb = _p(m, T=64, E=8, k=2, gating="batchwise", noise=False)
    st = m.BatchwiseState(**{n: 0x1000 for n in m.BATCHWISE_STATE_FIELDS})
    st.tok_gate = 0x1008
    assert m._lib.moe_dispatch_batchwise(ctypes.byref(pb), ok, ctypes.byref(st), ok, None) == -1
    ph, h = _p(m, T=64, E=8, k=2), m.hier(2, 1)
    hs = m.HierState(**{n: 0x1000 for n in m.HIER_STATE_FIELDS})
    hs.clean_s = 0x1002
    assert m._lib.moe_route_hier(ctypes.byref(ph), ctypes.byref(h), *([ok] * 7),
                                 ctypes.byref(hs), ok, big, None) == -1

def test_batchwise_validation(m):
    p = _p(m, T=64, E=8, k=2, gating="batchwise", noise=False)
    assert m.moe_batchwise_m(p) == 16
    assert m.moe_batchwise_workspace_size(p, m.MOE_WS_ROUTE) > 0
    assert m.moe_workspace_size(p, m.MOE_WS_ROUTE) == 0  # the top-k entry points refuse it
    fake0 = ctypes.c_void_p(0x1000)
    assert m._lib.moe_route(ctypes.byref(p), *([fake0] * 10), fake0, 1 << 30, None) == -1
    assert m._lib.moe_batchwise_m(ctypes.byref(_p(m, T=3, E=8, k=2, gating="batchwise",
                                                  noise=False))) == -1  # k T < E
    assert m._lib.moe_batchwise_m(ctypes.byref(_p(m, gating="batchwise", noise=True))) == -1
    assert m._lib.moe_batchwise_m(ctypes.byref(_p(m))) == -1  # not a batchwise problem
    fake = ctypes.c_void_p(0x1000)
    st = m.BatchwiseState(**{n: 0x1000 for n in m.BATCHWISE_STATE_FIELDS})
    need = m.moe_batchwise_workspace_size(p, m.MOE_WS_ROUTE)
    assert m._lib.moe_route_batchwise(ctypes.byref(p), fake, fake, None, fake, ctypes.byref(st),
                                      fake, need - 1, None) == -5
    st.tok_gate = None
    assert m._lib.moe_route_batchwise(ctypes.byref(p), fake, fake, None, fake, ctypes.byref(st),
                                      fake, need, None) == -1


def test_backward_validation(m):
    p = _p(m, T=64, E=8, k=2)
    assert m.moe_backward_workspace_size(p) > 0
    sw = _p(m, T=64, E=8, k=1, gating="switch", noise=False)
    assert m.moe_backward_workspace_size(sw) > 0
    bw = _p(m, T=64, E=8, k=2, gating="batchwise", noise=False)
    assert m.moe_backward_workspace_size(bw) == 0
    fake = ctypes.c_void_p(0x1000)
    # every call below is rejected by the host checks before anything is enqueued
    assert m._lib.moe_combine_backward(ctypes.byref(bw), *([fake] * 9), None) == -1
    assert m._lib.moe_combine_backward(ctypes.byref(p), fake, None, *([fake] * 7), None) == -1
    args = [fake] * 13 + [ctypes.c_float(0.0), ctypes.c_float(0.0)] + [fake] * 9
    need = m.moe_backward_workspace_size(p)
    assert m._lib.moe_route_backward(ctypes.byref(p), *args, fake, need - 1, None) == -5
    args_nan = [fake] * 13 + [ctypes.c_float(float("nan")), ctypes.c_float(0.0)] + [fake] * 9
    assert m._lib.moe_route_backward(ctypes.byref(p), *args_nan, fake, need, None) == -1
    # each gate has its own route-backward entry point
    assert m._lib.moe_route_backward(ctypes.byref(sw), *args, fake, need, None) == -1
    sargs = [fake] * 7 + [ctypes.c_float(0.0), ctypes.c_float(0.1)] + [fake] * 8
    need_sw = m.moe_backward_workspace_size(sw)
    assert m._lib.moe_route_backward_switch(ctypes.byref(p), *sargs, fake, need, None) == -1
    assert m._lib.moe_route_backward_switch(ctypes.byref(sw), *sargs, fake, need_sw - 1,
                                            None) == -5
    no_counts = list(sargs)
    no_counts[6] = None  # counts, needed for w_switch != 0
    assert m._lib.moe_route_backward_switch(ctypes.byref(sw), *no_counts, fake, need_sw,
                                            None) == -1


def test_weight_grad_validation(m):
    p = _p(m, T=64, E=8, k=2)
    fake = ctypes.c_void_p(0x1000)
    assert m._lib.moe_expert_weight_grad(ctypes.byref(p), 3, *([fake] * 4), None) == -1
    assert m._lib.moe_expert_weight_grad(ctypes.byref(p), 1, fake, None, fake, fake, None) == -1
    bw = _p(m, T=64, E=8, k=2, gating="batchwise", noise=False)
    assert m._lib.moe_expert_weight_grad(ctypes.byref(bw), 1, *([fake] * 4), None) == -1


def test_recompute_validation(m):
    p = _p(m, T=64, E=8, k=2)
    fake = ctypes.c_void_p(0x1000)
    args = [fake] * 11
    args_missing = list(args)
    args_missing[6] = None  # Hd scratch
    assert m._lib.moe_expert_ffn_backward_recompute(ctypes.byref(p), *args_missing, None) == -1
    bw = _p(m, T=64, E=8, k=2, gating="batchwise", noise=False)
    assert m._lib.moe_expert_ffn_backward_recompute(ctypes.byref(bw), *args, None) == -1


def test_route_scores_address(m):
    """The noisy scores sit after the packed router weights in the route workspace; a gate
    without noise has none (no device access: pure address arithmetic)."""
    p = _p(m, T=64, E=8, k=2)
    base = 0x10000000
    a = m._lib.moe_route_scores(ctypes.byref(p), ctypes.c_void_p(base))
    assert a is not None and base < a < base + m.moe_workspace_size(p, m.MOE_WS_ROUTE)
    assert (a - base) % 256 == 0
    assert a + 64 * 8 * 4 <= base + m.moe_workspace_size(p, m.MOE_WS_ROUTE)
    off = _p(m, T=64, E=8, k=2, noise=False)
    assert m._lib.moe_route_scores(ctypes.byref(off), ctypes.c_void_p(base)) is None
    sw = _p(m, T=64, E=8, k=1, gating="switch", noise=False)
    assert m._lib.moe_route_scores(ctypes.byref(sw), ctypes.c_void_p(base)) is None


def test_gathered_entry_points_need_their_pointers(m):
    """The gathered layer-1 entry points reject a missing pointer (argument error, nothing
    enqueued); moe_dispatch accepts Xd = NULL (slots only) but not a missing row_token."""
    p = _p(m)
    ok = ctypes.c_void_p(0x1000)
    for i in range(5):
        a = [ok] * 5
        a[i] = None
        assert m._lib.moe_grouped_gemm_gather(ctypes.byref(p), *a, None) == -1, i
    for i in range(7):
        a = [ok] * 7
        a[i] = None
        assert m._lib.moe_expert_ffn_gather(ctypes.byref(p), *a, None) == -1, i
    a = [ok] * 9  # X, ids, pos, accepted, counts, offsets, row_token, Xd, workspace
    a[6] = None
    assert m._lib.moe_dispatch(ctypes.byref(p), *a, 1 << 30, None) == -1
