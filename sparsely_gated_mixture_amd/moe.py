"""Python binding of the MoE C ABI (libmoe.so): argument marshalling only.

Every step of the layer runs in the HIP kernels behind the C ABI; this module
turns torch CUDA tensors into device pointers and the current HIP stream, and
raises MoEError on a negative status. PyTorch is used for device memory and
streams only. If the library is missing the import of this module fails:
there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_GATE_NOISY_TOPK, MOE_GATE_SWITCH_TOP1, MOE_GATE_BATCHWISE = 0, 1, 2
MOE_WS_ROUTE, MOE_WS_DISPATCH, MOE_WS_AUX = 0, 1, 2
MOE_MAX_K = 8

STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED",
          -3: "MOE_ERR_NONFINITE", -4: "MOE_ERR_HIP", -5: "MOE_ERR_WORKSPACE"}

ENTRY_POINTS = [
    "moe_capacity", "moe_max_rows", "moe_workspace_size", "moe_packed_weight_bytes",
    "moe_route", "moe_dispatch", "moe_pack_expert_weights", "moe_grouped_gemm",
    "moe_expert_ffn", "moe_combine", "moe_aux_loss", "moe_check_finite", "moe_status_string",
    "moe_hier_workspace_size", "moe_route_hier", "moe_aux_loss_hier",
    "moe_batchwise_m", "moe_batchwise_workspace_size", "moe_route_batchwise",
    "moe_dispatch_batchwise", "moe_combine_batchwise", "moe_aux_loss_batchwise",
    "moe_pack_expert_weights_t", "moe_combine_backward", "moe_expert_ffn_backward",
    "moe_route_backward", "moe_backward_workspace_size", "moe_expert_weight_grad",
    "moe_expert_ffn_backward_recompute", "moe_route_backward_switch", "moe_route_scores",
    "moe_grouped_gemm_gather", "moe_expert_ffn_gather", "moe_dispatch_noalloc",
]


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({_text(status)})")


class Problem(ctypes.Structure):
    """Mirror of moe_problem (include/moe.h)."""
    _fields_ = [
        ("T", ctypes.c_int32), ("D", ctypes.c_int32), ("E", ctypes.c_int32),
        ("H", ctypes.c_int32), ("k", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("gating", ctypes.c_int32), ("noise", ctypes.c_int32),
        ("capacity_factor", ctypes.c_float), ("min_capacity", ctypes.c_int32),
        ("seed", ctypes.c_uint64), ("check_finite", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
    ]


class Hier(ctypes.Structure):
    """Mirror of moe_hier."""
    _fields_ = [("groups", ctypes.c_int32), ("k_primary", ctypes.c_int32)]


HIER_STATE_FIELDS = ["ids_p", "gates_p", "clean_p", "std_p", "row_stats_p", "pos_p", "accepted_p",
                     "counts_p", "offsets_p", "row_token_p", "clean_s", "std_s", "row_stats_s",
                     "ids_s", "gates_s"]


class HierState(ctypes.Structure):
    """Mirror of moe_hier_state (device pointers)."""
    _fields_ = [(n, ctypes.c_void_p) for n in HIER_STATE_FIELDS]


BATCHWISE_STATE_FIELDS = ["probs_t", "sel", "offsets", "mask", "tok_count", "tok_off", "tok_row",
                          "tok_gate", "slot_pair"]


class BatchwiseState(ctypes.Structure):
    """Mirror of moe_batchwise_state (device pointers)."""
    _fields_ = [(n, ctypes.c_void_p) for n in BATCHWISE_STATE_FIELDS]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"HIP library not built: {path} (run python -m sparsely_gated_mixture_amd.build)")
    lib = ctypes.CDLL(path)
    vp, sz, i32, i64 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64
    P = ctypes.POINTER(Problem)
    sig = {
        "moe_capacity": (i32, [P]),
        "moe_max_rows": (i64, [P]),
        "moe_workspace_size": (sz, [P, ctypes.c_int]),
        "moe_packed_weight_bytes": (sz, [P, ctypes.c_int]),
        "moe_route": (ctypes.c_int, [P] + [vp] * 10 + [vp, sz, vp]),
        "moe_dispatch": (ctypes.c_int, [P] + [vp] * 8 + [vp, sz, vp]),
        "moe_dispatch_noalloc": (ctypes.c_int, [P] + [vp] * 8 + [vp]),
        "moe_pack_expert_weights": (ctypes.c_int, [P, vp, vp, vp, vp, vp]),
        "moe_grouped_gemm": (ctypes.c_int, [P, ctypes.c_int, vp, vp, vp, vp, vp]),
        "moe_expert_ffn": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp, vp]),
        "moe_grouped_gemm_gather": (ctypes.c_int, [P, vp, vp, vp, vp, vp, vp]),
        "moe_expert_ffn_gather": (ctypes.c_int, [P] + [vp] * 8),
        "moe_combine": (ctypes.c_int, [P] + [vp] * 8 + [vp]),
        "moe_aux_loss": (ctypes.c_int, [P] + [vp] * 9 + [vp, sz, vp]),
        "moe_check_finite": (ctypes.c_int, [vp]),
        "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_hier_workspace_size": (sz, [P, ctypes.POINTER(Hier), ctypes.c_int]),
        "moe_route_hier": (ctypes.c_int, [P, ctypes.POINTER(Hier)] + [vp] * 7 +
                           [ctypes.POINTER(HierState), vp, sz, vp]),
        "moe_aux_loss_hier": (ctypes.c_int, [P, ctypes.POINTER(Hier), ctypes.POINTER(HierState)] +
                              [vp] * 4 + [sz, vp]),
        "moe_pack_expert_weights_t": (ctypes.c_int, [P, vp, vp, vp, vp, vp]),
        "moe_combine_backward": (ctypes.c_int, [P] + [vp] * 9 + [vp]),
        "moe_expert_ffn_backward": (ctypes.c_int, [P] + [vp] * 10 + [vp]),
        "moe_route_scores": (vp, [P, vp]),
        "moe_route_backward": (ctypes.c_int, [P] + [vp] * 13 + [ctypes.c_float, ctypes.c_float] +
                               [vp] * 9 + [vp, sz, vp]),
        "moe_backward_workspace_size": (sz, [P]),
        "moe_expert_weight_grad": (ctypes.c_int, [P, i32, vp, vp, vp, vp, vp]),
        "moe_expert_ffn_backward_recompute": (ctypes.c_int, [P] + [vp] * 11 + [vp]),
        "moe_route_backward_switch": (ctypes.c_int, [P] + [vp] * 7 + [ctypes.c_float] * 2 +
                                      [vp] * 9 + [sz, vp]),
        "moe_batchwise_m": (i32, [P]),
        "moe_batchwise_workspace_size": (sz, [P, ctypes.c_int]),
        "moe_route_batchwise": (ctypes.c_int, [P, vp, vp, vp, vp, ctypes.POINTER(BatchwiseState),
                                               vp, sz, vp]),
        "moe_dispatch_batchwise": (ctypes.c_int, [P, vp, ctypes.POINTER(BatchwiseState), vp, vp]),
        "moe_combine_batchwise": (ctypes.c_int, [P, vp, ctypes.POINTER(BatchwiseState), vp, vp, vp]),
        "moe_aux_loss_batchwise": (ctypes.c_int, [P, ctypes.POINTER(BatchwiseState), vp, vp, vp,
                                                  vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = load_library()


def _text(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def _check(status: int, where: str):
    if status != 0:
        raise MoEError(status, where)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def problem(T, D, E, H, k, dtype="bf16", gating="noisy", noise=True, capacity_factor=0.0,
            min_capacity=1, seed=0, check_finite=False) -> Problem:
    return Problem(T=T, D=D, E=E, H=H, k=k,
                   dtype=MOE_BF16 if dtype == "bf16" else MOE_F32,
                   gating={"switch": MOE_GATE_SWITCH_TOP1,
                           "batchwise": MOE_GATE_BATCHWISE}.get(gating, MOE_GATE_NOISY_TOPK),
                   noise=1 if noise else 0, capacity_factor=float(capacity_factor),
                   min_capacity=int(min_capacity), seed=int(seed),
                   check_finite=1 if check_finite else 0, reserved=0)


def torch_dtype(p: Problem):
    return torch.bfloat16 if p.dtype == MOE_BF16 else torch.float32


# ------------------------------------------------------------------ sizes
def moe_capacity(p: Problem) -> int:
    c = _lib.moe_capacity(ctypes.byref(p))
    if c < 0:
        raise MoEError(-1, "moe_capacity")
    return c


def moe_max_rows(p: Problem) -> int:
    r = _lib.moe_max_rows(ctypes.byref(p))
    if r < 0:
        raise MoEError(-1, "moe_max_rows")
    return r


def moe_workspace_size(p: Problem, which: int) -> int:
    return _lib.moe_workspace_size(ctypes.byref(p), which)


def moe_packed_weight_bytes(p: Problem, layer: int) -> int:
    return _lib.moe_packed_weight_bytes(ctypes.byref(p), layer)


# ------------------------------------------------------------------ stages
def moe_route(p, X, Wg, Wnoise, bias, eps, ids, gates, clean, noise_std, row_stats, ws, stream=None):
    _check(_lib.moe_route(ctypes.byref(p), _ptr(X), _ptr(Wg), _ptr(Wnoise), _ptr(bias), _ptr(eps),
                          _ptr(ids), _ptr(gates), _ptr(clean), _ptr(noise_std), _ptr(row_stats),
                          _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)), "moe_route")


def moe_dispatch(p, X, ids, pos, accepted, counts, offsets, row_token, Xd, ws, stream=None):
    _check(_lib.moe_dispatch(ctypes.byref(p), _ptr(X), _ptr(ids), _ptr(pos), _ptr(accepted),
                             _ptr(counts), _ptr(offsets), _ptr(row_token), _ptr(Xd), _ptr(ws),
                             ws.numel() if ws is not None else 0, _stream(stream)), "moe_dispatch")


def moe_dispatch_noalloc(p, X, ids, pos, accepted, counts, offsets, row_token, Xd, stream=None):
    _check(_lib.moe_dispatch_noalloc(ctypes.byref(p), _ptr(X), _ptr(ids), _ptr(pos),
                                     _ptr(accepted), _ptr(counts), _ptr(offsets),
                                     _ptr(row_token), _ptr(Xd), _stream(stream)),
           "moe_dispatch_noalloc")


def moe_pack_expert_weights(p, W1, W2, W1p, W2p, stream=None):
    _check(_lib.moe_pack_expert_weights(ctypes.byref(p), _ptr(W1), _ptr(W2), _ptr(W1p), _ptr(W2p),
                                        _stream(stream)), "moe_pack_expert_weights")


def moe_grouped_gemm(p, layer, A, Wp, offsets, C, stream=None):
    _check(_lib.moe_grouped_gemm(ctypes.byref(p), layer, _ptr(A), _ptr(Wp), _ptr(offsets), _ptr(C),
                                 _stream(stream)), "moe_grouped_gemm")


def moe_grouped_gemm_gather(p, X, row_token, W1p, offsets, Hd, stream=None):
    _check(_lib.moe_grouped_gemm_gather(ctypes.byref(p), _ptr(X), _ptr(row_token), _ptr(W1p),
                                        _ptr(offsets), _ptr(Hd), _stream(stream)),
           "moe_grouped_gemm_gather")


def moe_expert_ffn_gather(p, X, row_token, W1p, W2p, offsets, Hd, Z, stream=None):
    _check(_lib.moe_expert_ffn_gather(ctypes.byref(p), _ptr(X), _ptr(row_token), _ptr(W1p),
                                      _ptr(W2p), _ptr(offsets), _ptr(Hd), _ptr(Z),
                                      _stream(stream)), "moe_expert_ffn_gather")


def moe_expert_ffn(p, Xd, W1p, W2p, offsets, Hd, Z, stream=None):
    _check(_lib.moe_expert_ffn(ctypes.byref(p), _ptr(Xd), _ptr(W1p), _ptr(W2p), _ptr(offsets),
                               _ptr(Hd), _ptr(Z), _stream(stream)), "moe_expert_ffn")


def moe_combine(p, Z, ids, gates, pos, accepted, offsets, residual, Y, stream=None):
    _check(_lib.moe_combine(ctypes.byref(p), _ptr(Z), _ptr(ids), _ptr(gates), _ptr(pos),
                            _ptr(accepted), _ptr(offsets), _ptr(residual), _ptr(Y), _stream(stream)),
           "moe_combine")


def moe_aux_loss(p, ids, gates, clean, noise_std, row_stats, counts, importance, load, out, ws,
                 stream=None):
    _check(_lib.moe_aux_loss(ctypes.byref(p), _ptr(ids), _ptr(gates), _ptr(clean), _ptr(noise_std),
                             _ptr(row_stats), _ptr(counts), _ptr(importance), _ptr(load), _ptr(out),
                             _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)),
           "moe_aux_loss")


def hier(groups: int, k_primary: int) -> Hier:
    return Hier(groups=int(groups), k_primary=int(k_primary))


def hier_state(st: dict) -> HierState:
    """HierState from a dict of device tensors (missing / None fields are NULL)."""
    return HierState(**{n: (_ptr(st[n]).value if st.get(n) is not None else None)
                        for n in HIER_STATE_FIELDS})


def moe_hier_workspace_size(p: Problem, h: Hier, which: int) -> int:
    return _lib.moe_hier_workspace_size(ctypes.byref(p), ctypes.byref(h), which)


def moe_route_hier(p, h, X, Wpg, Wpn, Wsg, Wsn, ids, gates, st: dict, ws, stream=None):
    hs = hier_state(st)
    _check(_lib.moe_route_hier(ctypes.byref(p), ctypes.byref(h), _ptr(X), _ptr(Wpg), _ptr(Wpn),
                               _ptr(Wsg), _ptr(Wsn), _ptr(ids), _ptr(gates), ctypes.byref(hs),
                               _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)),
           "moe_route_hier")


def moe_aux_loss_hier(p, h, st: dict, importance, load, out, ws, stream=None):
    hs = hier_state(st)
    _check(_lib.moe_aux_loss_hier(ctypes.byref(p), ctypes.byref(h), ctypes.byref(hs),
                                  _ptr(importance), _ptr(load), _ptr(out), _ptr(ws),
                                  ws.numel() if ws is not None else 0, _stream(stream)),
           "moe_aux_loss_hier")


def batchwise_state(st: dict) -> BatchwiseState:
    return BatchwiseState(**{n: (_ptr(st[n]).value if st.get(n) is not None else None)
                             for n in BATCHWISE_STATE_FIELDS})


def moe_batchwise_m(p: Problem) -> int:
    m = _lib.moe_batchwise_m(ctypes.byref(p))
    if m < 0:
        raise MoEError(-1, "moe_batchwise_m")
    return m


def moe_batchwise_workspace_size(p: Problem, which: int) -> int:
    return _lib.moe_batchwise_workspace_size(ctypes.byref(p), which)


def moe_route_batchwise(p, X, Wg, bias, clean, st: dict, ws, stream=None):
    bs = batchwise_state(st)
    _check(_lib.moe_route_batchwise(ctypes.byref(p), _ptr(X), _ptr(Wg), _ptr(bias), _ptr(clean),
                                    ctypes.byref(bs), _ptr(ws), ws.numel() if ws is not None else 0,
                                    _stream(stream)), "moe_route_batchwise")


def moe_dispatch_batchwise(p, X, st: dict, Xd, stream=None):
    bs = batchwise_state(st)
    _check(_lib.moe_dispatch_batchwise(ctypes.byref(p), _ptr(X), ctypes.byref(bs), _ptr(Xd),
                                       _stream(stream)), "moe_dispatch_batchwise")


def moe_combine_batchwise(p, Z, st: dict, residual, Y, stream=None):
    bs = batchwise_state(st)
    _check(_lib.moe_combine_batchwise(ctypes.byref(p), _ptr(Z), ctypes.byref(bs), _ptr(residual),
                                      _ptr(Y), _stream(stream)), "moe_combine_batchwise")


def moe_aux_loss_batchwise(p, st: dict, thresholds, importance, out, ws, stream=None):
    bs = batchwise_state(st)
    _check(_lib.moe_aux_loss_batchwise(ctypes.byref(p), ctypes.byref(bs), _ptr(thresholds),
                                       _ptr(importance), _ptr(out), _ptr(ws),
                                       ws.numel() if ws is not None else 0, _stream(stream)),
           "moe_aux_loss_batchwise")


def moe_pack_expert_weights_t(p, W1, W2, W1t, W2t, stream=None):
    _check(_lib.moe_pack_expert_weights_t(ctypes.byref(p), _ptr(W1), _ptr(W2), _ptr(W1t),
                                          _ptr(W2t), _stream(stream)), "moe_pack_expert_weights_t")


def moe_combine_backward(p, dY, Z, ids, gates, pos, accepted, offsets, dZ, dgates, stream=None):
    _check(_lib.moe_combine_backward(ctypes.byref(p), _ptr(dY), _ptr(Z), _ptr(ids), _ptr(gates),
                                     _ptr(pos), _ptr(accepted), _ptr(offsets), _ptr(dZ),
                                     _ptr(dgates), _stream(stream)), "moe_combine_backward")


def moe_expert_ffn_backward(p, Xd, Hd, dZ, W1t, W2t, offsets, dHp, dXd, dW1, dW2, stream=None):
    _check(_lib.moe_expert_ffn_backward(ctypes.byref(p), _ptr(Xd), _ptr(Hd), _ptr(dZ), _ptr(W1t),
                                        _ptr(W2t), _ptr(offsets), _ptr(dHp), _ptr(dXd), _ptr(dW1),
                                        _ptr(dW2), _stream(stream)), "moe_expert_ffn_backward")


def moe_expert_ffn_backward_recompute(p, Xd, W1p, dZ, W1t, W2t, offsets, Hd_scratch, dHp, dXd,
                                      dW1, dW2, stream=None):
    _check(_lib.moe_expert_ffn_backward_recompute(
        ctypes.byref(p), _ptr(Xd), _ptr(W1p), _ptr(dZ), _ptr(W1t), _ptr(W2t), _ptr(offsets),
        _ptr(Hd_scratch), _ptr(dHp), _ptr(dXd), _ptr(dW1), _ptr(dW2), _stream(stream)),
        "moe_expert_ffn_backward_recompute")


def moe_expert_weight_grad(p, which, A, B, offsets, C, stream=None):
    _check(_lib.moe_expert_weight_grad(ctypes.byref(p), int(which), _ptr(A), _ptr(B),
                                       _ptr(offsets), _ptr(C), _stream(stream)),
           "moe_expert_weight_grad")


def moe_route_backward_switch(p, X, Wg, ids, clean, dgates, importance, counts, w_imp, w_switch,
                              dY_residual, dXd, pos, accepted, offsets, dX, dWg, dbias, ws,
                              stream=None):
    _check(_lib.moe_route_backward_switch(
        ctypes.byref(p), _ptr(X), _ptr(Wg), _ptr(ids), _ptr(clean), _ptr(dgates),
        _ptr(importance), _ptr(counts), float(w_imp), float(w_switch), _ptr(dY_residual),
        _ptr(dXd), _ptr(pos), _ptr(accepted), _ptr(offsets), _ptr(dX), _ptr(dWg), _ptr(dbias),
        _ptr(ws), ws.numel() if ws is not None else 0, _stream(stream)),
        "moe_route_backward_switch")


def moe_backward_workspace_size(p: Problem) -> int:
    return _lib.moe_backward_workspace_size(ctypes.byref(p))


def moe_route_scores(p, route_ws) -> int:
    """Device address (int, 0 if none) of the noisy scores in a route workspace."""
    return _lib.moe_route_scores(ctypes.byref(p), _ptr(route_ws)) or 0


def moe_route_backward(p, X, Wg, Wnoise, eps, ids, gates, clean, noise_std, row_stats, dgates,
                       importance, load, w_imp, w_load, dY_residual, dXd, pos, accepted, offsets,
                       dX, dWg, dWnoise, dbias, ws, stream=None, scores=None):
    """scores: a device address from moe_route_scores (or None)."""
    _check(_lib.moe_route_backward(ctypes.byref(p), _ptr(X), _ptr(Wg), _ptr(Wnoise), _ptr(eps),
                                   ctypes.c_void_p(scores) if scores else None, _ptr(ids), _ptr(gates), _ptr(clean), _ptr(noise_std),
                                   _ptr(row_stats), _ptr(dgates), _ptr(importance), _ptr(load),
                                   float(w_imp), float(w_load), _ptr(dY_residual), _ptr(dXd),
                                   _ptr(pos), _ptr(accepted), _ptr(offsets), _ptr(dX), _ptr(dWg),
                                   _ptr(dWnoise), _ptr(dbias), _ptr(ws),
                                   ws.numel() if ws is not None else 0, _stream(stream)),
           "moe_route_backward")


def moe_check_finite(stream=None):
    _check(_lib.moe_check_finite(_stream(stream)), "moe_check_finite")


# ------------------------------------------------------------------ whole layer
@dataclass
class Buffers:
    ids: torch.Tensor
    gates: torch.Tensor
    clean: torch.Tensor
    noise_std: torch.Tensor | None
    row_stats: torch.Tensor
    pos: torch.Tensor
    accepted: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    row_token: torch.Tensor
    Xd: torch.Tensor
    Hd: torch.Tensor
    Z: torch.Tensor
    Y: torch.Tensor
    importance: torch.Tensor
    load: torch.Tensor
    aux_out: torch.Tensor
    ws_route: torch.Tensor
    ws_dispatch: torch.Tensor
    ws_aux: torch.Tensor


class Layer:
    """One MoE layer's device buffers plus the five C-ABI stages in order.

    Weights are given in the pages' layout (W1 [E,D,H], W2 [E,H,D]) and packed
    once at construction. forward() enqueues route, dispatch, expert FFN,
    combine and aux on the current stream and returns the buffers.
    """

    def __init__(self, p: Problem, Wg, Wnoise, bias, W1, W2, device="cuda"):
        self.p = p
        dt = torch_dtype(p)
        T, D, E, H, k = p.T, p.D, p.E, p.H, p.k
        rows = moe_max_rows(p)
        noisy = p.gating == MOE_GATE_NOISY_TOPK and p.noise == 1
        e = lambda *s, dtype=torch.float32: torch.empty(*s, dtype=dtype, device=device)
        self.Wg, self.Wnoise, self.bias = Wg, Wnoise, bias
        self.W1, self.W2 = W1, W2
        self.grads = None
        # True once a dispatch has copied the current rows into Xd; a slots-only dispatch
        # (rows gathered by layer 1) leaves Xd unwritten, and the backward needs it
        self.xd_current = False
        self.W1p = e(moe_packed_weight_bytes(p, 1), dtype=torch.uint8)
        self.W2p = e(moe_packed_weight_bytes(p, 2), dtype=torch.uint8)
        moe_pack_expert_weights(p, W1, W2, self.W1p, self.W2p)
        self.b = Buffers(
            ids=e(T, k, dtype=torch.int32), gates=e(T, k), clean=e(T, E),
            noise_std=e(T, E) if noisy else None, row_stats=e(T, 2),
            pos=e(T, k, dtype=torch.int32), accepted=e(T, k, dtype=torch.uint8),
            counts=e(E, dtype=torch.int32), offsets=e(E + 1, dtype=torch.int32),
            row_token=e(max(rows, 1), dtype=torch.int32), Xd=e(max(rows, 1), D, dtype=dt),
            Hd=e(max(rows, 1), H, dtype=dt), Z=e(max(rows, 1), D, dtype=dt), Y=e(T, D, dtype=dt),
            importance=e(E), load=e(E), aux_out=e(8),
            ws_route=e(max(moe_workspace_size(p, MOE_WS_ROUTE), 1), dtype=torch.uint8),
            ws_dispatch=e(max(moe_workspace_size(p, MOE_WS_DISPATCH), 1), dtype=torch.uint8),
            ws_aux=e(max(moe_workspace_size(p, MOE_WS_AUX), 1), dtype=torch.uint8),
        )

    def route(self, X, eps=None):
        b = self.b
        moe_route(self.p, X, self.Wg, self.Wnoise, self.bias, eps, b.ids, b.gates, b.clean,
                  b.noise_std, b.row_stats, b.ws_route)

    def dispatch(self, X, rows=True):
        """rows=False: slots and groups only; layer 1 then gathers X itself (gemm(1, X))."""
        b = self.b
        self.xd_current = False
        moe_dispatch(self.p, X, b.ids, b.pos, b.accepted, b.counts, b.offsets, b.row_token,
                     b.Xd if rows else None, b.ws_dispatch)
        self.xd_current = rows

    def ffn(self, X=None):
        """X given: layer 1 reads its rows through row_token (no Xd needed)."""
        b = self.b
        if X is not None:
            moe_expert_ffn_gather(self.p, X, b.row_token, self.W1p, self.W2p, b.offsets, b.Hd, b.Z)
        else:
            moe_expert_ffn(self.p, b.Xd, self.W1p, self.W2p, b.offsets, b.Hd, b.Z)

    def gemm(self, layer, X=None):
        b = self.b
        if layer == 1 and X is not None:
            moe_grouped_gemm_gather(self.p, X, b.row_token, self.W1p, b.offsets, b.Hd)
        elif layer == 1:
            moe_grouped_gemm(self.p, 1, b.Xd, self.W1p, b.offsets, b.Hd)
        else:
            moe_grouped_gemm(self.p, 2, b.Hd, self.W2p, b.offsets, b.Z)

    def combine(self, X, residual=True):
        b = self.b
        moe_combine(self.p, b.Z, b.ids, b.gates, b.pos, b.accepted, b.offsets,
                    X if residual else None, b.Y)

    def aux(self):
        b = self.b
        moe_aux_loss(self.p, b.ids, b.gates, b.clean, b.noise_std, b.row_stats, b.counts,
                     b.importance, b.load, b.aux_out, b.ws_aux)

    def backward_buffers(self, weight_grads=True) -> dict:
        """Gradient buffers (allocated on first use) and the transposed packed weights."""
        p = self.p
        if self.grads is None or (weight_grads and self.grads["dW1"] is None):
            e = lambda *s, dtype=torch.float32: torch.empty(*s, dtype=dtype, device=self.b.Y.device)
            dt = torch_dtype(p)
            rows = max(moe_max_rows(p), 1)
            noisy = p.gating == MOE_GATE_NOISY_TOPK and p.noise == 1
            if self.grads is None:
                self.W1t = e(moe_packed_weight_bytes(p, 4), dtype=torch.uint8)
                self.W2t = e(moe_packed_weight_bytes(p, 3), dtype=torch.uint8)
                moe_pack_expert_weights_t(p, self.W1, self.W2, self.W1t, self.W2t)
            self.grads = dict(
                dZ=e(rows, p.D, dtype=dt), dgates=e(p.T, p.k), dHp=e(rows, p.H, dtype=dt),
                dXd=e(rows, p.D, dtype=dt), dX=e(p.T, p.D, dtype=dt), dWg=e(p.D, p.E),
                dWnoise=e(p.D, p.E) if noisy else None, dbias=e(p.E),
                dW1=e(p.E, p.D, p.H) if weight_grads else None,
                dW2=e(p.E, p.H, p.D) if weight_grads else None,
                ws=e(max(moe_backward_workspace_size(p), 1), dtype=torch.uint8))
        return self.grads

    def backward_combine(self, dY):
        b, g = self.b, self.grads
        moe_combine_backward(self.p, dY, b.Z, b.ids, b.gates, b.pos, b.accepted, b.offsets,
                             g["dZ"], g["dgates"])

    def backward_ffn(self, weight_grads=True, recompute=False):
        """recompute: Hd is recomputed from Xd into a scratch buffer instead of read from
        the forward's (the memory-for-compute trade of not storing it)."""
        b, g = self.b, self.grads
        if not self.xd_current:
            raise RuntimeError("the expert backward reads the dispatched rows Xd, which the last "
                               "dispatch did not copy (forward(gather=True)); call "
                               "dispatch(X, rows=True) first, as backward(X, ...) does")
        dW1 = g["dW1"] if weight_grads else None
        dW2 = g["dW2"] if weight_grads else None
        if recompute:
            if "Hs" not in g:
                g["Hs"] = torch.empty_like(b.Hd)
            moe_expert_ffn_backward_recompute(self.p, b.Xd, self.W1p, g["dZ"], self.W1t, self.W2t,
                                              b.offsets, g["Hs"], g["dHp"], g["dXd"], dW1, dW2)
        else:
            moe_expert_ffn_backward(self.p, b.Xd, b.Hd, g["dZ"], self.W1t, self.W2t, b.offsets,
                                    g["dHp"], g["dXd"], dW1, dW2)

    def backward_route(self, X, dY, w_imp=0.0, w_load=0.0, residual=True, eps=None,
                       w_switch=0.0):
        """Noisy top-k: w_imp, w_load; Switch: w_imp, w_switch (the E * sum f * Pbar term)."""
        b, g = self.b, self.grads
        if self.p.gating == MOE_GATE_SWITCH_TOP1:
            if w_load or eps is not None:
                raise ValueError("the Switch gate has no load term and no noise")
            moe_route_backward_switch(self.p, X, self.Wg, b.ids, b.clean, g["dgates"],
                                      b.importance, b.counts, w_imp, w_switch,
                                      dY if residual else None, g["dXd"], b.pos, b.accepted,
                                      b.offsets, g["dX"], g["dWg"], g["dbias"], g["ws"])
            return
        if w_switch:
            raise ValueError("w_switch applies to the Switch gate")
        # the noisy scores the forward selected on (still in the route workspace)
        scores = moe_route_scores(self.p, b.ws_route)
        moe_route_backward(self.p, X, self.Wg, self.Wnoise, eps, b.ids, b.gates, b.clean,
                           b.noise_std, b.row_stats, g["dgates"], b.importance, b.load, w_imp,
                           w_load, dY if residual else None, g["dXd"], b.pos, b.accepted,
                           b.offsets, g["dX"], g["dWg"], g["dWnoise"], g["dbias"], g["ws"],
                           scores=scores)

    def backward(self, X, dY, w_imp=0.0, w_load=0.0, residual=True, eps=None,
                 weight_grads=True, recompute=False, w_switch=0.0) -> dict:
        """Gradients after forward(X) (with aux, whose importance and load the balancing
        terms use): dX, dWg, dWnoise, dbias, dW1, dW2 (fp32 weight gradients) of the
        objective <Y, dY> + w_imp CV^2(importance) + w_load CV^2(load)."""
        self.backward_buffers(weight_grads)
        if not self.xd_current:  # a gathered forward: copy the rows now (the same slots)
            self.dispatch(X, rows=True)
        self.backward_combine(dY)
        self.backward_ffn(weight_grads, recompute)
        self.backward_route(X, dY, w_imp, w_load, residual, eps, w_switch)
        return self.grads

    def forward(self, X, eps=None, residual=True, aux=True, gather=False) -> Buffers:
        """gather: the dispatch copies no rows and layer 1 reads X through row_token."""
        self.route(X, eps)
        self.dispatch(X, rows=not gather)
        self.ffn(X if gather else None)
        self.combine(X, residual)
        if aux:
            self.aux()
        return self.b


class HierLayer(Layer):
    """A hierarchical MoE layer: two-level routing (moe_route_hier), then the flat
    dispatch, expert FFN and combine over all E experts, and the hierarchical
    balancing terms (moe_aux_loss_hier)."""

    def __init__(self, p: Problem, h: Hier, Wpg, Wpn, Wsg, Wsn, W1, W2, device="cuda"):
        super().__init__(p, None, None, None, W1, W2, device=device)
        self.h = h
        self.Wpg, self.Wpn, self.Wsg, self.Wsn = Wpg, Wpn, Wsg, Wsn
        T, a, kp = p.T, h.groups, h.k_primary
        b, ks = p.E // a, p.k // kp
        R = T * kp
        noisy = p.noise == 1
        e = lambda *s, dtype=torch.float32: torch.empty(*s, dtype=dtype, device=device)
        self.st = dict(
            ids_p=e(T, kp, dtype=torch.int32), gates_p=e(T, kp), clean_p=e(T, a),
            std_p=e(T, a) if noisy else None, row_stats_p=e(T, 2),
            pos_p=e(T, kp, dtype=torch.int32), accepted_p=e(T, kp, dtype=torch.uint8),
            counts_p=e(a, dtype=torch.int32), offsets_p=e(a + 1, dtype=torch.int32),
            row_token_p=e(R, dtype=torch.int32), clean_s=e(R, b),
            std_s=e(R, b) if noisy else None, row_stats_s=e(R, 2),
            ids_s=e(R, ks, dtype=torch.int32), gates_s=e(R, ks))
        self.ws_route_h = e(max(moe_hier_workspace_size(p, h, MOE_WS_ROUTE), 1), dtype=torch.uint8)
        self.ws_aux_h = e(max(moe_hier_workspace_size(p, h, MOE_WS_AUX), 1), dtype=torch.uint8)

    def route(self, X, eps=None):
        if eps is not None:
            raise ValueError("the hierarchical router draws its own noise")
        b = self.b
        moe_route_hier(self.p, self.h, X, self.Wpg, self.Wpn, self.Wsg, self.Wsn, b.ids, b.gates,
                       self.st, self.ws_route_h)

    def aux(self):
        b = self.b
        moe_aux_loss_hier(self.p, self.h, self.st, b.importance, b.load, b.aux_out, self.ws_aux_h)

    def backward(self, *args, **kw):
        raise NotImplementedError("the hierarchical gate has no backward pass here")


class BatchwiseLayer:
    """The MoE layer with the batchwise mask: route (scores, mask, gates), dispatch
    (gather of the E*m rows), expert FFN (grouped GEMMs over offsets e*m), combine,
    aux; same stage names as Layer."""

    def __init__(self, p: Problem, Wg, bias, W1, W2, device="cuda", thresholds=None):
        self.p = p
        dt = torch_dtype(p)
        T, D, E, H = p.T, p.D, p.E, p.H
        m = moe_batchwise_m(p)
        R = E * m
        W = (E + 31) // 32
        e = lambda *s, dtype=torch.float32: torch.empty(*s, dtype=dtype, device=device)
        self.Wg, self.bias, self.thresholds = Wg, bias, thresholds
        self.W1p = e(moe_packed_weight_bytes(p, 1), dtype=torch.uint8)
        self.W2p = e(moe_packed_weight_bytes(p, 2), dtype=torch.uint8)
        moe_pack_expert_weights(p, W1, W2, self.W1p, self.W2p)
        self.m = m
        self.st = dict(probs_t=e(E, T), sel=e(R, dtype=torch.int32),
                       offsets=e(E + 1, dtype=torch.int32), mask=e(T, W, dtype=torch.int32),
                       tok_count=e(T, dtype=torch.int32), tok_off=e(T + 1, dtype=torch.int32),
                       tok_row=e(R, dtype=torch.int32), tok_gate=e(R),
                       slot_pair=e(R, dtype=torch.int32))
        self.clean = e(T, E)
        self.Xd, self.Hd, self.Z = e(R, D, dtype=dt), e(R, H, dtype=dt), e(R, D, dtype=dt)
        self.Y = e(T, D, dtype=dt)
        self.importance, self.aux_out = e(E), e(8)
        self.ws_route = e(max(moe_batchwise_workspace_size(p, MOE_WS_ROUTE), 1), dtype=torch.uint8)
        self.ws_aux = e(max(moe_batchwise_workspace_size(p, MOE_WS_AUX), 1), dtype=torch.uint8)

    def route(self, X):
        moe_route_batchwise(self.p, X, self.Wg, self.bias, self.clean, self.st, self.ws_route)

    def dispatch(self, X):
        moe_dispatch_batchwise(self.p, X, self.st, self.Xd)

    def gemm(self, layer):
        if layer == 1:
            moe_grouped_gemm(self.p, 1, self.Xd, self.W1p, self.st["offsets"], self.Hd)
        else:
            moe_grouped_gemm(self.p, 2, self.Hd, self.W2p, self.st["offsets"], self.Z)

    def ffn(self):
        moe_expert_ffn(self.p, self.Xd, self.W1p, self.W2p, self.st["offsets"], self.Hd, self.Z)

    def combine(self, X, residual=True):
        moe_combine_batchwise(self.p, self.Z, self.st, X if residual else None, self.Y)

    def aux(self):
        moe_aux_loss_batchwise(self.p, self.st, self.thresholds, self.importance, self.aux_out,
                               self.ws_aux)

    def forward(self, X, residual=True, aux=True):
        self.route(X)
        self.dispatch(X)
        self.ffn()
        self.combine(X, residual)
        if aux:
            self.aux()
        return self
