"""ctypes binding of the CPU oracle (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this module.  Arrays are numpy; bf16 data is passed as its raw uint16 bit
pattern.  Every call builds the oracle library first if it is missing.
"""
import ctypes
import dataclasses
import os
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

from . import build as _build

F32, BF16 = 0, 1
GATE_SOFTMAX_TOPK, GATE_TOPK_SOFTMAX = 0, 1
ACT_SWIGLU, ACT_RELU = 0, 1
DROP_TOKEN_ORDER, DROP_CHOICE_RANK = 0, 1

_lib = None


class _Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("N", ctypes.c_int32),
                ("K", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("d_ff_shared", ctypes.c_int32),
                ("capacity_factor", ctypes.c_float), ("noise_weight", ctypes.c_float),
                ("gating", ctypes.c_int32), ("act", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("drop_order", ctypes.c_int32)]


class _Inputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("u", "w_router", "b_router", "noise", "w_gate", "w_up", "w_down",
                 "ws_gate", "ws_up", "ws_down")]


@dataclass
class Problem:
    T: int
    d: int
    N: int
    K: int
    d_ff: int
    n_shared: int = 0
    d_ff_shared: int = 0
    capacity_factor: float = 0.0
    noise_weight: float = 0.0
    gating: int = GATE_TOPK_SOFTMAX
    act: int = ACT_SWIGLU
    dtype: int = F32
    drop_order: int = DROP_TOKEN_ORDER

    def c(self) -> _Problem:
        return _Problem(self.T, self.d, self.N, self.K, self.d_ff, self.n_shared,
                        self.d_ff_shared, self.capacity_factor, self.noise_weight,
                        self.gating, self.act, self.dtype, self.drop_order)


def nthreads_default() -> int:
    """Host threads for the oracle: the usable cores, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        P = ctypes.POINTER(_Problem)
        I = ctypes.POINTER(_Inputs)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.oracle_round_bf16.argtypes = [ctypes.c_double]
        L.oracle_round_bf16.restype = ctypes.c_double
        L.oracle_router_logits.argtypes = [P, I, vp, ctypes.c_int]
        L.oracle_route.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.oracle_capacity.argtypes = [i32, i32, i32, ctypes.c_float]
        L.oracle_capacity.restype = i32
        L.oracle_dispatch.argtypes = [P, vp, i32, vp, vp, vp, vp, vp]
        L.oracle_ffn_rows.argtypes = [P, I, i32, vp, vp, vp, ctypes.c_int]
        L.oracle_layer_rows.argtypes = [P, I, vp, vp, vp, i32, vp, vp, ctypes.c_int]
        L.oracle_combine.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.oracle_layer_forward.argtypes = [P, I] + [vp] * 11 + [ctypes.c_int]
        L.oracle_router_stats.argtypes = [P, vp, vp, vp, vp]
        L.oracle_ec_capacity.argtypes = [i32, i32, i32, ctypes.c_float]
        L.oracle_ec_capacity.restype = i32
        L.oracle_ec_select.argtypes = [P, vp, i32, vp, vp, vp, vp]
        L.oracle_combine_backward.argtypes = [P, vp, vp, vp, vp, vp, vp]
        L.oracle_route_backward.argtypes = [P, vp, vp, vp, vp, vp]
        L.oracle_router_param_grads.argtypes = [P, I, vp, vp, vp, vp, ctypes.c_int]
        L.oracle_ffn_backward_rows.argtypes = [P, I, i32, vp, vp, vp, vp, ctypes.c_int]
        L.oracle_ffn_weight_grads.argtypes = [P, I, i32, i32, vp, vp, i32, vp, vp, vp, vp,
                                              ctypes.c_int]
        L.oracle_layer_backward_rows.argtypes = [P, I, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp,
                                                 ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _elem_array(a, dtype: int) -> np.ndarray:
    a = np.ascontiguousarray(a)
    want = np.uint16 if dtype == BF16 else np.float32
    assert a.dtype == want, f"expected {want}, got {a.dtype}"
    return a


class Inputs:
    """Holds the numpy arrays (keeping them alive) and their C view."""

    def __init__(self, p: Problem, u, w_router=None, b_router=None, noise=None,
                 w_gate=None, w_up=None, w_down=None, ws_gate=None, ws_up=None,
                 ws_down=None):
        self.arrays = {}

        def keep(name, a, elem):
            if a is None:
                self.arrays[name] = None
                return
            if elem:
                a = _elem_array(a, p.dtype)
            else:
                a = np.ascontiguousarray(a, dtype=np.float32)
            self.arrays[name] = a

        keep("u", u, True)
        keep("w_router", w_router, False)
        keep("b_router", b_router, False)
        keep("noise", noise, False)
        for n, a in (("w_gate", w_gate), ("w_up", w_up), ("w_down", w_down),
                     ("ws_gate", ws_gate), ("ws_up", ws_up), ("ws_down", ws_down)):
            keep(n, a, True)
        self.c = _Inputs(*[_ptr(self.arrays[n]) for n, _ in _Inputs._fields_])


def round_bf16(v: float) -> float:
    return lib().oracle_round_bf16(float(v))


def router_logits(p: Problem, x: Inputs, nthreads: Optional[int] = None) -> np.ndarray:
    H = np.zeros((p.T, p.N), dtype=np.float32)
    lib().oracle_router_logits(ctypes.byref(p.c()), ctypes.byref(x.c), _ptr(H),
                               nthreads or nthreads_default())
    return H


def route(p: Problem, H: np.ndarray, want_probs: bool = False) -> Dict[str, np.ndarray]:
    H = np.ascontiguousarray(H, dtype=np.float32)
    assert H.shape == (p.T, p.N)
    out = dict(topk_idx=np.zeros((p.T, p.K), np.int32),
               topk_gate=np.zeros((p.T, p.K), np.float64),
               lse_sq=np.zeros(p.T, np.float64),
               mean_prob=np.zeros(p.N, np.float64))
    if want_probs:
        out["probs"] = np.zeros((p.T, p.N), np.float64)
    lib().oracle_route(ctypes.byref(p.c()), _ptr(H), _ptr(out["topk_idx"]),
                       _ptr(out["topk_gate"]), _ptr(out["lse_sq"]),
                       _ptr(out["mean_prob"]), _ptr(out.get("probs")))
    return out


def capacity(T: int, K: int, N: int, cf: float) -> int:
    return int(lib().oracle_capacity(T, K, N, cf))


def dispatch(p: Problem, topk_idx: np.ndarray, C: Optional[int] = None) -> Dict[str, np.ndarray]:
    if C is None:
        C = capacity(p.T, p.K, p.N, p.capacity_factor)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    assert idx.shape == (p.T, p.K)
    out = dict(expert_counts=np.zeros(p.N, np.int32), kept_counts=np.zeros(p.N, np.int32),
               offsets=np.zeros(p.N + 1, np.int32), row_of=np.zeros((p.T, p.K), np.int32),
               token_of_row=np.zeros(p.T * p.K, np.int32))
    lib().oracle_dispatch(ctypes.byref(p.c()), _ptr(idx), int(C), _ptr(out["expert_counts"]),
                          _ptr(out["kept_counts"]), _ptr(out["offsets"]), _ptr(out["row_of"]),
                          _ptr(out["token_of_row"]))
    out["capacity"] = C
    return out


def ffn_rows(p: Problem, x: Inputs, rows: np.ndarray, expert_of_row: np.ndarray,
             nthreads: Optional[int] = None) -> np.ndarray:
    rows = _elem_array(rows, p.dtype)
    e = np.ascontiguousarray(expert_of_row, dtype=np.int32)
    n = e.shape[0]
    assert rows.shape == (n, p.d)
    y = np.zeros((n, p.d), np.float64)
    lib().oracle_ffn_rows(ctypes.byref(p.c()), ctypes.byref(x.c), n, _ptr(rows), _ptr(e),
                          _ptr(y), nthreads or nthreads_default())
    return y


def layer_rows(p: Problem, x: Inputs, topk_idx, topk_gate, row_of, tokens=None,
               nthreads: Optional[int] = None) -> np.ndarray:
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    gate = np.ascontiguousarray(topk_gate, dtype=np.float64)
    rof = np.ascontiguousarray(row_of, dtype=np.int32)
    if tokens is None:
        n, tok = p.T, None
    else:
        tok = np.ascontiguousarray(tokens, dtype=np.int32)
        n = tok.shape[0]
    out = np.zeros((n, p.d), np.float64)
    lib().oracle_layer_rows(ctypes.byref(p.c()), ctypes.byref(x.c), _ptr(idx), _ptr(gate),
                            _ptr(rof), n, _ptr(tok), _ptr(out), nthreads or nthreads_default())
    return out


def combine(p: Problem, u, y, row_of, topk_gate, y_shared=None) -> np.ndarray:
    u = _elem_array(u, p.dtype)
    y = _elem_array(y, p.dtype)
    ys = None if y_shared is None else _elem_array(y_shared, p.dtype)
    rof = np.ascontiguousarray(row_of, dtype=np.int32)
    gate = np.ascontiguousarray(topk_gate, dtype=np.float64)
    assert u.shape == (p.T, p.d) and y.shape == (p.T * p.K, p.d) and rof.shape == (p.T, p.K)
    out = np.zeros((p.T, p.d), np.float64)
    lib().oracle_combine(ctypes.byref(p.c()), _ptr(u), _ptr(y), _ptr(rof), _ptr(gate), _ptr(ys),
                         _ptr(out))
    return out


def layer_forward(p: Problem, x: Inputs, nthreads: Optional[int] = None) -> Dict[str, np.ndarray]:
    T, N, K = p.T, p.N, p.K
    o = dict(scores=np.zeros((T, N), np.float32), topk_idx=np.zeros((T, K), np.int32),
             topk_gate=np.zeros((T, K), np.float64), lse_sq=np.zeros(T, np.float64),
             mean_prob=np.zeros(N, np.float64), expert_counts=np.zeros(N, np.int32),
             kept_counts=np.zeros(N, np.int32), offsets=np.zeros(N + 1, np.int32),
             row_of=np.zeros((T, K), np.int32), token_of_row=np.zeros(T * K, np.int32),
             out=np.zeros((T, p.d), np.float64))
    names = ["scores", "topk_idx", "topk_gate", "lse_sq", "mean_prob", "expert_counts",
             "kept_counts", "offsets", "row_of", "token_of_row", "out"]
    lib().oracle_layer_forward(ctypes.byref(p.c()), ctypes.byref(x.c),
                               *[_ptr(o[n]) for n in names], nthreads or nthreads_default())
    return o


STAT_NAMES = ("f_var", "p_var", "p_entropy", "z_loss")


def router_stats(p: Problem, expert_counts, mean_prob, lse_sq) -> Dict[str, float]:
    """Variance of the assignment fractions, variance and entropy of the mean
    probabilities, and the mean of lse^2 (see oracle_router_stats)."""
    cnt = np.ascontiguousarray(expert_counts, dtype=np.int32)
    mp = np.ascontiguousarray(mean_prob, dtype=np.float64)
    ls = np.ascontiguousarray(lse_sq, dtype=np.float64)
    assert cnt.shape == (p.N,) and mp.shape == (p.N,) and ls.shape == (p.T,)
    st = np.zeros(4, np.float64)
    lib().oracle_router_stats(ctypes.byref(p.c()), _ptr(cnt), _ptr(mp), _ptr(ls), _ptr(st))
    return dict(zip(STAT_NAMES, st.tolist()))


def ec_capacity(T: int, K: int, N: int, cf: float) -> int:
    return int(lib().oracle_ec_capacity(T, K, N, float(cf)))


def ec_select(p: Problem, probs, C: int) -> Dict[str, np.ndarray]:
    """Expert-choice selection from affinities probs [T][N] (see
    oracle_ec_select)."""
    pr = np.ascontiguousarray(probs, dtype=np.float64)
    assert pr.shape == (p.T, p.N) and 0 <= C <= p.T
    o = dict(expert_tokens=np.zeros((p.N, C), np.int32), expert_gates=np.zeros((p.N, C), np.float64),
             row_of=np.zeros((p.T, p.N), np.int32), gate_of=np.zeros((p.T, p.N), np.float64))
    lib().oracle_ec_select(ctypes.byref(p.c()), _ptr(pr), C, _ptr(o["expert_tokens"]),
                           _ptr(o["expert_gates"]), _ptr(o["row_of"]), _ptr(o["gate_of"]))
    return o


def ec_layer_rows(p: Problem, x: Inputs, sel: Dict[str, np.ndarray], tokens=None,
                  nthreads: Optional[int] = None) -> np.ndarray:
    """Layer output of expert choice: u_t + sum over the experts that chose
    t, in ascending expert order, of s * FFN_e(u_t) (+ shared experts) -- the
    token-choice sum with one slot per expert."""
    pe = dataclasses.replace(p, K=p.N)
    idx = np.tile(np.arange(p.N, dtype=np.int32), (p.T, 1))
    return layer_rows(pe, x, idx, sel["gate_of"], sel["row_of"], tokens, nthreads)


# ------------------------------------------------------------------ backward

def _f64(a, shape=None):
    a = np.ascontiguousarray(a, dtype=np.float64)
    if shape is not None:
        assert a.shape == tuple(shape), (a.shape, shape)
    return a


def combine_backward(p: Problem, d_out, y, row_of, gate) -> Dict[str, np.ndarray]:
    """dy [T*K][d] (rows no kept assignment references are 0) and d_gate [T][K]."""
    do = _f64(d_out, (p.T, p.d))
    yy = _elem_array(y, p.dtype)
    rof = np.ascontiguousarray(row_of, dtype=np.int32)
    g = _f64(gate, (p.T, p.K))
    assert yy.shape == (p.T * p.K, p.d) and rof.shape == (p.T, p.K)
    o = dict(dy=np.zeros((p.T * p.K, p.d)), d_gate=np.zeros((p.T, p.K)))
    lib().oracle_combine_backward(ctypes.byref(p.c()), _ptr(do), _ptr(yy), _ptr(rof), _ptr(g),
                                  _ptr(o["dy"]), _ptr(o["d_gate"]))
    return o


def route_backward(p: Problem, H, topk_idx, topk_gate, d_gate) -> np.ndarray:
    """dH [T][N]: the gating Jacobian applied to d_gate."""
    h = np.ascontiguousarray(H, dtype=np.float32)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    g = _f64(topk_gate, (p.T, p.K))
    dg = _f64(d_gate, (p.T, p.K))
    dH = np.zeros((p.T, p.N))
    lib().oracle_route_backward(ctypes.byref(p.c()), _ptr(h), _ptr(idx), _ptr(g), _ptr(dg), _ptr(dH))
    return dH


def router_param_grads(p: Problem, x: Inputs, dH, nthreads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """dw_router [N][d], db_router [N], du_router [T][d] from dH [T][N]."""
    h = _f64(dH, (p.T, p.N))
    o = dict(dw_router=np.zeros((p.N, p.d)), db_router=np.zeros(p.N), du_router=np.zeros((p.T, p.d)))
    lib().oracle_router_param_grads(ctypes.byref(p.c()), ctypes.byref(x.c), _ptr(h),
                                    _ptr(o["dw_router"]), _ptr(o["db_router"]), _ptr(o["du_router"]),
                                    nthreads or nthreads_default())
    return o


def ffn_backward_rows(p: Problem, x: Inputs, rows, expert_of_row, dy,
                      nthreads: Optional[int] = None) -> np.ndarray:
    """dx [n][d] of the expert FFN of each row (-1: the shared experts)."""
    xr = _elem_array(rows, p.dtype)
    eor = np.ascontiguousarray(expert_of_row, dtype=np.int32)
    n = len(eor)
    dyy = _f64(dy, (n, p.d))
    dx = np.zeros((n, p.d))
    lib().oracle_ffn_backward_rows(ctypes.byref(p.c()), ctypes.byref(x.c), n, _ptr(xr), _ptr(eor),
                                   _ptr(dyy), _ptr(dx), nthreads or nthreads_default())
    return dx


def ffn_weight_grads(p: Problem, x: Inputs, expert: int, rows, dy, f_list,
                     nthreads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Rows f of dW_gate and dW_up, columns f of dW_down (as [n_f][d]) of one
    expert (routed 0..N-1, shared s as -1-s) over the given rows."""
    xr = _elem_array(rows, p.dtype)
    n = xr.shape[0]
    dyy = _f64(dy, (n, p.d))
    fl = np.ascontiguousarray(f_list, dtype=np.int32)
    o = dict(dw_gate=np.zeros((len(fl), p.d)), dw_up=np.zeros((len(fl), p.d)),
             dw_down=np.zeros((len(fl), p.d)))
    lib().oracle_ffn_weight_grads(ctypes.byref(p.c()), ctypes.byref(x.c), int(expert), n, _ptr(xr),
                                  _ptr(dyy), len(fl), _ptr(fl), _ptr(o["dw_gate"]), _ptr(o["dw_up"]),
                                  _ptr(o["dw_down"]), nthreads or nthreads_default())
    return o


def layer_backward_rows(p: Problem, x: Inputs, H, topk_idx, topk_gate, row_of, d_out, tokens=None,
                        nthreads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """du, d_gate and dH of the listed tokens (all when tokens is None)."""
    h = np.ascontiguousarray(H, dtype=np.float32)
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    g = _f64(topk_gate, (p.T, p.K))
    rof = np.ascontiguousarray(row_of, dtype=np.int32)
    do = _f64(d_out, (p.T, p.d))
    tk = None if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    n = p.T if tk is None else len(tk)
    o = dict(du=np.zeros((n, p.d)), d_gate=np.zeros((n, p.K)), dH=np.zeros((n, p.N)))
    lib().oracle_layer_backward_rows(ctypes.byref(p.c()), ctypes.byref(x.c), _ptr(h), _ptr(idx), _ptr(g),
                                     _ptr(rof), _ptr(do), n, _ptr(tk), _ptr(o["du"]), _ptr(o["d_gate"]),
                                     _ptr(o["dH"]), nthreads or nthreads_default())
    return o
