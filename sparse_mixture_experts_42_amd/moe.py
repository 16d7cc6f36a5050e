"""Python binding of libmoe (include/moe.h): argument marshalling only.

Every function of the C ABI is exposed under its own name.  Tensors are
torch tensors on a ROCm device; outputs are allocated with torch and filled
by the HIP kernels.  The work is enqueued on torch's current stream.  If the
library is not built, every call raises: there is no fallback path.
"""
import ctypes
import os
import threading
from typing import Dict, Optional

import torch  # imported first: libmoe then binds to the HIP runtime torch loaded

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_GATE_SOFTMAX_TOPK, MOE_GATE_TOPK_SOFTMAX = 0, 1
MOE_ACT_SWIGLU, MOE_ACT_RELU = 0, 1
MOE_F32, MOE_BF16 = 0, 1
MOE_DROP_TOKEN_ORDER, MOE_DROP_CHOICE_RANK = 0, 1
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20   # static scratch of moe_layer_forward_noalloc, per GPU

GATING = {"softmax_topk": MOE_GATE_SOFTMAX_TOPK, "topk_softmax": MOE_GATE_TOPK_SOFTMAX}
ACT = {"swiglu": MOE_ACT_SWIGLU, "relu": MOE_ACT_RELU}
DTYPE = {"f32": MOE_F32, "bf16": MOE_BF16}
DROP = {"token": MOE_DROP_TOKEN_ORDER, "choice": MOE_DROP_CHOICE_RANK}
TORCH_DTYPE = {MOE_F32: torch.float32, MOE_BF16: torch.bfloat16}


class MoeProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d", ctypes.c_int32), ("N", ctypes.c_int32),
                ("K", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("d_ff_shared", ctypes.c_int32), ("capacity_factor", ctypes.c_float),
                ("noise_weight", ctypes.c_float), ("gating", ctypes.c_int32),
                ("act", ctypes.c_int32), ("dtype", ctypes.c_int32), ("drop_order", ctypes.c_int32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w_router", "b_router", "w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down")]


class MoeLayerOutputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("scores", "topk_idx", "topk_gate", "mean_prob", "lse_sq", "expert_counts",
                 "kept_counts", "offsets", "row_of", "token_of_row", "x_perm", "y_perm",
                 "y_shared", "pre", "pre_shared")]


class MoeEcOutputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("scores", "probs", "expert_tokens", "expert_gates", "row_of", "gate_of",
                 "offsets", "mean_prob", "lse_sq", "x_perm", "y_perm", "y_shared")]


class MoeSaved(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("scores", "topk_idx", "topk_gate", "row_of", "offsets", "x_perm", "y_perm",
                 "pre", "pre_shared")]


class MoeGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("du", "dw_router", "db_router", "dw_gate", "dw_up", "dw_down", "dws_gate",
                 "dws_up", "dws_down", "d_gate", "d_scores", "dy_perm", "dx_perm")]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {moe_status_string(status)}")
        self.status = status


_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded libmoe; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"libmoe is not built ({LIB_PATH} missing): run "
                    "`python -m sparse_mixture_experts_42_amd.build` or __graft_entry__.build()")
            L = ctypes.CDLL(LIB_PATH)
            vp, P, i32, sz = ctypes.c_void_p, ctypes.POINTER(MoeProblem), ctypes.c_int32, ctypes.c_size_t
            L.moe_status_string.argtypes = [ctypes.c_int]
            L.moe_status_string.restype = ctypes.c_char_p
            L.moe_workspace_size.argtypes = [P]
            L.moe_workspace_size.restype = sz
            L.moe_capacity.argtypes = [i32, i32, i32, ctypes.c_float]
            L.moe_capacity.restype = i32
            L.moe_ffn_row_tile.argtypes = [i32, i32, i32]
            L.moe_ffn_row_tile.restype = i32
            L.moe_route.argtypes = [P] + [vp] * 10 + [sz, vp]
            L.moe_dispatch.argtypes = [P] + [vp] * 9 + [sz, vp]
            L.moe_grouped_ffn.argtypes = [P] + [vp] * 12 + [sz, vp]
            L.moe_combine.argtypes = [P] + [vp] * 7 + [sz, vp]
            L.moe_layer_forward.argtypes = [P, vp, vp, ctypes.POINTER(MoeWeights),
                                            ctypes.POINTER(MoeLayerOutputs), vp, vp, sz, vp]
            L.moe_layer_forward_noalloc.argtypes = [P, vp, vp, ctypes.POINTER(MoeWeights),
                                                    ctypes.POINTER(MoeLayerOutputs), vp, vp]
            L.moe_router_stats.argtypes = [P] + [vp] * 5
            L.moe_ec_capacity.argtypes = [i32, i32, i32, ctypes.c_float]
            L.moe_ec_capacity.restype = i32
            L.moe_ec_workspace_size.argtypes = [P]
            L.moe_ec_workspace_size.restype = sz
            L.moe_ec_route.argtypes = [P] + [vp] * 14 + [sz, vp]
            L.moe_ec_dispatch.argtypes = [P] + [vp] * 4
            L.moe_ec_combine.argtypes = [P] + [vp] * 7
            L.moe_ec_layer_forward.argtypes = [P, vp, vp, ctypes.POINTER(MoeWeights),
                                               ctypes.POINTER(MoeEcOutputs), vp, vp, sz, vp]
            L.moe_backward_workspace_size.argtypes = [P]
            L.moe_backward_workspace_size.restype = sz
            L.moe_layer_backward.argtypes = [P, vp, ctypes.POINTER(MoeWeights), ctypes.POINTER(MoeSaved),
                                             vp, ctypes.POINTER(MoeGrads), vp, sz, vp]
            for f in ("moe_route", "moe_dispatch", "moe_grouped_ffn", "moe_combine",
                      "moe_layer_forward", "moe_layer_forward_noalloc", "moe_router_stats", "moe_ec_route",
                      "moe_ec_dispatch", "moe_ec_combine", "moe_ec_layer_forward",
                      "moe_layer_backward"):
                getattr(L, f).restype = ctypes.c_int
            _lib = L
    return _lib


def problem(T, d, N, K, d_ff, n_shared=0, d_ff_shared=0, capacity_factor=0.0, noise_weight=0.0,
            gating=MOE_GATE_TOPK_SOFTMAX, act=MOE_ACT_SWIGLU, dtype=MOE_BF16,
            drop_order=MOE_DROP_TOKEN_ORDER) -> MoeProblem:
    gating = GATING.get(gating, gating)
    act = ACT.get(act, act)
    dtype = DTYPE.get(dtype, dtype)
    drop_order = DROP.get(drop_order, drop_order)
    return MoeProblem(T, d, N, K, d_ff, n_shared, d_ff_shared, capacity_factor, noise_weight,
                      gating, act, dtype, drop_order)


def problem_of(w, **over) -> MoeProblem:
    """Problem descriptor of a workload description (workloads.Workload)."""
    kw = dict(T=w.T, d=w.d, N=w.N, K=w.K, d_ff=w.d_ff, n_shared=w.n_shared,
              d_ff_shared=w.d_ff_shared, capacity_factor=w.capacity_factor,
              noise_weight=w.noise_weight, gating=w.gating, act=w.act, dtype=w.dtype,
              drop_order=w.drop_order)
    kw.update(over)
    return problem(**kw)


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def moe_workspace_size(p: MoeProblem) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(p)))


def moe_capacity(T: int, K: int, N: int, cf: float) -> int:
    return int(lib().moe_capacity(int(T), int(K), int(N), float(cf)))


def moe_ffn_row_tile(rows: int, groups: int, dtype="bf16") -> int:
    """Row-tile height of the grouped GEMMs over `rows` rows in `groups` groups."""
    return int(lib().moe_ffn_row_tile(int(rows), int(groups), int(DTYPE.get(dtype, dtype))))


# ------------------------------------------------------------------ helpers

_ws_cache: Dict[int, torch.Tensor] = {}


def workspace(p: MoeProblem, device) -> torch.Tensor:
    """A cached workspace buffer (uint8) big enough for problem p."""
    n = max(moe_workspace_size(p), 256)
    dev = torch.device(device)
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < n:
        buf = torch.empty(n, dtype=torch.uint8, device=dev)
        _ws_cache[key] = buf
    return buf


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: Optional[torch.Tensor], name: str, shape, dtype, device, optional=False):
    if t is None:
        if optional:
            return
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _call(fn: str, *args):
    st = getattr(lib(), fn)(*args)
    if st != MOE_OK:
        raise MoeError(fn, st)


def _empty(shape, dtype, device):
    return torch.empty(shape, dtype=dtype, device=device)


# ------------------------------------------------------------------ stages

def moe_route(p: MoeProblem, u, w_router, b_router=None, noise=None, want_scores=True,
              ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    dev = u.device
    et = TORCH_DTYPE[p.dtype]
    _check(u, "u", (p.T, p.d), et, dev)
    _check(w_router, "w_router", (p.N, p.d), torch.float32, dev)
    _check(b_router, "b_router", (p.N,), torch.float32, dev, optional=True)
    _check(noise, "noise", (p.T, p.N), torch.float32, dev, optional=True)
    o = dict(scores=_empty((p.T, p.N), torch.float32, dev) if want_scores else None,
             topk_idx=_empty((p.T, p.K), torch.int32, dev),
             topk_gate=_empty((p.T, p.K), torch.float32, dev),
             mean_prob=_empty((p.N,), torch.float32, dev),
             lse_sq=_empty((p.T,), torch.float32, dev))
    ws = workspace(p, dev) if ws is None else ws
    _call("moe_route", ctypes.byref(p), _ptr(u), _ptr(w_router), _ptr(b_router), _ptr(noise),
          _ptr(o["scores"]), _ptr(o["topk_idx"]), _ptr(o["topk_gate"]), _ptr(o["mean_prob"]),
          _ptr(o["lse_sq"]), _ptr(ws), ws.numel(), _stream(dev))
    return o


def moe_dispatch(p: MoeProblem, u, topk_idx, ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    dev = u.device
    et = TORCH_DTYPE[p.dtype]
    _check(u, "u", (p.T, p.d), et, dev)
    _check(topk_idx, "topk_idx", (p.T, p.K), torch.int32, dev)
    o = dict(expert_counts=_empty((p.N,), torch.int32, dev),
             kept_counts=_empty((p.N,), torch.int32, dev),
             offsets=_empty((p.N + 1,), torch.int32, dev),
             row_of=_empty((p.T, p.K), torch.int32, dev),
             token_of_row=_empty((p.T * p.K,), torch.int32, dev),
             x_perm=_empty((p.T * p.K, p.d), et, dev))
    ws = workspace(p, dev) if ws is None else ws
    _call("moe_dispatch", ctypes.byref(p), _ptr(u), _ptr(topk_idx), _ptr(o["expert_counts"]),
          _ptr(o["kept_counts"]), _ptr(o["offsets"]), _ptr(o["row_of"]), _ptr(o["token_of_row"]),
          _ptr(o["x_perm"]), _ptr(ws), ws.numel(), _stream(dev))
    return o


def moe_grouped_ffn(p: MoeProblem, x_perm, offsets, w_gate, w_up, w_down, u=None, ws_gate=None,
                    ws_up=None, ws_down=None, ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    dev = x_perm.device
    et = TORCH_DTYPE[p.dtype]
    _check(x_perm, "x_perm", (p.T * p.K, p.d), et, dev)
    _check(offsets, "offsets", (p.N + 1,), torch.int32, dev)
    _check(w_gate, "w_gate", (p.N, p.d_ff, p.d), et, dev)
    _check(w_up, "w_up", (p.N, p.d_ff, p.d), et, dev, optional=p.act == MOE_ACT_RELU)
    _check(w_down, "w_down", (p.N, p.d, p.d_ff), et, dev)
    if p.n_shared > 0:
        _check(u, "u", (p.T, p.d), et, dev)
        _check(ws_gate, "ws_gate", (p.n_shared, p.d_ff_shared, p.d), et, dev)
        _check(ws_up, "ws_up", (p.n_shared, p.d_ff_shared, p.d), et, dev, optional=p.act == MOE_ACT_RELU)
        _check(ws_down, "ws_down", (p.n_shared, p.d, p.d_ff_shared), et, dev)
    o = dict(y_perm=_empty((p.T * p.K, p.d), et, dev),
             y_shared=_empty((p.T, p.d), et, dev) if p.n_shared > 0 else None)
    ws = workspace(p, dev) if ws is None else ws
    _call("moe_grouped_ffn", ctypes.byref(p), _ptr(x_perm), _ptr(offsets), _ptr(w_gate),
          _ptr(w_up), _ptr(w_down), _ptr(u), _ptr(ws_gate), _ptr(ws_up), _ptr(ws_down),
          _ptr(o["y_perm"]), _ptr(o["y_shared"]), _ptr(ws), ws.numel(), _stream(dev))
    return o


STAT_NAMES = ("f_var", "p_var", "p_entropy", "z_loss")


def moe_router_stats(p: MoeProblem, expert_counts, mean_prob, lse_sq) -> torch.Tensor:
    """stats [4] fp32 on the device: variance of the assignment fractions,
    variance and entropy of the mean probabilities, mean of lse^2."""
    dev = mean_prob.device
    _check(expert_counts, "expert_counts", (p.N,), torch.int32, dev)
    _check(mean_prob, "mean_prob", (p.N,), torch.float32, dev)
    _check(lse_sq, "lse_sq", (p.T,), torch.float32, dev)
    stats = _empty((4,), torch.float32, dev)
    _call("moe_router_stats", ctypes.byref(p), _ptr(expert_counts), _ptr(mean_prob), _ptr(lse_sq),
          _ptr(stats), _stream(dev))
    return stats


def moe_combine(p: MoeProblem, u, y_perm, row_of, topk_gate, y_shared=None) -> torch.Tensor:
    dev = u.device
    et = TORCH_DTYPE[p.dtype]
    _check(u, "u", (p.T, p.d), et, dev)
    _check(y_perm, "y_perm", (p.T * p.K, p.d), et, dev)
    _check(row_of, "row_of", (p.T, p.K), torch.int32, dev)
    _check(topk_gate, "topk_gate", (p.T, p.K), torch.float32, dev)
    _check(y_shared, "y_shared", (p.T, p.d), et, dev, optional=p.n_shared == 0)
    out = _empty((p.T, p.d), et, dev)
    _call("moe_combine", ctypes.byref(p), _ptr(u), _ptr(y_perm), _ptr(row_of), _ptr(topk_gate),
          _ptr(y_shared), _ptr(out), None, 0, _stream(dev))
    return out


class LayerBuffers:
    """Preallocated outputs and intermediates of moe_layer_forward."""

    def __init__(self, p: MoeProblem, device, want_scores=True, keep_pre=False):
        et = TORCH_DTYPE[p.dtype]
        e = lambda shape, dt: _empty(shape, dt, device)
        gu = 2 if p.act == MOE_ACT_SWIGLU else 1
        self.t = dict(
            pre=e((p.T * p.K, gu * p.d_ff), torch.float32) if keep_pre else None,
            pre_shared=(e((p.T, gu * p.n_shared * p.d_ff_shared), torch.float32)
                        if keep_pre and p.n_shared > 0 else None),
            scores=e((p.T, p.N), torch.float32) if want_scores else None,
            topk_idx=e((p.T, p.K), torch.int32), topk_gate=e((p.T, p.K), torch.float32),
            mean_prob=e((p.N,), torch.float32), lse_sq=e((p.T,), torch.float32),
            expert_counts=e((p.N,), torch.int32), kept_counts=e((p.N,), torch.int32),
            offsets=e((p.N + 1,), torch.int32), row_of=e((p.T, p.K), torch.int32),
            token_of_row=e((p.T * p.K,), torch.int32), x_perm=e((p.T * p.K, p.d), et),
            y_perm=e((p.T * p.K, p.d), et),
            y_shared=e((p.T, p.d), et) if p.n_shared > 0 else None,
            out=e((p.T, p.d), et))
        self.c = MoeLayerOutputs(*[None if self.t[n] is None else self.t[n].data_ptr()
                                   for n, _ in MoeLayerOutputs._fields_])


def make_weights(p: MoeProblem, w_router, b_router, w_gate, w_up, w_down, ws_gate=None,
                 ws_up=None, ws_down=None) -> MoeWeights:
    dev = w_router.device
    et = TORCH_DTYPE[p.dtype]
    _check(w_router, "w_router", (p.N, p.d), torch.float32, dev)
    _check(b_router, "b_router", (p.N,), torch.float32, dev, optional=True)
    _check(w_gate, "w_gate", (p.N, p.d_ff, p.d), et, dev)
    _check(w_up, "w_up", (p.N, p.d_ff, p.d), et, dev, optional=p.act == MOE_ACT_RELU)
    _check(w_down, "w_down", (p.N, p.d, p.d_ff), et, dev)
    if p.n_shared > 0:
        _check(ws_gate, "ws_gate", (p.n_shared, p.d_ff_shared, p.d), et, dev)
        _check(ws_up, "ws_up", (p.n_shared, p.d_ff_shared, p.d), et, dev, optional=p.act == MOE_ACT_RELU)
        _check(ws_down, "ws_down", (p.n_shared, p.d, p.d_ff_shared), et, dev)
    ptr = lambda t: None if t is None else t.data_ptr()
    return MoeWeights(ptr(w_router), ptr(b_router), ptr(w_gate), ptr(w_up), ptr(w_down),
                      ptr(ws_gate), ptr(ws_up), ptr(ws_down))


def moe_layer_forward(p: MoeProblem, u, noise, weights: MoeWeights, bufs: LayerBuffers,
                      ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The chained forward pass into preallocated buffers; returns bufs.t['out'].
    The tensors behind `weights` must stay alive while the work runs."""
    dev = u.device
    _check(u, "u", (p.T, p.d), TORCH_DTYPE[p.dtype], dev)
    _check(noise, "noise", (p.T, p.N), torch.float32, dev, optional=True)
    ws = workspace(p, dev) if ws is None else ws
    _call("moe_layer_forward", ctypes.byref(p), _ptr(u), _ptr(noise), ctypes.byref(weights),
          ctypes.byref(bufs.c), _ptr(bufs.t["out"]), _ptr(ws), ws.numel(), _stream(dev))
    return bufs.t["out"]


def moe_layer_forward_noalloc(p: MoeProblem, u, noise, weights: MoeWeights,
                              bufs: LayerBuffers) -> torch.Tensor:
    """moe_layer_forward with the library's static scratch instead of a
    workspace (no allocation in the call); returns bufs.t['out']."""
    dev = u.device
    _check(u, "u", (p.T, p.d), TORCH_DTYPE[p.dtype], dev)
    _check(noise, "noise", (p.T, p.N), torch.float32, dev, optional=True)
    _call("moe_layer_forward_noalloc", ctypes.byref(p), _ptr(u), _ptr(noise),
          ctypes.byref(weights), ctypes.byref(bufs.c), _ptr(bufs.t["out"]), _stream(dev))
    return bufs.t["out"]


def layer_forward(p: MoeProblem, u, x: Dict[str, Optional[torch.Tensor]], want_scores=True,
                  keep_pre=False) -> Dict[str, torch.Tensor]:
    """Convenience: allocate buffers and run the whole pass on workload tensors
    x (keys as produced by workloads.generate, already on the GPU).  keep_pre:
    also keep GEMM-1's fp32 pre-activations ('pre', 'pre_shared') for the
    backward pass."""
    w = make_weights(p, x["w_router"], x.get("b_router"), x["w_gate"], x.get("w_up"), x["w_down"],
                     x.get("ws_gate"), x.get("ws_up"), x.get("ws_down"))
    bufs = LayerBuffers(p, u.device, want_scores, keep_pre)
    moe_layer_forward(p, u, x.get("noise"), w, bufs)
    return bufs.t


# ------------------------------------------------------------ expert choice

def moe_ec_capacity(T: int, K: int, N: int, cf: float) -> int:
    return int(lib().moe_ec_capacity(int(T), int(K), int(N), float(cf)))


def moe_ec_workspace_size(p: MoeProblem) -> int:
    return int(lib().moe_ec_workspace_size(ctypes.byref(p)))


_ec_ws_cache: Dict[int, torch.Tensor] = {}


def ec_workspace(p: MoeProblem, device) -> torch.Tensor:
    """A cached workspace buffer (uint8) big enough for the expert-choice calls of p."""
    n = max(moe_ec_workspace_size(p), 256)
    dev = torch.device(device)
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    buf = _ec_ws_cache.get(key)
    if buf is None or buf.numel() < n:
        buf = torch.empty(n, dtype=torch.uint8, device=dev)
        _ec_ws_cache[key] = buf
    return buf


def moe_ec_route(p: MoeProblem, u, w_router, b_router=None, noise=None, want_scores=True,
                 ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    dev = u.device
    C = moe_ec_capacity(p.T, p.K, p.N, p.capacity_factor)
    _check(u, "u", (p.T, p.d), TORCH_DTYPE[p.dtype], dev)
    _check(w_router, "w_router", (p.N, p.d), torch.float32, dev)
    _check(b_router, "b_router", (p.N,), torch.float32, dev, optional=True)
    _check(noise, "noise", (p.T, p.N), torch.float32, dev, optional=True)
    f32, i32 = torch.float32, torch.int32
    o = dict(scores=_empty((p.T, p.N), f32, dev) if want_scores else None,
             probs=_empty((p.N, p.T), f32, dev),
             expert_tokens=_empty((p.N, C), i32, dev), expert_gates=_empty((p.N, C), f32, dev),
             row_of=_empty((p.T, p.N), i32, dev), gate_of=_empty((p.T, p.N), f32, dev),
             offsets=_empty((p.N + 1,), i32, dev), mean_prob=_empty((p.N,), f32, dev),
             lse_sq=_empty((p.T,), f32, dev))
    ws = ec_workspace(p, dev) if ws is None else ws
    _call("moe_ec_route", ctypes.byref(p), _ptr(u), _ptr(w_router), _ptr(b_router), _ptr(noise),
          _ptr(o["scores"]), _ptr(o["probs"]), _ptr(o["expert_tokens"]), _ptr(o["expert_gates"]),
          _ptr(o["row_of"]), _ptr(o["gate_of"]), _ptr(o["offsets"]), _ptr(o["mean_prob"]),
          _ptr(o["lse_sq"]), _ptr(ws), ws.numel(), _stream(dev))
    return o


def moe_ec_dispatch(p: MoeProblem, u, expert_tokens) -> torch.Tensor:
    dev = u.device
    et = TORCH_DTYPE[p.dtype]
    C = moe_ec_capacity(p.T, p.K, p.N, p.capacity_factor)
    _check(u, "u", (p.T, p.d), et, dev)
    _check(expert_tokens, "expert_tokens", (p.N, C), torch.int32, dev)
    x_perm = _empty((p.N * C, p.d), et, dev)
    _call("moe_ec_dispatch", ctypes.byref(p), _ptr(u), _ptr(expert_tokens), _ptr(x_perm),
          _stream(dev))
    return x_perm


def moe_ec_combine(p: MoeProblem, u, y_perm, row_of, gate_of, y_shared=None) -> torch.Tensor:
    dev = u.device
    et = TORCH_DTYPE[p.dtype]
    C = moe_ec_capacity(p.T, p.K, p.N, p.capacity_factor)
    _check(u, "u", (p.T, p.d), et, dev)
    _check(y_perm, "y_perm", (p.N * C, p.d), et, dev)
    _check(row_of, "row_of", (p.T, p.N), torch.int32, dev)
    _check(gate_of, "gate_of", (p.T, p.N), torch.float32, dev)
    _check(y_shared, "y_shared", (p.T, p.d), et, dev, optional=p.n_shared == 0)
    out = _empty((p.T, p.d), et, dev)
    _call("moe_ec_combine", ctypes.byref(p), _ptr(u), _ptr(y_perm), _ptr(row_of), _ptr(gate_of),
          _ptr(y_shared), _ptr(out), _stream(dev))
    return out


class EcBuffers:
    """Preallocated outputs and intermediates of moe_ec_layer_forward."""

    def __init__(self, p: MoeProblem, device, want_scores=True):
        et = TORCH_DTYPE[p.dtype]
        C = moe_ec_capacity(p.T, p.K, p.N, p.capacity_factor)
        e = lambda shape, dt: _empty(shape, dt, device)
        f32, i32 = torch.float32, torch.int32
        self.C = C
        self.t = dict(
            scores=e((p.T, p.N), f32) if want_scores else None, probs=e((p.N, p.T), f32),
            expert_tokens=e((p.N, C), i32), expert_gates=e((p.N, C), f32),
            row_of=e((p.T, p.N), i32), gate_of=e((p.T, p.N), f32), offsets=e((p.N + 1,), i32),
            mean_prob=e((p.N,), f32), lse_sq=e((p.T,), f32),
            x_perm=e((p.N * C, p.d), et), y_perm=e((p.N * C, p.d), et),
            y_shared=e((p.T, p.d), et) if p.n_shared > 0 else None,
            out=e((p.T, p.d), et))
        self.c = MoeEcOutputs(*[None if self.t[n] is None else self.t[n].data_ptr()
                                for n, _ in MoeEcOutputs._fields_])


def moe_ec_layer_forward(p: MoeProblem, u, noise, weights: MoeWeights, bufs: EcBuffers,
                         ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The chained expert-choice pass into preallocated buffers; returns
    bufs.t['out'].  The tensors behind `weights` must stay alive while the work runs."""
    dev = u.device
    _check(u, "u", (p.T, p.d), TORCH_DTYPE[p.dtype], dev)
    _check(noise, "noise", (p.T, p.N), torch.float32, dev, optional=True)
    ws = ec_workspace(p, dev) if ws is None else ws
    _call("moe_ec_layer_forward", ctypes.byref(p), _ptr(u), _ptr(noise), ctypes.byref(weights),
          ctypes.byref(bufs.c), _ptr(bufs.t["out"]), _ptr(ws), ws.numel(), _stream(dev))
    return bufs.t["out"]


def ec_layer_forward(p: MoeProblem, u, x: Dict[str, Optional[torch.Tensor]], want_scores=True) -> Dict[str, torch.Tensor]:
    """Convenience: allocate buffers and run the expert-choice pass on
    workload tensors x (keys as produced by workloads.generate, on the GPU)."""
    w = make_weights(p, x["w_router"], x.get("b_router"), x["w_gate"], x.get("w_up"), x["w_down"],
                     x.get("ws_gate"), x.get("ws_up"), x.get("ws_down"))
    bufs = EcBuffers(p, u.device, want_scores)
    moe_ec_layer_forward(p, u, x.get("noise"), w, bufs)
    return bufs.t


# ------------------------------------------------------------------ backward

def moe_backward_workspace_size(p: MoeProblem) -> int:
    return int(lib().moe_backward_workspace_size(ctypes.byref(p)))


_bwd_ws_cache: Dict[int, torch.Tensor] = {}


def backward_workspace(p: MoeProblem, device) -> torch.Tensor:
    """A cached workspace buffer (uint8) big enough for moe_layer_backward of p."""
    n = max(moe_backward_workspace_size(p), 256)
    dev = torch.device(device)
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    buf = _bwd_ws_cache.get(key)
    if buf is None or buf.numel() < n:
        _bwd_ws_cache.pop(key, None)
        buf = torch.empty(n, dtype=torch.uint8, device=dev)
        _bwd_ws_cache[key] = buf
    return buf


def saved_of(fwd: Dict[str, torch.Tensor]) -> MoeSaved:
    """The forward outputs the backward reads (LayerBuffers.t or layer_forward's dict)."""
    ptr = lambda n: None if fwd.get(n) is None else fwd[n].data_ptr()
    return MoeSaved(*[ptr(n) for n, _ in MoeSaved._fields_])


class BwdBuffers:
    """Gradients (and, if asked, the intermediates d_gate, d_scores, dy_perm,
    dx_perm) of moe_layer_backward."""

    def __init__(self, p: MoeProblem, device, intermediates=True):
        et = TORCH_DTYPE[p.dtype]
        e = lambda shape, dt: _empty(shape, dt, device)
        relu = p.act == MOE_ACT_RELU
        sh = p.n_shared > 0
        f32 = torch.float32
        self.t = dict(
            du=e((p.T, p.d), et), dw_router=e((p.N, p.d), f32), db_router=e((p.N,), f32),
            dw_gate=e((p.N, p.d_ff, p.d), et), dw_up=None if relu else e((p.N, p.d_ff, p.d), et),
            dw_down=e((p.N, p.d, p.d_ff), et),
            dws_gate=e((p.n_shared, p.d_ff_shared, p.d), et) if sh else None,
            dws_up=e((p.n_shared, p.d_ff_shared, p.d), et) if sh and not relu else None,
            dws_down=e((p.n_shared, p.d, p.d_ff_shared), et) if sh else None,
            d_gate=e((p.T, p.K), f32) if intermediates else None,
            d_scores=e((p.T, p.N), f32) if intermediates else None,
            dy_perm=e((p.T * p.K, p.d), et) if intermediates else None,
            dx_perm=e((p.T * p.K, p.d), et) if intermediates else None)
        self.c = MoeGrads(*[None if self.t[n] is None else self.t[n].data_ptr()
                            for n, _ in MoeGrads._fields_])


def moe_layer_backward(p: MoeProblem, u, weights: MoeWeights, fwd: Dict[str, torch.Tensor], d_out,
                       bufs: BwdBuffers, ws: Optional[torch.Tensor] = None) -> Dict[str, torch.Tensor]:
    """The backward pass into preallocated gradient buffers; fwd holds the
    forward's outputs (scores may be None for top-K-then-softmax gating)."""
    dev = u.device
    et = TORCH_DTYPE[p.dtype]
    _check(u, "u", (p.T, p.d), et, dev)
    _check(d_out, "d_out", (p.T, p.d), et, dev)
    saved = saved_of(fwd)
    ws = backward_workspace(p, dev) if ws is None else ws
    _call("moe_layer_backward", ctypes.byref(p), _ptr(u), ctypes.byref(weights), ctypes.byref(saved),
          _ptr(d_out), ctypes.byref(bufs.c), _ptr(ws), ws.numel(), _stream(dev))
    return bufs.t


def layer_backward(p: MoeProblem, x: Dict[str, Optional[torch.Tensor]], fwd: Dict[str, torch.Tensor],
                   d_out, intermediates=True) -> Dict[str, torch.Tensor]:
    """Convenience: allocate gradients and run the backward on workload
    tensors x (on the GPU) and the forward outputs fwd."""
    w = make_weights(p, x["w_router"], x.get("b_router"), x["w_gate"], x.get("w_up"), x["w_down"],
                     x.get("ws_gate"), x.get("ws_up"), x.get("ws_down"))
    bufs = BwdBuffers(p, x["u"].device, intermediates)
    return moe_layer_backward(p, x["u"], w, fwd, d_out, bufs)
