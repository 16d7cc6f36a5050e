"""Test helpers: turn a seeded workload (torch CPU tensors) into the oracle's
numpy inputs.  bf16 tensors travel as their raw 16-bit patterns."""
import numpy as np
import torch

from oracle import oracle as O

GATING = {"softmax_topk": O.GATE_SOFTMAX_TOPK, "topk_softmax": O.GATE_TOPK_SOFTMAX}
ACT = {"swiglu": O.ACT_SWIGLU, "relu": O.ACT_RELU}
DT = {"f32": O.F32, "bf16": O.BF16}
DROP = {"token": O.DROP_TOKEN_ORDER, "choice": O.DROP_CHOICE_RANK}


def to_np(t):
    """CPU numpy view of a tensor: bf16 -> uint16 bit patterns, f32 as is."""
    if t is None:
        return None
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def elems_to_f64(a, dtype):
    """Stored elements (uint16 bf16 patterns or float32) as float64."""
    if dtype == O.BF16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def problem(w, **over):
    kw = dict(T=w.T, d=w.d, N=w.N, K=w.K, d_ff=w.d_ff, n_shared=w.n_shared,
              d_ff_shared=w.d_ff_shared, capacity_factor=w.capacity_factor,
              noise_weight=w.noise_weight, gating=GATING[w.gating], act=ACT[w.act],
              dtype=DT[w.dtype], drop_order=DROP[w.drop_order])
    kw.update(over)
    return O.Problem(**kw)


def inputs(p, x):
    return O.Inputs(p, to_np(x["u"]), to_np(x["w_router"]), to_np(x.get("b_router")),
                    to_np(x.get("noise")), to_np(x["w_gate"]), to_np(x.get("w_up")),
                    to_np(x["w_down"]), to_np(x.get("ws_gate")), to_np(x.get("ws_up")),
                    to_np(x.get("ws_down")))
