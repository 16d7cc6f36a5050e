"""Parity of the expert-choice path (moe_ec_*, through the C ABI) with the
CPU oracle.

The selection is an integer decision taken on fp32 affinities: the oracle
selects from the GPU's own affinities and must agree bit for bit (tokens,
rows, gates), and the oracle's selection from its own double affinities must
agree wherever a token is further from the expert's C-th affinity than the
measured affinity error.  Layer outputs are compared with the oracle's
expert-choice rows on that selection within the bf16 / fp32 tolerances."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_mixture_experts_42_amd import moe as M
from sparse_mixture_experts_42_amd import workloads as W
from tests import _io
from tests._gpu import DEV, PROB_TOL, SCORE_TOL, assert_close, elems, gpu, host, say, workload

pytestmark = pytest.mark.gpu


def _ec_checks(w, x, r):
    """Scores, affinities, selection and side outputs of moe_ec_route."""
    po = _io.problem(w)
    C = O.ec_capacity(w.T, w.K, w.N, w.capacity_factor)
    assert M.moe_ec_capacity(w.T, w.K, w.N, w.capacity_factor) == C
    H_o = O.router_logits(po, _io.inputs(po, x))
    H_g = host(r["scores"])
    assert np.abs(H_g.astype(np.float64) - H_o).max() <= SCORE_TOL
    # affinities: the double softmax of the GPU's fp32 scores
    ro = O.route(po, H_g, want_probs=True)
    probs_g = host(r["probs"]).T.astype(np.float64)          # [T][N]
    assert np.abs(probs_g - ro["probs"]).max() <= PROB_TOL
    assert np.abs(host(r["mean_prob"]) - ro["mean_prob"]).max() <= PROB_TOL
    lse_g = host(r["lse_sq"]).astype(np.float64)
    assert np.all(np.abs(lse_g - ro["lse_sq"]) <= PROB_TOL * np.maximum(1.0, ro["lse_sq"]))
    # selection from the GPU's affinities: bit-exact
    sel = O.ec_select(po, probs_g, C)
    assert np.array_equal(host(r["expert_tokens"]), sel["expert_tokens"]), "expert_tokens"
    assert np.array_equal(host(r["row_of"]), sel["row_of"]), "row_of"
    assert np.array_equal(host(r["expert_gates"]).astype(np.float64), sel["expert_gates"])
    assert np.array_equal(host(r["gate_of"]).astype(np.float64), sel["gate_of"])
    assert host(r["offsets"]).tolist() == [i * C for i in range(w.N + 1)]
    # independent: the oracle's selection from its own affinities, away
    # from the expert's C-th affinity by more than twice the affinity error
    own = O.route(po, H_o, want_probs=True)["probs"]
    delta = np.abs(probs_g - own).max() + 1e-12
    say(f"{w.name}: C={C}, scores max|err| {np.abs(H_g - H_o).max():.2e}, "
        f"affinity max|err| {delta:.2e}")
    chosen = host(r["row_of"]) >= 0
    ambiguous = 0
    if 0 < C < w.T:
        thr = -np.sort(-own, axis=0)[C - 1]                 # C-th largest per expert
        above = own > thr + 2 * delta
        below = own < thr - 2 * delta
        assert chosen[above].all(), "a token well above the C-th affinity was not chosen"
        assert not chosen[below].any(), "a token well below the C-th affinity was chosen"
        ambiguous = int((~(above | below)).sum())
    elif C == w.T:
        assert chosen.all()
    else:
        assert not chosen.any()
    say(f"{w.name}: {ambiguous} (token, expert) pairs within a near tie of the C-th affinity")
    assert ambiguous <= max(4 * w.N, w.T * w.N // 100)
    return sel


# ------------------------------------------------------------------ route

@pytest.mark.parametrize("name", W.ORDER)
def test_ec_route_full_size(name):
    w = W.WORKLOADS[name]
    say(f"ec route {name} T={w.T} N={w.N} K={w.K} cf={w.capacity_factor}")
    x = W.generate(w, only=W.ROUTER)
    xg = gpu(x)
    r = M.moe_ec_route(M.problem_of(w), xg["u"], xg["w_router"], xg["b_router"], xg["noise"])
    torch.cuda.synchronize()
    _ec_checks(w, x, r)


@pytest.mark.parametrize("T,N,K,cf", [(1, 4, 1, 0.0), (37, 5, 3, 0.0), (300, 256, 16, 0.5),
                                      (2000, 8, 2, 4.0), (1500, 3, 1, 0.01), (5000, 64, 6, 1.0),
                                      (1025, 2, 1, 1.5), (129, 100, 7, 0.0)])
def test_ec_route_edges(T, N, K, cf):
    w = W.Workload("ecedge", T=T, d=128, N=N, K=K, d_ff=64, capacity_factor=cf,
                   seed=T * 7 + N, noise=True, noise_weight=0.5, bias="zipf")
    say(f"ec route edge T={T} N={N} K={K} cf={cf}")
    x = W.generate(w, only=W.ROUTER)
    xg = gpu(x)
    r = M.moe_ec_route(M.problem_of(w), xg["u"], xg["w_router"], xg["b_router"], xg["noise"])
    _ec_checks(w, x, r)


def test_ec_route_equal_affinities_take_lowest_tokens():
    """Zero router: every affinity is 1/N, so every expert takes tokens
    0 .. C-1 with gate 1/N."""
    say("ec route ties")
    T, N, K = 3000, 6, 2
    p = M.problem(T=T, d=64, N=N, K=K, d_ff=64)
    C = M.moe_ec_capacity(T, K, N, 0.0)
    r = M.moe_ec_route(p, torch.zeros(T, 64, dtype=torch.bfloat16, device=DEV),
                       torch.zeros(N, 64, device=DEV))
    assert (host(r["expert_tokens"]) == np.arange(C)).all()
    assert np.abs(host(r["expert_gates"]) - 1.0 / N).max() <= 1e-7
    ro = host(r["row_of"])
    assert (ro[:C] == np.arange(N) * C + np.arange(C)[:, None]).all()
    assert (ro[C:] == -1).all() and (host(r["gate_of"])[C:] == 0).all()


def test_ec_route_ties_at_the_threshold_across_token_chunks():
    """Affinities that depend on t mod 3 only: each expert's C-th affinity is
    shared by thousands of tokens on both sides of the 8192-token chunks the
    selection walks, and the lowest-index tokens of that tie must be the
    ones taken, in ascending order.  Checked bit for bit against the
    oracle's selection from the GPU's affinities."""
    T, N, K, dm = 20000, 4, 1, 64
    say(f"ec route threshold ties T={T} N={N}")
    p = M.problem(T=T, d=dm, N=N, K=K, d_ff=64)
    C = M.moe_ec_capacity(T, K, N, 0.0)
    u = torch.zeros(T, dm, dtype=torch.bfloat16)
    u[:, 0] = (torch.arange(T) % 3).to(torch.bfloat16)
    wr = torch.zeros(N, dm)
    wr[:, 0] = 0.5 * torch.arange(N, dtype=torch.float32)
    r = M.moe_ec_route(p, u.to(DEV), wr.to(DEV))
    probs = host(r["probs"]).T.astype(np.float64)
    sel = O.ec_select(O.Problem(T=T, d=dm, N=N, K=K, d_ff=64, dtype=O.BF16), probs, C)
    assert np.array_equal(host(r["expert_tokens"]), sel["expert_tokens"])
    assert np.array_equal(host(r["row_of"]), sel["row_of"])
    assert np.array_equal(host(r["expert_gates"]).astype(np.float64), sel["expert_gates"])
    # expert N-1 prefers t = 2 mod 3 (6667 tokens, more than C = 5000): its
    # rows are the first C of them
    assert (host(r["expert_tokens"]).reshape(N, C)[N - 1] == 2 + 3 * np.arange(C)).all()


def test_ec_route_without_scores_matches():
    w = W.WORKLOADS["switch_top1"]
    xg = gpu(W.generate(w, only=W.ROUTER))
    p = M.problem_of(w)
    a = M.moe_ec_route(p, xg["u"], xg["w_router"], xg["b_router"], xg["noise"])
    b = M.moe_ec_route(p, xg["u"], xg["w_router"], xg["b_router"], xg["noise"], want_scores=False)
    for k in ("probs", "expert_tokens", "expert_gates", "row_of", "gate_of", "offsets"):
        assert torch.equal(a[k], b[k]), k


# -------------------------------------------------------- dispatch, combine

@pytest.mark.parametrize("name", ["tiny_fp32", "deepseekmoe"])
def test_ec_dispatch_is_a_row_gather(name):
    w = W.WORKLOADS[name]
    x = W.generate(w, only=W.ROUTER)
    xg = gpu(x)
    p = M.problem_of(w)
    r = M.moe_ec_route(p, xg["u"], xg["w_router"], xg["b_router"], xg["noise"])
    xp = M.moe_ec_dispatch(p, xg["u"], r["expert_tokens"])
    ref = xg["u"].index_select(0, r["expert_tokens"].reshape(-1).long())
    assert torch.equal(xp, ref)


@pytest.mark.parametrize("T,N,K,d,dtype,cf,shared", [(256, 4, 2, 64, "f32", 0.0, 0),
                                                     (300, 8, 1, 768, "bf16", 2.0, 0),
                                                     (999, 16, 4, 256, "bf16", 1.0, 1),
                                                     (50, 256, 16, 128, "bf16", 3.0, 0)])
def test_ec_combine(T, N, K, d, dtype, cf, shared):
    w = W.Workload("eccomb", T=T, d=d, N=N, K=K, d_ff=64, dtype=dtype, capacity_factor=cf,
                   n_shared=shared, d_ff_shared=64 if shared else 0, seed=T + N)
    say(f"ec combine T={T} N={N} d={d} {dtype} cf={cf} shared={shared}")
    x = W.generate(w, only=W.ROUTER)
    xg = gpu(x)
    p = M.problem_of(w)
    r = M.moe_ec_route(p, xg["u"], xg["w_router"], xg["b_router"], xg["noise"])
    C = r["expert_tokens"].shape[1]
    et = M.TORCH_DTYPE[p.dtype]
    g = torch.Generator().manual_seed(T)
    y = torch.randn(N * C, d, generator=g).to(et)
    ys = torch.randn(T, d, generator=g).to(et) if shared else None
    out = M.moe_ec_combine(p, xg["u"], y.to(DEV), r["row_of"], r["gate_of"],
                           None if ys is None else ys.to(DEV))
    po = _io.problem(w)
    pe = dataclasses.replace(po, K=N)
    # the oracle's combine takes T*K rows (K = N here): the N*C expert
    # rows, then zero rows that no token references
    y_rows = torch.cat([y, torch.zeros(T * N - N * C, d, dtype=et)])
    ref = O.combine(pe, elems(xg["u"]), elems(y_rows), host(r["row_of"]),
                    host(r["gate_of"]).astype(np.float64), None if ys is None else elems(ys))
    assert_close(host(out), ref, dtype, "ec combine out")
    if dtype == "bf16":
        exact = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy()
        assert np.mean(host(out) == exact) > 0.99


# ------------------------------------------------------------ whole layer

def _ec_sample(w, row_of, n):
    if n >= w.T:
        return np.arange(w.T)
    rng = np.random.default_rng(w.seed + 1)
    nsel = (row_of >= 0).sum(axis=1)
    toks = set(range(min(4, w.T))) | set(range(max(0, w.T - 4), w.T))
    toks |= set(int(t) for t in np.nonzero(nsel == 0)[0][:6])
    toks |= set(int(t) for t in np.argsort(-nsel, kind="stable")[:4])
    toks |= set(int(t) for t in rng.choice(w.T, n, replace=False))
    return np.array(sorted(toks), dtype=np.int64)


EC_SAMPLE = dict(tiny_fp32=256, switch_top1=384, mixtral=16, deepseekmoe=64, decode_noisy=128)


def _ec_layer(w, x, sample=None):
    p = M.problem_of(w)
    xg = gpu(x)
    t = M.ec_layer_forward(p, xg["u"], xg)
    torch.cuda.synchronize()
    sel = _ec_checks(w, x, t)
    po = _io.problem(w)
    toks = np.arange(w.T) if sample is None else _ec_sample(w, sel["row_of"], sample)
    ref = O.ec_layer_rows(po, _io.inputs(po, x), sel, toks)
    got = host(t["out"][torch.from_numpy(toks).to(DEV)])
    assert_close(got, ref, w.dtype, f"{w.name} ec out ({len(toks)} tokens)")
    # tokens no expert chose keep the residual (plus shared experts) exactly
    none = np.nonzero((sel["row_of"] < 0).all(axis=1))[0]
    say(f"{w.name}: {len(none)} tokens chosen by no expert")
    if len(none) and w.n_shared == 0:
        ix = torch.from_numpy(none).to(DEV)
        assert torch.equal(t["out"][ix], xg["u"][ix])
    return t, xg


@pytest.mark.parametrize("name", W.ORDER)
def test_ec_layer_full_size(name):
    w, x = workload(name)
    say(f"ec layer {name} T={w.T}")
    _ec_layer(w, x, EC_SAMPLE[name])


@pytest.mark.parametrize("T,N,K,act,cf,shared,dtype", [
    (1, 4, 2, "swiglu", 0.0, 0, "bf16"),
    (17, 3, 1, "relu", 0.0, 0, "bf16"),
    (300, 6, 2, "swiglu", 0.3, 0, "bf16"),
    (200, 8, 3, "swiglu", 0.0, 2, "bf16"),
    (150, 1, 1, "swiglu", 0.0, 0, "bf16"),
    (100, 5, 2, "relu", 0.0, 1, "f32"),
    (333, 16, 16, "swiglu", 0.0, 0, "bf16"),
    (90, 4, 2, "swiglu", 9.0, 1, "bf16"),
    (700, 32, 2, "relu", 1.7, 0, "bf16")])
def test_ec_layer_small_shapes(T, N, K, act, cf, shared, dtype):
    w = W.Workload("ecsmall", T=T, d=128, N=N, K=K, d_ff=192, act=act, capacity_factor=cf,
                   n_shared=shared, d_ff_shared=64 if shared else 0, dtype=dtype,
                   seed=T * 13 + N, noise=True, noise_weight=0.5)
    say(f"ec layer small T={T} N={N} K={K} {act} cf={cf} shared={shared} {dtype}")
    _ec_layer(w, W.generate(w))


def test_ec_layer_c_equal_t_is_the_dense_mixture():
    """C = T: every expert takes every token, so each output is the dense
    softmax mixture of all experts (the token-choice oracle with K = N and
    softmax-then-top-K gating)."""
    w = W.Workload("ecdense", T=96, d=128, N=4, K=4, d_ff=128, gating="softmax_topk",
                   capacity_factor=1.0, seed=41)
    x = W.generate(w)
    t, _ = _ec_layer(w, x)
    po = _io.problem(w)
    xi = _io.inputs(po, x)
    ro = O.route(po, host(t["scores"]))
    dsp = O.dispatch(po, ro["topk_idx"])
    dense = O.layer_rows(po, xi, ro["topk_idx"], ro["topk_gate"], dsp["row_of"])
    assert_close(host(t["out"]), dense, "bf16", "ec dense mixture")


def test_ec_layer_determinism_and_zero_down():
    w = W.WORKLOADS["switch_top1"].replace(T=1500)
    xg = gpu(W.generate(w))
    p = M.problem_of(w)
    a = {k: (None if v is None else v.clone()) for k, v in M.ec_layer_forward(p, xg["u"], xg).items()}
    b = M.ec_layer_forward(p, xg["u"], xg)
    for k, v in a.items():
        if v is not None:
            assert torch.equal(v, b[k]), k
    xg["w_down"] = torch.zeros_like(xg["w_down"])
    c = M.ec_layer_forward(p, xg["u"], xg)
    assert torch.equal(c["out"], xg["u"])


def test_ec_t_zero_is_a_no_op():
    p = M.problem(T=0, d=64, N=4, K=2, d_ff=64)
    u = torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)
    r = M.moe_ec_route(p, u, torch.zeros(4, 64, device=DEV))
    assert r["expert_tokens"].numel() == 0
