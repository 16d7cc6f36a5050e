"""Parity of moe_layer_backward (through the C ABI) with the oracle's
backward pass.

The routing of the backward is the forward's: the oracle routes from the
GPU's fp32 scores (bit-exact, as in the forward tests) and the dispatch
maps must agree exactly.  Gradients are floating point with bf16
intermediates (dY, dA, a, dG, dU, dX) and fp32 accumulation; they are
compared two ways:

    ||got - ref|| <= 1e-2 ||ref||                  (whole tensor)
    |got - ref|   <= 2e-2 |ref| + 8e-2 rms(ref)    (every element)

A bf16 rounding moves a value by at most 2^-9 of itself.  The path from
d_out to du or to a weight gradient rounds four times (dY, dA, dG/dU, dX);
each rounding error spreads through the next sum like noise of about 2^-9
of the scale of its terms, so the whole-tensor error is a few 1e-3 (4 x
2^-9 = 7.8e-3 at most if every rounding went the same way).  Single
elements can be sums of a few large terms that cancel (a weight gradient of
an expert with four rows), so the element bound is looser; that the
indexing is exact is pinned separately by integer data, where every
gradient must match bit for bit.  The GPU's y_perm, which d_gate reads,
differs from the oracle's recomputed y by at most one bf16 step in a few
elements.  fp32 router gradients get the same bounds."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from sparse_mixture_experts_42_amd import moe as M
from sparse_mixture_experts_42_amd import workloads as W
from tests import _io
from tests._gpu import DEV, gpu, host, say, workload

pytestmark = pytest.mark.gpu

RTOL, AFRAC, FROB = 2e-2, 8e-2, 1e-2


def close(got, ref, what, rtol=RTOL, afrac=AFRAC, frob=FROB):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return
    scale = float(np.sqrt(np.mean(ref * ref)))
    bound = afrac * scale + rtol * np.abs(ref) + 1e-30
    ratio = np.abs(got - ref) / bound
    rel = float(np.linalg.norm(got - ref) / (np.linalg.norm(ref) + 1e-30))
    say(f"{what}: rms(ref) {scale:.3e}, ||err||/||ref|| {rel:.2e}, max err/bound {ratio.max():.3f}, "
        f"n={ref.size}")
    assert rel <= frob or scale == 0.0, f"{what}: relative error {rel:.3e}"
    assert (ratio <= 1.0).all(), f"{what}: {(ratio > 1).sum()} of {ratio.size} outside tolerance"


def _d_out(w, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(w.T, w.d, generator=g).to(torch.bfloat16)


def _expert_rows(dsp, ro, e):
    """Tokens and gates of expert e's kept rows, in row order."""
    lo, hi = int(dsp["offsets"][e]), int(dsp["offsets"][e + 1])
    toks = dsp["token_of_row"][lo:hi].astype(np.int64)
    K = ro["topk_idx"].shape[1]
    gates = np.array([ro["topk_gate"][t][list(ro["topk_idx"][t]).index(e)] for t in toks]) \
        if len(toks) else np.zeros(0)
    assert all(e in ro["topk_idx"][t][:K] for t in toks)
    return toks, gates


def _run(w, x, seed):
    p = M.problem_of(w)
    xg = gpu(x)
    fwd = M.layer_forward(p, xg["u"], xg)
    d_out = _d_out(w, seed)
    t = M.layer_backward(p, xg, fwd, d_out.to(DEV))
    torch.cuda.synchronize()
    po = _io.problem(w)
    H = host(fwd["scores"])
    ro = O.route(po, H)
    assert np.array_equal(host(fwd["topk_idx"]), ro["topk_idx"])
    dsp = O.dispatch(po, ro["topk_idx"])
    for k in ("offsets", "row_of", "token_of_row"):
        assert np.array_equal(host(fwd[k]), dsp[k]), k
    dO = d_out.to(torch.float64).numpy()
    return p, po, xg, fwd, t, H, ro, dsp, dO


def _check_weight_grads(w, po, xi, x, t, ro, dsp, dO, experts, f_of, shared_f=None):
    u = _io.to_np(x["u"])
    for e in experts:
        toks, gates = _expert_rows(dsp, ro, e)
        fl = np.asarray(f_of(e), np.int32)
        if len(toks) == 0:
            assert not host(t["dw_gate"][e]).any() and not host(t["dw_down"][e]).any()
            continue
        ref = O.ffn_weight_grads(po, xi, e, u[toks], gates[:, None] * dO[toks], fl)
        fl_t = torch.from_numpy(fl.astype(np.int64)).to(DEV)
        close(host(t["dw_gate"][e].index_select(0, fl_t)), ref["dw_gate"], f"dw_gate[{e}]")
        if w.act == "swiglu":
            close(host(t["dw_up"][e].index_select(0, fl_t)), ref["dw_up"], f"dw_up[{e}]")
        close(host(t["dw_down"][e].index_select(1, fl_t)).T, ref["dw_down"], f"dw_down[{e}]")
    if w.n_shared and shared_f is not None:
        for s in range(w.n_shared):
            fl = np.asarray(shared_f, np.int32)
            ref = O.ffn_weight_grads(po, xi, -1 - s, u, dO, fl)
            fl_t = torch.from_numpy(fl.astype(np.int64)).to(DEV)
            close(host(t["dws_gate"][s].index_select(0, fl_t)), ref["dw_gate"], f"dws_gate[{s}]")
            if w.act == "swiglu":
                close(host(t["dws_up"][s].index_select(0, fl_t)), ref["dw_up"], f"dws_up[{s}]")
            close(host(t["dws_down"][s].index_select(1, fl_t)).T, ref["dw_down"], f"dws_down[{s}]")


@pytest.mark.parametrize("T,N,K,gating,act,cf,shared", [
    (300, 6, 2, "topk_softmax", "swiglu", 0.3, 0),
    (200, 8, 3, "softmax_topk", "swiglu", 0.0, 2),
    (150, 4, 1, "softmax_topk", "relu", 1.0, 0),
    (129, 16, 4, "topk_softmax", "relu", 0.0, 1),
    (560, 2, 2, "topk_softmax", "swiglu", 0.0, 0),
    (64, 32, 2, "softmax_topk", "swiglu", 0.0, 1),
    (1300, 2, 2, "topk_softmax", "swiglu", 0.0, 0),
    (1, 4, 2, "softmax_topk", "swiglu", 0.0, 1),
    # router weight gradient over 256-token slices (wide router, long
    # batch), the last slice ragged
    (1100, 12, 2, "softmax_topk", "swiglu", 0.0, 0),
    # groups over 512 rows on average: transposed weight gradients, with
    # the shared experts' as a first set of long tiles in the same launches
    (1100, 4, 2, "softmax_topk", "swiglu", 0.0, 2)])
def test_backward_small_shapes(T, N, K, gating, act, cf, shared):
    """Every gradient and intermediate against the oracle.  The mean group
    T*K/N picks the GEMM tiles: 1300 tokens on both of two experts give two
    groups of 1300 rows (256-row tiles, each group's last tile extended by
    20 rows); 560 rows over two experts and 300 over six run 128-row tiles;
    64 tokens over 32 experts run 32-row tiles."""
    w = W.Workload("bwd", T=T, d=128, N=N, K=K, d_ff=192, gating=gating, act=act,
                   capacity_factor=cf, n_shared=shared, d_ff_shared=64 if shared else 0,
                   seed=T * 17 + N, noise=True, noise_weight=0.5, bias="zipf")
    want = 256 if T * K >= 1024 * N else 128 if T * K >= 128 * N else 32
    assert M.moe_ffn_row_tile(T * K, N) == want
    say(f"backward T={T} N={N} K={K} {gating} {act} cf={cf} shared={shared}")
    x = W.generate(w)
    p, po, xg, fwd, t, H, ro, dsp, dO = _run(w, x, seed=T)
    xi = _io.inputs(po, x)
    lb = O.layer_backward_rows(po, xi, H, ro["topk_idx"], ro["topk_gate"], dsp["row_of"], dO)
    close(host(t["d_gate"]), lb["d_gate"], "d_gate")
    close(host(t["d_scores"]), lb["dH"], "d_scores")
    close(host(t["du"]), lb["du"], "du")
    rp = O.router_param_grads(po, xi, lb["dH"])
    close(host(t["dw_router"]), rp["dw_router"], "dw_router")
    close(host(t["db_router"]), rp["db_router"], "db_router")
    # intermediates: dY rows and dX rows
    R = int(dsp["offsets"][-1])
    tor = dsp["token_of_row"][:R].astype(np.int64)
    eor = np.repeat(np.arange(N, dtype=np.int32), np.diff(dsp["offsets"]))
    gate_of_row = np.zeros(R)
    for tt in range(T):
        for k in range(K):
            r = dsp["row_of"][tt, k]
            if r >= 0:
                gate_of_row[r] = ro["topk_gate"][tt, k]
    dy_ref = gate_of_row[:, None] * dO[tor]
    close(host(t["dy_perm"][:R]), dy_ref, "dy_perm")
    if R:
        u = _io.to_np(x["u"])
        dx_ref = O.ffn_backward_rows(po, xi, u[tor], eor, dy_ref)
        close(host(t["dx_perm"][:R]), dx_ref, "dx_perm")
    _check_weight_grads(w, po, xi, x, t, ro, dsp, dO, range(N), lambda e: np.arange(w.d_ff),
                        np.arange(w.d_ff_shared) if shared else None)


SAMPLE_TOKENS = dict(switch_top1=64, mixtral=6, deepseekmoe=12, decode_noisy=16)


@pytest.mark.parametrize("name", ["switch_top1", "mixtral", "deepseekmoe", "decode_noisy"])
def test_backward_full_size(name):
    """Sampled tokens (du, d_gate, d_scores), sampled hidden units of a few
    experts (weight gradients) and properties of the router gradients that
    hold at any size (the scores' gradient sums to zero over the experts)."""
    w, x = workload(name)
    say(f"backward {name} T={w.T}")
    p, po, xg, fwd, t, H, ro, dsp, dO = _run(w, x, seed=7)
    xi = _io.inputs(po, x)
    rng = np.random.default_rng(w.seed)
    toks = np.unique(np.concatenate([[0, w.T - 1], rng.choice(w.T, SAMPLE_TOKENS[name], replace=False)]))
    lb = O.layer_backward_rows(po, xi, H, ro["topk_idx"], ro["topk_gate"], dsp["row_of"], dO,
                               tokens=toks.astype(np.int32))
    sel = torch.from_numpy(toks).to(DEV)
    close(host(t["d_gate"][sel]), lb["d_gate"], f"{name} d_gate")
    close(host(t["d_scores"][sel]), lb["dH"], f"{name} d_scores")
    close(host(t["du"][sel]), lb["du"], f"{name} du")
    # router gradients: sum_i dH[t][i] = 0, so the column sums of dW_router
    # and the sum of db vanish up to fp32 rounding
    dwr = host(t["dw_router"]).astype(np.float64)
    assert np.abs(dwr.sum(axis=0)).max() <= 1e-3 * np.abs(dwr).max()
    db = host(t["db_router"]).astype(np.float64)
    assert abs(db.sum()) <= 1e-3 * np.abs(db).max() + 1e-30
    # (fp32 gates sum to one only up to rounding: the row sums are that
    # rounding times sum_k g_k dg_k)
    dH = host(t["d_scores"]).astype(np.float64)
    dg = np.abs(host(t["d_gate"]).astype(np.float64)).sum(axis=1)
    assert (np.abs(dH.sum(axis=1)) <= 1e-5 * (np.abs(dH).sum(axis=1) + dg) + 1e-30).all()
    experts = sorted(set([0, w.N - 1]) | set(int(e) for e in rng.choice(w.N, 1)))
    f_of = lambda e: np.unique(np.concatenate([[0, w.d_ff - 1], rng.choice(w.d_ff, 2, replace=False)]))
    sf = np.unique([0, w.d_ff_shared - 1, 7]) if w.n_shared else None
    _check_weight_grads(w, po, xi, x, t, ro, dsp, dO, experts, f_of, sf)


def test_backward_is_deterministic_and_fp32_is_refused():
    w = W.WORKLOADS["switch_top1"].replace(T=2000)
    x = W.generate(w)
    p = M.problem_of(w)
    xg = gpu(x)
    fwd = M.layer_forward(p, xg["u"], xg)
    d_out = _d_out(w, 3).to(DEV)
    a = {k: (None if v is None else v.clone()) for k, v in M.layer_backward(p, xg, fwd, d_out).items()}
    b = M.layer_backward(p, xg, fwd, d_out)
    R = int(fwd["offsets"][-1])
    for k, v in a.items():
        if v is None:
            continue
        if k in ("dy_perm", "dx_perm"):
            assert torch.equal(v[:R], b[k][:R]), k
        else:
            assert torch.equal(v, b[k]), k
    wf = W.WORKLOADS["tiny_fp32"]
    xf = gpu(W.generate(wf))
    pf = M.problem_of(wf)
    ff = M.layer_forward(pf, xf["u"], xf)
    with pytest.raises(M.MoeError):
        M.layer_backward(pf, xf, ff, torch.zeros_like(xf["u"]))


def _cold_bias(w, x, lo, hi):
    """Router bias that leaves expert N-1 with between lo and hi tokens: 0 for
    the others, and for N-1 minus the midpoint of a wide gap in the sorted
    margins H[N-1] - max_{i<N-1} H[i] of the unbiased scores (wide enough that
    the GPU's fp32 scores, within 1e-4 of the oracle's, choose the same
    tokens)."""
    N = w.N
    b = torch.zeros(N, dtype=torch.float32)
    x["b_router"] = b
    po = _io.problem(w, noise_weight=0.0)
    H = O.router_logits(po, _io.inputs(po, x)).astype(np.float64)
    srt = np.sort(H[:, N - 1] - H[:, :N - 1].max(axis=1))[::-1]
    m = max(range(lo, hi + 1), key=lambda m: srt[m - 1] - srt[m])
    assert srt[m - 1] - srt[m] > 1e-3
    b[N - 1] = -float(srt[m - 1] + srt[m]) / 2
    return m


@pytest.mark.parametrize("T,shared,cold", [(300, 0, None), (300, 1, None), (2100, 0, "empty"),
                                           (2100, 1, None), (4200, 0, "short")])
def test_backward_integer_data_is_exact(T, shared, cold):
    """ReLU experts, top-1 with softmax over the one selected score (gate 1,
    so no gradient reaches the router), sparse weights and inputs in
    {-1, 0, 1}: every product, sum and stored bf16 value is a small integer,
    so every gradient must equal the oracle's bit for bit.  With 2100 tokens
    the experts average over 512 rows, so the weight gradients take the
    transposed form; the last expert's bias keeps it empty, and its weight
    gradients must come out zero; with a shared expert, its weight gradients
    (every token) run as the first tiles of the same launches.  With 4200
    tokens the groups average 1050
    rows, so the GEMMs run 256-row tiles; the last expert's bias leaves it
    24 to 56 rows, which run as a 64-row tail tile."""
    N, d, dff = 4, 128, 192
    w = W.Workload("bwdint", T=T, d=d, N=N, K=1, d_ff=dff, gating="topk_softmax", act="relu",
                   n_shared=shared, d_ff_shared=64 if shared else 0, seed=5)
    assert M.moe_ffn_row_tile(T, N) == (256 if T >= 1024 * N else 128 if T >= 128 * N else 32)
    x = W.generate(w)
    if cold == "empty":
        x["b_router"] = torch.zeros(N, dtype=torch.float32)
        x["b_router"][N - 1] = -1.0e4
    g = torch.Generator().manual_seed(11)
    tern = lambda *s, p=0.15: (torch.randint(-1, 2, s, generator=g) *
                               (torch.rand(s, generator=g) < p)).to(torch.bfloat16)
    # sparser inputs for the longer groups keep every sum within bf16's
    # exact integers (|v| <= 256)
    dens = 0.5 if T < 1000 else 0.15 if T < 3000 else 0.1
    x["u"] = tern(T, d, p=dens)
    x["w_gate"] = tern(N, dff, d)
    x["w_down"] = tern(N, d, dff)
    if shared:
        x["ws_gate"] = tern(1, 64, d)
        x["ws_down"] = tern(1, d, 64)
    x["noise"] = None
    d_out = tern(T, d, p=dens)
    if cold == "short":
        m = _cold_bias(w, x, 24, 56)
        say(f"integer backward: expert {N - 1} biased to {m} tokens")
    p = M.problem_of(w, noise_weight=0.0)
    xg = gpu(x)
    fwd = M.layer_forward(p, xg["u"], xg)
    t = M.layer_backward(p, xg, fwd, d_out.to(DEV))
    torch.cuda.synchronize()
    po = _io.problem(w, noise_weight=0.0)
    xi = _io.inputs(po, x)
    H = host(fwd["scores"])
    ro = O.route(po, H)
    dsp = O.dispatch(po, ro["topk_idx"])
    assert np.array_equal(host(fwd["row_of"]), dsp["row_of"])
    assert (ro["topk_gate"] == 1.0).all()
    dO = d_out.to(torch.float64).numpy()
    lb = O.layer_backward_rows(po, xi, H, ro["topk_idx"], ro["topk_gate"], dsp["row_of"], dO)
    assert np.abs(lb["du"]).max() <= 256 and np.array_equal(lb["du"], np.round(lb["du"]))
    assert np.array_equal(host(t["du"]), lb["du"]), "du"
    assert np.array_equal(host(t["d_gate"]), lb["d_gate"]), "d_gate"
    assert not host(t["dw_router"]).any() and not host(t["d_scores"]).any()
    u = _io.to_np(x["u"])
    sizes = np.diff(dsp["offsets"])
    if cold == "empty":
        assert sizes[N - 1] == 0
        assert not host(t["dw_gate"][N - 1]).any() and not host(t["dw_down"][N - 1]).any()
    if cold == "short":
        assert sizes[N - 1] == m and 1 <= m <= 64 and sizes.mean() >= 1024
    for e in range(N):
        toks, gates = _expert_rows(dsp, ro, e)
        ref = O.ffn_weight_grads(po, xi, e, u[toks], dO[toks], np.arange(dff, dtype=np.int32))
        assert np.abs(ref["dw_gate"]).max() <= 256 and np.abs(ref["dw_down"]).max() <= 256
        assert np.array_equal(host(t["dw_gate"][e]), ref["dw_gate"]), f"dw_gate[{e}]"
        assert np.array_equal(host(t["dw_down"][e]).T, ref["dw_down"]), f"dw_down[{e}]"
    if shared:
        ref = O.ffn_weight_grads(po, xi, -1, u, dO, np.arange(64, dtype=np.int32))
        assert np.abs(ref["dw_gate"]).max() <= 256 and np.abs(ref["dw_down"]).max() <= 256
        assert np.array_equal(host(t["dws_gate"][0]), ref["dw_gate"])
        assert np.array_equal(host(t["dws_down"][0]).T, ref["dw_down"])


@pytest.mark.parametrize("T,N,K,act,shared", [
    (300, 6, 2, "swiglu", 0),       # 128-row tiles
    (200, 8, 3, "swiglu", 2),       # shared experts (one group over every token)
    (129, 16, 4, "relu", 1),        # 32-row tiles, ReLU
    (1300, 2, 2, "swiglu", 0),      # 256-row tiles, each group's last tile extended
    (4200, 4, 1, "relu", 0)])       # 256-row tiles, ragged groups
def test_backward_from_kept_pre_activations(T, N, K, act, shared):
    """A forward that keeps GEMM-1's fp32 pre-activations changes none of its
    other outputs, and a backward that takes them instead of recomputing
    GEMM-1 gives the same gradients bit for bit: the kept values are the
    recompute GEMM's own accumulators, and both paths share the activation
    backward's arithmetic.  The kept g (and v) are checked against the
    oracle's products x_perm W^T (shared experts: u Ws^T) on sampled rows,
    to the fp32 accumulation bound."""
    dffs = 64 if shared else 0
    w = W.Workload("keep", T=T, d=256, N=N, K=K, d_ff=192, gating="topk_softmax", act=act,
                   n_shared=shared, d_ff_shared=dffs, seed=T + N)
    say(f"kept pre-activations T={T} N={N} K={K} {act} shared={shared} "
        f"(row tile {M.moe_ffn_row_tile(T * K, N)})")
    x = W.generate(w)
    xg = gpu(x)
    p = M.problem_of(w)
    a = M.layer_forward(p, xg["u"], xg)
    b = M.layer_forward(p, xg["u"], xg, keep_pre=True)
    torch.cuda.synchronize()
    R = int(a["offsets"][-1])
    for k, v in a.items():
        if v is None or k in ("pre", "pre_shared"):
            continue
        vb = b[k]
        if k in ("x_perm", "y_perm"):
            assert torch.equal(v[:R], vb[:R]), k
        else:
            assert torch.equal(v, vb), k
    # kept values against the oracle's products on sampled rows
    gu = 2 if act == "swiglu" else 1
    pre = host(b["pre"])
    assert pre.shape == (T * K, gu * w.d_ff)
    xp = host(b["x_perm"]).astype(np.float64)
    off = host(b["offsets"])
    f64 = lambda t: t.to(torch.float64).numpy()
    mats = [f64(x["w_gate"])] + ([f64(x["w_up"])] if gu == 2 else [])
    rng = np.random.default_rng(T)
    for r in np.unique(np.concatenate([off[:-1], np.maximum(off[1:] - 1, 0), rng.integers(0, max(R, 1), 24)])):
        if r >= R:
            continue
        e = int(np.searchsorted(off, r, side="right") - 1)
        for h, Wm in enumerate(mats):
            ref = Wm[e] @ xp[r]
            bound = 2e-5 * (np.abs(Wm[e]) @ np.abs(xp[r])) + 1e-30
            got = pre[r, h * w.d_ff:(h + 1) * w.d_ff]
            assert (np.abs(got - ref) <= bound).all(), f"pre row {r} part {h}"
    if shared:
        ps = host(b["pre_shared"])
        uu = f64(x["u"])
        smats = [f64(x["ws_gate"]).reshape(-1, w.d)] + \
            ([f64(x["ws_up"]).reshape(-1, w.d)] if gu == 2 else [])
        wsw = shared * dffs
        for t in (0, T // 2, T - 1):
            for h, Wm in enumerate(smats):
                ref = Wm @ uu[t]
                bound = 2e-5 * (np.abs(Wm) @ np.abs(uu[t])) + 1e-30
                assert (np.abs(ps[t, h * wsw:(h + 1) * wsw] - ref) <= bound).all(), f"pre_shared {t}"
    # the backward from the kept values equals the recomputing one
    d_out = _d_out(w, 7).to(DEV)
    ga = {k: (None if v is None else v.clone()) for k, v in M.layer_backward(p, xg, a, d_out).items()}
    gb = M.layer_backward(p, xg, b, d_out)
    torch.cuda.synchronize()
    for k, v in ga.items():
        if v is None:
            continue
        if k in ("dy_perm", "dx_perm"):
            assert torch.equal(v[:R], gb[k][:R]), k
        else:
            assert torch.equal(v, gb[k]), k
