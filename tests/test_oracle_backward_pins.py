"""Pins of the oracle's backward pass against the oracle's forward pass:
central finite differences (with one Richardson step) of L = sum(d_out * h)
in fp32 problems, where the forward rounds only to fp32, must match the
analytic gradients; plus invariants of the gating Jacobian.  CPU only.

The forward pass is the pages' layer; its gradient is the calculus of that
definition with the routing held fixed, so the finite differences only move
parameters by amounts that leave every Top-K set and capacity decision
unchanged (asserted)."""
import numpy as np
import pytest

from oracle import oracle as O

F32 = O.F32


def _problem(gating, act, **kw):
    base = dict(T=6, d=64, N=4, K=2, d_ff=32, n_shared=1, d_ff_shared=16, capacity_factor=0.5,
                noise_weight=0.3, gating=gating, act=act, dtype=F32)
    base.update(kw)
    return O.Problem(**base)


def _data(p, seed):
    rng = np.random.default_rng(seed)
    f = lambda *s, std=1.0: (rng.standard_normal(s) * std).astype(np.float32)
    x = dict(u=f(p.T, p.d), w_router=f(p.N, p.d, std=0.5), b_router=f(p.N, std=0.5),
             noise=f(p.T, p.N), w_gate=f(p.N, p.d_ff, p.d, std=p.d ** -0.5),
             w_up=f(p.N, p.d_ff, p.d, std=p.d ** -0.5) if p.act == O.ACT_SWIGLU else None,
             w_down=f(p.N, p.d, p.d_ff, std=p.d_ff ** -0.5))
    if p.n_shared:
        x.update(ws_gate=f(p.n_shared, p.d_ff_shared, p.d, std=p.d ** -0.5),
                 ws_up=f(p.n_shared, p.d_ff_shared, p.d, std=p.d ** -0.5) if p.act == O.ACT_SWIGLU else None,
                 ws_down=f(p.n_shared, p.d, p.d_ff_shared, std=p.d_ff_shared ** -0.5))
    d_out = rng.standard_normal((p.T, p.d))
    return x, d_out


def _separated_data(p, seed, gap=0.25):
    """The first of a fixed sequence of seeds whose tokens all have their
    K-th and (K+1)-th scores at least `gap` apart (steps then cannot move
    the Top-K sets) and, with a capacity, drop at least one assignment."""
    for s in range(seed, seed + 1000 * 50, 1000):
        x, d_out = _data(p, s)
        o = O.layer_forward(p, _inputs(p, x))
        srt = -np.sort(-o["scores"].astype(np.float64), axis=1)
        ok = p.K >= p.N or (srt[:, p.K - 1] - srt[:, p.K]).min() >= gap
        if ok and (p.capacity_factor <= 0 or (o["row_of"] < 0).any()):
            return x, d_out
    raise AssertionError("no seed found")


def _inputs(p, x):
    return O.Inputs(p, x["u"], x["w_router"], x["b_router"], x["noise"], x["w_gate"], x["w_up"],
                    x["w_down"], x.get("ws_gate"), x.get("ws_up"), x.get("ws_down"))


class _FD:
    """Finite differences of L = sum(d_out * h) through the forward oracle."""

    def __init__(self, p, x, d_out):
        self.p, self.x, self.d_out = p, x, d_out
        self.ref = O.layer_forward(p, _inputs(p, x))

    def loss(self, name, idx, value):
        xx = dict(self.x)
        a = xx[name].copy()
        a[idx] = value
        xx[name] = a
        o = O.layer_forward(self.p, _inputs(self.p, xx))
        # the routing must not move: the gradient holds it fixed
        assert np.array_equal(o["topk_idx"], self.ref["topk_idx"])
        assert np.array_equal(o["row_of"], self.ref["row_of"])
        return float(np.sum(self.d_out * o["out"]))

    def grad(self, name, idx, h):
        a0 = float(self.x[name][idx])

        def central(hh):
            lo, hi = np.float32(a0 - hh), np.float32(a0 + hh)
            return (self.loss(name, idx, hi) - self.loss(name, idx, lo)) / (float(hi) - float(lo))

        return (4.0 * central(h / 2) - central(h)) / 3.0


def _analytic(p, x, d_out, ref):
    """Every gradient the backward oracle gives, assembled per parameter."""
    xi = _inputs(p, x)
    lb = O.layer_backward_rows(p, xi, ref["scores"], ref["topk_idx"], ref["topk_gate"], ref["row_of"], d_out)
    rp = O.router_param_grads(p, xi, lb["dH"])
    g = dict(u=lb["du"], w_router=rp["dw_router"], b_router=rp["db_router"], d_gate=lb["d_gate"], dH=lb["dH"])
    for name in ("w_gate", "w_up", "w_down"):
        g[name] = np.zeros((p.N,) + x["w_gate" if name != "w_down" else "w_down"].shape[1:])
    f_all = np.arange(p.d_ff, dtype=np.int32)
    for e in range(p.N):
        toks, gates = [], []
        for t in range(p.T):
            for k in range(p.K):
                if ref["topk_idx"][t, k] == e and ref["row_of"][t, k] >= 0:
                    toks.append(t)
                    gates.append(ref["topk_gate"][t, k])
        if not toks:
            continue
        dy = np.array(gates)[:, None] * d_out[toks]
        wg = O.ffn_weight_grads(p, xi, e, x["u"][toks], dy, f_all)
        g["w_gate"][e] = wg["dw_gate"]
        g["w_up"][e] = wg["dw_up"]
        g["w_down"][e] = wg["dw_down"].T
    if p.n_shared:
        fs = np.arange(p.d_ff_shared, dtype=np.int32)
        g["ws_gate"] = np.zeros(x["ws_gate"].shape)
        g["ws_up"] = np.zeros(x["ws_gate"].shape)
        g["ws_down"] = np.zeros(x["ws_down"].shape)
        for s in range(p.n_shared):
            wg = O.ffn_weight_grads(p, xi, -1 - s, x["u"], d_out, fs)
            g["ws_gate"][s] = wg["dw_gate"]
            g["ws_up"][s] = wg["dw_up"]
            g["ws_down"][s] = wg["dw_down"].T
    return g


def _check(fd, g, name, positions, h=4e-2, atol=5e-4, rtol=2e-3):
    worst = 0.0
    for idx in positions:
        num = fd.grad(name, idx, h)
        ana = float(g[name][idx])
        err = abs(num - ana)
        worst = max(worst, err / (atol + rtol * abs(ana)))
        assert err <= atol + rtol * abs(ana), (name, idx, num, ana)
    return worst


def _positions(rng, shape, n):
    return [tuple(int(rng.integers(0, s)) for s in shape) for _ in range(n)]


@pytest.mark.parametrize("gating", [O.GATE_TOPK_SOFTMAX, O.GATE_SOFTMAX_TOPK])
def test_layer_backward_matches_finite_differences_swiglu(gating):
    p = _problem(gating, O.ACT_SWIGLU)
    x, d_out = _separated_data(p, 11 + gating)
    fd = _FD(p, x, d_out)
    ref = fd.ref
    assert (ref["row_of"] < 0).any(), "the case must drop an assignment"
    g = _analytic(p, x, d_out, ref)
    rng = np.random.default_rng(5)
    _check(fd, g, "u", [(t, int(j)) for t in range(p.T) for j in rng.integers(0, p.d, 3)])
    _check(fd, g, "w_router", _positions(rng, x["w_router"].shape, 10))
    _check(fd, g, "b_router", [(i,) for i in range(p.N)])
    for name in ("w_gate", "w_up", "w_down", "ws_gate", "ws_up", "ws_down"):
        _check(fd, g, name, _positions(rng, x[name].shape, 8))


def test_layer_backward_matches_finite_differences_relu():
    """ReLU FFN: differences only in the weights, whose steps move few
    pre-activations (the check fails loudly if one crosses zero)."""
    p = _problem(O.GATE_SOFTMAX_TOPK, O.ACT_RELU, n_shared=0, d_ff_shared=0, capacity_factor=0.0)
    x, d_out = _separated_data(p, 23)
    fd = _FD(p, x, d_out)
    g = _analytic(p, x, d_out, fd.ref)
    rng = np.random.default_rng(6)
    _check(fd, g, "w_down", _positions(rng, x["w_down"].shape, 12), h=1e-2)
    _check(fd, g, "w_gate", _positions(rng, x["w_gate"].shape, 12), h=1e-2)
    _check(fd, g, "w_router", _positions(rng, x["w_router"].shape, 6), h=1e-2)


def test_score_gradient_sums_to_zero():
    """Softmax is unchanged by adding one constant to every score, so
    sum_i dH[t][i] = 0 for every token in both gating variants, hence the
    bias gradient sums to zero over the experts."""
    for gating in (O.GATE_TOPK_SOFTMAX, O.GATE_SOFTMAX_TOPK):
        p = _problem(gating, O.ACT_SWIGLU, T=12)
        x, d_out = _data(p, 31)
        ref = O.layer_forward(p, _inputs(p, x))
        lb = O.layer_backward_rows(p, _inputs(p, x), ref["scores"], ref["topk_idx"], ref["topk_gate"],
                                   ref["row_of"], d_out)
        assert np.abs(lb["dH"].sum(axis=1)).max() <= 1e-14
        rp = O.router_param_grads(p, _inputs(p, x), lb["dH"])
        assert abs(rp["db_router"].sum()) <= 1e-13
        assert np.abs(rp["db_router"]).max() > 1e-3


@pytest.mark.parametrize("gating", [O.GATE_TOPK_SOFTMAX, O.GATE_SOFTMAX_TOPK])
def test_gating_jacobian_matches_finite_differences(gating):
    """dH from route_backward against central differences of sum_k dg_k g_k
    under steps of 2^-12 on the fp32 scores (exact in fp32, gates in double)."""
    rng = np.random.default_rng(41)
    T, N, K = 20, 7, 3
    p = O.Problem(T=T, d=8, N=N, K=K, d_ff=8, gating=gating)
    H = rng.standard_normal((T, N)).astype(np.float32)
    r = O.route(p, H)
    dg = rng.standard_normal((T, K))
    dH = O.route_backward(p, H, r["topk_idx"], r["topk_gate"], dg)
    h = 2.0 ** -12
    for t in range(T):
        for i in range(N):
            vals = []
            for s in (h, -h):
                Hp = H.copy()
                Hp[t, i] += np.float32(s)
                rp = O.route(p, Hp)
                assert np.array_equal(rp["topk_idx"], r["topk_idx"])
                vals.append(float(np.sum(dg[t] * rp["topk_gate"][t])))
            assert (vals[0] - vals[1]) / (2 * h) == pytest.approx(dH[t, i], abs=1e-6)


def test_gating_variants_agree_when_every_expert_is_selected():
    """K = N: both variants are the softmax over all experts, so their
    Jacobians (computed by different formulas) agree and equal
    s * (dg - <s, dg>) in expert order."""
    rng = np.random.default_rng(42)
    T, N = 9, 5
    H = rng.standard_normal((T, N)).astype(np.float32)
    out = []
    for gating in (O.GATE_TOPK_SOFTMAX, O.GATE_SOFTMAX_TOPK):
        p = O.Problem(T=T, d=8, N=N, K=N, d_ff=8, gating=gating)
        r = O.route(p, H)
        dg = np.take_along_axis(np.tile(np.arange(1.0, N + 1), (T, 1)), r["topk_idx"], axis=1)
        out.append(O.route_backward(p, H, r["topk_idx"], r["topk_gate"], dg))
    assert np.allclose(out[0], out[1], rtol=1e-13, atol=1e-15)
    H64 = H.astype(np.float64)
    s = np.exp(H64 - H64.max(axis=1, keepdims=True))
    s = s / s.sum(axis=1, keepdims=True)
    v = np.arange(1.0, N + 1)
    assert np.allclose(out[0], s * (v - (s * v).sum(axis=1, keepdims=True)), rtol=1e-12, atol=1e-14)


def test_combine_backward_is_the_derivative_of_combine():
    """Combine is linear in the gates and in y: differences of any size are
    exact up to rounding.  Dropped assignments get d_gate = 0 and no dy."""
    rng = np.random.default_rng(43)
    T, N, K, d = 7, 4, 2, 16
    p = O.Problem(T=T, d=d, N=N, K=K, d_ff=8, dtype=F32)
    u = rng.standard_normal((T, d)).astype(np.float32)
    y = rng.standard_normal((T * K, d)).astype(np.float32)
    row_of = rng.permutation(T * K).astype(np.int32).reshape(T, K)
    row_of[2, 1] = -1
    row_of[5, 0] = -1
    gate = rng.random((T, K))
    d_out = rng.standard_normal((T, d))
    b = O.combine_backward(p, d_out, y, row_of, gate)
    L = lambda g, yy: float(np.sum(d_out * O.combine(p, u, yy, row_of, g)))
    for t in range(T):
        for k in range(K):
            gp, gm = gate.copy(), gate.copy()
            gp[t, k] += 0.5
            gm[t, k] -= 0.5
            assert (L(gp, y) - L(gm, y)) == pytest.approx(b["d_gate"][t, k], abs=1e-12)
    assert b["d_gate"][2, 1] == 0.0 and b["d_gate"][5, 0] == 0.0
    for r in range(T * K):
        for j in (0, d - 1):
            yp, ym = y.copy(), y.copy()
            yp[r, j] += 0.5
            ym[r, j] -= 0.5
            step = float(yp[r, j]) - float(ym[r, j])        # the fp32 step actually taken
            assert (L(gate, yp) - L(gate, ym)) / step == pytest.approx(b["dy"][r, j], abs=1e-12)
    unused = np.setdiff1d(np.arange(T * K), row_of[row_of >= 0])
    assert np.all(b["dy"][unused] == 0.0)


@pytest.mark.parametrize("act", [O.ACT_SWIGLU, O.ACT_RELU])
def test_ffn_backward_rows_matches_finite_differences(act):
    """dx of single experts and of two shared experts against differences of
    the forward expert outputs in the input."""
    p = O.Problem(T=4, d=32, N=3, K=1, d_ff=24, n_shared=2, d_ff_shared=16, act=act, dtype=F32)
    x, _ = _data(p, 51)
    xi = _inputs(p, x)
    rng = np.random.default_rng(52)
    rows = rng.standard_normal((5, p.d)).astype(np.float32)
    eor = np.array([0, 1, 2, -1, 1], np.int32)
    dy = rng.standard_normal((5, p.d))
    dx = O.ffn_backward_rows(p, xi, rows, eor, dy)
    h = 1e-3
    for r in range(5):
        for j in rng.integers(0, p.d, 6):
            vals = []
            for s in (h, -h):
                rr = rows[r:r + 1].copy()
                rr[0, j] = np.float32(rows[r, j] + s)
                vals.append((float(np.sum(dy[r] * O.ffn_rows(p, xi, rr, eor[r:r + 1])[0])), float(rr[0, j])))
            num = (vals[0][0] - vals[1][0]) / (vals[0][1] - vals[1][1])
            assert num == pytest.approx(dx[r, j], abs=2e-3, rel=2e-3)
