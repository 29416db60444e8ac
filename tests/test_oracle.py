"""Pins of the float64 oracle against what the pages and the mathematics fix (CPU only).

Every check here is independent of the oracle's own code path:
  * torch.autograd in float64 of the forward the pages define (a library routine);
  * central finite differences of the forward, evaluated in mpmath at 40 digits;
  * closed forms of the Swish derivative (Lambert W root, extrema, symmetry);
  * invariants linking the three stages (ones-column trick, adjoint identity);
  * brute-force loops on tiny inputs;
  * the Swish page's worked example (section 4.1: grad all ones, x = 1..6,
    beta = 1.1), with values derived at 40 digits.
A planted-mistake test then mutates the oracle and checks that a pin catches it.
"""
from __future__ import annotations

import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch

import oracle.ref as R

HERE = os.path.dirname(os.path.abspath(__file__))
mpmath.mp.dps = 40


# ----------------------------------------------------------------------------------
# pin functions: each takes the oracle callables so a mutated oracle can be checked
# ----------------------------------------------------------------------------------

def _mp_swish(x, beta):
    return x / (1 + mpmath.exp(-beta * x))


def _mp_swish_grad(x, beta):
    """d/dx [x * sigmoid(beta x)] by mpmath numerical differentiation (40 digits)."""
    return mpmath.diff(lambda u: _mp_swish(u, beta), x)


def pin_swish_autograd(swish_grad_ref):
    rng = np.random.default_rng(11)
    x = np.concatenate([np.linspace(-40, 40, 801), rng.normal(0, 3, 500),
                        [0.0, -1e-300, 1e-8, -700.0, 700.0]])
    grad = rng.normal(0, 1, x.shape)
    for beta in (1.0, 1.702, 0.5, 1.1, 0.01, -0.7, 0.0):
        b32 = float(np.float32(beta))
        xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
        y = xt * torch.sigmoid(b32 * xt)
        (gx,) = torch.autograd.grad(y, xt, grad_outputs=torch.tensor(grad))
        got, want = swish_grad_ref(grad, x, beta), gx.numpy()
        # near the zero of s' both float64 evaluations cancel: allow 1e-15 * |grad|
        assert np.all(np.abs(got - want) <= 1e-12 * np.abs(want) + 1e-15 * np.abs(grad)), beta


def pin_swish_mpmath(swish_grad_ref):
    xs = [-9.5, -3.0, -1.2784645, -0.3, 0.0, 0.25, 1.0, 2.5, 7.0, 19.0]
    for beta in (1.0, 1.702, 0.5, 1.1):
        b = mpmath.mpf(float(np.float32(beta)))
        for x in xs:
            want = float(_mp_swish_grad(mpmath.mpf(x), b))
            got = float(swish_grad_ref(np.array([1.0]), np.array([x]), beta)[0])
            assert abs(got - want) <= 1e-13 * max(1.0, abs(want)), (beta, x, got, want)


def pin_swish_closed_forms(swish_grad_ref):
    one = np.ones(1)
    # s'(0) = 1/2 for every beta
    for beta in (1.0, 1.702, 0.5, 3.0, -2.0, 0.0):
        assert swish_grad_ref(one, np.zeros(1), beta)[0] == pytest.approx(0.5, abs=1e-15)
    # beta = 0: the Swish becomes x/2, the gradient grad/2
    xs = np.linspace(-5, 5, 11)
    np.testing.assert_allclose(swish_grad_ref(np.full(11, 3.0), xs, 0.0), 1.5, rtol=1e-15)
    # s'(t) + s'(-t) = 1, since SiLU(t) - SiLU(-t) = t
    t = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(swish_grad_ref(np.ones_like(t), t, 1.0)
                               + swish_grad_ref(np.ones_like(t), -t, 1.0), 1.0, atol=2e-15)
    # root of s' at t* = -1 - W(1/e); s' changes sign there
    tstar = float(-1 - mpmath.lambertw(1 / mpmath.e).real)
    assert tstar == pytest.approx(-1.2784645427610738, abs=1e-15)
    v = swish_grad_ref(one, np.array([tstar]), 1.0)[0]
    assert abs(v) < 1e-15
    assert swish_grad_ref(one, np.array([tstar - 1e-3]), 1.0)[0] < 0
    assert swish_grad_ref(one, np.array([tstar + 1e-3]), 1.0)[0] > 0
    # extrema of s' where s'' = 0 (found by mpmath root finding on the 2nd derivative)
    f2 = lambda u: mpmath.diff(lambda w: _mp_swish(w, 1), u, 2)  # noqa: E731
    tmax = mpmath.findroot(f2, 2.4)
    smax = float(mpmath.diff(lambda w: _mp_swish(w, 1), tmax))
    assert float(tmax) == pytest.approx(2.3993572805, abs=1e-9)
    assert smax == pytest.approx(1.0998393201, abs=1e-9)
    assert swish_grad_ref(one, np.array([float(tmax)]), 1.0)[0] == pytest.approx(smax, abs=1e-14)
    assert swish_grad_ref(one, np.array([-float(tmax)]), 1.0)[0] == pytest.approx(1 - smax, abs=1e-14)
    # scaling: swish_grad(g, x, beta) = swish_grad(g, beta x, 1) (beta = 0.5 is exact)
    x = np.random.default_rng(5).normal(0, 3, 1000)
    gr = np.random.default_rng(6).normal(0, 1, 1000)
    np.testing.assert_allclose(swish_grad_ref(gr, x, 0.5), swish_grad_ref(gr, 0.5 * x, 1.0),
                               rtol=1e-15, atol=1e-300)
    # saturation: finite for huge |t|
    big = swish_grad_ref(np.ones(2), np.array([-800.0, 800.0]), 1.0)
    assert np.all(np.isfinite(big)) and big[0] == 0.0 and big[1] == 1.0


def pin_swish_silu_identity(swish_grad_ref):
    """beta = 1: the Swish gradient is SiLU' (library: aten silu_backward, float64)."""
    x = torch.linspace(-25, 25, 2001, dtype=torch.float64)
    gr = torch.randn(2001, dtype=torch.float64, generator=torch.Generator().manual_seed(3))
    want = torch.ops.aten.silu_backward(gr, x).numpy()
    np.testing.assert_allclose(swish_grad_ref(gr.numpy(), x.numpy(), 1.0), want,
                               rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(swish_grad_ref(gr.numpy(), x.numpy(), None), want,
                               rtol=1e-13, atol=1e-300)


def pin_swish_example(swish_grad_ref):
    with open(os.path.join(HERE, "golden", "swish_example.json")) as f:
        ex = json.load(f)
    got = swish_grad_ref(np.array(ex["grad"]), np.array(ex["x"]), ex["beta"])
    # independently: 40-digit derivative with beta = float32(1.1)
    b = mpmath.mpf(float(np.float32(ex["beta"])))
    want = [float(_mp_swish_grad(mpmath.mpf(v), b)) for v in ex["x"]]
    np.testing.assert_allclose(got, want, rtol=1e-14)
    np.testing.assert_allclose(got, ex["expected"], rtol=1e-14)


def _swiglu_case(M, K, N, seed):
    gen = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, dtype=torch.float64, generator=gen)  # noqa: E731
    return {"x": r(M, K), "w_g": r(K, N) / math.sqrt(K), "w_fc": r(K, N) / math.sqrt(K),
            "b_g": 0.3 * r(N), "b_fc": 0.3 * r(N), "dy": r(M, N)}


def pin_swiglu_autograd(b_ref, w_ref, x_ref):
    """Reference gradients from torch.autograd of y = SiLU(xW_g+b_g)*(xW_fc+b_fc)."""
    for (M, K, N, seed) in ((5, 3, 4, 0), (37, 19, 23, 1), (64, 8, 16, 2)):
        c = _swiglu_case(M, K, N, seed)
        leaves = {k: c[k].clone().requires_grad_(True) for k in ("x", "w_g", "w_fc", "b_g", "b_fc")}
        g = leaves["x"] @ leaves["w_g"] + leaves["b_g"]
        fc = leaves["x"] @ leaves["w_fc"] + leaves["b_fc"]
        g.retain_grad()
        fc.retain_grad()
        y = torch.nn.functional.silu(g) * fc
        (y * c["dy"]).sum().backward()
        G, FC, DY = g.detach().numpy(), fc.detach().numpy(), c["dy"].numpy()
        dg, dfc, db_g, db_fc = b_ref(DY, G, FC)
        dw_g, dw_fc = w_ref(c["x"].numpy(), dg, dfc)
        dx = x_ref(dg, dfc, c["w_g"].numpy(), c["w_fc"].numpy())
        pairs = [(dg, g.grad), (dfc, fc.grad), (db_g, leaves["b_g"].grad),
                 (db_fc, leaves["b_fc"].grad), (dw_g, leaves["w_g"].grad),
                 (dw_fc, leaves["w_fc"].grad), (dx, leaves["x"].grad)]
        for got, want in pairs:
            np.testing.assert_allclose(got, want.numpy(), rtol=1e-11, atol=1e-13)


def pin_swiglu_chain(swiglu_bwd_ref):
    """The chained backward (b, then w and x on the dg and dfc that b produced) against
    torch.autograd in float64 of y = SiLU(xW_g+b_g)*(xW_fc+b_fc): all seven gradients,
    each under its own name, at three shapes (non-square, N != K, M > K)."""
    for (M, K, N, seed) in ((5, 3, 4, 0), (37, 19, 23, 1), (64, 8, 16, 2)):
        c = _swiglu_case(M, K, N, seed)
        leaves = {k: c[k].clone().requires_grad_(True) for k in ("x", "w_g", "w_fc", "b_g", "b_fc")}
        g = leaves["x"] @ leaves["w_g"] + leaves["b_g"]
        fc = leaves["x"] @ leaves["w_fc"] + leaves["b_fc"]
        g.retain_grad()
        fc.retain_grad()
        y = torch.nn.functional.silu(g) * fc
        (y * c["dy"]).sum().backward()
        out = swiglu_bwd_ref(c["dy"].numpy(), c["x"].numpy(), c["w_g"].numpy(),
                             c["w_fc"].numpy(), g.detach().numpy(), fc.detach().numpy())
        want = {"dg": g.grad, "dfc": fc.grad, "db_g": leaves["b_g"].grad,
                "db_fc": leaves["b_fc"].grad, "dw_g": leaves["w_g"].grad,
                "dw_fc": leaves["w_fc"].grad, "dx": leaves["x"].grad}
        assert set(out) == set(want)
        for k, v in want.items():
            np.testing.assert_allclose(out[k], v.numpy(), rtol=1e-11, atol=1e-13, err_msg=k)


def pin_swiglu_fd(b_ref, w_ref, x_ref):
    """Central differences of L = sum(dy * SiLU(xW_g+b_g) * (xW_fc+b_fc)) in mpmath."""
    M, K, N = 4, 3, 5
    c = {k: v.numpy() for k, v in _swiglu_case(M, K, N, 7).items()}

    def loss(p):
        tot = mpmath.mpf(0)
        for m in range(M):
            for n in range(N):
                gv = p["b_g"][n] + sum(p["x"][m][k] * p["w_g"][k][n] for k in range(K))
                fv = p["b_fc"][n] + sum(p["x"][m][k] * p["w_fc"][k][n] for k in range(K))
                tot += c["dy"][m, n] * gv / (1 + mpmath.exp(-gv)) * fv
        return tot

    P = {k: [[mpmath.mpf(float(v)) for v in row] for row in np.atleast_2d(c[k])]
         if c[k].ndim == 2 else [mpmath.mpf(float(v)) for v in c[k]]
         for k in ("x", "w_g", "w_fc", "b_g", "b_fc")}
    G = c["x"] @ c["w_g"] + c["b_g"]
    FC = c["x"] @ c["w_fc"] + c["b_fc"]
    dg, dfc, db_g, db_fc = b_ref(c["dy"], G, FC)
    dw_g, dw_fc = w_ref(c["x"], dg, dfc)
    dx = x_ref(dg, dfc, c["w_g"], c["w_fc"])
    got = {"x": dx, "w_g": dw_g, "w_fc": dw_fc, "b_g": db_g, "b_fc": db_fc}
    h = mpmath.mpf("1e-12")
    for name, arr in got.items():
        for idx in np.ndindex(arr.shape):
            def at(delta):
                Q = {k: ([row[:] for row in v] if isinstance(v[0], list) else v[:])
                     for k, v in P.items()}
                if len(idx) == 2:
                    Q[name][idx[0]][idx[1]] += delta
                else:
                    Q[name][idx[0]] += delta
                return loss(Q)
            fd = float((at(h) - at(-h)) / (2 * h))
            assert abs(arr[idx] - fd) <= 1e-10 * max(1.0, abs(fd)), (name, idx, arr[idx], fd)


def pin_swiglu_invariants(b_ref, w_ref, x_ref):
    rng = np.random.default_rng(21)
    M, K, N = 50, 7, 9
    x = rng.normal(size=(M, K))
    w_g, w_fc = rng.normal(size=(K, N)), rng.normal(size=(K, N))
    dy, g, fc = rng.normal(size=(M, N)), rng.normal(size=(M, N)) * 2, rng.normal(size=(M, N))
    dg, dfc, db_g, db_fc = b_ref(dy, g, fc)
    # a column of ones appended to x: that row of dw equals db (links w to b)
    x1 = np.concatenate([x, np.ones((M, 1))], axis=1)
    dw_g1, dw_fc1 = w_ref(x1, dg, dfc)
    np.testing.assert_allclose(dw_g1[K], db_g, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw_fc1[K], db_fc, rtol=1e-12, atol=1e-12)
    # adjoint identity: <dx, x> = <dw_g, W_g> + <dw_fc, W_fc>
    dw_g, dw_fc = w_ref(x, dg, dfc)
    dx = x_ref(dg, dfc, w_g, w_fc)
    lhs = np.sum(dx * x)
    rhs = np.sum(dw_g * w_g) + np.sum(dw_fc * w_fc)
    assert lhs == pytest.approx(rhs, rel=1e-11)
    # accumulators are added exactly
    db0 = rng.normal(size=N)
    _, _, db_g2, db_fc2 = b_ref(dy, g, fc, db0, -db0)
    np.testing.assert_allclose(db_g2 - db0, db_g, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(db_fc2 + db0, db_fc, rtol=1e-12, atol=1e-12)
    dw0 = rng.normal(size=(K, N))
    dw_g3, dw_fc3 = w_ref(x, dg, dfc, dw0, 2 * dw0)
    np.testing.assert_allclose(dw_g3 - dw0, dw_g, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dw_fc3 - 2 * dw0, dw_fc, rtol=1e-12, atol=1e-12)
    # dg and dfc at g = 0: SiLU'(0) = 1/2 and SiLU(0) = 0
    z = np.zeros((3, 4))
    dg0, dfc0, _, _ = b_ref(np.ones((3, 4)), z, np.full((3, 4), 2.0))
    np.testing.assert_allclose(dg0, 1.0)
    np.testing.assert_allclose(dfc0, 0.0)


def pin_swiglu_bruteforce(b_ref, w_ref, x_ref):
    rng = np.random.default_rng(4)
    M, K, N = 6, 5, 7
    x = rng.normal(size=(M, K))
    w_g, w_fc = rng.normal(size=(K, N)), rng.normal(size=(K, N))
    dy, g, fc = rng.normal(size=(M, N)), rng.normal(size=(M, N)), rng.normal(size=(M, N))
    dg, dfc, db_g, db_fc = b_ref(dy, g, fc)
    for m in range(M):
        for n in range(N):
            s = 1.0 / (1.0 + math.exp(-g[m, n]))
            assert dg[m, n] == pytest.approx(dy[m, n] * fc[m, n] * (s + g[m, n] * s * (1 - s)), rel=1e-13)
            assert dfc[m, n] == pytest.approx(dy[m, n] * g[m, n] * s, rel=1e-13)
    for n in range(N):
        assert db_g[n] == pytest.approx(sum(dg[m, n] for m in range(M)), rel=1e-12, abs=1e-14)
        assert db_fc[n] == pytest.approx(sum(dfc[m, n] for m in range(M)), rel=1e-12, abs=1e-14)
    dw_g, dw_fc = w_ref(x, dg, dfc)
    for k in range(K):
        for n in range(N):
            assert dw_g[k, n] == pytest.approx(sum(x[m, k] * dg[m, n] for m in range(M)), rel=1e-12, abs=1e-14)
            assert dw_fc[k, n] == pytest.approx(sum(x[m, k] * dfc[m, n] for m in range(M)), rel=1e-12, abs=1e-14)
    dx = x_ref(dg, dfc, w_g, w_fc)
    for m in range(M):
        for k in range(K):
            want = sum(dg[m, n] * w_g[k, n] + dfc[m, n] * w_fc[k, n] for n in range(N))
            assert dx[m, k] == pytest.approx(want, rel=1e-12, abs=1e-14)


SWISH_PINS = [pin_swish_autograd, pin_swish_mpmath, pin_swish_closed_forms,
              pin_swish_silu_identity, pin_swish_example]
SWIGLU_PINS = [pin_swiglu_autograd, pin_swiglu_fd, pin_swiglu_invariants,
               pin_swiglu_bruteforce]


@pytest.mark.parametrize("pin", SWISH_PINS, ids=lambda f: f.__name__)
def test_swish_pins(pin):
    pin(R.swish_grad_ref)


@pytest.mark.parametrize("pin", SWIGLU_PINS, ids=lambda f: f.__name__)
def test_swiglu_pins(pin):
    pin(R.b_ref, R.w_ref, R.x_ref)


def test_swiglu_chain_pin():
    pin_swiglu_chain(R.swiglu_bwd_ref)


def test_forward_ref_matches_definition():
    rng = np.random.default_rng(2)
    x, w_g, w_fc = rng.normal(size=(4, 3)), rng.normal(size=(3, 5)), rng.normal(size=(3, 5))
    b_g, b_fc = rng.normal(size=5), rng.normal(size=5)
    g, fc, y = R.swiglu_forward_ref(x, w_g, b_g, w_fc, b_fc)
    want = torch.nn.functional.silu(torch.tensor(x @ w_g + b_g)) * torch.tensor(x @ w_fc + b_fc)
    np.testing.assert_allclose(y, want.numpy(), rtol=1e-13)
    # g and fc against the sums written out term by term
    for m in range(4):
        for n in range(5):
            sg = b_g[n] + sum(x[m, k] * w_g[k, n] for k in range(3))
            sf = b_fc[n] + sum(x[m, k] * w_fc[k, n] for k in range(3))
            assert abs(g[m, n] - sg) <= 1e-12 * (1 + abs(sg))
            assert abs(fc[m, n] - sf) <= 1e-12 * (1 + abs(sf))


# ----------------------------------------------------------------------------------
# planted mistakes: each mutation of the oracle must fail at least one pin
# ----------------------------------------------------------------------------------

def _sig(t):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-np.asarray(t, dtype=np.float64)))


def _swish_variant(kind):
    def f(grad, x, beta=1.0):
        b = 1.0 if beta is None else float(np.float32(beta))
        x = np.asarray(x, dtype=np.float64)
        t = b * x
        s = _sig(t)
        if kind == "drop_one":
            fac = s * (t * (1 - s))
        elif kind == "sign":
            fac = s * (1 - t * (1 - s))
        elif kind == "beta_lost_in_factor":
            fac = s * (1 + x * (1 - s))
        elif kind == "sigma_of_x":
            s = _sig(x)
            fac = s * (1 + t * (1 - s))
        elif kind == "beta_not_float32":
            t = (1.0 if beta is None else float(beta)) * x
            s = _sig(t)
            fac = s * (1 + t * (1 - s))
        elif kind == "silu_not_grad":
            fac = t * s
        return np.asarray(grad, dtype=np.float64) * fac
    return f


def _b_variant(kind):
    def f(dy, g, fc, db_g0=None, db_fc0=None):
        dy, g, fc = (np.asarray(a, dtype=np.float64) for a in (dy, g, fc))
        N = dy.shape[-1]
        s = _sig(g)
        dg = dy * fc * s * (1 + g * (1 - s))
        dfc = dy * g * s
        if kind == "dg_no_fc":
            dg = dy * s * (1 + g * (1 - s))
        elif kind == "dfc_no_g":
            dfc = dy * s
        elif kind == "swap":
            dg, dfc = dfc, dg
        elif kind == "dg_sign":
            dg = dy * fc * s * (1 - g * (1 - s))
        db_g = (np.zeros(N) if db_g0 is None else np.asarray(db_g0, dtype=np.float64)) + dg.sum(0)
        db_fc = (np.zeros(N) if db_fc0 is None else np.asarray(db_fc0, dtype=np.float64)) + dfc.sum(0)
        if kind == "db_drop_init":
            db_g = dg.sum(0)
        if kind == "db_mean":
            db_g = db_g / dy.shape[0]
        return dg, dfc, db_g, db_fc
    return f


def _w_variant(kind):
    def f(x, dg, dfc, dw_g0=None, dw_fc0=None):
        x, dg, dfc = (np.asarray(a, dtype=np.float64) for a in (x, dg, dfc))
        dw_g, dw_fc = x.T @ dg, x.T @ dfc
        if kind == "swap":
            dw_g, dw_fc = dw_fc, dw_g
        elif kind == "reverse_rows":
            dw_g = x[::-1].T @ dg
        if dw_g0 is not None:
            dw_g = dw_g + dw_g0
        if dw_fc0 is not None:
            dw_fc = dw_fc + (dw_fc0 if kind != "drop_init" else 0)
        return dw_g, dw_fc
    return f


def _x_variant(kind):
    def f(dg, dfc, w_g, w_fc):
        dg, dfc, w_g, w_fc = (np.asarray(a, dtype=np.float64) for a in (dg, dfc, w_g, w_fc))
        if kind == "swap_weights":
            return dg @ w_fc.T + dfc @ w_g.T
        if kind == "drop_fc":
            return dg @ w_g.T
        if kind == "minus":
            return dg @ w_g.T - dfc @ w_fc.T
        return dg @ w_g.T + dfc @ w_fc.T
    return f


def _fails_some(pins, *fns):
    for pin in pins:
        try:
            pin(*fns)
        except (AssertionError, ValueError):
            return True
    return False


@pytest.mark.parametrize("kind", ["drop_one", "sign", "beta_lost_in_factor", "sigma_of_x",
                                  "beta_not_float32", "silu_not_grad"])
def test_planted_swish_mistake_is_caught(kind):
    assert _fails_some(SWISH_PINS, _swish_variant(kind))


@pytest.mark.parametrize("stage,kind", [
    ("b", "dg_no_fc"), ("b", "dfc_no_g"), ("b", "swap"), ("b", "dg_sign"),
    ("b", "db_drop_init"), ("b", "db_mean"),
    ("w", "swap"), ("w", "reverse_rows"), ("w", "drop_init"),
    ("x", "swap_weights"), ("x", "drop_fc"), ("x", "minus")])
def test_planted_swiglu_mistake_is_caught(stage, kind):
    fns = [R.b_ref, R.w_ref, R.x_ref]
    fns[{"b": 0, "w": 1, "x": 2}[stage]] = {"b": _b_variant, "w": _w_variant,
                                            "x": _x_variant}[stage](kind)
    # the FD pin is slow; the others suffice to catch every planted mistake
    assert _fails_some([p for p in SWIGLU_PINS if p is not pin_swiglu_fd], *fns)


def _chain_variant(kind):
    """The chained backward with one plausible mistake in how the stages are wired."""
    def f(dy, x, w_g, w_fc, g, fc):
        if kind == "swap_g_fc":             # b stage given fc as the gate
            dg, dfc, db_g, db_fc = R.b_ref(dy, fc, g)
        else:
            dg, dfc, db_g, db_fc = R.b_ref(dy, g, fc)
        if kind == "swap_dg_dfc_into_w":
            dw_g, dw_fc = R.w_ref(x, dfc, dg)
        else:
            dw_g, dw_fc = R.w_ref(x, dg, dfc)
        if kind == "swap_weights_in_x":
            dx = R.x_ref(dg, dfc, w_fc, w_g)
        elif kind == "x_from_dg_only":
            dx = R.x_ref(dg, 0 * dfc, w_g, w_fc)
        else:
            dx = R.x_ref(dg, dfc, w_g, w_fc)
        out = {"dg": dg, "dfc": dfc, "db_g": db_g, "db_fc": db_fc,
               "dw_g": dw_g, "dw_fc": dw_fc, "dx": dx}
        if kind == "swap_db":
            out["db_g"], out["db_fc"] = db_fc, db_g
        return out
    return f


@pytest.mark.parametrize("kind", ["swap_g_fc", "swap_dg_dfc_into_w", "swap_weights_in_x",
                                  "x_from_dg_only", "swap_db"])
def test_planted_chain_mistake_is_caught(kind):
    with pytest.raises(AssertionError):
        pin_swiglu_chain(_chain_variant(kind))
