"""Pins of the fp64 oracle against things other than itself (CPU only).

  * a library routine: PyTorch CPU float64 batch_norm + activation, with autograd;
  * central finite differences of the oracle's own forward (pins the backward);
  * the chain-rule form of the BN gradient from Ioffe & Szegedy (cited by the
    pages), written independently of the oracle's compact form;
  * an exact rational worked example (fractions.Fraction);
  * invariants: mean(xhat) = 0, mean(xhat^2) = v/(v+eps), sum dx = 0 per channel;
  * brute force (pure Python loops) for the statistics on a tiny case;
  * closed form of the running statistics after k steps;
  * storage rounding against numpy / torch casts;
  * the backward with frozen statistics against PyTorch's inference-mode
    batch_norm + activation under autograd, and against finite differences.
"""
import dataclasses
from fractions import Fraction
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = np.sqrt(np.mean(b * b)) + 1e-300
    return float(np.max(np.abs(a - b)) / scale)


def _draw(wl, seed=None):
    inp = workloads.make_inputs(wl, seed=seed)
    x = workloads.from_storage(inp.x, wl.N, wl.C, wl.H, wl.W, wl.layout, wl.dtype)
    dy = workloads.from_storage(inp.dy, wl.N, wl.C, wl.H, wl.W, wl.layout, wl.dtype)
    return inp, x, dy


def _torch_act(z, act, p):
    if act == "leaky_relu":
        return F.leaky_relu(z, negative_slope=p)
    if act == "elu":
        return F.elu(z, alpha=p)
    return z


def _torch_reference(x, dy, gamma, beta, act, p, eps, momentum=0.1, rm=None, rv=None):
    xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    gt = torch.tensor(np.asarray(gamma, np.float64), requires_grad=True)
    bt = torch.tensor(np.asarray(beta, np.float64), requires_grad=True)
    rmt = None if rm is None else torch.tensor(np.asarray(rm, np.float64))
    rvt = None if rv is None else torch.tensor(np.asarray(rv, np.float64))
    z = F.batch_norm(xt, rmt, rvt, gt, bt, training=True, momentum=momentum, eps=eps)
    y = _torch_act(z, act, p)
    y.backward(torch.tensor(dy, dtype=torch.float64))
    return {"y": y.detach().numpy(), "dx": xt.grad.numpy(), "dgamma": gt.grad.numpy(),
            "dbeta": bt.grad.numpy(),
            "running_mean": None if rmt is None else rmt.numpy(),
            "running_var": None if rvt is None else rvt.numpy()}


# small shapes that keep every recipe's character (config 1 as is; 2-5 shrunk)
SMALL = [
    workloads.config(1),
    workloads.config(2).with_shape(4, 8, 6, 7),
    workloads.config(3).with_shape(2, 8, 5, 9),
    workloads.config(4).with_shape(3, 16, 7, 5),
    workloads.config(5).with_shape(4, 16, 7, 7),
    # ELU with alpha != 1, so that alpha-dependent terms cannot hide behind alpha = 1
    dataclasses.replace(workloads.config(4).with_shape(2, 8, 6, 5), act_param=0.5,
                        name="stress_elu_alpha_half"),
]


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_forward_and_backward_match_torch_fp64(wl):
    _, x, dy = _draw(wl)
    inp = workloads.make_inputs(wl)
    ref = _torch_reference(x, dy, inp.gamma, inp.beta, wl.act, wl.act_param, wl.eps,
                           wl.momentum, inp.running_mean, inp.running_var)
    f = oracle.forward_train(x, inp.gamma, inp.beta, wl.act, wl.act_param, wl.eps, wl.momentum,
                             inp.running_mean, inp.running_var)
    assert _rel(f["y"], ref["y"]) < 1e-12
    assert _rel(f["running_mean"], ref["running_mean"]) < 1e-12
    assert _rel(f["running_var"], ref["running_var"]) < 1e-12
    var_t, mean_t = torch.var_mean(torch.tensor(x), dim=(0, 2, 3), unbiased=False)
    assert _rel(f["mean"], mean_t.numpy()) < 1e-12
    assert _rel(f["var"], var_t.numpy()) < 1e-12
    assert _rel(f["invstd"], 1.0 / np.sqrt(var_t.numpy() + wl.eps)) < 1e-12

    # backward from y (form I), form II and the conventional backward from x
    b1 = oracle.backward_from_y(f["y"], dy, inp.gamma, inp.beta, f["invstd"], wl.act, wl.act_param)
    b2 = oracle.backward_from_y_form2(f["y"], dy, inp.gamma, inp.beta, f["invstd"], wl.act,
                                      wl.act_param)
    bx = oracle.backward_from_x(x, dy, inp.gamma, inp.beta, wl.act, wl.act_param, wl.eps)
    tol = 1e-9 if wl.act == "elu" else 1e-11   # ELU: log1p(expm1(z)) round trip at z << 0
    for b in (b1, b2, bx):
        assert _rel(b["dx"], ref["dx"]) < tol
        assert _rel(b["dgamma"], ref["dgamma"]) < tol
        assert _rel(b["dbeta"], ref["dbeta"]) < tol


@pytest.mark.parametrize("act,p", [("leaky_relu", 0.01), ("elu", 1.0), ("elu", 0.5),
                                   ("identity", 0.0), ("leaky_relu", 0.2)])
def test_eval_forward_matches_torch(act, p):
    rng = np.random.default_rng(7)
    x = rng.normal(0.3, 2.0, size=(3, 5, 4, 3))
    g = rng.uniform(-1.5, 1.5, 5)
    b = rng.normal(0, 0.3, 5)
    rm = rng.normal(0, 1, 5)
    rv = rng.uniform(0.2, 3.0, 5)
    y = oracle.forward_eval(x, g, b, rm, rv, act, p, 1e-4)
    z = F.batch_norm(torch.tensor(x), torch.tensor(rm), torch.tensor(rv), torch.tensor(g),
                     torch.tensor(b), training=False, eps=1e-4)
    assert _rel(y, _torch_act(z, act, p).numpy()) < 1e-13


EVAL_ACTS = [("leaky_relu", 0.01), ("elu", 1.0), ("elu", 0.5), ("identity", 0.0),
             ("leaky_relu", 0.2)]


def _eval_case(seed=17, shape=(3, 5, 4, 3)):
    rng = np.random.default_rng(seed)
    C = shape[1]
    x = rng.normal(0.3, 2.0, size=shape)
    dy = rng.normal(size=shape)
    g = rng.uniform(0.5, 1.5, C) * np.where(np.arange(C) % 2 == 0, 1.0, -1.0)
    b = rng.normal(0, 0.3, C)
    rm = rng.normal(0, 1, C)
    rv = rng.uniform(0.2, 3.0, C)
    return x, dy, g, b, rm, rv


@pytest.mark.parametrize("act,p", EVAL_ACTS)
def test_eval_backward_matches_torch(act, p):
    """Frozen statistics: torch's inference-mode batch_norm treats the running
    statistics as constants, so its autograd is the reference."""
    x, dy, g, b, rm, rv = _eval_case()
    eps = 1e-4
    y = oracle.forward_eval(x, g, b, rm, rv, act, p, eps)
    bw = oracle.backward_eval(y, dy, g, b, rv, act, p, eps)
    xt = torch.tensor(x, requires_grad=True)
    gt = torch.tensor(g, requires_grad=True)
    bt = torch.tensor(b, requires_grad=True)
    z = F.batch_norm(xt, torch.tensor(rm), torch.tensor(rv), gt, bt, training=False, eps=eps)
    _torch_act(z, act, p).backward(torch.tensor(dy))
    tol = 1e-9 if act == "elu" else 1e-12
    assert _rel(bw["dx"], xt.grad.numpy()) < tol
    assert _rel(bw["dgamma"], gt.grad.numpy()) < tol
    assert _rel(bw["dbeta"], bt.grad.numpy()) < tol


def test_eval_backward_matches_finite_differences():
    x, dy, g, b, rm, rv = _eval_case(seed=23, shape=(2, 3, 3, 2))
    act, p, eps = "elu", 0.7, 1e-3

    def loss(xx, gg, bb):
        return float(np.sum(dy * oracle.forward_eval(xx, gg, bb, rm, rv, act, p, eps)))

    y = oracle.forward_eval(x, g, b, rm, rv, act, p, eps)
    bw = oracle.backward_eval(y, dy, g, b, rv, act, p, eps)
    h = 1e-6
    for i in range(x.size):
        xp, xm = x.copy(), x.copy()
        xp.reshape(-1)[i] += h
        xm.reshape(-1)[i] -= h
        fd = (loss(xp, g, b) - loss(xm, g, b)) / (2 * h)
        assert abs(fd - bw["dx"].reshape(-1)[i]) <= 1e-6 * (abs(fd) + 1.0)
    for c in range(x.shape[1]):
        gp, gm = g.copy(), g.copy()
        gp[c] += h
        gm[c] -= h
        fd = (loss(x, gp, b) - loss(x, gm, b)) / (2 * h)
        assert abs(fd - bw["dgamma"][c]) <= 1e-6 * (abs(fd) + 1.0)
        bp, bm = b.copy(), b.copy()
        bp[c] += h
        bm[c] -= h
        fd = (loss(x, g, bp) - loss(x, g, bm)) / (2 * h)
        assert abs(fd - bw["dbeta"][c]) <= 1e-6 * (abs(fd) + 1.0)


def test_backward_matches_finite_differences():
    wl = workloads.config(1)
    inp, x, dy = _draw(wl)
    g = inp.gamma.astype(np.float64)
    b = inp.beta.astype(np.float64)

    def loss(xx, gg, bb):
        return float(np.sum(dy * oracle.forward_train(xx, gg, bb, wl.act, wl.act_param,
                                                      wl.eps)["y"]))

    f = oracle.forward_train(x, g, b, wl.act, wl.act_param, wl.eps)
    bw = oracle.backward_from_y(f["y"], dy, g, b, f["invstd"], wl.act, wl.act_param)
    h = 1e-6
    z = (f["y"] > 0) * f["y"] + (f["y"] <= 0) * f["y"] / wl.act_param
    rng = np.random.default_rng(3)
    flat = [i for i in rng.permutation(x.size) if abs(z.reshape(-1)[i]) > 1e-3][:40]
    for i in flat:
        xp, xm = x.copy(), x.copy()
        xp.reshape(-1)[i] += h
        xm.reshape(-1)[i] -= h
        fd = (loss(xp, g, b) - loss(xm, g, b)) / (2 * h)
        an = bw["dx"].reshape(-1)[i]
        assert abs(fd - an) <= 1e-6 * (abs(an) + 1.0), (i, fd, an)
    for c in range(wl.C):
        gp, gm = g.copy(), g.copy()
        gp[c] += h
        gm[c] -= h
        fd = (loss(x, gp, b) - loss(x, gm, b)) / (2 * h)
        assert abs(fd - bw["dgamma"][c]) <= 1e-6 * (abs(fd) + 1.0)
        bp, bm = b.copy(), b.copy()
        bp[c] += h
        bm[c] -= h
        fd = (loss(x, g, bp) - loss(x, g, bm)) / (2 * h)
        assert abs(fd - bw["dbeta"][c]) <= 1e-6 * (abs(fd) + 1.0)


def _chain_rule_bn_backward(x, dz, gamma, eps):
    """BN backward as the chain rule of Ioffe & Szegedy (Algorithm 1 and its
    back-propagation), per channel: through xhat, then var, then mean."""
    m = x.shape[0] * x.shape[2] * x.shape[3]
    mu = x.mean(axis=(0, 2, 3), keepdims=True)
    var = ((x - mu) ** 2).mean(axis=(0, 2, 3), keepdims=True)
    g = gamma.reshape(1, -1, 1, 1)
    dxhat = dz * g
    dvar = np.sum(dxhat * (x - mu) * -0.5 * (var + eps) ** -1.5, axis=(0, 2, 3), keepdims=True)
    dmu = (np.sum(dxhat * -1.0 / np.sqrt(var + eps), axis=(0, 2, 3), keepdims=True)
           + dvar * np.sum(-2.0 * (x - mu), axis=(0, 2, 3), keepdims=True) / m)
    return dxhat / np.sqrt(var + eps) + dvar * 2.0 * (x - mu) / m + dmu / m


@pytest.mark.parametrize("gamma_one", [True, False])
def test_identity_activation_is_textbook_bn(gamma_one):
    rng = np.random.default_rng(11)
    x = rng.normal(1.0, 3.0, size=(4, 3, 5, 5))
    dy = rng.normal(size=x.shape)
    g = np.ones(3) if gamma_one else rng.uniform(-2, 2, 3)
    b = np.zeros(3) if gamma_one else rng.normal(size=3)
    f = oracle.forward_train(x, g, b, "identity", 0.0, 1e-3)
    bw = oracle.backward_from_y(f["y"], dy, g, b, f["invstd"], "identity", 0.0)
    assert _rel(bw["dx"], _chain_rule_bn_backward(x, dy, g, 1e-3)) < 1e-12
    # leaky ReLU with slope 1 is the identity
    f1 = oracle.forward_train(x, g, b, "leaky_relu", 1.0, 1e-3)
    bw1 = oracle.backward_from_y(f1["y"], dy, g, b, f1["invstd"], "leaky_relu", 1.0)
    assert np.array_equal(f1["y"], f["y"])
    assert _rel(bw1["dx"], bw["dx"]) < 1e-15


def test_exact_rational_example():
    """Hand example, eps = 0: x = (-7, -1, 1, 7) has mean 0 and variance 25, so
    invstd = 1/5 and xhat = (-7, -1, 1, 7)/5.  gamma = 2, beta = 1/2, leaky slope
    1/100, dy = (1, 1, 1, 1).  Expected values in exact rational arithmetic, through
    the chain rule (not the oracle's compact formula)."""
    xs = [Fraction(v) for v in (-7, -1, 1, 7)]
    g, b, a = Fraction(2), Fraction(1, 2), Fraction(1, 100)
    m = len(xs)
    mu = sum(xs) / m
    var = sum((v - mu) ** 2 for v in xs) / m
    assert var == 25
    inv = Fraction(1, 5)
    xh = [(v - mu) * inv for v in xs]
    z = [g * t + b for t in xh]
    y = [t if t > 0 else a * t for t in z]
    dy = [Fraction(1)] * 4
    dz = [d if t > 0 else a * d for d, t in zip(dy, z)]
    dbeta = sum(dz)
    dgamma = sum(d * t for d, t in zip(dz, xh))
    # chain rule with eps = 0: dvar = sum dxhat (x-mu) (-1/2) var^-3/2, var^-3/2 = inv^3
    dxh = [d * g for d in dz]
    dvar = sum(d * (v - mu) for d, v in zip(dxh, xs)) * Fraction(-1, 2) * inv ** 3
    dmu = -inv * sum(dxh) + dvar * sum(-2 * (v - mu) for v in xs) / m
    dx = [d * inv + dvar * 2 * (v - mu) / m + dmu / m for d, v in zip(dxh, xs)]
    assert sum(dx) == 0

    x = np.array([float(v) for v in xs]).reshape(1, 1, 1, 4)
    f = oracle.forward_train(x, [2.0], [0.5], "leaky_relu", 0.01, 0.0)
    assert np.allclose(f["y"].reshape(-1), [float(v) for v in y], rtol=0, atol=1e-15)
    assert abs(f["invstd"][0] - 0.2) < 1e-16
    bw = oracle.backward_from_y(f["y"], np.ones_like(x), [2.0], [0.5], f["invstd"], "leaky_relu",
                                0.01)
    assert np.allclose(bw["dx"].reshape(-1), [float(v) for v in dx], rtol=0, atol=1e-14)
    assert abs(bw["dbeta"][0] - float(dbeta)) < 1e-14
    assert abs(bw["dgamma"][0] - float(dgamma)) < 1e-14
    assert float(dbeta) == 3.01 and abs(float(dgamma) - 1.386) < 1e-15


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_invariants(wl):
    inp, x, dy = _draw(wl)
    f = oracle.forward_train(x, inp.gamma, inp.beta, wl.act, wl.act_param, wl.eps)
    bw = oracle.backward_from_y(f["y"], dy, inp.gamma, inp.beta, f["invstd"], wl.act,
                                wl.act_param, want_xhat=True)
    xh = bw["xhat"]
    tol = 1e-8 if wl.act == "elu" else 1e-12
    # xhat rebuilt from y alone has zero mean and second moment v/(v+eps)
    assert np.max(np.abs(xh.mean(axis=(0, 2, 3)))) < tol
    v = f["var"]
    assert np.max(np.abs((xh ** 2).mean(axis=(0, 2, 3)) - v / (v + wl.eps))) < tol
    # the rebuilt xhat is the forward's xhat: exact inversion y -> xhat
    xh_fwd = (x - f["mean"][None, :, None, None]) * f["invstd"][None, :, None, None]
    assert np.max(np.abs(xh - xh_fwd)) < tol
    # per channel, the input gradient sums to zero (the mean is subtracted)
    s = bw["dx"].sum(axis=(0, 2, 3))
    assert np.max(np.abs(s)) < 1e-10 * np.max(np.abs(bw["dx"])) * wl.m


def test_eps_zero_gives_unit_variance_and_orthogonal_gradient():
    rng = np.random.default_rng(5)
    x = rng.normal(-2.0, 0.7, size=(3, 4, 6, 6))
    dy = rng.normal(size=x.shape)
    g, b = rng.uniform(0.5, 1.5, 4), rng.normal(0, 0.3, 4)
    f = oracle.forward_train(x, g, b, "elu", 1.0, 0.0)
    bw = oracle.backward_from_y(f["y"], dy, g, b, f["invstd"], "elu", 1.0, want_xhat=True)
    xh = bw["xhat"]
    assert np.max(np.abs((xh ** 2).mean(axis=(0, 2, 3)) - 1.0)) < 1e-12
    assert np.max(np.abs((bw["dx"] * xh).sum(axis=(0, 2, 3)))) < 1e-11


def test_statistics_brute_force():
    wl = workloads.config(1)
    inp, x, _ = _draw(wl)
    f = oracle.forward_train(x, inp.gamma, inp.beta, wl.act, wl.act_param, wl.eps)
    for c in range(wl.C):
        vals = [x[n, c, h, w] for n in range(wl.N) for h in range(wl.H) for w in range(wl.W)]
        mu = math.fsum(vals) / len(vals)
        var = math.fsum((v - mu) ** 2 for v in vals) / len(vals)
        assert abs(f["mean"][c] - mu) < 1e-14 * (1 + abs(mu))
        assert abs(f["var"][c] - var) < 1e-13 * var
        for n in range(wl.N):
            for h in range(wl.H):
                for w in range(wl.W):
                    z = inp.gamma[c] * (x[n, c, h, w] - mu) / math.sqrt(var + wl.eps) + inp.beta[c]
                    yy = z if z > 0 else wl.act_param * z
                    assert abs(f["y"][n, c, h, w] - yy) < 1e-13 * (1 + abs(yy))


def test_running_statistics_closed_form():
    rng = np.random.default_rng(2)
    x = rng.normal(0.7, 1.3, size=(2, 3, 4, 4))
    g, b = np.ones(3), np.zeros(3)
    rm0, rv0 = rng.normal(size=3), rng.uniform(0.5, 2, 3)
    rm, rv = rm0.copy(), rv0.copy()
    mom, k = 0.1, 7
    for _ in range(k):
        f = oracle.forward_train(x, g, b, "leaky_relu", 0.01, 1e-5, mom, rm, rv)
        rm, rv = f["running_mean"], f["running_var"]
    m = x.size // 3
    keep = (1 - mom) ** k
    mu = x.mean(axis=(0, 2, 3))
    unb = x.var(axis=(0, 2, 3), ddof=1)
    assert np.allclose(rm, keep * rm0 + (1 - keep) * mu, rtol=1e-13, atol=1e-14)
    assert np.allclose(rv, keep * rv0 + (1 - keep) * unb, rtol=1e-13, atol=1e-14)
    assert np.allclose(f["var"] * m / (m - 1), unb, rtol=1e-13)


def test_elu_inverse_tail_clamp():
    # y = -alpha exactly can only come from rounding; the clamp keeps z finite
    y = np.array([-1.0, -0.5, -1e-3, 0.0, 2.0]).reshape(1, 1, 1, 5)
    bw = oracle.backward_from_y(y, np.ones_like(y), [1.0], [0.0], [1.0], "elu", 1.0,
                                want_xhat=True)
    xh = bw["xhat"].reshape(-1)
    assert abs(xh[0] - math.log1p(-1.0 + 2.0 ** -24)) < 1e-15
    assert abs(xh[1] - math.log(0.5)) < 1e-15
    assert xh[3] == 0.0 and xh[4] == 2.0


def test_round_storage_f32_matches_numpy():
    rng = np.random.default_rng(9)
    v = np.concatenate([rng.normal(size=1000) * 10.0 ** rng.uniform(-40, 38, 1000),
                        [0.0, -0.0, np.inf, -np.inf, 1e-45, 3.4028235677973366e38]])
    r = oracle.round_storage(v.copy(), "f32")
    assert np.array_equal(r, v.astype(np.float32).astype(np.float64))


def test_round_storage_bf16_matches_torch_on_f32_values():
    rng = np.random.default_rng(10)
    f32 = np.concatenate([
        (rng.normal(size=4000) * 10.0 ** rng.uniform(-40, 38, 4000)).astype(np.float32),
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 2 ** -130, 3e38, -3.39e38],
                 np.float32)])
    r = oracle.round_storage(f32.astype(np.float64), "bf16")
    t = torch.from_numpy(f32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(r, t)
    # halfway cases round to even
    assert oracle.round_storage(np.array([1.0 + 2 ** -8]), "bf16")[0] == 1.0
    assert oracle.round_storage(np.array([1.0 + 3 * 2 ** -8]), "bf16")[0] == 1.0 + 2 ** -6


def test_round_storage_f16_matches_numpy_on_f32_values():
    """numpy's float32 -> float16 cast rounds to nearest even, with subnormals and
    overflow to infinity; on float32 inputs one rounding from fp64 is the same."""
    rng = np.random.default_rng(12)
    f32 = np.concatenate([
        (rng.normal(size=4000) * 10.0 ** rng.uniform(-9, 5, 4000)).astype(np.float32),
        np.array([1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11, -(1.0 + 2 ** -11), 2 ** -25, 3 * 2 ** -26,
                  2 ** -24, 65504.0, 65519.0, 65520.0, -70000.0, 6.1e-5], np.float32)])
    r = oracle.round_storage(f32.astype(np.float64), "f16")
    with np.errstate(over="ignore"):
        ref = f32.astype(np.float16).astype(np.float64)
    assert np.array_equal(r, ref)
    assert oracle.round_storage(np.array([1.0 + 2 ** -11]), "f16")[0] == 1.0
    assert oracle.round_storage(np.array([65520.0]), "f16")[0] == np.inf


def test_oracle_rejects_invalid_arguments():
    x = np.zeros((1, 2, 1, 1))
    with pytest.raises(ValueError):
        oracle.forward_train(x, [1, 1], [0, 0])          # m = 1
    x = np.zeros((2, 2, 1, 1))
    with pytest.raises(ValueError):
        oracle.forward_train(x, [1, 1], [0, 0], "leaky_relu", 0.0)
    with pytest.raises(ValueError):
        oracle.forward_train(x, [1, 1], [0, 0], "elu", -1.0)


# ---------------------------------------------------------------------------
# optimized checkpointing (the block keeps xhat instead of x)

@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_ckpt_forward_matches_torch_fp64(wl):
    """xhat against (x - mean)/sqrt(var + eps) from torch's statistics, y against
    torch's batch_norm + activation, running statistics against torch's update."""
    _, x, dy = _draw(wl)
    inp = workloads.make_inputs(wl)
    ref = _torch_reference(x, dy, inp.gamma, inp.beta, wl.act, wl.act_param, wl.eps,
                           wl.momentum, inp.running_mean, inp.running_var)
    f = oracle.forward_train_ckpt(x, inp.gamma, inp.beta, wl.act, wl.act_param, wl.eps,
                                  wl.momentum, inp.running_mean, inp.running_var)
    xt = torch.tensor(x)
    var_t, mean_t = torch.var_mean(xt, dim=(0, 2, 3), unbiased=False, keepdim=True)
    xhat_t = ((xt - mean_t) / torch.sqrt(var_t + wl.eps)).numpy()
    assert _rel(f["xhat"], xhat_t) < 1e-12
    assert _rel(f["y"], ref["y"]) < 1e-12
    assert _rel(f["running_mean"], ref["running_mean"]) < 1e-12
    assert _rel(f["running_var"], ref["running_var"]) < 1e-12
    assert _rel(f["invstd"], 1.0 / np.sqrt(var_t.numpy().reshape(-1) + wl.eps)) < 1e-12
    # the layer output rebuilt from the checkpoint: act(gamma xhat + beta) by torch
    yr = oracle.recompute_from_xhat(f["xhat"], inp.gamma, inp.beta, wl.act, wl.act_param)
    g = torch.tensor(inp.gamma.astype(np.float64)).view(1, -1, 1, 1)
    b = torch.tensor(inp.beta.astype(np.float64)).view(1, -1, 1, 1)
    yt = _torch_act(g * torch.tensor(f["xhat"]) + b, wl.act, wl.act_param).numpy()
    assert _rel(yr, yt) < 1e-13
    assert _rel(yr, ref["y"]) < 1e-12


@pytest.mark.parametrize("wl", SMALL, ids=lambda w: w.name)
def test_ckpt_backward_matches_torch_fp64(wl):
    """The backward from xhat (computed from x by torch) against torch's autograd of
    batch_norm + activation taken from x."""
    _, x, dy = _draw(wl)
    inp = workloads.make_inputs(wl)
    ref = _torch_reference(x, dy, inp.gamma, inp.beta, wl.act, wl.act_param, wl.eps)
    xt = torch.tensor(x)
    var_t, mean_t = torch.var_mean(xt, dim=(0, 2, 3), unbiased=False, keepdim=True)
    inv_t = 1.0 / torch.sqrt(var_t + wl.eps)
    xhat = ((xt - mean_t) * inv_t).numpy()
    b = oracle.backward_from_xhat(xhat, dy, inp.gamma, inp.beta, inv_t.numpy().reshape(-1),
                                  wl.act, wl.act_param)
    assert _rel(b["dx"], ref["dx"]) < 1e-11
    assert _rel(b["dgamma"], ref["dgamma"]) < 1e-11
    assert _rel(b["dbeta"], ref["dbeta"]) < 1e-11


def test_ckpt_backward_matches_finite_differences():
    """Central differences of the checkpointing forward's y (loss sum dy*y) against
    the backward from its xhat: dx, dgamma, dbeta."""
    wl = dataclasses.replace(workloads.config(4).with_shape(2, 3, 4, 5), act_param=0.5)
    inp, x, dy = _draw(wl)
    g = inp.gamma.astype(np.float64)
    b = inp.beta.astype(np.float64)

    def loss(xx, gg, bb):
        return float(np.sum(dy * oracle.forward_train_ckpt(xx, gg, bb, wl.act, wl.act_param,
                                                           wl.eps)["y"]))

    f = oracle.forward_train_ckpt(x, g, b, wl.act, wl.act_param, wl.eps)
    bw = oracle.backward_from_xhat(f["xhat"], dy, g, b, f["invstd"], wl.act, wl.act_param)
    h = 1e-6
    for i in range(x.size):
        xp, xm = x.copy(), x.copy()
        xp.reshape(-1)[i] += h
        xm.reshape(-1)[i] -= h
        fd = (loss(xp, g, b) - loss(xm, g, b)) / (2 * h)
        an = bw["dx"].reshape(-1)[i]
        assert abs(fd - an) <= 1e-6 * (abs(an) + 1.0), (i, fd, an)
    for c in range(wl.C):
        for vec, key in ((g, "dgamma"), (b, "dbeta")):
            vp, vm = vec.copy(), vec.copy()
            vp[c] += h
            vm[c] -= h
            args_p = (x, vp, b) if key == "dgamma" else (x, g, vp)
            args_m = (x, vm, b) if key == "dgamma" else (x, g, vm)
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - bw[key][c]) <= 1e-6 * (abs(fd) + 1.0), (key, c)


def test_ckpt_backward_branches_on_the_exact_sign_of_z():
    """Leaky ReLU slope where gamma*xhat + beta is within a rounding of zero: the side
    is that of the exact value.  gamma = xhat = 1 + 2^-30 make gamma*xhat =
    1 + 2^-29 + 2^-60, which fp64 rounds to 1 + 2^-29; with beta = -(1 + 2^-29)
    the exact z is +2^-60 (slope 1), although a multiply then an add gives 0
    (slope a).  With beta = -(1 + 2^-28) the exact z is negative (slope a)."""
    a = 0.01
    e = 1.0 + 2.0 ** -30
    xh = np.full((1, 1, 1, 1), e)
    dy = np.ones((1, 1, 1, 1))
    g = np.array([e])
    for beta, slope in ((-(1.0 + 2.0 ** -29), 1.0), (-(1.0 + 2.0 ** -28), a)):
        r = oracle.backward_from_xhat(xh, dy, g, np.array([beta]), np.ones(1), "leaky_relu", a)
        assert r["dbeta"][0] == slope, (beta, r["dbeta"][0])
