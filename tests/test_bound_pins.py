"""Pins for oracle.bounds: the running-error bound of the bfloat16 backward.

The bound says: if every quantity the model rounds carries a relative error
of at most u, and every float32 sum and logit an error of at most
n * 2^-24 times the sum of its terms' magnitudes, then each gradient element
moves by at most u * E (to first order).  The checks below evaluate that
model directly, by brute force: ``perturbed`` recomputes the backward from
the oracle's records with an explicit perturbation at every site, and

* on one-term layers (T = P = h = 1, depth 0; d = 1 or 4096), where no
  site is shared between terms, the largest change over all sign patterns
  of the sites equals u * E (the bound is tight, so no term is missing or
  doubled);
* on small random layers, random perturbations at every site stay within
  u * E (the bound holds where terms share sites and cancel);
* GELU's first and second derivatives match finite differences, and
  ``bounds.gelu`` matches the oracle's own GELU (depth-0 layer).
"""
import importlib.util
import itertools
import os
import tempfile

import numpy as np
import pytest

import oracle
from oracle import bounds

U = bounds.U_BF16
R = bounds.R_F32


def _records(x, W, b, V, Wo, variant):
    f = oracle.forward(x, W, b, V, Wo, want_y=False, want_records=True, variant=variant)
    return f["rec_node"].astype(np.int64), f["rec_a"]


SITES = ("a", "Hacc", "H", "dHacc", "dH", "gacc", "dS", "da", "G", "Wacc", "xacc", "dx", "dWacc",
         "dbacc", "dVacc")


def perturbed(x, W, V, Wo, dy, node, a, variant, delta):
    """The backward with each model site perturbed: delta[site] (broadcast to
    the site's quantity, values in [-1, 1]) times u times the site's error
    scale.  delta = {} gives the exact gradients."""
    def dl(name, shape):
        v = delta.get(name, 0.0)
        return np.broadcast_to(v, shape) if np.ndim(v) else np.full(shape, float(v))

    T, d = x.shape
    P, N, _ = W.shape
    h = V.shape[2]
    L = node.shape[2]
    pidx = np.arange(P)[None, :, None]
    Wn, Vn = W[pidx, node], V[pidx, node]
    a = a + U * dl("a", a.shape) * d * R * np.einsum("tc,tplc->tpl", np.abs(x), np.abs(Wn))
    G, G1 = bounds.gelu(a), bounds.gelu_d1(a)
    if variant == 0:
        terms = G[..., None] * Vn
    else:
        terms = a[..., None] * Vn
    acc = terms.sum(axis=2) + U * dl("Hacc", (T, P, h)) * L * R * np.abs(terms).sum(axis=2)
    S = acc
    H = (acc if variant == 0 else bounds.gelu(acc)) * (1 + U * dl("H", (T, P, h)))
    dH = dy @ Wo.T + U * dl("dHacc", (T, P * h)) * d * R * (np.abs(dy) @ np.abs(Wo).T)
    dH = (dH * (1 + U * dl("dH", (T, P * h)))).reshape(T, P, h)
    if variant == 0:
        src = dH
    else:
        src = bounds.gelu_d1(S) * dH * (1 + U * dl("dS", (T, P, h)))
    g = np.einsum("tpj,tplj->tpl", src, Vn)
    g = g + U * dl("gacc", g.shape) * h * R * np.einsum("tpj,tplj->tpl", np.abs(src), np.abs(Vn))
    da = (g * G1 if variant == 0 else g) * (1 + U * dl("da", g.shape))
    wgt = (G if variant == 0 else a) * (1 + U * dl("G", a.shape))

    out = {}
    Hf = H.reshape(T, P * h)
    out["dW_out"] = Hf.T @ dy + U * dl("Wacc", (P * h, d)) * T * R * (np.abs(Hf).T @ np.abs(dy))
    dx = np.einsum("tpl,tplc->tc", da, Wn)
    dx = dx + U * dl("xacc", (T, d)) * P * L * R * np.einsum("tpl,tplc->tc", np.abs(da), np.abs(Wn))
    out["dx"] = dx * (1 + U * dl("dx", (T, d)))
    dW = np.zeros((P, N, d))
    adW = np.zeros((P, N, d))
    db = np.zeros((P, N))
    adb = np.zeros((P, N))
    dV = np.zeros((P, N, h))
    adV = np.zeros((P, N, h))
    for t in range(T):
        for p in range(P):
            for l in range(L):
                n = node[t, p, l]
                dW[p, n] += da[t, p, l] * x[t]
                adW[p, n] += np.abs(da[t, p, l] * x[t])
                db[p, n] += da[t, p, l]
                adb[p, n] += abs(da[t, p, l])
                dV[p, n] += wgt[t, p, l] * src[t, p]
                adV[p, n] += np.abs(wgt[t, p, l] * src[t, p])
    out["dW_node"] = dW + U * dl("dWacc", dW.shape) * T * R * adW
    out["db_node"] = db + U * dl("dbacc", db.shape) * T * R * adb
    out["dV_node"] = dV + U * dl("dVacc", dV.shape) * T * R * adV
    return out


def _layer(rng, T, d, P, D, h, scale_x=1.0):
    N = (1 << (D + 1)) - 1
    x = rng.standard_normal((T, d)) * scale_x
    W = rng.standard_normal((P, N, d)) / np.sqrt(d)
    b = rng.standard_normal((P, N)) * 0.3
    V = rng.standard_normal((P, N, h))
    Wo = rng.standard_normal((P * h, d)) / np.sqrt(P * h)
    dy = rng.standard_normal((T, d))
    return x, W, b, V, Wo, dy


def check_tight(mod, variant, seed, d):
    """One term per gradient element: the worst sign pattern of the sites
    moves each gradient by u * E, up to O(u^2)."""
    rng = np.random.default_rng(seed)
    x, W, b, V, Wo, dy = _layer(rng, 1, d, 1, 0, 1, scale_x=1.5)
    node, a = _records(x, W, b, V, Wo, variant)
    E = mod.backward_bound(x, W, V, Wo, dy, node, a, variant)
    ref = perturbed(x, W, V, Wo, dy, node, a, variant, {})
    # Every sign pattern of the sites whose share of E is not negligible (the
    # float32 sums other than the logit's add about 2^-16 of it each; they
    # are held at +1).
    sites = [s for s in ("a", "H", "dH", "dS", "da", "G", "dx") if not (variant == 0 and s == "dS")]
    fixed = {s: 1.0 for s in SITES if s not in sites}
    worst = {k: np.zeros_like(ref[k]) for k in ref}
    for signs in itertools.product((-1.0, 1.0), repeat=len(sites)):
        g = perturbed(x, W, V, Wo, dy, node, a, variant, dict(fixed, **dict(zip(sites, signs))))
        for k in ref:
            worst[k] = np.maximum(worst[k], np.abs(g[k] - ref[k]))
    for k in ref:
        assert (E[k] > 0).all(), k
        ratio = worst[k] / (U * E[k])
        assert (ratio < 1.0 + 4 * U).all(), (k, float(ratio.max()))  # the bound holds
        if variant == 1 and k == "dV_node":
            # FFF-post's dV term a * GELU'(S) dH takes the logit's error
            # twice (through a and through S = a v); the bound adds the two
            # magnitudes, so it is not tight there when they differ in sign.
            assert (ratio > 0.5).all(), (k, float(ratio.min()))
        else:
            assert (ratio > 1.0 - 4 * U).all(), (k, float(ratio.min()))  # and is reached


def check_random(mod, variant, shape):
    """Random perturbations at every site stay within u * E, including sums
    that cancel (two tokens with opposite output gradients)."""
    T, d, P, D, h = shape
    rng = np.random.default_rng(sum(shape) + variant)
    x, W, b, V, Wo, dy = _layer(rng, T, d, P, D, h)
    dy[1] = -dy[0]
    x[1] = x[0]
    node, a = _records(x, W, b, V, Wo, variant)
    E = mod.backward_bound(x, W, V, Wo, dy, node, a, variant)
    ref = perturbed(x, W, V, Wo, dy, node, a, variant, {})
    for k in ref:
        assert (E[k] >= np.abs(ref[k]) * (1 - 1e-12)).all(), k  # never below the value itself
    L = D + 1
    N = (1 << L) - 1
    shapes = {"a": (T, P, L), "Hacc": (T, P, h), "H": (T, P, h), "dHacc": (T, P * h),
              "dH": (T, P * h), "gacc": (T, P, L), "dS": (T, P, h), "da": (T, P, L),
              "G": (T, P, L), "Wacc": (P * h, d), "xacc": (T, d), "dx": (T, d),
              "dWacc": (P, N, d), "dbacc": (P, N), "dVacc": (P, N, h)}
    worst = 0.0
    for trial in range(20):
        r = np.random.default_rng(100 + trial)
        delta = {s: (r.choice([-1.0, 1.0], size=shp) if trial % 2 else r.uniform(-1, 1, shp))
                 for s, shp in shapes.items()}
        g = perturbed(x, W, V, Wo, dy, node, a, variant, delta)
        for k in ref:
            lim = U * E[k] * (1 + 4 * U) + 1e-300
            ratio = np.abs(g[k] - ref[k]) / lim
            worst = max(worst, float(ratio.max()))
            assert (ratio <= 1.0).all(), (k, float(ratio.max()))
    assert worst > 0.05  # the perturbations are not vanishingly small against the bound


@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("seed,d", [(0, 1), (1, 1), (2, 4096)])
def test_one_term_bound_is_tight(variant, seed, d):
    # d = 4096: the logit's float32 sum carries an error comparable to u.
    check_tight(bounds, variant, seed, d)


@pytest.mark.parametrize("variant", [0, 1])
@pytest.mark.parametrize("shape", [(5, 8, 2, 2, 4), (7, 16, 3, 3, 2), (12, 4, 1, 1, 8)])
def test_random_perturbations_stay_within_bound(variant, shape):
    check_random(bounds, variant, shape)


# Plausible mistakes in the bound; each must fail one of the checks above.
MUTANTS = [
    ("dv_drops_dH_error", "                     + np.abs(G)[..., None] * E_dH[:, :, None, :])",
     "                     + 0.0 * E_dH[:, :, None, :])"),
    ("da_drops_gelu2_term", "E_da = np.abs(G1) * E_g + np.abs(g) * np.abs(G2) * e_a + np.abs(da)",
     "E_da = np.abs(G1) * E_g + np.abs(da)"),
    ("da_drops_own_rounding", "E_da = np.abs(G1) * E_g + np.abs(g) * np.abs(G2) * e_a + np.abs(da)",
     "E_da = np.abs(G1) * E_g + np.abs(g) * np.abs(G2) * e_a"),
    ("dx_drops_output_rounding", "                 + np.abs(dx))", "                 )"),
    ("logit_error_dropped", "e_a = d * R_F32 * np.einsum", "e_a = 0.0 * np.einsum"),
    ("dH_rounding_dropped", "E_dH = np.abs(dH) + d * R_F32", "E_dH = 0.0 * np.abs(dH) + d * R_F32"),
    ("H_rounding_doubled", "        E_H = (np.abs(H) + np.einsum", "        E_H = (2 * np.abs(H) + np.einsum"),
    ("post_dS_rounding_dropped",
     "E_dS = np.abs(G1S) * E_dH + np.abs(gelu_d2(S)) * E_S * np.abs(dH) + np.abs(dS)",
     "E_dS = np.abs(G1S) * E_dH + np.abs(gelu_d2(S)) * E_S * np.abs(dH)"),
    ("post_weight_error_dropped", "((np.abs(a) + e_a)[..., None] * np.abs(dS)[:, :, None, :]",
     "((np.abs(a) + 0.0)[..., None] * np.abs(dS)[:, :, None, :]"),
    ("gelu_d2_sign", "return sech2 * s1 + 0.5 * a * sech2 * (s2 - 2.0 * t * s1 * s1)",
     "return sech2 * s1 + 0.5 * a * sech2 * (s2 + 2.0 * t * s1 * s1)"),
    ("node_sum_uses_first_token_only", "    np.add.at(E_onehot, (pp, node, tt), E_da)",
     "    np.add.at(E_onehot, (pp[:1], node[:1], tt[:1]), E_da[:1])"),
]


def _load_mutant(path):
    spec = importlib.util.spec_from_file_location("bounds_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,anchor,replacement", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_bound_mutant_is_caught(name, anchor, replacement):
    with open(bounds.__file__) as f:
        src = f.read()
    assert src.count(anchor) == 1, f"anchor for {name} must occur exactly once"
    with tempfile.TemporaryDirectory() as tmp:
        path = os.path.join(tmp, f"bounds_{name}.py")
        with open(path, "w") as f:
            f.write(src.replace(anchor, replacement))
        mod = _load_mutant(path)
        caught = False
        for check in (lambda: check_tight(mod, 0, 2, 4096), lambda: check_tight(mod, 1, 2, 4096),
                      lambda: check_random(mod, 0, (5, 8, 2, 2, 4)),
                      lambda: check_random(mod, 1, (5, 8, 2, 2, 4))):
            try:
                check()
            except AssertionError:
                caught = True
                break
        assert caught, f"mutant {name} passed every check"


def test_gelu_derivatives_and_oracle_gelu():
    a = np.linspace(-6, 6, 241)
    eps = 1e-5
    fd1 = (bounds.gelu(a + eps) - bounds.gelu(a - eps)) / (2 * eps)
    fd2 = (bounds.gelu_d1(a + eps) - bounds.gelu_d1(a - eps)) / (2 * eps)
    assert np.allclose(bounds.gelu_d1(a), fd1, rtol=1e-7, atol=1e-9)
    assert np.allclose(bounds.gelu_d2(a), fd2, rtol=1e-6, atol=1e-8)
    # The oracle's GELU: a depth-0 layer with one output is y = GELU(x w + b).
    T = a.size
    x = a[:, None]
    ones = np.ones
    f = oracle.forward(x, ones((1, 1, 1)), np.zeros((1, 1)), ones((1, 1, 1)), ones((1, 1)))
    assert np.allclose(f["y"][:, 0], bounds.gelu(a), rtol=1e-14, atol=1e-15)
    assert T == f["y"].shape[0]
