"""Running-error bound for the backward pass in bfloat16 (test infrastructure).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``: the tests use it to
decide how far a bfloat16 gradient may lie from the oracle's float64 one.

What the bound covers.  The gradients of sum(y * dy) with the forward's paths
held fixed (explainer page, section 3.B: only the visited nodes receive
gradient) are sums of products.  A bfloat16 implementation rounds some
intermediate quantities to bfloat16 once each (unit roundoff u = 2^-8) before
the sums that use them, and accumulates every sum and every logit in float32
(unit roundoff 2^-24 = r u with r = 2^-16).  For such a computation, to first
order in u, each element of each gradient g obeys

    |g_computed - g| <= u * E

where E, computed here in float64 from the oracle's own forward records, adds
up the magnitude each rounding can contribute (a running-error bound in the
sense of Higham, "Accuracy and Stability of Numerical Algorithms", 2nd ed.,
section 3.3):

  * a quantity q rounded once contributes |q| times the magnitude of what it
    multiplies;
  * a float32 sum of n terms contributes n r times the sum of the terms'
    magnitudes (the standard n * unit-roundoff bound, here in units of u);
  * an error already carried by an input of a smooth function f (GELU, its
    derivative) is carried through by |f'|.

The rounded quantities are the ones the layer's backward has to hand from
one product to the next: the tree outputs H (or, for FFF-post, the summed
vector S goes through GELU in float32 and H is rounded), the output gradient
dH = dy . W_out^T, for FFF-post dS = GELU'(S) dH, the logit gradients da, the
per-node weights GELU(a) (or a itself for FFF-post) that multiply dH into
dV_node, and the input gradient dx, which is returned in bfloat16.  Nothing
here rounds anything: every E is a sum of magnitudes in float64.

Parity pins: ``tests/test_bound_pins.py`` (one-term cases where every
contribution is known by hand, a case with cancellation, random
perturbations of every rounded quantity within the model, and the GELU
derivatives against finite differences).
"""
from __future__ import annotations

from typing import Dict

import numpy as np

U_BF16 = 2.0 ** -8
R_F32 = 2.0 ** -16  # float32 unit roundoff in units of U_BF16

_C = np.sqrt(2.0 / np.pi)
_K = 0.044715


def gelu(a):
    """GELU, tanh form (explainer page, section 3.C uses GELU as the node
    activation; the tanh form is the one the layer computes)."""
    a = np.asarray(a, dtype=np.float64)
    return 0.5 * a * (1.0 + np.tanh(_C * (a + _K * a ** 3)))


def gelu_d1(a):
    """d GELU / da of the tanh form."""
    a = np.asarray(a, dtype=np.float64)
    t = np.tanh(_C * (a + _K * a ** 3))
    s1 = _C * (1.0 + 3.0 * _K * a * a)
    return 0.5 * (1.0 + t) + 0.5 * a * (1.0 - t * t) * s1


def gelu_d2(a):
    """d^2 GELU / da^2 of the tanh form."""
    a = np.asarray(a, dtype=np.float64)
    t = np.tanh(_C * (a + _K * a ** 3))
    s1 = _C * (1.0 + 3.0 * _K * a * a)
    s2 = 6.0 * _C * _K * a
    sech2 = 1.0 - t * t
    return sech2 * s1 + 0.5 * a * sech2 * (s2 - 2.0 * t * s1 * s1)


def backward_bound(x, W_node, V_node, W_out, dy, rec_node, rec_a, variant: int = 0
                   ) -> Dict[str, np.ndarray]:
    """E for every gradient element (the coefficient of u in the bound).

    x [T,d], W_node [P,N,d], V_node [P,N,h], W_out [P*h,d], dy [T,d] float64;
    rec_node [T,P,L] (heap index of the node visited at each level) and
    rec_a [T,P,L] (its logit) from the oracle's forward with want_records.
    Returns float64 arrays shaped like the gradients: dx [T,d],
    dW_node [P,N,d], db_node [P,N], dV_node [P,N,h], dW_out [P*h,d].
    """
    x = np.asarray(x, dtype=np.float64)
    W_node = np.asarray(W_node, dtype=np.float64)
    V_node = np.asarray(V_node, dtype=np.float64)
    W_out = np.asarray(W_out, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    T, d = x.shape
    P, N, _ = W_node.shape
    h = V_node.shape[2]
    L = rec_node.shape[2]
    node = np.asarray(rec_node, dtype=np.int64)
    a = np.asarray(rec_a, dtype=np.float64)
    pidx = np.arange(P)[None, :, None]
    Wn = W_node[pidx, node]            # [T,P,L,d] the visited nodes' rows
    Vn = V_node[pidx, node]            # [T,P,L,h]
    ax = np.abs(x)

    # Logits: a float32 sum of d products.
    e_a = d * R_F32 * np.einsum("tc,tplc->tpl", ax, np.abs(Wn))
    G, G1, G2 = gelu(a), gelu_d1(a), gelu_d2(a)

    # Tree outputs H [T,P,h] (rounded) and their bound.
    if variant == 0:
        terms = G[..., None] * Vn
        H = terms.sum(axis=2)
        E_H = (np.abs(H) + np.einsum("tpl,tplj->tpj", np.abs(G1) * e_a, np.abs(Vn))
               + L * R_F32 * np.abs(terms).sum(axis=2))
    else:
        terms = a[..., None] * Vn
        S = terms.sum(axis=2)
        E_S = np.einsum("tpl,tplj->tpj", e_a, np.abs(Vn)) + L * R_F32 * np.abs(terms).sum(axis=2)
        H = gelu(S)
        E_H = np.abs(H) + np.abs(gelu_d1(S)) * E_S

    # Output gradient dH = dy . W_out^T (rounded).
    dH = (dy @ W_out.T).reshape(T, P, h)
    E_dH = np.abs(dH) + d * R_F32 * (np.abs(dy) @ np.abs(W_out).T).reshape(T, P, h)

    # Logit gradients da (rounded) and the per-visit terms of dV_node.
    if variant == 0:
        g = np.einsum("tpj,tplj->tpl", dH, Vn)
        E_g = (np.einsum("tpj,tplj->tpl", E_dH, np.abs(Vn))
               + h * R_F32 * np.einsum("tpj,tplj->tpl", np.abs(dH), np.abs(Vn)))
        da = g * G1
        E_da = np.abs(G1) * E_g + np.abs(g) * np.abs(G2) * e_a + np.abs(da)
        # dV term G * dH_j: G rounded (|G|), G's error from a (|G1| e_a), dH's.
        dv_term = np.abs(G)[..., None] * np.abs(dH)[:, :, None, :]
        E_dv_term = ((np.abs(G) + np.abs(G1) * e_a)[..., None] * np.abs(dH)[:, :, None, :]
                     + np.abs(G)[..., None] * E_dH[:, :, None, :])
    else:
        G1S = gelu_d1(S)
        dS = G1S * dH
        E_dS = np.abs(G1S) * E_dH + np.abs(gelu_d2(S)) * E_S * np.abs(dH) + np.abs(dS)
        g = np.einsum("tpj,tplj->tpl", dS, Vn)
        E_g = (np.einsum("tpj,tplj->tpl", E_dS, np.abs(Vn))
               + h * R_F32 * np.einsum("tpj,tplj->tpl", np.abs(dS), np.abs(Vn)))
        da = g
        E_da = E_g + np.abs(da)
        # dV term a * dS_j: a rounded (|a|), a's own error (e_a), dS's.
        dv_term = np.abs(a)[..., None] * np.abs(dS)[:, :, None, :]
        E_dv_term = ((np.abs(a) + e_a)[..., None] * np.abs(dS)[:, :, None, :]
                     + np.abs(a)[..., None] * E_dS[:, :, None, :])

    out: Dict[str, np.ndarray] = {}
    # dW_out[k,c] = sum_t H[t,k] dy[t,c].
    Hf, EHf = H.reshape(T, P * h), E_H.reshape(T, P * h)
    out["dW_out"] = np.abs(EHf).T @ np.abs(dy) + T * R_F32 * (np.abs(Hf).T @ np.abs(dy))
    # dx[t,c] = sum over (p,l) of da W_n[c], returned rounded.
    dx = np.einsum("tpl,tplc->tc", da, Wn)
    out["dx"] = (np.einsum("tpl,tplc->tc", E_da, np.abs(Wn))
                 + P * L * R_F32 * np.einsum("tpl,tplc->tc", np.abs(da), np.abs(Wn))
                 + np.abs(dx))
    # Node gradients: sums over the tokens that visit each node.
    E_onehot = np.zeros((P, N, T))
    abs_onehot = np.zeros((P, N, T))
    EV = np.zeros((P, N, h))
    AV = np.zeros((P, N, h))
    tt = np.broadcast_to(np.arange(T)[:, None, None], node.shape)
    pp = np.broadcast_to(np.arange(P)[None, :, None], node.shape)
    np.add.at(E_onehot, (pp, node, tt), E_da)
    np.add.at(abs_onehot, (pp, node, tt), np.abs(da))
    np.add.at(EV, (pp, node), E_dv_term)
    np.add.at(AV, (pp, node), dv_term)
    out["dW_node"] = (np.einsum("pnt,tc->pnc", E_onehot, ax)
                      + T * R_F32 * np.einsum("pnt,tc->pnc", abs_onehot, ax))
    out["db_node"] = E_onehot.sum(axis=2) + T * R_F32 * abs_onehot.sum(axis=2)
    out["dV_node"] = EV + T * R_F32 * AV
    return out
