"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` function takes an oracle library handle (so the mutant test can
run the same battery against deliberately broken copies) and raises
AssertionError when the oracle disagrees with:

* brute force over every root-to-leaf path of tiny trees, using the "masked"
  formulation of the FFF explainer page (gist.science, section 2,
  Implementation): all node logits computed densely, then the unique path
  whose every decision agrees with its logit's sign selected as a mask;
* hand-built weights whose routing is known in closed form;
* the all-zero case (every logit exactly 0, so every decision is a tie);
* a constant negative bias (every path goes to leaf 0; closed-form H);
* the visit count against Table 4's MLP-block sparsity column and the
  Figure 7 caption (tests/golden/table4_mlp_sparsity.txt);
* depth 0, which the paper's Figure 5 caption calls the dense FF case, against
  a dense one-hidden-layer MLP written with torch library routines;
* forced paths against the brute-force masked sum along those paths;
* invariances: positive rescaling of a node's (w, b), token and tree
  permutation, linearity in V and W_out, batch invariance.

The FFF-post variant (explainer page, section 3.C: GELU after the sum of the
node outputs a_n v_n instead of on each a_n) has its own pins: the masked
brute force with GELU moved outside the masked sum, hand routing with an
all-ones V column (where the two placements give different closed forms),
the constant-bias and depth-0 closed forms, and routing identical to FFF's.

GELU references come from ``torch.nn.functional.gelu(approximate="tanh")``
in float64, a library implementation independent of the oracle's C code.
"""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def gelu_ref(a: np.ndarray) -> np.ndarray:
    return torch.nn.functional.gelu(torch.from_numpy(np.asarray(a, dtype=np.float64)),
                                    approximate="tanh").numpy()


def rand_layer(rng, T, d, P, D, h):
    N = (1 << (D + 1)) - 1
    return dict(
        x=rng.standard_normal((T, d)),
        W_node=rng.standard_normal((P, N, d)) / np.sqrt(d),
        b_node=0.1 * rng.standard_normal((P, N)),
        V_node=rng.standard_normal((P, N, h)) / np.sqrt(h),
        W_out=rng.standard_normal((P * h, d)) / np.sqrt(P * h),
    )


def ancestors_of_leaf(leaf: int, D: int):
    """Heap ids of the nodes on the path to a leaf, root first (bottom-up walk)."""
    n = leaf + (1 << D) - 1
    nodes = [n]
    while n > 0:
        n = (n - 1) // 2
        nodes.append(n)
    return nodes[::-1]


def brute_force(L, forced=None, variant=0):
    """Masked formulation: dense logits, enumerate all 2^D paths.

    variant 0 sums GELU(a_n) v_n over the path's nodes; variant 1 (FFF-post)
    sums a_n v_n and applies GELU to the result."""
    x, W, b, V, Wo = L["x"], L["W_node"], L["b_node"], L["V_node"], L["W_out"]
    T, d = x.shape
    P, N, _ = W.shape
    h = V.shape[2]
    D = int(np.log2(N + 1)) - 1
    A = np.einsum("td,pnd->tpn", x, W) + b[None, :, :]
    G = gelu_ref(A)
    path = np.zeros((T, P), dtype=np.int32)
    H = np.zeros((T, P * h))
    for t in range(T):
        for p in range(P):
            if forced is None:
                ok = []
                for leaf in range(1 << D):
                    nodes = ancestors_of_leaf(leaf, D)
                    good = True
                    for lvl in range(D):
                        child_is_right = nodes[lvl + 1] == 2 * nodes[lvl] + 2
                        if child_is_right != (not (A[t, p, nodes[lvl]] < 0)):
                            good = False
                            break
                    if good:
                        ok.append(leaf)
                assert len(ok) == 1, "exactly one path must agree with every sign"
                leaf = ok[0]
            else:
                leaf = int(forced[t, p])
            mask = np.zeros(N)
            mask[ancestors_of_leaf(leaf, D)] = 1.0
            path[t, p] = leaf
            if variant == 0:
                H[t, p * h:(p + 1) * h] = (mask * G[t, p]) @ V[p]
            else:
                H[t, p * h:(p + 1) * h] = gelu_ref((mask * A[t, p]) @ V[p])
    return path, H, H @ Wo


def _close(a, b, rtol=1e-12, atol=1e-12):
    np.testing.assert_allclose(a, b, rtol=rtol, atol=atol)


def pin_brute_force(lib, n_cases=24):
    rng = np.random.default_rng(1234)
    shapes = [(7, 5, 3, 3, 4), (4, 8, 2, 5, 3), (9, 3, 1, 2, 6), (3, 16, 2, 4, 5), (5, 4, 3, 1, 2)]
    for i in range(n_cases):
        T, d, P, D, h = shapes[i % len(shapes)]
        L = rand_layer(rng, T, d, P, D, h)
        r = oracle.forward(**L, want_H=True, lib=lib, nthreads=2)
        path, H, y = brute_force(L)
        np.testing.assert_array_equal(r["path"], path)
        _close(r["H"], H)
        _close(r["y"], y)


def pin_hand_routing(lib):
    """x in {+-1}^(D+1), w_n = s_p * e_level(n), b = 0: every |a| = 1.

    Then leaf = sum over l < D of [s_p * x_l > 0] * 2^(D-1-l) exactly, and with
    V one-hot (v_n = e_n, h >= N) H[t, p*h + n] = GELU(s_p * x_level(n)) on the
    visited nodes and 0 elsewhere.
    """
    D, P, T = 4, 3, 32
    N = (1 << (D + 1)) - 1
    d, h = D + 3, N + 2
    rng = np.random.default_rng(7)
    s = np.array([1.0, -1.0, 1.0])
    x = np.zeros((T, d))
    x[:, :D + 1] = rng.choice([-1.0, 1.0], size=(T, D + 1))
    W = np.zeros((P, N, d))
    for p in range(P):
        for n in range(N):
            level = int(np.floor(np.log2(n + 1)))
            W[p, n, level] = s[p]
    V = np.zeros((P, N, h))
    for n in range(N):
        V[:, n, n] = 1.0
    b = np.zeros((P, N))
    Wo = rng.standard_normal((P * h, d))
    r = oracle.forward(x, W, b, V, Wo, want_H=True, lib=lib, nthreads=2)
    g_pos, g_neg = gelu_ref(np.array([1.0, -1.0]))
    for t in range(T):
        for p in range(P):
            bits = [(s[p] * x[t, lvl] > 0) for lvl in range(D + 1)]
            leaf = sum(int(bits[lvl]) << (D - 1 - lvl) for lvl in range(D))
            assert r["path"][t, p] == leaf
            expect = np.zeros(h)
            for lvl, n in enumerate(ancestors_of_leaf(leaf, D)):
                expect[n] = g_pos if bits[lvl] else g_neg
            _close(r["H"][t, p * h:(p + 1) * h], expect)
    _close(r["y"], r["H"] @ Wo)


def pin_zero_ties(lib):
    """W = 0, b = 0: every logit is exactly 0 and goes right; GELU(0) = 0."""
    T, d, P, D, h = 6, 5, 2, 3, 4
    rng = np.random.default_rng(3)
    L = rand_layer(rng, T, d, P, D, h)
    L["W_node"][:] = 0.0
    L["b_node"][:] = 0.0
    r = oracle.forward(**L, want_H=True, lib=lib, nthreads=1)
    assert (r["path"] == (1 << D) - 1).all()
    assert (r["H"] == 0).all() and (r["y"] == 0).all()


def pin_nan_goes_right(lib):
    """A NaN logit is not below zero: every decision goes right (the
    rightmost leaf), and the outputs are NaN."""
    T, d, P, D, h = 4, 5, 2, 3, 3
    rng = np.random.default_rng(12)
    L = rand_layer(rng, T, d, P, D, h)
    L["W_node"][:] = 0.0
    L["b_node"][:] = np.nan
    r = oracle.forward(**L, want_H=True, lib=lib, nthreads=1)
    assert (r["path"] == (1 << D) - 1).all()
    assert np.isnan(r["y"]).all()


def pin_negative_bias(lib):
    """W = 0, b = -beta: every path is leaf 0 (the leftmost spine) and
    H_p = GELU(-beta) * sum over levels of V[p, 2^l - 1]."""
    T, d, P, D, h = 5, 4, 3, 4, 6
    beta = 0.75
    rng = np.random.default_rng(4)
    L = rand_layer(rng, T, d, P, D, h)
    L["W_node"][:] = 0.0
    L["b_node"][:] = -beta
    r = oracle.forward(**L, want_H=True, lib=lib, nthreads=1)
    assert (r["path"] == 0).all()
    g = gelu_ref(np.array([-beta]))[0]
    for p in range(P):
        spine = sum(L["V_node"][p, (1 << lvl) - 1] for lvl in range(D + 1))
        for t in range(T):
            _close(r["H"][t, p * h:(p + 1) * h], g * spine)


def read_table4():
    rows = []
    with open(os.path.join(GOLDEN, "table4_mlp_sparsity.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                depth, pct, mode = line.split()
                rows.append((int(depth), int(pct), mode))
    return rows


def pin_visit_count_table4(lib):
    """Evaluated nodes per (token, tree), counted from the oracle's records,
    against the printed sparsity 1 - evaluated / nodes-per-tree."""
    for depth, pct, mode in read_table4():
        T, d, P, h = 3, 2, 1, 1
        rng = np.random.default_rng(depth)
        L = rand_layer(rng, T, d, P, depth, h)
        r = oracle.forward(**L, want_y=False, want_records=True, lib=lib, nthreads=1)
        evaluated = (r["rec_node"] >= 0).sum(axis=2)
        assert (evaluated == evaluated[0, 0]).all()
        nodes_per_tree = L["W_node"].shape[1]
        sparsity = 100.0 * (1.0 - evaluated[0, 0] / nodes_per_tree)
        got = int(np.floor(sparsity)) if mode == "floor" else int(np.floor(sparsity + 0.5))
        assert got == pct, (depth, sparsity, pct)
        # The recorded nodes form a root-to-leaf chain ending at the reported leaf.
        for t in range(T):
            chain = list(r["rec_node"][t, 0])
            assert chain == ancestors_of_leaf(int(r["path"][t, 0]), depth)


def pin_depth0_dense(lib):
    """D = 0: one node per tree, so the layer is a dense MLP with P hidden
    units: y = GELU(x W0^T + b0) M with M[p] = v_p W_out[p*h:(p+1)*h]."""
    T, d, P, h = 11, 9, 5, 3
    rng = np.random.default_rng(5)
    L = rand_layer(rng, T, d, P, 0, h)
    r = oracle.forward(**L, want_H=True, lib=lib, nthreads=1)
    assert (r["path"] == 0).all()
    xt = torch.from_numpy(L["x"])
    W0 = torch.from_numpy(L["W_node"][:, 0, :])
    b0 = torch.from_numpy(L["b_node"][:, 0])
    hidden = torch.nn.functional.gelu(torch.nn.functional.linear(xt, W0, b0), approximate="tanh")
    M = torch.stack([torch.from_numpy(L["V_node"][p, 0]) @ torch.from_numpy(
        L["W_out"][p * h:(p + 1) * h]) for p in range(P)])
    _close(r["y"], (hidden @ M).numpy(), rtol=1e-11, atol=1e-12)


def pin_forced_paths(lib):
    rng = np.random.default_rng(6)
    T, d, P, D, h = 6, 7, 2, 3, 4
    L = rand_layer(rng, T, d, P, D, h)
    natural = oracle.forward(**L, want_H=True, lib=lib, nthreads=1)
    same = oracle.forward(**L, forced=natural["path"], want_H=True, lib=lib, nthreads=1)
    np.testing.assert_array_equal(same["path"], natural["path"])
    _close(same["y"], natural["y"])
    forced = rng.integers(0, 1 << D, size=(T, P)).astype(np.int32)
    r = oracle.forward(**L, forced=forced, want_H=True, lib=lib, nthreads=1)
    path, H, y = brute_force(L, forced=forced)
    np.testing.assert_array_equal(r["path"], forced)
    _close(r["H"], H)
    _close(r["y"], y)


def pin_invariants(lib):
    rng = np.random.default_rng(8)
    T, d, P, D, h = 10, 6, 3, 3, 4
    L = rand_layer(rng, T, d, P, D, h)
    base = oracle.forward(**L, want_H=True, lib=lib, nthreads=2)
    # Only the sign of a logit routes: rescaling (w_n, b_n) by c > 0 keeps paths.
    L2 = dict(L)
    c = rng.uniform(0.1, 10.0, size=L["b_node"].shape)
    L2["W_node"] = L["W_node"] * c[:, :, None]
    L2["b_node"] = L["b_node"] * c
    np.testing.assert_array_equal(oracle.forward(**L2, want_y=False, lib=lib)["path"], base["path"])
    # Token permutation is equivariant.
    perm = rng.permutation(T)
    L3 = dict(L, x=L["x"][perm])
    r3 = oracle.forward(**L3, lib=lib)
    np.testing.assert_array_equal(r3["path"], base["path"][perm])
    _close(r3["y"], base["y"][perm])
    # Permuting trees together with W_out's row blocks leaves y unchanged.
    tp = rng.permutation(P)
    rows = np.concatenate([np.arange(p * h, (p + 1) * h) for p in tp])
    L4 = dict(L, W_node=L["W_node"][tp], b_node=L["b_node"][tp], V_node=L["V_node"][tp],
              W_out=L["W_out"][rows])
    r4 = oracle.forward(**L4, lib=lib)
    np.testing.assert_array_equal(r4["path"], base["path"][:, tp])
    _close(r4["y"], base["y"], rtol=1e-11, atol=1e-12)
    # H is linear in V; y is linear in W_out.
    V2 = rng.standard_normal(L["V_node"].shape)
    rv = oracle.forward(**dict(L, V_node=V2), want_H=True, lib=lib)
    rs = oracle.forward(**dict(L, V_node=2.0 * L["V_node"] - 3.0 * V2), want_H=True, lib=lib)
    _close(rs["H"], 2.0 * base["H"] - 3.0 * rv["H"], rtol=1e-10, atol=1e-11)
    Wo2 = rng.standard_normal(L["W_out"].shape)
    rw = oracle.forward(**dict(L, W_out=Wo2), lib=lib)
    rsw = oracle.forward(**dict(L, W_out=L["W_out"] + 0.5 * Wo2), lib=lib)
    _close(rsw["y"], base["y"] + 0.5 * rw["y"], rtol=1e-10, atol=1e-11)
    # Batch invariance: one token alone gives its batched row.
    for t in (0, T - 1):
        r1 = oracle.forward(**dict(L, x=L["x"][t:t + 1]), lib=lib, nthreads=1)
        np.testing.assert_array_equal(r1["path"][0], base["path"][t])
        np.testing.assert_array_equal(r1["y"][0], base["y"][t])


def pin_tie_threshold(lib):
    """rec_thr = 1e-4 * ||x_t|| * ||w_n|| for each visited node."""
    rng = np.random.default_rng(9)
    T, d, P, D, h = 4, 6, 2, 2, 3
    L = rand_layer(rng, T, d, P, D, h)
    r = oracle.forward(**L, want_records=True, lib=lib, nthreads=1)
    for t in range(T):
        for p in range(P):
            for lvl in range(D + 1):
                n = r["rec_node"][t, p, lvl]
                expect = 1e-4 * np.linalg.norm(L["x"][t]) * np.linalg.norm(L["W_node"][p, n])
                _close(r["rec_thr"][t, p, lvl], expect)
                _close(r["rec_a"][t, p, lvl], L["x"][t] @ L["W_node"][p, n] + L["b_node"][p, n])


def pin_post_brute_force(lib, n_cases=16):
    rng = np.random.default_rng(4321)
    shapes = [(7, 5, 3, 3, 4), (4, 8, 2, 5, 3), (9, 3, 1, 2, 6), (5, 4, 3, 1, 2)]
    for i in range(n_cases):
        T, d, P, D, h = shapes[i % len(shapes)]
        L = rand_layer(rng, T, d, P, D, h)
        r = oracle.forward(**L, want_H=True, variant=1, lib=lib, nthreads=2)
        path, H, y = brute_force(L, variant=1)
        np.testing.assert_array_equal(r["path"], path)
        _close(r["H"], H)
        _close(r["y"], y)
    # Forced paths follow the same masked sum along the given leaves.
    T, d, P, D, h = 6, 7, 2, 3, 4
    L = rand_layer(rng, T, d, P, D, h)
    forced = rng.integers(0, 1 << D, size=(T, P)).astype(np.int32)
    r = oracle.forward(**L, forced=forced, want_H=True, variant=1, lib=lib, nthreads=1)
    _, H, y = brute_force(L, forced=forced, variant=1)
    _close(r["H"], H)
    _close(r["y"], y)


def pin_post_hand_routing(lib):
    """Hand routing as in pin_hand_routing (every |a| = 1) with an all-ones
    first V column: FFF-post gives H[t, p*h] = GELU(#right - #left) along the
    path, where FFF would give #right GELU(1) + #left GELU(-1)."""
    D, P, T = 4, 2, 32
    N = (1 << (D + 1)) - 1
    d, h = D + 3, 3
    rng = np.random.default_rng(17)
    s = np.array([1.0, -1.0])
    x = np.zeros((T, d))
    x[:, :D + 1] = rng.choice([-1.0, 1.0], size=(T, D + 1))
    W = np.zeros((P, N, d))
    for p in range(P):
        for n in range(N):
            W[p, n, int(np.floor(np.log2(n + 1)))] = s[p]
    V = np.zeros((P, N, h))
    V[:, :, 0] = 1.0
    b = np.zeros((P, N))
    Wo = rng.standard_normal((P * h, d))
    post = oracle.forward(x, W, b, V, Wo, want_H=True, variant=1, lib=lib, nthreads=2)
    pre = oracle.forward(x, W, b, V, Wo, want_H=True, variant=0, lib=lib, nthreads=2)
    np.testing.assert_array_equal(post["path"], pre["path"])
    g_pos, g_neg = gelu_ref(np.array([1.0, -1.0]))
    for t in range(T):
        for p in range(P):
            n_right = sum(int(s[p] * x[t, lvl] > 0) for lvl in range(D + 1))
            n_left = D + 1 - n_right
            leaf = sum(int(s[p] * x[t, lvl] > 0) << (D - 1 - lvl) for lvl in range(D))
            assert post["path"][t, p] == leaf
            _close(post["H"][t, p * h], gelu_ref(np.array([float(n_right - n_left)]))[0])
            _close(pre["H"][t, p * h], n_right * g_pos + n_left * g_neg)
            assert (post["H"][t, p * h + 1:(p + 1) * h] == 0).all()
    _close(post["y"], post["H"] @ Wo)


def pin_post_closed_forms(lib):
    """Constant bias -beta (W = 0): H_p = GELU(-beta * sum of the spine's v);
    depth 0: H[t, p*h + j] = GELU((x_t . w_p + b_p) v_p[j]), checked against
    torch's linear and GELU."""
    T, d, P, D, h = 5, 4, 3, 4, 6
    beta = 0.75
    rng = np.random.default_rng(14)
    L = rand_layer(rng, T, d, P, D, h)
    L["W_node"][:] = 0.0
    L["b_node"][:] = -beta
    r = oracle.forward(**L, want_H=True, variant=1, lib=lib, nthreads=1)
    assert (r["path"] == 0).all()
    for p in range(P):
        spine = sum(L["V_node"][p, (1 << lvl) - 1] for lvl in range(D + 1))
        for t in range(T):
            _close(r["H"][t, p * h:(p + 1) * h], gelu_ref(-beta * spine))
    T, d, P, h = 11, 9, 5, 3
    L = rand_layer(rng, T, d, P, 0, h)
    r = oracle.forward(**L, want_H=True, variant=1, lib=lib, nthreads=1)
    logits = torch.nn.functional.linear(torch.from_numpy(L["x"]),
                                        torch.from_numpy(L["W_node"][:, 0, :]),
                                        torch.from_numpy(L["b_node"][:, 0]))
    H = torch.nn.functional.gelu(logits[:, :, None] * torch.from_numpy(L["V_node"][:, 0, :])[None],
                                 approximate="tanh").reshape(T, P * h)
    _close(r["H"], H.numpy(), rtol=1e-11, atol=1e-12)
    _close(r["y"], (H @ torch.from_numpy(L["W_out"])).numpy(), rtol=1e-11, atol=1e-12)


def pin_post_routing_unchanged(lib):
    """Routing depends on the logits only, so both variants take the same
    paths and record the same per-visit logits."""
    rng = np.random.default_rng(15)
    L = rand_layer(rng, 12, 6, 3, 5, 4)
    a = oracle.forward(**L, want_records=True, variant=0, lib=lib, nthreads=2)
    b = oracle.forward(**L, want_records=True, variant=1, lib=lib, nthreads=2)
    np.testing.assert_array_equal(a["path"], b["path"])
    np.testing.assert_array_equal(a["rec_node"], b["rec_node"])
    np.testing.assert_array_equal(a["rec_a"], b["rec_a"])
    assert not np.allclose(a["y"], b["y"])


def subtree_alive(leaf_alive_p: np.ndarray, D: int, n: int) -> bool:
    """Whether any leaf below heap node n is alive (leaf range by level)."""
    level = int(np.floor(np.log2(n + 1)))
    span = 1 << (D - level)
    first = (n - ((1 << level) - 1)) * span
    return bool(leaf_alive_p[first:first + span].any())


def brute_force_pruned(L, leaf_alive):
    """Enumerate the alive leaves; keep the one whose every step either
    follows its logit's sign or is forced because the preferred child's
    subtree has no alive leaf."""
    x, W, b, V, Wo = L["x"], L["W_node"], L["b_node"], L["V_node"], L["W_out"]
    T = x.shape[0]
    P, N, _ = W.shape
    h = V.shape[2]
    D = int(np.log2(N + 1)) - 1
    A = np.einsum("td,pnd->tpn", x, W) + b[None, :, :]
    G = gelu_ref(A)
    path = np.zeros((T, P), dtype=np.int32)
    H = np.zeros((T, P * h))
    for t in range(T):
        for p in range(P):
            ok = []
            for leaf in np.flatnonzero(leaf_alive[p]):
                nodes = ancestors_of_leaf(int(leaf), D)
                good = True
                for lvl in range(D):
                    n = nodes[lvl]
                    pref = 2 * n + 1 if A[t, p, n] < 0 else 2 * n + 2
                    if nodes[lvl + 1] != pref and subtree_alive(leaf_alive[p], D, pref):
                        good = False
                        break
                if good:
                    ok.append(int(leaf))
            assert len(ok) == 1, "exactly one alive leaf is consistent"
            mask = np.zeros(N)
            mask[ancestors_of_leaf(ok[0], D)] = 1.0
            path[t, p] = ok[0]
            H[t, p * h:(p + 1) * h] = (mask * G[t, p]) @ V[p]
    return path, H, H @ Wo


def pin_prune_brute_force(lib):
    rng = np.random.default_rng(77)
    for i, (T, d, P, D, h) in enumerate([(9, 5, 3, 3, 4), (6, 8, 2, 5, 3), (7, 4, 2, 1, 2),
                                         (5, 6, 4, 4, 3)]):
        L = rand_layer(rng, T, d, P, D, h)
        for frac in (0.3, 0.7):
            alive = (rng.random((P, 1 << D)) > frac).astype(np.uint8)
            alive[np.arange(P), rng.integers(0, 1 << D, size=P)] = 1  # every tree keeps a leaf
            r = oracle.forward(**L, leaf_alive=alive, want_H=True, lib=lib, nthreads=2)
            path, H, y = brute_force_pruned(L, alive)
            np.testing.assert_array_equal(r["path"], path)
            assert alive[np.arange(P)[None, :], r["path"]].all()
            _close(r["H"], H)
            _close(r["y"], y)


def pin_prune_reductions(lib):
    """All leaves alive: the unpruned result bit for bit.  One alive leaf per
    tree: every token takes it, exactly as the forced-path mode computes.
    Pruning only leaves that no token reaches: nothing changes."""
    rng = np.random.default_rng(78)
    T, d, P, D, h = 40, 6, 3, 4, 5
    L = rand_layer(rng, T, d, P, D, h)
    base = oracle.forward(**L, want_H=True, lib=lib, nthreads=2)
    full = oracle.forward(**L, want_H=True, leaf_alive=np.ones((P, 1 << D), np.uint8), lib=lib,
                          nthreads=2)
    for k in ("path", "H", "y"):
        np.testing.assert_array_equal(full[k], base[k])
    only = rng.integers(0, 1 << D, size=P)
    alive = np.zeros((P, 1 << D), np.uint8)
    alive[np.arange(P), only] = 1
    one = oracle.forward(**L, want_H=True, leaf_alive=alive, lib=lib, nthreads=2)
    assert (one["path"] == only[None, :]).all()
    forced = oracle.forward(**L, want_H=True, forced=np.tile(only.astype(np.int32), (T, 1)),
                            lib=lib, nthreads=2)
    np.testing.assert_array_equal(one["y"], forced["y"])
    np.testing.assert_array_equal(one["H"], forced["H"])
    visited = np.zeros((P, 1 << D), np.uint8)
    visited[np.arange(P)[None, :], base["path"]] = 1
    same = oracle.forward(**L, want_H=True, leaf_alive=visited, lib=lib, nthreads=2)
    for k in ("path", "H", "y"):
        np.testing.assert_array_equal(same[k], base[k])


def _fd_layer(rng, T, d, P, D, h, margin=0.05):
    """A random tiny layer whose logits are all at least `margin` from 0."""
    for _ in range(1000):
        L = rand_layer(rng, T, d, P, D, h)
        A = np.einsum("td,pnd->tpn", L["x"], L["W_node"]) + L["b_node"][None]
        if np.abs(A).min() > margin:
            return L
    raise AssertionError("no layer with logits away from zero")


def _check_fd(lib, L, dy, variant=0, leaf_alive=None, eps=1e-6):
    g = oracle.backward(**L, dy=dy, variant=variant, leaf_alive=leaf_alive, lib=lib, nthreads=1)
    base_path = oracle.forward(**L, variant=variant, leaf_alive=leaf_alive, lib=lib,
                               nthreads=1)["path"]
    names = {"x": "dx", "W_node": "dW_node", "b_node": "db_node", "V_node": "dV_node",
             "W_out": "dW_out"}
    for key, gname in names.items():
        arr = L[key]
        fd = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            vals = []
            for sgn in (1.0, -1.0):
                L2 = dict(L)
                L2[key] = arr.copy()
                L2[key][idx] += sgn * eps
                r = oracle.forward(**L2, variant=variant, leaf_alive=leaf_alive, lib=lib,
                                   nthreads=1)
                np.testing.assert_array_equal(r["path"], base_path)
                vals.append(float((r["y"] * dy).sum()))
            fd[idx] = (vals[0] - vals[1]) / (2 * eps)
        np.testing.assert_allclose(g[gname], fd, rtol=1e-5, atol=1e-7, err_msg=gname)


def pin_backward_finite_differences(lib):
    rng = np.random.default_rng(90)
    for variant in (0, 1):
        L = _fd_layer(rng, 3, 4, 2, 2, 3)
        dy = rng.standard_normal((3, 4))
        _check_fd(lib, L, dy, variant=variant)
    # Pruned trees: the forced steps are part of the fixed paths.
    L = _fd_layer(rng, 4, 3, 2, 3, 2)
    alive = np.array([[1, 0, 0, 1, 1, 0, 0, 0], [0, 0, 0, 0, 1, 1, 0, 1]], np.uint8)
    _check_fd(lib, L, rng.standard_normal((4, 3)), variant=0, leaf_alive=alive)
    _check_fd(lib, L, rng.standard_normal((4, 3)), variant=1, leaf_alive=alive)


def pin_backward_dense_autograd(lib):
    """Depth 0 is a dense layer: torch autograd in float64 gives every
    gradient (both variants)."""
    rng = np.random.default_rng(91)
    T, d, P, h = 7, 5, 4, 3
    L = rand_layer(rng, T, d, P, 0, h)
    dy = rng.standard_normal((T, d))
    for variant in (0, 1):
        t = {k: torch.from_numpy(L[k].copy()).requires_grad_(True) for k in L}
        logits = torch.nn.functional.linear(t["x"], t["W_node"][:, 0, :], t["b_node"][:, 0])
        if variant == 0:
            hid = torch.nn.functional.gelu(logits, approximate="tanh")[:, :, None] * \
                t["V_node"][:, 0, :][None]
        else:
            hid = torch.nn.functional.gelu(logits[:, :, None] * t["V_node"][:, 0, :][None],
                                           approximate="tanh")
        y = hid.reshape(T, P * h) @ t["W_out"]
        (y * torch.from_numpy(dy)).sum().backward()
        g = oracle.backward(**L, dy=dy, variant=variant, lib=lib, nthreads=2)
        for key, gname in (("x", "dx"), ("W_node", "dW_node"), ("b_node", "db_node"),
                           ("V_node", "dV_node"), ("W_out", "dW_out")):
            _close(g[gname], t[key].grad.numpy(), rtol=1e-11, atol=1e-12)


def pin_backward_linear_in_dy(lib):
    rng = np.random.default_rng(92)
    L = rand_layer(rng, 9, 6, 3, 4, 5)
    dy1, dy2 = rng.standard_normal((2, 9, 6))
    g1 = oracle.backward(**L, dy=dy1, lib=lib)
    g2 = oracle.backward(**L, dy=dy2, lib=lib)
    g3 = oracle.backward(**L, dy=dy1 - 2.0 * dy2, lib=lib)
    for k in g1:
        _close(g3[k], g1[k] - 2.0 * g2[k], rtol=1e-10, atol=1e-11)
    # Nodes off every path get no gradient.
    paths = oracle.forward(**L, lib=lib)["path"]
    visited = np.zeros(L["b_node"].shape, bool)
    for t in range(9):
        for p in range(3):
            visited[p, ancestors_of_leaf(int(paths[t, p]), 4)] = True
    assert (g1["db_node"][~visited] == 0).all() and (g1["dW_node"][~visited] == 0).all()


ALL_PINS = [pin_brute_force, pin_hand_routing, pin_zero_ties, pin_nan_goes_right,
            pin_negative_bias, pin_visit_count_table4, pin_depth0_dense, pin_forced_paths, pin_invariants,
            pin_tie_threshold, pin_post_brute_force, pin_post_hand_routing,
            pin_post_closed_forms, pin_post_routing_unchanged, pin_prune_brute_force,
            pin_prune_reductions, pin_backward_finite_differences, pin_backward_dense_autograd,
            pin_backward_linear_in_dy]
