"""Comparison of a device result with the oracle (test infrastructure).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: the tests, the smoke
check and the benchmark's sampled error report use it; the HIP library never
does.

Routing parity (the sign rule of the explainer page, gist.science, section 2,
Methodology: a node's logit sign picks the child).  A device leaf index must
equal the oracle's, except where the two paths first part at a node whose
oracle logit is a near-tie, |a| <= 1e-4 * ||x_t|| * ||w_n||; such flips are
excused and counted.  After a flip the device walks a subtree the oracle did
not, so the oracle is run again along the device's own path
(``check_path_signs``): every later decision on that path must follow its own
logit's sign, or be a near-tie itself.

y parity: elementwise relative error with the denominator floored at the
token's RMS of the reference row,
    err = max |y_dev - y_ref| / max(|y_ref|, rms(y_ref[t, :])).
A reference row that is exactly zero has no scale of its own; its error is
the absolute difference (denominator 1).  Tokens whose paths all match are
compared with the oracle's own y; flipped tokens with the oracle's y along
the device's paths.

Bit layout shared with the library: bit (D-1-l) of a leaf index is the
level-l decision, 1 = right; heap node n has children 2n+1 (left), 2n+2.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

import numpy as np


def parting_level(leaf_a: int, leaf_b: int, D: int) -> int:
    """First level at which two distinct leaf indices of a depth-D tree take
    different branches: the level of their highest differing bit."""
    diff = int(leaf_a) ^ int(leaf_b)
    if diff == 0:
        raise ValueError("identical leaves do not part")
    return D - diff.bit_length()


def classify_paths(path_dev: np.ndarray, ref: Dict[str, np.ndarray], D: int) -> Dict[str, object]:
    """Sort every (token, tree) whose device leaf differs from the oracle's
    into excused near-tie flips and failures.

    ``ref`` holds the oracle's ``path`` [T,P] and per-visit ``rec_a``,
    ``rec_thr`` [T,P,D+1].  A device leaf outside [0, 2^D) fails."""
    path_dev = np.asarray(path_dev, dtype=np.int64)
    path_ref = np.asarray(ref["path"], dtype=np.int64)
    T, P = path_ref.shape
    if path_dev.shape != (T, P):
        raise ValueError(f"device paths {path_dev.shape} against reference {(T, P)}")
    mism = np.argwhere(path_dev != path_ref)
    excused: List[Tuple[int, int, int]] = []
    bad: List[Tuple[int, int, Optional[int]]] = []
    for t, p in mism:
        leaf = int(path_dev[t, p])
        if leaf < 0 or leaf >= (1 << D):
            bad.append((int(t), int(p), None))
            continue
        level = parting_level(leaf, int(path_ref[t, p]), D)
        a = ref["rec_a"][t, p, level]
        thr = ref["rec_thr"][t, p, level]
        (excused if abs(a) <= thr else bad).append((int(t), int(p), level))
    ok_tokens = np.ones(T, dtype=bool)
    for t, _, _ in excused + bad:
        ok_tokens[t] = False
    return {"mismatches": int(len(mism)), "excused": excused, "bad": bad,
            "flips_near_tie": len(excused), "tokens_ok": ok_tokens}


def node_alive_from_leaves(leaf_alive: np.ndarray, D: int) -> np.ndarray:
    """[P, N] alive flags from a [P, 2^D] leaf mask: a leaf as given, an inner
    node alive when either child is."""
    leaf_alive = np.asarray(leaf_alive) != 0
    P = leaf_alive.shape[0]
    first = (1 << D) - 1
    alive = np.zeros((P, 2 * first + 1), dtype=bool)
    alive[:, first:] = leaf_alive
    for n in range(first - 1, -1, -1):
        alive[:, n] = alive[:, 2 * n + 1] | alive[:, 2 * n + 2]
    return alive


def check_path_signs(path: np.ndarray, rec: Dict[str, np.ndarray], D: int,
                     node_alive: Optional[np.ndarray] = None) -> List[Tuple[int, int, int]]:
    """Decisions along given paths that their own logits do not allow.

    ``rec`` is the oracle run *forced* along ``path`` [R,P] (records
    ``rec_a``, ``rec_thr``, ``rec_node`` [R,P,D+1]).  At each level l < D the
    taken branch (bit D-1-l of the leaf) must be right = !(a < 0), unless
    |a| <= thr (a near-tie, either branch).  On pruned trees (``node_alive``
    [P,N]) the taken child must be alive, and a step whose sign-preferred
    child is pruned must take the sibling.  Returns (row, tree, level)
    triples that break the rule (empty when the paths are valid)."""
    path = np.asarray(path, dtype=np.int64)
    R, P = path.shape
    viol: List[Tuple[int, int, int]] = []
    for r in range(R):
        for p in range(P):
            leaf = int(path[r, p])
            if leaf < 0 or leaf >= (1 << D):
                viol.append((r, p, -1))
                continue
            for lvl in range(D):
                n = int(rec["rec_node"][r, p, lvl])
                a = rec["rec_a"][r, p, lvl]
                thr = rec["rec_thr"][r, p, lvl]
                took_right = (leaf >> (D - 1 - lvl)) & 1
                want_right = 0 if a < 0 else 1
                if node_alive is not None:
                    if not node_alive[p, 2 * n + 1 + took_right]:
                        viol.append((r, p, lvl))
                        continue
                    if not node_alive[p, 2 * n + 1 + want_right]:
                        want_right ^= 1  # a pruned preference forces the sibling
                        if took_right != want_right:
                            viol.append((r, p, lvl))
                        continue
                if took_right != want_right and not abs(a) <= thr:
                    viol.append((r, p, lvl))
    return viol


def y_error(y_dev: np.ndarray, y_ref: np.ndarray, rows_ok=None) -> Dict[str, float]:
    """Error of y_dev against y_ref [R, d] (rows limited to ``rows_ok``):
    ``err`` the RMS-floored elementwise relative error, ``err_unfloored``
    the plain relative error over elements with |y_ref| >= the row RMS,
    ``normwise`` the largest ||dy_t|| / ||y_ref,t|| (zero rows: absolute)."""
    y_dev = np.asarray(y_dev, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    if y_dev.shape != y_ref.shape:
        raise ValueError(f"y shapes differ: {y_dev.shape} against {y_ref.shape}")
    if rows_ok is not None:
        y_dev, y_ref = y_dev[rows_ok], y_ref[rows_ok]
    if y_ref.size == 0:
        return {"err": 0.0, "err_unfloored": 0.0, "normwise": 0.0, "rows": 0}
    rms = np.sqrt(np.mean(y_ref * y_ref, axis=1, keepdims=True))
    diff = np.abs(y_dev - y_ref)
    den = np.maximum(np.abs(y_ref), rms)
    den = np.where(den > 0, den, 1.0)
    big = np.abs(y_ref) >= rms
    nrm = np.linalg.norm(y_ref, axis=1)
    nrm = np.where(nrm > 0, nrm, 1.0)
    return {
        "err": float(np.max(diff / den)),
        "err_unfloored": float(np.max(np.where(big, diff / np.where(big & (y_ref != 0), np.abs(y_ref), 1.0), 0.0))),
        "normwise": float(np.max(np.linalg.norm(y_dev - y_ref, axis=1) / nrm)),
        "rows": int(y_ref.shape[0]),
    }
