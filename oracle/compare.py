"""Comparison of a device result with the oracle (test infrastructure).

Routing parity: a device leaf index must equal the oracle's, except where the
two paths first part at a node whose oracle logit is a near-tie,
|a| <= 1e-4 * ||x_t|| * ||w_n||; such flips are excused and counted, and the
token is left out of the y comparison.

y parity: elementwise relative error with the denominator floored at the
token's RMS of the reference row,
    err = max |y_dev - y_ref| / max(|y_ref|, rms(y_ref[t, :])).
"""
from __future__ import annotations

from typing import Dict

import numpy as np


def classify_paths(path_dev: np.ndarray, ref: Dict[str, np.ndarray], D: int) -> Dict[str, object]:
    path_dev = np.asarray(path_dev, dtype=np.int64)
    path_ref = np.asarray(ref["path"], dtype=np.int64)
    T, P = path_ref.shape
    mism = np.argwhere(path_dev != path_ref)
    excused, bad = [], []
    for t, p in mism:
        diff = int(path_dev[t, p] ^ path_ref[t, p])
        if path_dev[t, p] < 0 or path_dev[t, p] >= (1 << D) or D == 0:
            bad.append((int(t), int(p), None))
            continue
        level = D - diff.bit_length()  # highest differing bit -> first level that parts
        a = ref["rec_a"][t, p, level]
        thr = ref["rec_thr"][t, p, level]
        (excused if abs(a) <= thr else bad).append((int(t), int(p), level))
    ok_tokens = np.ones(T, dtype=bool)
    for t, _, _ in excused + bad:
        ok_tokens[t] = False
    return {"mismatches": int(len(mism)), "excused": excused, "bad": bad,
            "flips_near_tie": len(excused), "tokens_ok": ok_tokens}


def y_error(y_dev: np.ndarray, y_ref: np.ndarray, rows_ok=None) -> Dict[str, float]:
    y_dev = np.asarray(y_dev, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
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
        "err_unfloored": float(np.max(np.where(big, diff / np.where(big, np.abs(y_ref), 1.0), 0.0))),
        "normwise": float(np.max(np.linalg.norm(y_dev - y_ref, axis=1) / nrm)),
        "rows": int(y_ref.shape[0]),
    }
