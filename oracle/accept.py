"""Acceptance rules for comparing a block selection with the oracle's.

TEST INFRASTRUCTURE (same restriction as the rest of ``oracle``).

Where the (k-1)-th and k-th best non-local pooled scores of a row are more than
1e-3 apart (relative), the selected set is unique and must match the oracle's
bit for bit.  Inside that gap any selection that is structurally valid and
epsilon-valid (no unselected candidate beats a selected one by more than the
relative tolerance) is a correct answer.
"""
from __future__ import annotations

import numpy as np

GAP_REL = 1e-3


def gap_rel(pooled_row, local: int, k: int) -> float:
    """Relative gap between the (k-1)-th and k-th best non-local candidates.

    Rows with at most k visible blocks select everything: returns +inf.
    """
    if local + 1 <= k:
        return float("inf")
    c = np.sort(np.asarray(pooled_row[:local], dtype=np.float64))[::-1]
    a, b = c[k - 2], c[k - 1]
    return float((a - b) / max(abs(a), abs(b), 1e-30))


def structure_ok(sel_row, local: int, k: int) -> bool:
    """Ascending, no duplicates, local block present as the last valid entry,
    -1 padding at the tail, and exactly min(k, local+1) valid entries."""
    s = np.asarray(sel_row)
    valid = s[s >= 0]
    n = min(k, local + 1)
    if len(valid) != n or np.any(s[n:] != -1) or np.any(s[:n] < 0):
        return False
    if np.any(np.diff(valid) <= 0):
        return False
    return int(valid[-1]) == local and int(valid[0]) >= 0


def eps_valid(sel_row, pooled_row, local: int, k: int, eps: float = GAP_REL) -> bool:
    """Structure plus: every selected non-local candidate a and unselected c
    satisfy P_a >= P_c - eps * max(|P_a|, |P_c|)."""
    if not structure_ok(sel_row, local, k):
        return False
    if local + 1 <= k:
        return True
    s = np.asarray(sel_row)
    chosen = np.zeros(local, bool)
    chosen[s[(s >= 0) & (s < local)]] = True
    P = np.asarray(pooled_row[:local], dtype=np.float64)
    pa, pc = P[chosen][:, None], P[~chosen][None, :]
    return bool(np.all(pa >= pc - eps * np.maximum(np.abs(pa), np.abs(pc))))


def check_indices(sel_gpu, sel_ref, pooled_ref, local, k: int):
    """Row-wise verdict: 'exact' where the gap rule demands equality and it
    holds, 'eps' where an in-gap row is epsilon-valid, 'FAIL' otherwise."""
    verdicts = []
    for r in range(len(sel_gpu)):
        g = gap_rel(pooled_ref[r], int(local[r]), k)
        if g > GAP_REL:
            ok = np.array_equal(np.asarray(sel_gpu[r]), np.asarray(sel_ref[r]))
            verdicts.append("exact" if ok else "FAIL")
        else:
            ok = eps_valid(sel_gpu[r], pooled_ref[r], int(local[r]), k)
            verdicts.append("eps" if ok else "FAIL")
    return verdicts
