"""Comparison rules between the HIP path and the oracle (test-only helpers).

Floating point: normwise max error, max|g - o| / max|o| per output tensor,
and for attention outputs per query row (the scale is that row's own max|o|
over its d elements, so a row with small outputs is held to the same
relative bound as the tensor's largest).
Integers (token ids, commit sets, counts): bit-exact, except positions the
rules exclude because their decision sits within `eps` of a boundary in the
oracle's own values:
  * a token id is excluded when the oracle's top-2 probabilities differ by
    less than eps (the argmax is then decided by rounding);
  * a commit decision is excluded when the oracle's confidence lies within
    eps of tau; when no candidate is surely above tau and one is near it,
    whether the fallback fires is itself undecided and the whole sequence is
    excluded; a fallback (or top-k / factor boundary) whose deciding
    confidences differ by less than eps excludes the sequence too.
Everything excluded is counted and returned.
"""
from __future__ import annotations

import numpy as np

from oracle import fdl_oracle as O


def normwise(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (scale if scale > 0 else 1.0))


def rowwise(got, ref) -> dict:
    """Per-row normwise error over the last axis: for each row,
    max_d |g - o| / max_d |o|.  Returns the worst row's error ("max") with
    element-wise diagnostics: the largest absolute error, the median and 99th
    percentile of the per-row errors, and the row count."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = ref.shape[-1]
    g2, r2 = got.reshape(-1, d), ref.reshape(-1, d)
    scale = np.abs(r2).max(axis=1)
    err = np.abs(g2 - r2).max(axis=1) / np.where(scale > 0, scale, 1.0)
    return dict(max=float(err.max()), p50=float(np.median(err)), p99=float(np.percentile(err, 99)),
                abs_max=float(np.abs(g2 - r2).max()), rows=int(err.size))


def compare_select(ref: dict, got: dict, masked, tau, mode=O.SELECT_THRESHOLD, k=0, factor=1.0,
                   eps=1e-3) -> dict:
    """ref: oracle conf_select result; got: dict of numpy arrays token/conf/commit/n_commit.
    Returns counts; raises AssertionError on a mismatch outside the exclusions."""
    masked = np.asarray(masked).astype(bool)
    tau = np.asarray(tau, dtype=np.float64).reshape(-1)
    B, R = masked.shape
    stats = dict(rows=B * R, token_excluded=0, token_checked=0, commit_excluded_rows=0,
                 seq_excluded=0, seq_checked=0, commits=int(np.asarray(got["n_commit"]).sum()))
    c, p2 = ref["conf"], ref["p2"]
    for b in range(B):
        for r in range(R):
            if c[b, r] - p2[b, r] < eps:
                stats["token_excluded"] += 1
                continue
            stats["token_checked"] += 1
            assert int(got["token"][b, r]) == int(ref["token"][b, r]), (b, r, got["token"][b, r], ref["token"][b, r])
        cands = [r for r in range(R) if masked[b, r]]
        order = sorted(cands, key=lambda r: (-c[b, r], r))
        excluded_rows = set()
        seq_ok = True
        if mode == O.SELECT_THRESHOLD:
            near = [r for r in cands if abs(c[b, r] - tau[b]) < eps]
            sure = [r for r in cands if c[b, r] > tau[b] + eps]
            if sure:
                excluded_rows = set(near)
            elif near:
                seq_ok = False
            elif len(order) >= 2 and c[b, order[0]] - c[b, order[1]] < eps:
                seq_ok = False
        elif mode == O.SELECT_TOPK:
            if 0 < k < len(order) and c[b, order[k - 1]] - c[b, order[k]] < eps:
                seq_ok = False
        else:
            for n in range(1, len(order) + 1):
                if abs((n + 1) * (1 - c[b, order[n - 1]]) - factor) < (n + 1) * eps:
                    seq_ok = False
                if n < len(order) and c[b, order[n - 1]] - c[b, order[n]] < eps:
                    seq_ok = False
        if not seq_ok:
            stats["seq_excluded"] += 1
            continue
        stats["seq_checked"] += 1
        stats["commit_excluded_rows"] += len(excluded_rows)
        for r in range(R):
            if r in excluded_rows:
                continue
            assert bool(got["commit"][b, r]) == bool(ref["commit"][b, r]), (b, r, c[b, r], tau[b])
        if not excluded_rows:
            assert int(got["n_commit"][b]) == int(ref["n_commit"][b]), (b, got["n_commit"][b], ref["n_commit"][b])
    return stats
