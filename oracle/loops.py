"""Scalar pure-Python versions of the oracle, for tiny shapes only (test infrastructure).

Only tests may use this. These loops restate the same definitions as
``oracle.ref`` without NumPy vector operations, matrix products or array
indexing tricks, so that a slip in ``ref`` (a transposed operand, a wrong
group index, a dropped term) shows up as a disagreement.
"""

from __future__ import annotations

import math


def dequant_value(q: int, s: float, z: int) -> float:
    """One AWQ weight: (q - z) * s (PR #522, Purpose: {FP16 scale, u8 zero} records)."""
    return (float(q) - float(z)) * float(s)


def dequant_loop(q, s, z):
    K, N = len(q), len(q[0])
    return [[dequant_value(int(q[k][n]), float(s[k // 32][n]), int(z[k // 32][n])) for n in range(N)]
            for k in range(K)]


def route_brute(ids, num_experts: int):
    """Canonical compaction by sorting (expert, slot) keys with ``sorted``."""
    flat = [int(v) for row in ids for v in row]
    n = len(flat)
    valid = [s for s in range(n) if 0 <= flat[s] < num_experts]
    invalid = [s for s in range(n) if not (0 <= flat[s] < num_experts)]
    rows = sorted(valid, key=lambda s: (flat[s], s))
    experts, offsets = [], [0]
    for i, s in enumerate(rows):
        if i == 0 or flat[s] != flat[rows[i - 1]]:
            if i:
                offsets.append(i)
            experts.append(flat[s])
    if rows:
        offsets.append(len(rows))
    return dict(experts=experts, offsets=offsets, sorted_slots=rows + invalid,
                status=1 if invalid else 0)


def _dot(a, col_of_b, K):
    acc = 0.0
    for k in range(K):
        acc += a[k] * col_of_b(k)
    return acc


def _silu(g: float) -> float:
    if g >= 0:
        return g / (1.0 + math.exp(-g))
    e = math.exp(g)
    return g * e / (1.0 + e)


def stage_loops(x, ids, w, num_experts: int, weights_of):
    """out[t][n] = sum_j w[t][j] * sum_i act_tj[i] * Wd[i][n], by explicit loops.

    x [M][H] (numbers), ids [M][k], w [M][k]; ``weights_of(e)`` returns an
    ``ExpertWeights``. Invalid ids contribute nothing.
    """
    M, k = len(ids), len(ids[0])
    H = len(x[0])
    out = [[0.0] * H for _ in range(M)]
    cache = {}
    for t in range(M):
        xt = [float(v) for v in x[t]]
        for j in range(k):
            e = int(ids[t][j])
            if not (0 <= e < num_experts):
                continue
            if e not in cache:
                ew = weights_of(e)
                cache[e] = (dequant_loop(ew.q_gate, ew.s_gate, ew.z_gate),
                            dequant_loop(ew.q_up, ew.s_up, ew.z_up),
                            dequant_loop(ew.q_down, ew.s_down, ew.z_down))
            Wg, Wu, Wd = cache[e]
            I = len(Wg[0])
            act = []
            for i in range(I):
                gsum = _dot(xt, lambda kk: Wg[kk][i], H)
                usum = _dot(xt, lambda kk: Wu[kk][i], H)
                act.append(_silu(gsum) * usum)
            wt = float(w[t][j])
            for n in range(H):
                y = _dot(act, lambda i: Wd[i][n], I)
                out[t][n] += wt * y
    return out
