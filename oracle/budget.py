"""Verify-budget scheduling, plain Python in float64.  TEST INFRASTRUCTURE ONLY
(see oracle/__init__.py); it shares nothing with the library.

Follows DSpark ("Hardware-aware prefix scheduler"; method section on
confidence-scheduled verification) step by step:
  1. cumulative survival of each draft position: S[i][k] = prod_{m<=k} c[i][m];
  2. all (request, position) candidates sorted by S, largest first (equal S:
     earlier position, then lower request);
  3. the batch grows one candidate at a time from the requests' root rows;
     for each size B (verify rows) the expected emitted tokens
     tau = (one bonus token per request) + (sum of the admitted S) and
     Theta = tau * SPS(B), SPS linearly interpolated in the measured table and
     clamped at its ends;
  4. the first batch with the largest Theta is kept; request i verifies the
     drafts up to its last admitted position.
Readings (the page leaves them open): B counts verify rows including each
request's root; tau counts the bonus token; ties keep the smaller batch."""
from __future__ import annotations


def sps_at(rows, value, b):
    rows = [float(x) for x in rows]
    value = [float(x) for x in value]
    b = float(b)
    if b <= rows[0]:
        return float(value[0])
    if b >= rows[-1]:
        return float(value[-1])
    j = 1
    while rows[j] < b:
        j += 1
    t = (b - rows[j - 1]) / (float(rows[j]) - float(rows[j - 1]))
    return float(value[j - 1]) + t * (float(value[j]) - float(value[j - 1]))


def verify_budget(cond, gammas, sps_rows, sps_value):
    """cond: list per request of conditional survival values (position 1..gamma_i).
    Returns (verify_len per request, batch rows, Theta)."""
    n = len(gammas)
    cand = []
    for i in range(n):
        s = 1.0
        for k in range(1, gammas[i] + 1):
            s *= float(cond[i][k - 1])
            cand.append((s, i, k))
    cand.sort(key=lambda c: (-c[0], c[2], c[1]))
    tau = float(n)
    best = tau * sps_at(sps_rows, sps_value, n) if n > 0 else 0.0
    best_m = 0
    for m in range(1, len(cand) + 1):
        tau += cand[m - 1][0]
        th = tau * sps_at(sps_rows, sps_value, n + m)
        if th > best:
            best, best_m = th, m
    verify = [0] * n
    for s, i, k in cand[:best_m]:
        verify[i] = max(verify[i], k)
    return verify, n + best_m, best
