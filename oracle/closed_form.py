"""TEST INFRASTRUCTURE ONLY: exact counting results for TDT lattices.

With every token and duration logit equal to zero, every emission weighs
-log V - log D - sigma, so

    P = sum over k >= 1 of N(k) * (V * D * e^sigma) ** -(U + k),

where N(k) is the number of alignments with U labels and k blanks.  An alignment is an
arrangement of the U labels and k - 1 blanks in any order followed by the final blank
(which must be the last move, at u = U), with label durations in the duration set and
blank durations in its positive part, all summing to T:

    N(k) = C(U + k - 1, U) * [x^T] (sum_{d in D} x^d)^U (sum_{d in D, d > 0} x^d)^k.

Integers are exact (Python big ints); only the final log is rounded.  The move rules
are the ones stated in ``bruteforce.py``.
"""
from __future__ import annotations

import math


def _poly_mul(a, b, deg):
    out = [0] * (deg + 1)
    for i, x in enumerate(a):
        if x == 0:
            continue
        for j, y in enumerate(b):
            if i + j > deg:
                break
            out[i + j] += x * y
    return out


def _poly_pow(p, e, deg):
    res = [1] + [0] * deg
    base = p[:]
    while e:
        if e & 1:
            res = _poly_mul(res, base, deg)
        base = _poly_mul(base, base, deg)
        e >>= 1
    return res


def alignment_counts(T: int, U: int, durations) -> dict:
    """{k: N(k)} for every number of blanks k >= 1 with N(k) > 0."""
    durations = list(durations)
    if T <= 0:
        return {}
    lab = [0] * (T + 1)
    for d in durations:
        if d <= T:
            lab[d] += 1
    blk = [0] * (T + 1)
    for d in durations:
        if 0 < d <= T:
            blk[d] += 1
    lab_pow = _poly_pow(lab, U, T)
    out = {}
    blk_pow = [1] + [0] * T
    for k in range(1, T + 1):
        blk_pow = _poly_mul(blk_pow, blk, T)
        if not any(blk_pow):
            break
        c = sum(lab_pow[j] * blk_pow[T - j] for j in range(T + 1))
        if c:
            out[k] = math.comb(U + k - 1, U) * c
    return out


def count_alignments(T: int, U: int, durations) -> int:
    return sum(alignment_counts(T, U, durations).values())


def zero_logit_loss(T: int, U: int, V: int, durations, sigma: float = 0.0) -> float:
    """Exact -log P when every token and duration logit is zero (+inf if no alignment)."""
    D = len(list(durations))
    counts = alignment_counts(T, U, durations)
    if not counts:
        return math.inf
    per = math.log(V) + math.log(D) + sigma
    terms = [math.log(n) - (U + k) * per for k, n in counts.items()]
    m = max(terms)
    return -(m + math.log(math.fsum(math.exp(x - m) for x in terms)))
