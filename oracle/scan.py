"""Exact affine-map scans over time (rational arithmetic).

A Newton iteration leaves the linear recurrence s_t = A_t s_{t-1} + b_t.  An
affine map is the pair (A, b); applying m = (A, b) to s gives A s + b, and
"m2 after m1" is (A2 A1, A2 b1 + b2).  That composition is associative, so
the recurrence can be solved by any bracketing of the product, which is what
the parallel scan exploits ("Newton+scan", FAQs; a segment head is the map
(0, b), shapes/layout page).

Everything here works on Python Fractions (or ints), so equality between the
serial loop, every bracketing and the chunked three-phase scan is exact.
Maps are (A, b) with A an S x S list of lists and b a length-S list.
"""
from __future__ import annotations

from fractions import Fraction
from functools import lru_cache


def identity(S):
    return ([[Fraction(int(p == q)) for q in range(S)] for p in range(S)], [Fraction(0)] * S)


def apply(m, s):
    A, b = m
    S = len(b)
    return [sum(A[p][q] * s[q] for q in range(S)) + b[p] for p in range(S)]


def compose(m2, m1):
    """m2 after m1: x -> m2(m1(x))."""
    A2, b2 = m2
    A1, b1 = m1
    S = len(b2)
    A = [[sum(A2[p][r] * A1[r][q] for r in range(S)) for q in range(S)] for p in range(S)]
    b = [sum(A2[p][r] * b1[r] for r in range(S)) + b2[p] for p in range(S)]
    return (A, b)


def freeze(m):
    A, b = m
    return (tuple(tuple(r) for r in A), tuple(b))


def serial_states(maps, s0):
    """s_t = m_t(s_{t-1}) for t = 1..T, one after the other."""
    out = []
    s = list(s0)
    for m in maps:
        s = apply(m, s)
        out.append(s)
    return out


def all_bracketings(maps):
    """Every full bracketing of m_T after ... after m_1, as a set of frozen maps."""
    maps = [freeze(m) for m in maps]

    @lru_cache(maxsize=None)
    def rec(i, j):  # composite of maps[i..j]
        if i == j:
            return {maps[i]}
        res = set()
        for k in range(i, j):
            for left in rec(i, k):          # earlier block
                for right in rec(k + 1, j):  # later block
                    res.add(freeze(compose(right, left)))
        return res

    return rec(0, len(maps) - 1)


def count_bracketings(n):
    """Catalan number C_{n-1}: how many bracketings a product of n maps has."""
    from math import comb
    return comb(2 * (n - 1), n - 1) // n


def three_phase(maps, s0, L):
    """Chunked scan with chunk length L.

    phase 1  reduce each chunk's maps to one aggregate (in time order);
    phase 2  exclusive scan of the aggregates as maps, applied to s0, giving
             each chunk's carry-in state;
    phase 3  run every chunk from its carry-in.
    """
    S = len(s0)
    chunks = [maps[i:i + L] for i in range(0, len(maps), L)]
    aggs = []
    for ch in chunks:
        agg = identity(S)
        for m in ch:
            agg = compose(m, agg)
        aggs.append(agg)
    prefix = identity(S)
    carries = []
    for agg in aggs:
        carries.append(apply(prefix, s0))
        prefix = compose(agg, prefix)
    out = []
    for ch, carry in zip(chunks, carries):
        s = carry
        for m in ch:
            s = apply(m, s)
            out.append(s)
    return out
