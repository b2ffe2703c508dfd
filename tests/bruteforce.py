"""Brute-force enumerators for tiny inputs (pure Python, test-only).

Written independently of oracle.c, from the same definitions but by other
means: top-k membership by counting the experts strictly ahead, buffer
positions by a full sort of (rank, expert, token) keys, dedup rows from a set,
combine by exact rational arithmetic (the exact sum, and the fp32 chain with
every rounding step done by bisection over fp32 bit patterns).
"""
from __future__ import annotations

import math
import struct
from collections import Counter
from fractions import Fraction


def topk(logits_row, k):
    """Expert e takes slot s iff exactly s experts are strictly ahead of it,
    where e' is ahead of e if l[e'] > l[e], or l[e'] == l[e] and e' < e."""
    E = len(logits_row)
    slots = [None] * k
    for e in range(E):
        ahead = sum(1 for f in range(E)
                    if logits_row[f] > logits_row[e]
                    or (logits_row[f] == logits_row[e] and f < e))
        if ahead < k:
            slots[ahead] = e
    return slots


def nondedup_layout(idx, place):
    """Row position of every (t, j): sort all (place[e], e, t) keys."""
    keys = []
    for t, row in enumerate(idx):
        for j, e in enumerate(row):
            keys.append((place[e], e, t, j))
    keys.sort()
    pos = {}
    for p, (_, e, t, j) in enumerate(keys):
        pos[(t, j)] = p
    return keys, pos


def dedup_layout(idx, place):
    """Rows = sorted set of (rank, token)."""
    pairs = sorted({(place[e], t) for t, row in enumerate(idx) for e in row})
    return pairs


def bf16_to_fraction(bits):
    f = struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]
    return Fraction(f)


def _bf16_value(bits):
    return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]


def nearest_bf16(q: Fraction, negative_zero=False):
    """Nearest bf16 to an exact rational, ties to the even bit pattern, found by
    comparing q with the finite bf16 values around it (no overflow handling:
    |q| must be below the largest finite bf16)."""
    if q == 0:
        return 0x8000 if negative_zero else 0x0000
    sign = 0x8000 if q < 0 else 0
    a = abs(q)
    # Bisect over non-negative finite bf16 patterns 0x0000..0x7F7F (monotone).
    lo, hi = 0, 0x7F7F
    while lo < hi:                      # smallest pattern with value >= a
        mid = (lo + hi) // 2
        if Fraction(_bf16_value(mid)) >= a:
            hi = mid
        else:
            lo = mid + 1
    up = lo
    if Fraction(_bf16_value(up)) == a:
        return sign | up
    down = up - 1
    du = Fraction(_bf16_value(up)) - a
    dd = a - Fraction(_bf16_value(down))
    if du < dd:
        b = up
    elif dd < du:
        b = down
    else:
        b = up if (up & 1) == 0 else down
    return sign | b


def e4m3_to_fraction(b):
    """fp8 E4M3 (OCP) value of byte b as an exact fraction (NaN excluded)."""
    b = int(b) & 0xFF
    s, e, m = b >> 7, (b >> 3) & 15, b & 7
    assert not (e == 15 and m == 7), "NaN"
    v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v


def combine(rows_bits, weights, slot_row, fp8=False):
    """Exact rational weighted sum of the distinct rows of each token; rows are
    bf16 bit patterns, or fp8 E4M3 bytes with fp8=True."""
    T, k = len(slot_row), len(slot_row[0])
    H = len(rows_bits[0])
    out = []
    for t in range(T):
        rs = sorted({r for r in slot_row[t] if r >= 0})
        o = []
        for h in range(H):
            acc = Fraction(0)
            all_neg_zero = True
            for r in rs:
                w = Fraction(1) if weights is None else Fraction(float(weights[r]))
                v = e4m3_to_fraction(rows_bits[r][h]) if fp8 else bf16_to_fraction(rows_bits[r][h])
                acc += w * v
                b = int(rows_bits[r][h])
                neg_zero = b == (0x80 if fp8 else 0x8000)
                if not (neg_zero and (weights is None or float(weights[r]) > 0)):
                    all_neg_zero = False
            # the sum starts at -0.0: it stays -0 only if every term is -0 (or none)
            o.append(nearest_bf16(acc, negative_zero=(acc == 0 and all_neg_zero)))
        out.append(o)
    return out


def _f32_value(bits):
    return struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0]


_F32_MAX = Fraction(_f32_value(0x7F7FFFFF))
_F32_OVERFLOW = _F32_MAX + Fraction(2) ** 103     # halfway from the largest fp32 to 2^128


def nearest_f32(q: Fraction):
    """Nearest fp32 to an exact rational, ties to the even bit pattern, by
    bisection over the finite non-negative fp32 patterns; magnitudes from the
    halfway point above the largest fp32 on round to infinity.  Returns a
    Python float (zero comes back as +0.0: callers fix its sign)."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    if a >= _F32_OVERFLOW:
        return sign * math.inf
    lo, hi = 0, 0x7F7FFFFF
    while lo < hi:                      # smallest pattern with value >= a
        mid = (lo + hi) // 2
        if Fraction(_f32_value(mid)) >= a:
            hi = mid
        else:
            lo = mid + 1
    up = lo
    if Fraction(_f32_value(up)) == a:
        return sign * _f32_value(up)
    down = up - 1
    du = Fraction(_f32_value(up)) - a
    dd = a - Fraction(_f32_value(down))
    if du < dd or (du == dd and (up & 1) == 0):
        return sign * _f32_value(up)
    return sign * _f32_value(down)


def fma_f32(w, y, acc):
    """fp32 fused multiply-add of finite fp32 values: w*y + acc computed
    exactly as rationals and rounded once.  An exact zero takes IEEE's sign:
    -0 only when both w*y and acc are zeros of negative sign."""
    p = Fraction(w) * Fraction(y)
    s = p + Fraction(acc)
    if s == 0:
        p_neg = p == 0 and (math.copysign(1.0, w) * math.copysign(1.0, y)) < 0
        acc_neg = acc == 0 and math.copysign(1.0, acc) < 0
        return -0.0 if (p_neg and acc_neg) else 0.0
    return nearest_f32(s)


def combine_chain(rows_bits, weights, slot_row, fp8=False):
    """The combine as its fp32 chain, emulated one rounding at a time with
    exact rationals: distinct rows in ascending index, acc = -0.0, acc =
    fma_f32(w, y, acc) per row, then bf16 round-to-nearest-even of acc.
    Finite values only (no overflow to bf16 infinity)."""
    T = len(slot_row)
    H = len(rows_bits[0])
    out = []
    for t in range(T):
        rs = sorted({r for r in slot_row[t] if r >= 0})
        o = []
        for h in range(H):
            acc = -0.0
            for r in rs:
                w = 1.0 if weights is None else float(weights[r])
                y = (float(e4m3_to_fraction(rows_bits[r][h])) if fp8
                     else _bf16_value(int(rows_bits[r][h])))
                acc = fma_f32(w, y, acc)
            o.append(nearest_bf16(Fraction(acc), negative_zero=math.copysign(1.0, acc) < 0))
        out.append(o)
    return out


def coselect(idx, n_experts, n_tokens):
    c = Counter()
    for t in range(min(n_tokens, len(idx))):
        s = list(idx[t])
        for a in s:
            for b in s:
                c[(a, b)] += 1
    return [[c[(a, b)] for b in range(n_experts)] for a in range(n_experts)]


def softmax_desc(values):
    """Full softmax of a list, in descending order of the values (textbook form)."""
    m = max(values)
    ex = [math.exp(v - m) for v in values]
    s = math.fsum(ex)
    return sorted((e / s for e in ex), reverse=True)


def expand_layout(row_experts, n_rows, place):
    """Receive-side expansion: position of every listed (row p, column c), by a
    full sort of the (rank, expert, row) keys of the non-padding entries."""
    keys = sorted((place[e], e, p, c) for p in range(n_rows)
                  for c, e in enumerate(row_experts[p]) if e >= 0)
    return {(p, c): q for q, (_, e, p, c) in enumerate(keys)}
