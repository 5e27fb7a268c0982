"""Brute-force collectives in pure Python, for tiny inputs.

TEST INFRASTRUCTURE, written independently of ``oracle.c``: values are
decoded from their bit patterns into exact rationals, every binary32
addition is the exact rational sum rounded to binary32 by an explicit
nearest-even search, and the final narrowing to the element type is the same
generic rounding. Layouts are explicit index loops over Python lists.

Inputs and outputs are lists of integer bit patterns (bf16: 16-bit, fp32:
32-bit words). A NaN result is returned as that format's canonical quiet NaN;
callers compare NaNs by class, not by payload.
"""

from __future__ import annotations

from fractions import Fraction

# (exponent bits, fraction bits)
FMT = {"bf16": (8, 7), "f32": (8, 23)}


class Val:
    """An IEEE value: kind is 'fin', 'inf' or 'nan'. For 'fin', q is the exact
    value and neg the sign bit (which only matters when q == 0)."""

    __slots__ = ("kind", "q", "neg")

    def __init__(self, kind, q=Fraction(0), neg=False):
        self.kind, self.q, self.neg = kind, q, neg


def decode(bits: int, fmt: str) -> Val:
    E, M = FMT[fmt]
    sign = (bits >> (E + M)) & 1
    e = (bits >> M) & ((1 << E) - 1)
    m = bits & ((1 << M) - 1)
    bias = (1 << (E - 1)) - 1
    if e == (1 << E) - 1:
        return Val("nan") if m else Val("inf", neg=bool(sign))
    if e == 0:
        q = Fraction(m, 1 << M) * Fraction(2) ** (1 - bias)
    else:
        q = (1 + Fraction(m, 1 << M)) * Fraction(2) ** (e - bias)
    return Val("fin", -q if sign else q, bool(sign))


def _floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # 2^e <= a < 2^(e+1) after at most one correction either way
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def encode(v: Val, fmt: str) -> int:
    """Round v to the format, nearest with ties to even, and return its bits."""
    E, M = FMT[fmt]
    bias = (1 << (E - 1)) - 1
    emin, emax = 1 - bias, bias
    exp_all = (1 << E) - 1
    if v.kind == "nan":
        return (exp_all << M) | (1 << (M - 1))
    if v.kind == "inf":
        return (int(v.neg) << (E + M)) | (exp_all << M)
    q = v.q
    neg = v.neg if q == 0 else q < 0
    a = abs(q)
    if a == 0:
        return int(neg) << (E + M)
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - M)
    N = round(a / quantum)            # Fraction.__round__: half to even
    if N == 0:
        return int(neg) << (E + M)
    if N >= (1 << (M + 1)):           # carried into the next binade
        N //= 2
        e += 1
    if e > emax:
        return (int(neg) << (E + M)) | (exp_all << M)
    if N < (1 << M):                  # subnormal (e == emin)
        return (int(neg) << (E + M)) | N
    return (int(neg) << (E + M)) | ((e + bias) << M) | (N - (1 << M))


def add_f32(a: Val, b: Val) -> Val:
    """One IEEE binary32 addition (round to nearest even)."""
    if a.kind == "nan" or b.kind == "nan":
        return Val("nan")
    if a.kind == "inf" and b.kind == "inf":
        return Val("inf", neg=a.neg) if a.neg == b.neg else Val("nan")
    if a.kind == "inf":
        return a
    if b.kind == "inf":
        return b
    s = a.q + b.q
    if s == 0:
        # exact zero: -0 only for (-0) + (-0); x + (-x) is +0
        neg = a.q == 0 and b.q == 0 and a.neg and b.neg
        return Val("fin", Fraction(0), neg)
    return decode(encode(Val("fin", s, s < 0), "f32"), "f32")


def widen(bits: int, fmt: str) -> Val:
    """Element -> binary32 value (exact for both formats)."""
    return decode(bits, fmt)


def reduce_elem(vals_bits: list[int], fmt: str) -> int:
    acc = widen(vals_bits[0], fmt)
    for b in vals_bits[1:]:
        acc = add_f32(acc, widen(b, fmt))
    return encode(acc, fmt)


def reduce(srcs: list[list[int]], fmt: str) -> list[int]:
    m = len(srcs[0])
    return [reduce_elem([s[i] for s in srcs], fmt) for i in range(m)]


def reduce_scatter(xs: list[list[int]], fmt: str) -> list[list[int]]:
    P = len(xs)
    n = len(xs[0]) // P
    ys = []
    for k in range(P):
        yk = []
        for i in range(n):
            yk.append(reduce_elem([xs[r][k * n + i] for r in range(P)], fmt))
        ys.append(yk)
    return ys


def all_gather(zs: list[list[int]]) -> list[list[int]]:
    P = len(zs)
    n = len(zs[0])
    outs = []
    for j in range(P):
        o = [None] * (P * n)
        for k in range(P):
            for i in range(n):
                o[k * n + i] = zs[k][i]
        outs.append(o)
    return outs


def all_to_all(xs: list[list[int]]) -> list[list[int]]:
    P = len(xs)
    n = len(xs[0]) // P
    outs = []
    for j in range(P):
        o = [None] * (P * n)
        for r in range(P):
            for i in range(n):
                o[r * n + i] = xs[r][j * n + i]
        outs.append(o)
    return outs


def all_to_all_v(xs: list[list[int]], C: list[list[int]], row: int):
    """Source r's rows are grouped by destination in destination order;
    destination j receives every source's group for j, sources in order."""
    P = len(xs)
    outs = [[] for _ in range(P)]
    for j in range(P):
        for r in range(P):
            start = sum(C[r][jj] for jj in range(j))
            for t in range(start, start + C[r][j]):
                outs[j].extend(xs[r][t * row:(t + 1) * row])
    return outs


def all_reduce(xs: list[list[int]], fmt: str) -> list[list[int]]:
    return all_gather(reduce_scatter(xs, fmt))


def reduce_scatter_v(xs: list[list[int]], cnt: list[int], fmt: str):
    P = len(xs)
    ys = []
    off = 0
    for k in range(P):
        ys.append([reduce_elem([xs[r][off + i] for r in range(P)], fmt)
                   for i in range(cnt[k])])
        off += cnt[k]
    return ys


def all_gather_v(zs: list[list[int]]) -> list[list[int]]:
    P = len(zs)
    flat = []
    for k in range(P):
        flat.extend(zs[k])
    return [list(flat) for _ in range(P)]


def fma_f32(a: Val, b: Val, c: Val) -> Val:
    """One IEEE binary32 fused multiply-add a*b + c (round to nearest even):
    the exact rational result, rounded once."""
    if "nan" in (a.kind, b.kind, c.kind):
        return Val("nan")
    if a.kind == "inf" or b.kind == "inf":
        other = b if a.kind == "inf" else a
        if other.kind == "fin" and other.q == 0:
            return Val("nan")                       # inf * 0
        neg = (a.q < 0 or (a.q == 0 and a.neg)) if a.kind == "fin" else a.neg
        neg ^= (b.q < 0 or (b.q == 0 and b.neg)) if b.kind == "fin" else b.neg
        if c.kind == "inf" and c.neg != neg:
            return Val("nan")
        return Val("inf", neg=neg)
    if c.kind == "inf":
        return c
    p = a.q * b.q
    s = p + c.q
    if s == 0:
        pneg = (a.q < 0 or (a.q == 0 and a.neg)) != (b.q < 0 or (b.q == 0 and b.neg))
        neg = p == 0 and c.q == 0 and pneg and c.neg
        return Val("fin", Fraction(0), neg)
    return decode(encode(Val("fin", s, s < 0), "f32"), "f32")


def moe_route(ids: list[list[int]], E: int, k: int):
    """Positions by sorting: the entries bound for the experts of rank j,
    ordered by (expert, source rank, entry index), take rows 0, 1, ... in
    that order. Returns (pos, counts, recv) as Python lists."""
    P = len(ids)
    per = E // P
    pos = [[-1] * len(ids[r]) for r in range(P)]
    counts = [[0] * E for _ in range(P)]
    recv = [0] * P
    for j in range(P):
        keys = sorted((ids[r][i], r, i) for r in range(P) for i in range(len(ids[r]))
                      if j * per <= ids[r][i] < (j + 1) * per)
        for row, (e, r, i) in enumerate(keys):
            pos[r][i] = row
            counts[r][e] += 1
        recv[j] = len(keys)
    return pos, counts, recv


def moe_combine(ys: list[list[int]], ids, pos, w_bits, E: int, k: int, H: int, cap: int, fmt: str):
    """out_r[t][h] = fma chain over the token's k choices in order, from +0,
    one rounding to the element type. w_bits: binary32 weight bit patterns."""
    P = len(ys)
    per = E // P
    outs = []
    for r in range(P):
        T = len(ids[r]) // k
        o = []
        for t in range(T):
            for h in range(H):
                acc = Val("fin", Fraction(0), False)
                for c in range(k):
                    i = t * k + c
                    e = ids[r][i]
                    if not (0 <= e < E) or pos[r][i] < 0 or pos[r][i] >= cap:
                        continue
                    v = widen(ys[e // per][pos[r][i] * H + h], fmt)
                    acc = fma_f32(decode(w_bits[r][i], "f32"), v, acc)
                o.append(encode(acc, fmt))
        outs.append(o)
    return outs


def is_nan_bits(bits: int, fmt: str) -> bool:
    return decode(bits, fmt).kind == "nan"
