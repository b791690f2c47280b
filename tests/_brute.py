"""Pure-Python brute force for tiny inputs, used to pin the oracle.

Written independently of ``oracle/`` (different algorithms, exact rational
arithmetic with ``fractions.Fraction``), so that a slip in either one shows
up as a disagreement.  Tiny inputs only: everything here is O(slow).
"""
from __future__ import annotations

import struct
from fractions import Fraction

SENT = 0xFFFFFFFF
E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def mask(rows, real_count, tp_rank):
    """rows: list of lists of ints.  Row r is padding iff r + tp_rank*N >= real_count."""
    n = len(rows)
    out = []
    for r, row in enumerate(rows):
        if r + tp_rank * n >= real_count:
            out.append([-1] * len(row))
        else:
            out.append(list(row))
    return out


def indices(flat_ids, n_experts):
    """Bucket enumeration: for each expert in ascending order, walk every slot."""
    s = len(flat_ids)
    teo, counts = [], []
    for e in range(n_experts):
        c = 0
        for i in range(s):
            if flat_ids[i] == e:
                teo.append(i)
                c += 1
        counts.append(c)
    v = len(teo)
    restore = [SENT] * s
    for p, i in enumerate(teo):
        restore[i] = p
    teo = teo + [SENT] * (s - v)
    expert_ids, starts = [], [0]
    for e in range(n_experts):
        if counts[e] > 0:
            expert_ids.append(e)
            starts.append(starts[-1] + counts[e])
    a = len(expert_ids)
    expert_ids += [-1] * (n_experts - a)
    starts += [v] * (n_experts + 1 - len(starts))
    stats = [max(counts) if v else 0, a]
    return dict(token_expert_order=teo, restore_token_order=restore, expert_ids=expert_ids,
                expert_start_indices=starts, expert_usage_stats=stats, n_routed=v)


# ---------------------------------------------------------------- numbers
def bf16_value(bits):
    """Exact value of a finite bf16 pattern, and its sign bit."""
    f = struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]
    return Fraction(f), (bits >> 15) & 1


def floor_log2(a: Fraction) -> int:
    """Largest integer e with 2**e <= a (a > 0), by stepping."""
    e = 0
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_binary(q: Fraction, p: int, emin: int) -> Fraction:
    """Round q to p significant bits, exponent floor emin (gradual underflow),
    to nearest with ties to even.  No overflow handling (not needed here)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(floor_log2(a), emin)
    quantum = Fraction(2) ** (e - p + 1)
    m = a / quantum
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * quantum


def f32(q: Fraction) -> Fraction:
    return round_binary(q, 24, -126)


def bf16(q: Fraction) -> Fraction:
    return round_binary(q, 8, -126)


# ---------------------------------------------------------------- MXFP4
def mxfp4_block(bits32):
    """One 32-element block -> (scale byte, 32 nibbles).  Exact search."""
    vals = [bf16_value(b) for b in bits32]
    amax = max(abs(v) for v, _ in vals)
    if amax == 0:
        se = -127
    else:
        se = min(max(floor_log2(amax) - 2, -127), 127)
    unit = Fraction(2) ** se
    nibs = []
    for v, sgn in vals:
        a = abs(v) / unit
        best, best_d = None, None
        for code, g in enumerate(E2M1):
            d = abs(a - g)
            if best is None or d < best_d or (d == best_d and code % 2 == 0):
                best, best_d = code, d
        nibs.append(best | (8 if sgn else 0))
    return se + 127, nibs


def mxfp4_row(bits_row):
    payload, scales = [], []
    for b0 in range(0, len(bits_row), 32):
        sc, nibs = mxfp4_block(bits_row[b0:b0 + 32])
        scales.append(sc)
        for m in range(16):
            payload.append(nibs[2 * m] | (nibs[2 * m + 1] << 4))
    return payload, scales


# ---------------------------------------------------------------- combine
def combine_row(weights_row, y_rows, positions):
    """Exact per-operation fp32 rounding, j in order; returns exact bf16 values."""
    h = len(y_rows[0]) if y_rows else 0
    out = []
    for c in range(h):
        acc = Fraction(0)
        for j, p in enumerate(positions):
            if p == SENT:
                continue
            w = Fraction(float(weights_row[j]))
            y, _ = bf16_value(y_rows[p][c])
            prod = f32(w * y)
            acc = f32(acc + prod)
        out.append(bf16(acc))
    return out


# ---------------------------------------------------------------- next rows
def scales_offset(flat_ids, n_experts, align):
    """Walk the experts in id order; each active one starts at the running
    total, which then grows by its count rounded up to `align`."""
    counts = [0] * n_experts
    for f in flat_ids:
        if 0 <= f < n_experts:
            counts[f] += 1
    out, run = [], 0
    for e in range(n_experts):
        if counts[e] > 0:
            out.append(run)
            c = counts[e]
            while c % align:
                c += 1
            run += c
    return out + [run] * (n_experts + 1 - len(out))


def even_scale_byte(bits32):
    """Scale byte under the even-mode rule: round max |x| to one mantissa bit
    (halves up) and take floor(log2) of the rounded value."""
    amax = max(abs(bf16_value(b)[0]) for b in bits32)
    if amax == 0:
        return 0
    e = floor_log2(amax)
    unit = Fraction(2) ** (e - 1)            # one mantissa bit below the leading bit
    n = amax / unit
    q = n.numerator // n.denominator
    if n - q >= Fraction(1, 2):
        q += 1
    rounded = q * unit
    se = min(max(floor_log2(rounded) - 2, -127), 127)
    return se + 127


def combine_epilogue_row(weights_row, y_rows, positions, scale, residual_row):
    plain = combine_row_f32(weights_row, y_rows, positions)
    out = []
    for c, acc in enumerate(plain):
        r = f32(Fraction(float(scale)) * acc) if scale is not None else acc
        if residual_row is not None:
            r = f32(r + bf16_value(residual_row[c])[0])
        out.append(bf16(r))
    return out


def combine_row_f32(weights_row, y_rows, positions):
    h = len(y_rows[0]) if y_rows else 0
    out = []
    for c in range(h):
        acc = Fraction(0)
        for j, p in enumerate(positions):
            if p == SENT:
                continue
            w = Fraction(float(weights_row[j]))
            y, _ = bf16_value(y_rows[p][c])
            acc = f32(acc + f32(w * y))
        out.append(acc)
    return out
