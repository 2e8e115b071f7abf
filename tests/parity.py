"""Comparators for parity checks: bf16 step distances (plain, and at the
larger addend of a residual add), the teacher-forced near-tie judge, the exact
row comparator, and logit statistics.

The near-tie rule follows the pull request "llama: Nanbeige4.3-33B on Metal,
the bf16 release served as published", review reply "Teacher-forced misses":
where two sides choose different tokens, the choice is a near-tie when the two
contenders lie within one bf16 step of each other on both sides (0.125 below
32, 0.25 from 32 to 64); a third token within that step of the top makes the
row red (reply "1. Row 1370"); rows holding NaN or +-Inf on either side are
refused before any comparison (reply "Non-finite rows").
"""
import math

import numpy as np


class Refused(ValueError):
    """A row holding NaN or +-Inf reached a comparator."""


def bf16_bits_to_f64(b):
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_step(v):
    """Spacing of bf16 at magnitude |v| (8 significant bits), floored at the
    spacing of the smallest normal, 2^-133."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    e = np.maximum(e, -126.0)
    return np.exp2(e - 7.0)


def ulp_distance(a_bits, b_bits):
    """|a - b| in bf16 steps at max(|a|, |b|)."""
    a = bf16_bits_to_f64(a_bits)
    b = bf16_bits_to_f64(b_bits)
    if not (np.isfinite(a).all() and np.isfinite(b).all()):
        raise Refused("non-finite activation")
    return np.abs(a - b) / bf16_step(np.maximum(np.abs(a), np.abs(b)))


def check_finite_row(row, side, pos):
    row = np.asarray(row, dtype=np.float64)
    if not np.isfinite(row).all():
        raise Refused(f"refused: {side} position {pos}: non-finite logit")


def top1(row):
    """Largest logit, ties to the lowest id."""
    row = np.asarray(row, dtype=np.float64)
    return int(np.argmax(row))  # numpy returns the first maximal index


def judge_row(ref, test, pos=0):
    """Returns 'equal', 'near-tie' or 'red' for one teacher-forced position.
    Both rows are logit values (binary64 of bf16, or any float)."""
    ref = np.asarray(ref, dtype=np.float64)
    test = np.asarray(test, dtype=np.float64)
    check_finite_row(ref, "reference", pos)
    check_finite_row(test, "native", pos)
    a, b = top1(ref), top1(test)
    if a == b:
        return "equal"
    for row in (ref, test):
        top = row.max()
        step = float(bf16_step(top))
        if abs(row[a] - row[b]) > step:
            return "red"
        close = np.nonzero(row >= top - step)[0]
        if any(c not in (a, b) for c in close.tolist()):
            return "red"
    return "near-tie"


def top1_gate(counts, rows):
    """Teacher-forced top-1 agreement of at least 99%, every miss a near-tie:
    no red row, and at most max(1, 1% of rows) near-ties (on a sample of
    under 100 positions one near-tie is the smallest possible miss)."""
    misses = counts["near-tie"]
    return counts["red"] == 0 and misses <= max(1, int(0.01 * rows))


def judge(ref_rows, test_rows):
    """Judges every position; returns (counts dict, list of (pos, verdict))."""
    counts = {"equal": 0, "near-tie": 0, "red": 0}
    detail = []
    for i, (r, t) in enumerate(zip(ref_rows, test_rows)):
        v = judge_row(r, t, i)
        counts[v] += 1
        if v != "equal":
            detail.append((i, v))
    return counts, detail


def differing_rows(a, b):
    """Exact comparator: indices of rows whose bit patterns differ anywhere."""
    a = np.asarray(a).reshape(len(a), -1)
    b = np.asarray(b).reshape(len(b), -1)
    if a.shape != b.shape:
        raise ValueError(f"shape mismatch {a.shape} vs {b.shape}")
    return np.nonzero((a != b).any(axis=1))[0].tolist()


def log_softmax(x):
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=-1, keepdims=True)
    z = x - m
    return z - np.log(np.exp(z).sum(axis=-1, keepdims=True))


def mean_kl(ref_logits, test_logits):
    """Mean over rows of KL(softmax(ref) || softmax(test)), in nats, over the
    full vocabulary."""
    lp = log_softmax(ref_logits)
    lq = log_softmax(test_logits)
    p = np.exp(lp)
    return float((p * (lp - lq)).sum(axis=-1).mean())


def within_ulps(a_bits, b_bits, ulps=2.0):
    """Fraction of elements within `ulps` bf16 steps (at max(|a|, |b|))."""
    d = ulp_distance(a_bits, b_bits)
    return float((d <= ulps).mean()), float(d.max()) if d.size else 0.0


def addend_ulps(got_bits, ref_bits, h_in_bits):
    """Distance of residual-stream elements in bf16 steps taken at the larger
    addend of the residual add that produced them: h_out = bf16(h_in + y) with
    y = h_out - h_in, scale max(|got|, |ref|, |h_in|, |ref - h_in|).  A 1-step
    difference in y moves a cancelling sum by a step of y, not of the small
    result; measuring at the result's own magnitude would count cancellation
    instead of error."""
    a = bf16_bits_to_f64(got_bits)
    b = bf16_bits_to_f64(ref_bits)
    h = bf16_bits_to_f64(h_in_bits)
    if not (np.isfinite(a).all() and np.isfinite(b).all()):
        raise Refused("non-finite activation")
    scale = np.maximum.reduce([np.abs(a), np.abs(b), np.abs(h), np.abs(b - h)])
    return np.abs(a - b) / bf16_step(scale)


def within_addend_ulps(got_bits, ref_bits, h_in_bits, ulps=2.0):
    d = addend_ulps(got_bits, ref_bits, h_in_bits)
    return float((d <= ulps).mean()), float(d.max()) if d.size else 0.0


def sum_bound_ok(got_bits, ref_bits, abs_sum, k):
    """For values that are sums of k exact products rounded once to bf16 (in
    any fp32 order on one side, exactly on the other): True where the two
    bf16 values differ by at most one bf16 step at the larger of them plus
    the worst fp32 summation error, (k - 1) * 2^-24 * sum |terms| (abs_sum).
    A missing, repeated or misplaced term breaks it; rounding order cannot."""
    a = bf16_bits_to_f64(got_bits)
    b = bf16_bits_to_f64(ref_bits)
    if not (np.isfinite(a).all() and np.isfinite(b).all()):
        raise Refused("non-finite value")
    step = bf16_step(np.maximum(np.abs(a), np.abs(b)))
    return np.abs(a - b) <= step + (k - 1) * 2.0 ** -24 * np.asarray(abs_sum, dtype=np.float64)


def bf16_round_f64(x):
    """Round binary64 to bf16 with ties to even, returning binary64 (used only
    on test fixtures)."""
    if x == 0 or not math.isfinite(x):
        return x
    m, e = math.frexp(abs(x))
    q = e - 8
    r = round(math.ldexp(abs(x), -q))  # Python's round: ties to even
    return math.copysign(math.ldexp(r, q), x)
