"""Pins of the oracle's seeded sampler (temperature, top-k, top-p, one draw
against a given uniform) against what the definitions fix independently of
its code: limits that reduce to the greedy choice, a two-candidate sigmoid,
the top-p cut of a three-candidate row, the uniform limit of a large
temperature, exact draw frequencies over a grid of uniforms, a brute-force
top-k by sorting, and refusal of non-finite rows."""
import math

import numpy as np

import oracle
import synth
from synth.workloads import TensorIds


def _row(n, seed, std=3.0):
    return synth.normal_bf16(n, seed, TensorIds.SAMPLE_LOGITS, 0.0, std)


def test_top_k_one_is_the_greedy_choice():
    for seed in range(5):
        row = _row(4096, 40 + seed)
        row[[7, 900]] = row[np.argmax(oracle.f64(row))]  # force ties with the maximum
        g = oracle.argmax(row)
        for u in (0.0, 0.37, 0.999999):
            assert oracle.sample(row, 0.6, 1, 0.95, u)[0] == g


def test_tiny_top_p_is_the_greedy_choice():
    row = _row(4096, 50)
    g = oracle.argmax(row)
    for u in (0.0, 0.5, 0.9999):
        assert oracle.sample(row, 1.0, 20, 1e-9, u)[0] == g


def test_two_candidates_sigmoid():
    # logits a = 1.5 (id 3) and b = 0.25 (id 9), the rest far below
    row = oracle.bf16(np.full(16, -60.0))
    row[3], row[9] = oracle.bf16(np.array([1.5, 0.25]))
    for T in (0.6, 1.0, 2.0):
        p0 = 1.0 / (1.0 + math.exp((0.25 - 1.5) / T))
        assert oracle.sample(row, T, 2, 1.0, p0 - 1e-9)[0] == 3
        assert oracle.sample(row, T, 2, 1.0, p0 + 1e-9)[0] == 9
        # margin: the draw target sits 0.5*p0 from the first boundary; the top-p
        # cut (top_p = 1) is the second candidate's mass 1 - p0 away
        tok, m = oracle.sample(row, T, 2, 1.0, 0.5 * p0)
        assert tok == 3 and abs(m - min(0.5 * p0, 1.0 - p0)) < 1e-12


def test_ties_are_ordered_by_id():
    row = oracle.bf16(np.zeros(10))
    for j, u in enumerate((0.1, 0.4, 0.9)):
        assert oracle.sample(row, 1.0, 3, 1.0, u)[0] == j


def test_top_p_cut_three_candidates():
    x = np.array([0.0, -0.5, -0.875])           # exact in bf16
    row = oracle.bf16(np.concatenate([x, np.full(5, -40.0)]))
    e = np.exp(x)
    p = e / e.sum()
    # candidate i stays while the mass before it is below top_p
    cases = [(0.4, 1), (p[0] - 1e-6, 1), (p[0] + 1e-6, 2), (0.75, 2), (p[0] + p[1] + 1e-6, 3), (1.0, 3)]
    for top_p, kept in cases:
        seen = {oracle.sample(row, 1.0, 3, top_p, (j + 0.5) / 64)[0] for j in range(64)}
        assert seen == set(range(kept)), (top_p, seen)


def test_large_temperature_is_uniform_over_top_k():
    row = _row(2048, 60)
    order = np.lexsort((np.arange(row.size), -oracle.f64(row)))  # value desc, then id
    K = 16
    for j in range(K):
        assert oracle.sample(row, 1e9, K, 1.0, (j + 0.5) / K)[0] == order[j]


def test_draw_frequencies_match_the_kept_distribution():
    row = _row(1000, 70, std=1.0)
    T, K, P = 0.7, 12, 0.8
    vals = oracle.f64(row)
    order = np.lexsort((np.arange(row.size), -vals))[:K]
    e = np.exp((vals[order] - vals[order[0]]) / T)
    keep = 1
    while keep < K and e[:keep].sum() < P * e.sum():
        keep += 1
    q = e[:keep] / e[:keep].sum()
    N = 20000
    counts = {}
    for j in range(N):
        t, _ = oracle.sample(row, T, K, P, (j + 0.5) / N)
        counts[t] = counts.get(t, 0) + 1
    assert set(counts) == set(order[:keep].tolist())
    for i, tok in enumerate(order[:keep]):
        assert abs(counts[int(tok)] / N - q[i]) <= 1.0 / N + 1e-12


def test_top_k_selection_equals_sorting():
    for seed in range(4):
        row = _row(166912, 80 + seed)
        vals = oracle.f64(row)
        order = np.lexsort((np.arange(row.size), -vals))
        K = 64
        for j in (0, 17, 63):
            assert oracle.sample(row, 1e9, K, 1.0, (j + 0.5) / K)[0] == order[j]


def test_nonfinite_rows_are_refused():
    row = _row(512, 90)
    for bad in (0x7FC0, 0x7F80, 0xFF80):
        r = row.copy()
        r[100] = bad
        assert oracle.sample(r, 1.0, 20, 0.95, 0.5)[0] == -1
