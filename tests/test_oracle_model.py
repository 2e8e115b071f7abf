"""Oracle forward-pass checks: the model-level invariants the pages hold the
engine to (bit-exact in the oracle by construction), an independent rewrite
on the tiny workload, the pages' size figures, and the comparators' planted
controls.  CPU only.

Invariants: one-row steps equal multi-row windows and a resumed prompt equals
a fresh one (pull request "llama: Nanbeige4.3-33B on Metal, the bf16 release
served as published", section "Measured"); continuations match across chunk
boundaries (NInfer model card, section "Validation").
"""
import csv
import dataclasses

import numpy as np
import pytest

import oracle
from oracle.model import OracleModel
from synth.workloads import CONFIGS, config
from tests import naive_llama, parity
from tests.host_inputs import HostWeights, prompt


@pytest.fixture(scope="module")
def tiny():
    g = config(1)
    return g, HostWeights(g)


def test_tiny_matches_independent_rewrite(tiny):
    """Whole-sequence numpy rewrite vs the C oracle on the 2-block workload:
    every bf16 logit and every execution's output residual agree."""
    g, W = tiny
    toks = prompt(g, n=24)
    m = OracleModel(g, W)
    s = m.new_sequence(64)
    r = m.forward(s, tokens=toks, logits="all", capture=True)
    ref64, outs = naive_llama.forward(g, W.all(), toks)
    assert (oracle.f64(r["logits"]) == naive_llama.rnd(ref64)).all()
    assert np.allclose(r["logits64"], ref64, rtol=0, atol=1e-9)
    for (mid, out), want in zip(r["capture"], outs):
        assert (oracle.f64(out) == want).all()


def test_looped_matches_independent_rewrite():
    """A small looped geometry (3 blocks x 2 loops, decoupled head width):
    each execution keeps its own cache and the final norm replaces the
    residual after every loop."""
    g = dataclasses.replace(config(1), name="tiny-looped", n_blocks=3, n_loops=2, hidden=256,
                            n_q_heads=4, n_kv_heads=2, head_dim=128, ffn=512, vocab=512)
    W = HostWeights(g)
    toks = prompt(g, n=12)
    m = OracleModel(g, W)
    s = m.new_sequence(16)
    r = m.forward(s, tokens=toks, logits="all", capture=True)
    ref64, outs = naive_llama.forward(g, W.all(), toks)
    assert len(r["capture"]) == 6
    assert (oracle.f64(r["logits"]) == naive_llama.rnd(ref64)).all()
    # loop 2's caches are distinct from loop 1's
    assert (s.kc[0] != s.kc[3]).any()


def test_window_equals_one_row_steps(tiny):
    g, W = tiny
    toks = prompt(g, n=40)
    m = OracleModel(g, W)
    a = m.new_sequence(64)
    b = m.new_sequence(64)
    m.forward(a, tokens=toks[:24], logits=None)
    m.forward(b, tokens=toks[:24], logits=None)
    wa = m.forward(a, tokens=toks[24:40], logits="all")["logits"]
    rows = [m.forward(b, tokens=toks[i:i + 1], logits="all")["logits"][0] for i in range(24, 40)]
    assert parity.differing_rows(wa, np.stack(rows)) == []
    assert (a.kc == b.kc).all() and (a.vc == b.vc).all()


def test_chunked_prefill_equals_single_chunk(tiny):
    g, W = tiny
    toks = prompt(g)
    m = OracleModel(g, W)
    one = m.new_sequence(64)
    many = m.new_sequence(64)
    full = m.forward(one, tokens=toks, logits="all")["logits"]
    parts = [m.forward(many, tokens=toks[i:i + 13], logits="all")["logits"]
             for i in range(0, 64, 13)]
    assert parity.differing_rows(full, np.concatenate(parts)) == []


def test_resumed_equals_fresh(tiny):
    """Keep the first 30 positions of a sequence, drop the rest, and run the
    continuation again: it equals a fresh run of the whole prompt."""
    g, W = tiny
    toks = prompt(g)
    m = OracleModel(g, W)
    fresh = m.new_sequence(64)
    lf = m.forward(fresh, tokens=toks, logits="all")["logits"]
    kept = m.new_sequence(64)
    m.forward(kept, tokens=toks[:30], logits=None)
    m.forward(kept, tokens=toks[30:50], logits=None)  # a turn that is later dropped
    kept.length = 30
    lr = m.forward(kept, tokens=toks[30:], logits="all")["logits"]
    assert parity.differing_rows(lf[30:], lr) == []


def test_greedy_generation_is_consistent(tiny):
    """generate() = prompt chunk, then one-row steps fed their own choices;
    every token equals the argmax of the logits a teacher-forced pass gives."""
    g, W = tiny
    toks = prompt(g)
    m = OracleModel(g, W)
    s = m.new_sequence(96)
    gen = m.generate(s, toks, g.decode_steps)
    s2 = m.new_sequence(96)
    full = np.concatenate([toks, gen[:-1]])
    lg = m.forward(s2, tokens=full, logits="all")["logits"]
    assert [oracle.argmax(r) for r in lg[63:]] == gen.tolist()


# ----------------------------------------------------------- size figures ---

def _golden(root, name):
    with open(f"{root}/tests/golden/{name}") as fh:
        return {r["quantity"]: float(r["value"]) for r in csv.DictReader(fh, delimiter="\t")}


def test_geometry_matches_the_pages(root):
    """Parameter count 33,118,977,024 (NInfer card, "Provenance and
    representation"); 61.7 GiB of bf16 (issue "A llama family on Metal:
    Nanbeige4.3-33B served from its bf16 release"); 16-bit KV of 208 KiB a
    token, 3.25 / 6.5 / 13 GiB at 16K / 32K / 64K (EXL3 card, "Which rung
    should I use?"); 44 executions and q_proj 3072 -> 6144 for the looped
    model (Nanbeige4.2-3B card, "About the architecture")."""
    gd = _golden(root, "geometry.tsv")
    g3 = config(3)
    assert g3.params() == gd["33b_stored_parameters"]
    assert round(g3.params() * 2 / 2 ** 30, 1) == gd["33b_release_gib"]
    assert g3.kv_bytes_per_position() == gd["kv_fp16_kib_per_token"] * 1024
    for k, n in (("kv_gib_at_16k", 16384), ("kv_gib_at_32k", 32768), ("kv_gib_at_64k", 65536)):
        assert g3.kv_bytes_per_position() * n / 2 ** 30 == gd[k]
    g4 = config(4)
    assert g4.n_exec == gd["looped_effective_layers"]
    assert (g4.hidden, g4.q_dim) == (gd["looped_q_proj_in"], gd["looped_q_proj_out"])
    # one 33B layer's projections are 1,181,745,152 bytes; its two norms add 28,672
    g2 = config(2)
    assert (g2.block_params() - 2 * g2.hidden) * 2 == 1181745152
    assert CONFIGS[5].params() == CONFIGS[3].params()


# ---------------------------------------------------------- comparators -----

def _rows_from_table(root):
    with open(f"{root}/tests/golden/misses_table.tsv") as fh:
        rows = list(csv.DictReader(fh, delimiter="\t"))
    V = 166912
    out = []
    for r in rows:
        a, b = int(r["hf_top1"]), int(r["engine_top1"])
        hf = np.zeros(V)
        en = np.zeros(V)
        hf[a], hf[b] = float(r["hf_a"]), float(r["hf_b"])
        en[a], en[b] = float(r["engine_a"]), float(r["engine_b"])
        out.append((int(r["position"]), a, b, hf, en))
    return out


def test_misses_table_ties_to_lower_id_and_near_ties(root):
    """Every printed choice follows 'largest logit, ties to the lower id', and
    each of the thirteen misses is a near-tie on its two contenders."""
    for pos, a, b, hf, en in _rows_from_table(root):
        assert parity.top1(hf) == a and parity.top1(en) == b
        assert parity.judge_row(hf, en, pos) == "near-tie"


def test_row_1370_third_contender_is_red(root):
    with open(f"{root}/tests/golden/row1370.tsv") as fh:
        third = {int(r["token_id"]): r for r in csv.DictReader(fh, delimiter="\t")}
    for pos, a, b, hf, en in _rows_from_table(root):
        if pos != 1370:
            continue
        hf[754] = float(third[754]["hf_bf16"])
        en[754] = float(third[754]["engine"])
        assert parity.judge_row(hf, en, pos) == "red"


def test_judge_planted_controls():
    base = np.zeros(16)
    base[3], base[5] = 10.0, 9.9375  # within one step (0.0625 at 8..16)
    other = base.copy()
    other[3], other[5] = 9.9375, 10.0
    assert parity.judge_row(base, other) == "near-tie"
    wide = other.copy()
    wide[5] = 10.25  # two steps above
    assert parity.judge_row(base, wide) == "red"
    third = other.copy()
    third[7] = 10.0
    assert parity.judge_row(base, third) == "red"
    for bad in (np.nan, np.inf, -np.inf):
        for side in (0, 1):
            x, y = base.copy(), base.copy()
            (x if side == 0 else y)[9] = bad  # away from the winner
            with pytest.raises(parity.Refused):
                parity.judge_row(x, y)
    both = np.array([np.nan, 0.0])
    with pytest.raises(parity.Refused):
        parity.judge_row(both, both.copy())  # same winner, still refused
    ninf = np.array([1.0, -np.inf])
    with pytest.raises(parity.Refused):
        parity.judge_row(ninf, ninf.copy())


def test_exact_comparator_reports_exactly_the_planted_row():
    g = np.random.default_rng(5)
    a = g.integers(0, 65536, size=(64, 100)).astype(np.uint16)
    for row in (0, 17, 63):
        b = a.copy()
        b[row, 42] ^= np.uint16(1)
        assert parity.differing_rows(a, b) == [row]
    assert parity.differing_rows(a, a.copy()) == []


def test_ulp_distance_and_kl():
    a = oracle.bf16([1.0, 38.25, -3.0])
    b = oracle.bf16([1.0 + 2.0 ** -7, 38.0, -3.0])
    assert parity.ulp_distance(a, b).tolist() == [1.0, 1.0, 0.0]
    x = np.random.default_rng(0).standard_normal((4, 50))
    assert parity.mean_kl(x, x) == 0.0
    assert parity.mean_kl(x, x + 3.0) < 1e-12  # shift invariance
    assert parity.mean_kl(x, x * 1.1) > 0


def test_block_rows_equals_block():
    """The sampled-rows composition of a block equals the block on every row
    it returns, bit for bit, and stores the same cache (tiny geometry, rows
    at positions 5.. over an earlier prefix)."""
    import synth
    from oracle.model import block_rows, mlp_half
    from synth.workloads import TensorIds
    g = config(1)
    W = HostWeights(g)
    w = {k: W(f"b1.{k}") for k in ("attn_norm", "q", "k", "v", "o", "mlp_norm", "gate", "up",
                                    "down")}
    T, n = 64, 40
    h = synth.normal_bf16(n * g.hidden, 3500, TensorIds.INPUT_ROWS).reshape(n, g.hidden)
    kc = synth.normal_bf16(T * g.kv_dim, 3500, TensorIds.K_CACHE).reshape(T, g.n_kv_heads,
                                                                          g.head_dim)
    vc = synth.normal_bf16(T * g.kv_dim, 3500, TensorIds.V_CACHE).reshape(T, g.n_kv_heads,
                                                                          g.head_dim)
    pos = np.arange(5, 5 + n, dtype=np.int32)
    k1, v1 = kc.copy(), vc.copy()
    out_all, mid_all = oracle.block(g, w, k1, v1, pos, h, want_mid=True)
    rows = np.array([0, 7, 22, 39])
    k2, v2 = kc.copy(), vc.copy()
    mid, out = block_rows(g, w, k2, v2, pos, h, rows)
    assert (mid == mid_all[rows]).all() and (out == out_all[rows]).all()
    assert (k1 == k2).all() and (v1 == v2).all()
    assert (mlp_half(g, w, mid_all) == out_all).all()
