"""Shared rounds and resumed prompts on the GPU, bit for bit (the pull request
"llama: Nanbeige4.3-33B on Metal, the bf16 release served as published",
sections "How" and "Measured": concurrent streams each equal their solo run;
a prompt resumed from a kept cache prefix equals the fresh prompt).

* Twelve sequences at different positions share every decode round (one-row
  steps and four-row windows); each sequence's logits equal its solo run.
* A prompt resumed at a kept length (the cache truncated, the rest prefilled
  as a new chunk) equals the prompt prefilled fresh in one chunk, rows and
  cache; so does any split of a prompt into chunks.  Prompt rows are
  computed independently of the chunk's size (the projections' k order and
  attention's key tiles are anchored at absolute positions)."""
import numpy as np
import pytest

from synth.workloads import config
from tests import parity
from tests.gpu_util import gpu_model, log, to_dev, u16
from tests.host_inputs import prompt

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

NSEQ = 12


def _prompts(g):
    base = prompt(g, n=g.prompt_len)
    # twelve prompts of different lengths and contents
    return [np.roll(base, 5 * i)[:20 + 3 * i].copy() for i in range(NSEQ)]


def test_twelve_streams_equal_solo():
    g = config(1)
    cap = 96
    model = gpu_model(g, cap, max_chunk_rows=64, max_seqs=NSEQ)
    ps = _prompts(g)
    steps, win = 6, 4
    # teacher-forced window tokens, the same for solo and shared rounds
    wtok = [np.roll(p, 1)[:win].astype(np.int32) for p in ps]

    def run(seqs, idx):
        """Prefill each of `idx`, then `steps` greedy rounds and one window
        round over all of them together; returns per-sequence logit rows."""
        firsts = []
        for s, i in zip(seqs, idx):
            firsts.append(model.prefill(s, tokens=to_dev(ps[i]), want_logits=False)["next"])
        nxt = torch.cat(firsts)
        out = {i: [] for i in idx}
        for _ in range(steps):
            o = model.decode(seqs, tokens=nxt)
            lg = u16(o["logits"])
            for k, i in enumerate(idx):
                out[i].append(lg[k:k + 1])
            nxt = o["next"]
        t = to_dev(np.concatenate([wtok[i] for i in idx]))
        o = model.decode(seqs, tokens=t, rows=win)
        lg = u16(o["logits"])
        for k, i in enumerate(idx):
            out[i].append(lg[k * win:(k + 1) * win])
        return {i: np.concatenate(v) for i, v in out.items()}

    solo = {}
    for i in range(NSEQ):
        solo.update(run([model.new_sequence(cap)], [i]))
    shared = run([model.new_sequence(cap) for _ in range(NSEQ)], list(range(NSEQ)))
    model.check_finite()
    bad = {i: parity.differing_rows(shared[i], solo[i]) for i in range(NSEQ)}
    log(f"twelve shared streams vs solo: differing rows {bad}")
    assert all(v == [] for v in bad.values())


def test_resumed_prompt_equals_fresh_tiny():
    g = config(1)
    cap = 128
    model = gpu_model(g, cap, max_chunk_rows=128, max_seqs=1)
    p = prompt(g, n=g.prompt_len)
    p = np.concatenate([p, p[::-1]])[:100].copy()
    fresh = model.new_sequence(cap)
    of = model.prefill(fresh, tokens=to_dev(p), all_rows=True)
    lf = u16(of["logits"])
    cf = u16(fresh.view())[:, :, :100]
    # resumed: a different continuation first, then truncated to 60 and resumed
    res = model.new_sequence(cap)
    model.prefill(res, tokens=to_dev(p[:60]), all_rows=True)
    model.prefill(res, tokens=to_dev(p[::-1][:40].copy()), all_rows=True)
    res.truncate(60)
    orr = model.prefill(res, tokens=to_dev(p[60:]), all_rows=True)
    assert np.array_equal(u16(orr["logits"]), lf[60:])
    assert np.array_equal(u16(res.view())[:, :, :100], cf)
    # any chunk split
    spl = model.new_sequence(cap)
    rows = []
    for a, b in ((0, 37), (37, 38), (38, 100)):
        rows.append(u16(model.prefill(spl, tokens=to_dev(p[a:b]), all_rows=True)["logits"]))
    assert np.array_equal(np.concatenate(rows), lf)
    assert np.array_equal(u16(spl.view())[:, :, :100], cf)
    # and the decode steps after it
    t = of["next"][-1:]
    a = model.decode([fresh], tokens=t)
    b = model.decode([res], tokens=t)
    assert np.array_equal(u16(a["logits"]), u16(b["logits"]))
    log("resumed and split prompts equal the fresh prompt bit for bit")


def test_resumed_prompt_equals_fresh_33b_layer():
    """The same on one 33B-shaped layer (head dim 128, 256x256 GEMM tiles,
    ragged chunk rows), through hidden rows."""
    import synth
    from synth.workloads import TensorIds
    g = config(2)
    cap = 320
    model = gpu_model(g, cap, max_chunk_rows=320, max_seqs=1)
    rows = synth.normal_bf16(300 * g.hidden, 3110, TensorIds.INPUT_ROWS).reshape(300, g.hidden)
    fresh = model.new_sequence(cap)
    hf = u16(model.prefill(fresh, hidden=to_dev(rows), want_hidden=True)["hidden"])
    cf = u16(fresh.view())[:, :, :300]
    spl = model.new_sequence(cap)
    parts = []
    for a, b in ((0, 137), (137, 300)):
        parts.append(u16(model.prefill(spl, hidden=to_dev(rows[a:b]), want_hidden=True)["hidden"]))
    assert np.array_equal(np.concatenate(parts), hf)
    assert np.array_equal(u16(spl.view())[:, :, :300], cf)
    spl.truncate(211)
    hr = u16(model.prefill(spl, hidden=to_dev(rows[211:]), want_hidden=True)["hidden"])
    assert np.array_equal(hr, hf[211:])
    log("33B layer: split and resumed chunks equal the single chunk bit for bit")


def test_chunk_sizes_select_other_tiles_same_bits_33b_layer():
    """Chunks of 2,048, 1,500, 1,048 and 548 rows of one 33B-shaped layer take
    different projection tilings (256 x 256 and 256 x 224 tiles on the
    alternating schedule, the q/k/v projection split at the q segment's end,
    256 x 128 and 128 x 128 tiles); every row still equals the single
    2,048-row chunk's, and so does the cache."""
    import synth
    from synth.workloads import TensorIds
    g = config(2)
    n = 2048
    model = gpu_model(g, n, max_chunk_rows=n, max_seqs=1)
    rows = synth.normal_bf16(n * g.hidden, 3111, TensorIds.INPUT_ROWS).reshape(n, g.hidden)
    fresh = model.new_sequence(n)
    hf = u16(model.prefill(fresh, hidden=to_dev(rows), want_hidden=True)["hidden"])
    cf = u16(fresh.view())[:, :, :n]
    spl = model.new_sequence(n)
    parts = []
    for a, b in ((0, 1500), (1500, n)):
        parts.append(u16(model.prefill(spl, hidden=to_dev(rows[a:b]), want_hidden=True)["hidden"]))
    assert np.array_equal(np.concatenate(parts), hf)
    assert np.array_equal(u16(spl.view())[:, :, :n], cf)
    spl.truncate(1000)
    hr = u16(model.prefill(spl, hidden=to_dev(rows[1000:]), want_hidden=True)["hidden"])
    assert np.array_equal(hr, hf[1000:])
    assert np.array_equal(u16(spl.view())[:, :, :n], cf)
    log("33B layer: chunks of 2048 / 1500 / 548 / 1048 rows equal the single chunk bit for bit")
