"""Drafted greedy decoding on the GPU (`llama_draft_round`) equals plain
greedy decoding, token for token and cache bit for bit (issue "A llama family
on Metal: Nanbeige4.3-33B served from its bf16 release", follow-ups: a
smaller Llama on the same tokenizer drafting with replies unchanged; pull
request "llama: Nanbeige4.3-33B on Metal, the bf16 release served as
published", reply "Drafting": drafted greedy equals plain greedy).

The target verifies each round's proposals in one window, and windows equal
one-row steps bit for bit, so the reply cannot depend on the draft.  Three
drafts on the tiny workload cover the acceptance range: the target's own
weights (every proposal taken), a model of another seed (almost none taken)
and the target with a quarter of its lm_head rows replaced (some taken);
rounds of 1 to 15 proposals."""
import dataclasses

import numpy as np
import pytest

from synth.workloads import TensorIds, config
from tests.gpu_util import gpu_model, log, to_dev, u16
from tests.host_inputs import prompt

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

CAP = 160
N_TOKENS = 48
SCHEDULE = (3, 7, 15, 1, 5, 11)


def _plain(model, p, n):
    s = model.new_sequence(CAP)
    tok = model.prefill(s, tokens=to_dev(p), want_logits=False)["next"]
    toks = [tok]
    for _ in range(n - 1):
        tok = model.decode([s], tokens=tok, want_logits=False)["next"]
        toks.append(tok)
    return torch.cat(toks).cpu().numpy().tolist(), s


def _drafted(target, draft, p, n):
    ts, ds = target.new_sequence(CAP), draft.new_sequence(CAP)
    last = target.prefill(ts, tokens=to_dev(p), want_logits=False)["next"]
    draft.prefill(ds, tokens=to_dev(p), want_logits=False)
    out, taken, i = [int(last.item())], [], 0
    while len(out) < n:
        k = SCHEDULE[i % len(SCHEDULE)]
        i += 1
        toks, m = target.draft_round(ts, draft, ds, k, last)
        assert 1 <= m <= k + 1
        assert ts.length == ds.length
        out += toks[:m].cpu().numpy().tolist()
        taken.append((m - 1, k))
        last = toks[m - 1:m].clone()
    return out, ts, taken


def _draft_weights(kind, g, w):
    from synth import device as sd
    if kind == "self":
        return w
    if kind == "other":
        return sd.weights(dataclasses.replace(g, weight_seed=g.weight_seed + 100))
    # a quarter of the lm_head rows from another stream
    d = dict(w)
    head = w["lm_head"].clone()
    q = g.vocab // 4
    head[:q] = sd.normal((q, g.hidden), g.weight_seed, TensorIds.SAMPLE_LOGITS, 0.0, 0.02)
    d["lm_head"] = head
    return d


@pytest.mark.parametrize("kind", ["self", "other", "lm_head_quarter"])
def test_drafted_greedy_equals_plain_greedy(kind):
    from synth import device as sd
    g = config(1)
    w = sd.weights(g)
    target = gpu_model(g, CAP, max_chunk_rows=64, max_window_rows=16, max_seqs=1, weights=w)
    draft = gpu_model(g, CAP, max_chunk_rows=64, max_window_rows=1, max_seqs=1,
                      weights=_draft_weights(kind, g, w))
    p = prompt(g, n=g.prompt_len)
    want, ps = _plain(target, p, N_TOKENS)
    got, ts, taken = _drafted(target, draft, p, N_TOKENS)
    target.check_finite()
    draft.check_finite()
    rate = sum(a for a, _ in taken) / max(1, sum(k for _, k in taken))
    log(f"draft {kind}: {len(taken)} rounds, proposals taken {rate:.2f}, (taken, proposed) {taken}")
    assert got[:N_TOKENS] == want
    # the target's cache, over the positions both runs hold, is the plain run's
    n = min(ts.length, ps.length)
    assert n >= len(p) + N_TOKENS - 1
    assert np.array_equal(u16(ts.view())[:, :, :n], u16(ps.view())[:, :, :n])
    if kind == "self":
        assert all(a == k for a, k in taken)
    if kind == "lm_head_quarter":
        assert 0 < rate < 1


def _plain_sampled(model, p, n, u, T, K, P):
    s = model.new_sequence(CAP)
    lg = model.prefill(s, tokens=to_dev(p))["logits"]
    toks = []
    for i in range(n):
        t = model.sample(lg, u[i:i + 1], T, K, P)
        toks.append(int(t.item()))
        if i + 1 < n:
            lg = model.decode([s], tokens=t)["logits"]
    return toks, s


def _drafted_sampled(target, draft, p, n, u, T, K, P):
    ts, ds = target.new_sequence(CAP), draft.new_sequence(CAP)
    lg = target.prefill(ts, tokens=to_dev(p))["logits"]
    draft.prefill(ds, tokens=to_dev(p), want_logits=False)
    last = target.sample(lg, u[0:1], T, K, P)
    out, taken, i = [int(last.item())], [], 0
    while len(out) < n:
        k = SCHEDULE[i % len(SCHEDULE)]
        i += 1
        j = len(out)  # the round's draws take uniforms j .. j + k
        toks, m = target.draft_round_sampled(ts, draft, ds, k, last, u[j:j + k + 1], T, K, P)
        assert ts.length == ds.length
        out += toks[:m].cpu().numpy().tolist()
        taken.append((m - 1, k))
        last = toks[m - 1:m].clone()
    return out, ts, taken


@pytest.mark.parametrize("kind", ["self", "lm_head_quarter"])
def test_drafted_sampling_equals_plain_sampling(kind):
    """Seeded sampling by drafted rounds (the target draws each window row's
    token with that position's uniform and keeps matching proposals) equals
    seeded sampling by plain steps with the same uniforms."""
    from synth import device as sd
    g = config(1)
    w = sd.weights(g)
    target = gpu_model(g, CAP, max_chunk_rows=64, max_window_rows=16, max_seqs=1, weights=w)
    draft = gpu_model(g, CAP, max_chunk_rows=64, max_window_rows=1, max_seqs=1,
                      weights=_draft_weights(kind, g, w))
    p = prompt(g, n=g.prompt_len)
    T, K, P = 0.6, 20, 0.95
    u = sd.uniform(N_TOKENS + 16, 4800, TensorIds.SAMPLE_UNIFORM)
    want, ps = _plain_sampled(target, p, N_TOKENS, u, T, K, P)
    got, ts, taken = _drafted_sampled(target, draft, p, N_TOKENS, u, T, K, P)
    target.check_finite()
    draft.check_finite()
    rate = sum(a for a, _ in taken) / max(1, sum(k for _, k in taken))
    log(f"sampled, draft {kind}: {len(taken)} rounds, proposals taken {rate:.2f}, {taken}")
    assert got[:N_TOKENS] == want
    n = min(ts.length, ps.length)
    assert n >= len(p) + N_TOKENS - 1
    assert np.array_equal(u16(ts.view())[:, :, :n], u16(ps.view())[:, :, :n])
    assert 0 < rate < 1
