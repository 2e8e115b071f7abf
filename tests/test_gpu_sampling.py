"""Seeded sampling on the GPU (`llama_sample`) against the oracle's sampler,
on the same bf16 logit rows and the same uniforms.  The GPU forms the
weights and the draw in fp32, the oracle in binary64, so a token may differ
only where the oracle's decision margin (the distance between a top-p or draw
threshold and the running weight it was compared with, relative to the sum)
is below 1e-5; anywhere else they must be equal.  Equal seeds must give equal
tokens (the pull request's "seeded sampling" check), and a sampled greedy-free
run of the tiny model must repeat exactly."""
import numpy as np
import pytest

import oracle
import synth
from synth.workloads import TensorIds, config
from tests.gpu_util import gpu_model, log, to_dev, u16
from tests.host_inputs import prompt

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

MARGIN = 1e-5
PARAMS = [(0.6, 20, 0.95), (1.0, 64, 1.0), (0.3, 1, 0.5), (2.0, 40, 0.5), (1.0, 5, 0.3)]


def _judge(rows, u, got, T, K, P, tag):
    misses, near = [], 0
    for r in range(rows.shape[0]):
        want, margin = oracle.sample(rows[r], T, K, P, float(u[r]))
        if got[r] != want:
            if margin < MARGIN:
                near += 1
            else:
                misses.append((r, int(got[r]), want, margin))
    log(f"{tag} T={T} top_k={K} top_p={P}: {rows.shape[0]} rows, {near} near-threshold "
        f"differences, misses {misses[:4]}")
    assert not misses


@pytest.mark.parametrize("V", [4096, 166912])
def test_sampling_matches_oracle(V):
    g = config(1) if V == 4096 else config(3)
    import dataclasses
    g = dataclasses.replace(g, n_blocks=1, vocab=V)
    model = gpu_model(g, 16, max_chunk_rows=16, max_seqs=1)
    n = 64
    rows = synth.normal_bf16(n * V, 4100 + V % 7, TensorIds.SAMPLE_LOGITS, 0.0, 3.0).reshape(n, V)
    # a few rows with ties at the top
    rows[3, [11, 500, 900]] = oracle.bf16(np.array([40.0]))[0]
    rows[4, :] = oracle.bf16(np.zeros(1))[0]
    dl = to_dev(rows)
    for i, (T, K, P) in enumerate(PARAMS):
        u = synth.uniform_f32(n, 4200 + i, TensorIds.SAMPLE_UNIFORM)
        got = model.sample(dl, to_dev(u), T, K, P).cpu().numpy()
        _judge(rows, u, got, T, K, P, f"V={V}")
    model.check_finite()


def test_sampling_is_seeded_and_refuses_nonfinite_rows():
    import dataclasses

    import dense_gqa_llama_amd as L
    g = dataclasses.replace(config(1), n_blocks=1)
    model = gpu_model(g, 16, max_chunk_rows=16, max_seqs=1)
    V, n = g.vocab, 32
    rows = synth.normal_bf16(n * V, 4300, TensorIds.SAMPLE_LOGITS, 0.0, 2.0).reshape(n, V)
    dl = to_dev(rows)
    from synth import device as sd
    a = model.sample(dl, sd.uniform(n, 4301, TensorIds.SAMPLE_UNIFORM), 1.0, 40, 0.95)
    b = model.sample(dl, sd.uniform(n, 4301, TensorIds.SAMPLE_UNIFORM), 1.0, 40, 0.95)
    c = model.sample(dl, sd.uniform(n, 4302, TensorIds.SAMPLE_UNIFORM), 1.0, 40, 0.95)
    assert torch.equal(a, b)
    assert not torch.equal(a, c)
    bad = rows.copy()
    bad[5, 77] = 0x7FC0
    bad[9, 4000] = 0xFF80
    got = model.sample(to_dev(bad), sd.uniform(n, 4301, TensorIds.SAMPLE_UNIFORM), 1.0, 40,
                       0.95).cpu().numpy()
    assert got[5] == -1 and got[9] == -1
    assert (np.delete(got, [5, 9]) == np.delete(a.cpu().numpy(), [5, 9])).all()
    with pytest.raises(L.LlamaError):
        model.check_finite()
    model.check_finite()  # the flag was cleared


def test_sampled_decode_repeats_and_follows_the_oracle_sampler():
    """Free-running sampled decode of the tiny model (temperature 0.6, top_k 20,
    top_p 0.95, one uniform per step from the seed): two runs give the same
    tokens, and every token is the oracle sampler's draw from the GPU's own
    logits of that step (up to near-threshold differences)."""
    g = config(1)
    p = prompt(g, n=g.prompt_len)
    T, K, P = 0.6, 20, 0.95
    steps = 16
    u = synth.uniform_f32(steps, 4400, TensorIds.SAMPLE_UNIFORM)

    def run():
        model = gpu_model(g, 96, max_chunk_rows=64, max_seqs=1)
        s = model.new_sequence(96)
        o = model.prefill(s, tokens=to_dev(p))
        lg = o["logits"]
        toks, rows = [], []
        for i in range(steps):
            t = model.sample(lg, to_dev(u[i:i + 1]), T, K, P)
            toks.append(int(t.item()))
            rows.append(u16(lg)[0])
            lg = model.decode([s], tokens=t)["logits"]
        return toks, np.stack(rows)

    t1, r1 = run()
    t2, r2 = run()
    assert t1 == t2 and np.array_equal(r1, r2)
    _judge(r1, u, np.array(t1), T, K, P, "tiny sampled decode")
    log(f"sampled tokens {t1}")
