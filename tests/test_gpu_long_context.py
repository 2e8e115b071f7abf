"""Two 33B-shaped sequences at long context (131,072-token prompts, each
prefilled in 2,048-row chunks into a position-major cache, then 64 greedy
decode rounds with both sequences batched into every step).

* Each reply must equal its solo run, bit for bit (the pull request "llama:
  Nanbeige4.3-33B on Metal, the bf16 release served as published", section
  "Measured": concurrent rows equal solo rows), and every greedy id must be
  the argmax of the GPU's own logits.
* The oracle cannot walk 131k rows through 52 blocks, and nothing the GPU
  computes is fed to it; its checks at this context are layer-local from
  synthetic states that reach both sides (tests/test_gpu_models.py: the last
  2,048-row chunk of the prompt over a 129,024-position cache of N(0,1) keys
  and values, and the last decode position), per kernel at 129k context
  (tests/test_gpu_kernels.py), and here the strict per-element gate where
  every key weighs the same: q projection zeroed, so each row averages the
  values of all its positions over a full 131,072-position N(0,1) cache, for
  a decode window and for a prompt chunk -- a missing or repeated key tile
  moves every output there."""
import numpy as np
import pytest

import oracle
from synth.workloads import config
from tests.gpu_util import half_report, log, u16
from tests.host_inputs import HostWeights

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

KINDS = ("attn_norm", "q", "k", "v", "o", "mlp_norm", "gate", "up", "down")


def test_two_long_sequences_equal_solo():
    import dense_gqa_llama_amd as L
    from synth import device as sd
    g = config(5)
    P, C, S = g.prompt_len, g.chunk_rows, g.decode_steps
    log(f"config 5: two sequences of {P} prompt tokens in {P // C} chunks, {S} decode rounds")
    w = sd.weights(g)
    torch.cuda.synchronize()
    model = L.Model(g, w, max_positions=P + S, max_chunk_rows=C, max_window_rows=16, max_seqs=2)
    seqs = [model.new_sequence(P + S) for _ in g.prompt_seeds]
    prompts = [sd.tokens(P, seed, 0, g.vocab) for seed in g.prompt_seeds]

    solo_tok, solo_bits, first = [], [], []
    for i, seq in enumerate(seqs):
        for c in range(P // C):
            last = c == P // C - 1
            out = model.prefill(seq, tokens=prompts[i][c * C:(c + 1) * C], want_logits=last)
            if c % 8 == 7 or last:
                torch.cuda.synchronize()
                log(f"sequence {i}: chunk {c + 1}/{P // C} done")
        assert int(out["next"].item()) == oracle.argmax(u16(out["logits"])[0])
        first.append(int(out["next"].item()))
        model.check_finite()
        # solo greedy decode
        tok = torch.tensor([first[i]], dtype=torch.int32, device="cuda")
        toks_i, bits_i = [first[i]], []
        for step in range(S):
            o = model.decode([seq], tokens=tok)
            bits_i.append(u16(o["logits"])[0])
            tok = o["next"]
            toks_i.append(int(tok.item()))
            assert toks_i[-1] == oracle.argmax(bits_i[-1])
        model.check_finite()
        solo_tok.append(toks_i)
        solo_bits.append(np.stack(bits_i))
        log(f"sequence {i} solo greedy: {toks_i[:8]} ...")

    # batched: both sequences in every step, from the same prompt caches
    for seq in seqs:
        seq.truncate(P)
    tok = torch.tensor(first, dtype=torch.int32, device="cuda")
    bat_tok = [[first[0]], [first[1]]]
    bat_bits = [[], []]
    for step in range(S):
        o = model.decode(seqs, tokens=tok)
        b = u16(o["logits"])
        for i in range(2):
            bat_bits[i].append(b[i])
        tok = o["next"]
        nt = tok.cpu().tolist()
        for i in range(2):
            bat_tok[i].append(nt[i])
    model.check_finite()
    for i in range(2):
        assert bat_tok[i] == solo_tok[i], f"sequence {i}: batched tokens differ from solo"
        assert np.array_equal(np.stack(bat_bits[i]), solo_bits[i]), \
            f"sequence {i}: batched logits differ from solo"
    log("batched replies equal the solo runs bit for bit")


# ------------------------------------------- uniform attention, full cache ----

def test_uniform_attention_over_full_cache():
    """One 33B-shaped layer with q_proj zeroed: every score is 0, so each row
    averages the values of all its positions.  The cache holds N(0,1) keys and
    values at 131,072 positions; a 16-row decode window after them and a
    64-row prompt chunk ending at the same place are checked per element
    against the oracle (attention half, strict gate)."""
    import dataclasses

    import synth
    from synth import device as sd
    from synth.workloads import TensorIds
    from tests.gpu_util import HalfRunner
    g = dataclasses.replace(config(2), name="33b-layer-long")
    T = config(5).prompt_len
    kvd = g.kv_dim
    cap = T + 16
    log(f"uniform attention: cache of {T} positions")
    kc = np.zeros((cap, g.n_kv_heads, g.head_dim), dtype=np.uint16)
    vc = np.zeros_like(kc)
    kc[:T] = synth.normal_bf16(T * kvd, 3005, TensorIds.K_CACHE).reshape(T, g.n_kv_heads, g.head_dim)
    vc[:T] = synth.normal_bf16(T * kvd, 3005, TensorIds.V_CACHE).reshape(T, g.n_kv_heads, g.head_dim)
    rows = synth.normal_bf16(64 * g.hidden, 3105, TensorIds.INPUT_ROWS).reshape(64, g.hidden)
    W = HostWeights(g)
    blk = {k: W(f"b0.{k}") for k in KINDS}
    blk["q"] = np.zeros_like(blk["q"])
    dev = sd.weights(g)
    dev["b0.q"] = torch.zeros_like(dev["b0.q"])
    runner = HalfRunner(g, dev, cap, 64)

    # a decode window of 16 rows at T .. T+15
    log("uniform attention: decode window at the end of the cache")
    got, _ = runner.run(0, rows[:16], kc, vc, T, "attn", chunk=False)
    kco, vco = kc.copy(), vc.copy()
    _, ref = oracle.block(g, blk, kco, vco, np.arange(T, T + 16, dtype=np.int32), rows[:16],
                          want_mid=True)
    assert half_report("uniform attention, decode window", got, ref, rows[:16]) >= 0.999

    # a 64-row prompt chunk ending at T (positions T-64 .. T-1)
    log("uniform attention: prompt chunk ending at the end of the cache")
    got, _ = runner.run(0, rows, kc, vc, T - 64, "attn", chunk=True)
    kco, vco = kc.copy(), vc.copy()
    _, ref = oracle.block(g, blk, kco, vco, np.arange(T - 64, T, dtype=np.int32), rows,
                          want_mid=True)
    assert half_report("uniform attention, prompt chunk", got, ref, rows) >= 0.999
