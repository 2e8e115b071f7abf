"""Teacher-forced greedy agreement at the pages' scale (pull request "llama:
Nanbeige4.3-33B on Metal, the bf16 release served as published", section
"Measured": 1,500 teacher-forced positions; reply "Teacher-forced misses":
every miss listed with its contenders, a near-tie when the two lie within one
bf16 step on both sides).

Six seeded 256-token prompts on the tiny workload (1,536 positions) and four
on a small looped geometry (3 blocks x 2 loops, 1,024 positions), each
position's logits from the GPU's prompt path (one chunk per prompt) and from
its decode path (sixteen 16-row windows per prompt), against the oracle.

On random-init weights the top two logits of a row are often within a
rounding-scale distance of each other, so the oracle itself changes its
greedy choice on ~1.5% of rows when one input row is moved by one bf16 step,
and an ordinary float32 implementation of the same spec (tests/fp32_ref.py)
differs from the binary64 oracle on about as many.  The gate is therefore
relative to those two in-spec references: with lam the larger of their miss
counts, the GPU may miss on at most lam + 3 sqrt(lam) + 2 rows (the upper end
of a Poisson count of that mean), and likewise for red rows (contenders
further apart than one step, or a third contender within it); and it must
agree with the oracle on at least as many rows as the nudged oracle does.
The absolute figure (the pages' 99%) is printed beside it.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from oracle.model import OracleModel
from synth.workloads import config
from tests import fp32_ref, parity
from tests.gpu_util import gpu_model, log, to_dev, u16
from tests.host_inputs import HostWeights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

ROWS = 256


def _geometry(name):
    if name == "tiny":
        return config(1), 6
    return dataclasses.replace(config(1), name="tiny-looped", n_blocks=3, n_loops=2, hidden=256,
                               n_q_heads=4, n_kv_heads=2, head_dim=128, ffn=512,
                               vocab=512), 4


def _oracle_rows(g, W, prompts):
    """The oracle's logits of every prompt row, and those of the oracle whose
    embedding row of each prompt's first token is moved by one bf16 step."""
    ref64, refb, nb = [], [], []
    for toks in prompts:
        om = OracleModel(g, W)
        r = om.forward(om.new_sequence(ROWS), tokens=toks, logits="all")

        class Nudged:
            def __call__(self, name, toks=toks):
                a = W(name)
                if name == "embed":
                    a = a.copy()
                    a[toks[0], :] += np.uint16(1)
                return a
        on = OracleModel(g, Nudged())
        rn = on.forward(on.new_sequence(ROWS), tokens=toks, logits="all")
        ref64.append(r["logits64"])
        refb.append(r["logits"])
        nb.append(rn["logits"])
    return np.concatenate(ref64), np.concatenate(refb), np.concatenate(nb)


@pytest.mark.parametrize("name", ["tiny", "looped"])
def test_teacher_forced_agreement(name):
    import synth
    g, n_prompts = _geometry(name)
    W = HostWeights(g)
    prompts = [synth.tokens(ROWS, 7100 + i, 0, g.vocab) for i in range(n_prompts)]
    ref64, refb, nudgedb = _oracle_rows(g, W, prompts)
    model = gpu_model(g, ROWS, max_chunk_rows=ROWS, max_window_rows=16, max_seqs=1)
    paths = {"prompt": ([], []), "decode": ([], [])}
    for toks in prompts:
        s = model.new_sequence(ROWS)
        out = model.prefill(s, tokens=to_dev(toks), all_rows=True)
        paths["prompt"][0].append(out["logits32"].cpu().numpy())
        paths["prompt"][1].append(u16(out["logits"]))
        assert out["next"].cpu().numpy().tolist() == [oracle.argmax(x) for x in u16(out["logits"])]
        s = model.new_sequence(ROWS)
        for w0 in range(0, ROWS, 16):
            out = model.decode([s], tokens=to_dev(toks[w0:w0 + 16]), rows=16)
            paths["decode"][0].append(out["logits32"].cpu().numpy())
            paths["decode"][1].append(u16(out["logits"]))
    model.check_finite()
    n = ref64.shape[0]
    ncounts, ndetail = parity.judge(parity.bf16_bits_to_f64(refb), parity.bf16_bits_to_f64(nudgedb))
    fb = np.concatenate([fp32_ref.forward(g, W, toks)[1] for toks in prompts])
    fcounts, fdetail = parity.judge(parity.bf16_bits_to_f64(refb), parity.bf16_bits_to_f64(fb))
    log(f"{name}: the oracle nudged by one step on the first row of each prompt: {ncounts} "
        f"({100 * ncounts['equal'] / n:.2f}% equal over {n} positions); the float32 "
        f"implementation: {fcounts} ({100 * fcounts['equal'] / n:.2f}% equal)")
    lam = max(n - ncounts["equal"], n - fcounts["equal"])
    lam_red = max(ncounts["red"], fcounts["red"])
    bound = lam + 3.0 * np.sqrt(lam) + 2
    bound_red = lam_red + 3.0 * np.sqrt(lam_red) + 2
    for path, (l32, lb) in paths.items():
        l32, lb = np.concatenate(l32), np.concatenate(lb)
        counts, detail = parity.judge(parity.bf16_bits_to_f64(refb), parity.bf16_bits_to_f64(lb))
        miss = n - counts["equal"]
        err = float(np.abs(l32 - ref64).max())
        kl = parity.mean_kl(ref64, l32)
        log(f"{name} {path} path, {n} teacher-forced positions: {counts} "
            f"({100 * counts['equal'] / n:.2f}% equal; the pages' bar is 99%), logits max|d| "
            f"{err:.3e}, KL {kl:.2e}; misses {detail[:12]}; bounds {bound:.1f} misses, "
            f"{bound_red:.1f} red")
        assert miss <= bound, (path, counts, ncounts, fcounts)
        # and at least as often as the oracle agrees with itself when one
        # input row moves by a step, on the same rows
        assert counts["equal"] >= ncounts["equal"], (path, counts, ncounts)
        assert counts["red"] <= bound_red, (path, counts, ncounts, fcounts)
        assert kl <= 1e-3
