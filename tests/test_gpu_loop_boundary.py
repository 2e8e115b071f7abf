"""GPU parity of the loop boundary of a looped model (card "Nanbeige4.2-3B --
MLX NVFP4", section "About the architecture": the block stack runs twice over
the same weights, each execution with its own cache, and the final norm is
applied at the end of every loop, its output replacing the residual).

1. Identity blocks: one block run twice with o_proj and down_proj zeroed, so
   each block leaves the residual exactly as it came (bf16(h + 0) = h).  The
   residual captured after the first execution of loop 2 is then the GPU's
   boundary-normed row itself, compared bit for bit with the oracle's
   RMSNorm of the embedding rows, for a prompt chunk, a decode window of four
   rows (the last loop's norm fused into lm_head) and one of eight rows
   (every norm by the norm kernel).
2. A small looped model (3 blocks x 2 loops, hidden 256, heads of 128) end to
   end: a prompt chunk and teacher-forced decode steps against the oracle
   with the logit gates (fp32 sums within 0.05, mean KL <= 1e-3, every top-1
   difference a near-tie, at most max(1, 1%) of rows), and every execution's
   halves layer-local from the oracle's own inputs -- the first execution of
   loop 2 from the oracle's boundary-normed rows -- held by
   tests/gpu_util.HalfGates.
"""
import dataclasses

import numpy as np
import pytest

import oracle
from oracle.model import OracleModel
from synth.workloads import config
from tests import parity
from tests.gpu_util import (HalfGates, HalfRunner, exec_inputs, f32_halves, gpu_model, log, to_dev,
                            u16)
from tests.host_inputs import HostWeights, prompt

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def looped_geometry(n_blocks):
    return dataclasses.replace(config(1), name="tiny-looped", n_blocks=n_blocks, n_loops=2,
                               hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=128, ffn=512,
                               vocab=512)


class ZeroedHost:
    """Host weights with o_proj and down_proj of every block zeroed."""

    def __init__(self, g):
        self.W = HostWeights(g)

    def __call__(self, name):
        a = self.W(name)
        if name.endswith(".o") or name.endswith(".down"):
            return np.zeros_like(a)
        return a


@pytest.mark.parametrize("mode", ["chunk", "window4", "window8"])
def test_boundary_norm_identity_blocks(mode):
    from synth import device as sd
    g = looped_geometry(1)
    Wz = ZeroedHost(g)
    dev = sd.weights(g)
    dev["b0.o"] = torch.zeros_like(dev["b0.o"])
    dev["b0.down"] = torch.zeros_like(dev["b0.down"])
    toks = prompt(g, n=20)
    model = gpu_model(g, 32, max_chunk_rows=16, max_window_rows=8, max_seqs=1, weights=dev)
    seq = model.new_sequence(32)
    om = OracleModel(g, Wz)
    oseq = om.new_sequence(32)
    if mode == "chunk":
        pre, rows = 0, 12
    else:
        pre, rows = 8, int(mode[len("window"):])
    if pre:  # a prompt first, so the window's rows attend to earlier slots
        model.prefill(seq, tokens=to_dev(toks[:pre]), want_logits=False)
        om.forward(oseq, tokens=toks[:pre], logits=None)
    t = toks[pre:pre + rows]
    model.set_capture(rows)
    if mode == "chunk":
        out = model.prefill(seq, tokens=to_dev(t), all_rows=True)
    else:
        out = model.decode([seq], tokens=to_dev(t), rows=rows)
    cap = u16(model.capture).copy()
    model.set_capture(0)
    r = om.forward(oseq, tokens=t, logits="all", capture=True)
    emb = oracle.embed(Wz("embed"), t)
    normed = oracle.rmsnorm(emb, Wz("final_norm"), g.rms_eps)
    # loop 1 leaves the embedding rows as they were; the boundary norm then
    # replaces them, and loop 2 leaves that as it is
    assert np.array_equal(cap[0, 0], emb) and np.array_equal(cap[0, 1], emb)
    assert np.array_equal(r["capture"][1][0], normed)  # the oracle agrees with itself
    diff = parity.differing_rows(cap[1, 0], normed)
    log(f"loop boundary ({mode}, {rows} rows): GPU boundary-normed rows differing from the "
        f"oracle's: {diff}")
    assert diff == []
    assert np.array_equal(cap[1, 1], normed)
    l32 = out["logits32"].cpu().numpy()
    err = float(np.abs(l32 - r["logits64"]).max())
    exact = float((u16(out["logits"]) == r["logits"]).mean())
    log(f"loop boundary ({mode}): logits max|d| {err:.2e}, bf16 exact {exact:.5f}")
    assert err <= 1e-3 and exact >= 0.999
    assert out["next"].cpu().numpy().tolist() == [oracle.argmax(x) for x in u16(out["logits"])]


@pytest.fixture(scope="module")
def looped():
    g = looped_geometry(3)
    W = HostWeights(g)
    om = OracleModel(g, W)
    seq = om.new_sequence(96)
    toks = prompt(g, n=64)
    r = om.forward(seq, tokens=toks, logits="all", capture=True)
    steps = [dict(tokens=toks, pos0=0, caps=r["capture"])]
    logits64, logits = [r["logits64"]], [r["logits"]]
    gen = [int(r["tokens"][-1])]
    for _ in range(15):
        pos0 = seq.length
        r = om.forward(seq, tokens=np.array([gen[-1]], dtype=np.int32), logits="all", capture=True)
        steps.append(dict(tokens=np.array([gen[-1]], dtype=np.int32), pos0=pos0, caps=r["capture"]))
        logits64.append(r["logits64"])
        logits.append(r["logits"])
        gen.append(int(r["tokens"][-1]))
    log("looped 3x2: oracle prompt 64 + 15 steps")
    return dict(g=g, W=W, toks=toks, gen=np.array(gen, dtype=np.int32), steps=steps,
                logits64=np.concatenate(logits64), logits=np.concatenate(logits),
                kc=seq.kc, vc=seq.vc)


def test_looped_model_end_to_end(looped):
    g = looped["g"]
    model = gpu_model(g, 96, max_chunk_rows=64, max_seqs=1)
    seq = model.new_sequence(96)
    out = model.prefill(seq, tokens=to_dev(looped["toks"]), all_rows=True)
    l32, lbf, nxt = [out["logits32"].cpu().numpy()], [u16(out["logits"])], [out["next"].cpu().numpy()]
    for t in looped["gen"][:-1]:
        out = model.decode([seq], tokens=to_dev(np.array([t], dtype=np.int32)))
        l32.append(out["logits32"].cpu().numpy())
        lbf.append(u16(out["logits"]))
        nxt.append(out["next"].cpu().numpy())
    model.check_finite()
    l32, lbf, nxt = np.concatenate(l32), np.concatenate(lbf), np.concatenate(nxt)
    ref64 = looped["logits64"]
    rows = ref64.shape[0]
    err = float(np.abs(l32 - ref64).max())
    kl = parity.mean_kl(ref64, l32)
    counts, detail = parity.judge(parity.bf16_bits_to_f64(looped["logits"]),
                                  parity.bf16_bits_to_f64(lbf))
    log(f"looped 3x2 end to end ({rows} rows): max|dlogit| {err:.3e} KL {kl:.2e} judge {counts} "
        f"{detail[:5]}")
    assert nxt.tolist() == [oracle.argmax(r) for r in lbf]
    assert err <= 0.05 and kl <= 1e-3
    assert counts["red"] == 0 and counts["near-tie"] <= max(1, int(0.01 * rows))


@pytest.mark.parametrize("step,exact", [(0, True), (0, False), (1, False), (15, False)])
def test_looped_layer_local(looped, step, exact):
    """Every execution's halves from the oracle's inputs; execution 3 (the
    first of loop 2) takes the oracle's boundary-normed rows.  The prompt
    chunk (step 0) in both prompt forms: exact at the literal gate, fast at
    the larger addend."""
    from synth import device as sd
    g, W = looped["g"], looped["W"]
    st = looped["steps"][step]
    runner = HalfRunner(g, sd.weights(g), 96, 64, prompt_exact=exact)
    hg = HalfGates(exact or step > 0)
    ins = exec_inputs(g, oracle.embed(W("embed"), st["tokens"]), st["caps"], W("final_norm"))
    for e in range(g.n_exec):
        b = e % g.n_blocks
        mid, outr = st["caps"][e]
        kc0, vc0 = looped["kc"][e], looped["vc"][e]
        got_mid, _ = runner.run(b, ins[e], kc0, vc0, st["pos0"], "attn")
        got_out, _ = runner.run(b, mid, kc0, vc0, st["pos0"], "mlp")
        f_mid, f_out = f32_halves(g, W, b, kc0, vc0, st["pos0"], ins[e], mid)
        tag = f"looped step {step} exec {e}" + (" (exact prompt form)" if exact else "")
        hg.check(tag + " attention half", got_mid, mid, ins[e], f_mid)
        hg.check(tag + " MLP half", got_out, outr, mid, f_out)
    hg.finish(f"looped step {step}" + (" (exact prompt form)" if exact else ""))
