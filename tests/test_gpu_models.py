"""GPU parity at the full model sizes, sampled.  The GPU runs the launch
configuration the benchmark times -- a whole prompt chunk (2,048 rows for the
33B shape, 512 for the looped model) -- and, because attention is causal, its
first rows are comparable with the oracle's forward of those rows alone.  The
oracle walks the blocks one at a time with weights generated on the host (as
the float64 reference in the pull request "llama: Nanbeige4.3-33B on Metal,
the bf16 release served as published" ran one layer's weights at a time).

Deep random-init stacks amplify rounding: a one-step change of a single
embedding element moves the oracle's own 33B logits by up to ~0.4.  So the
tolerance gates here are layer-local -- sampled executions per half, and the
head (final norm + lm_head) fed the oracle's final residual through an
identity block -- while end to end the greedy choices must agree, every miss a
near-tie or within the position's noise floor (how far the oracle's own logits
move when the first row's input is moved by one bf16 step), and the logit
distance is reported beside that floor."""
import numpy as np
import pytest

import oracle
from oracle.model import OracleModel
from synth.workloads import config
from tests import parity
from tests.gpu_util import HalfRunner, exec_inputs, half_report, log, to_dev, u16
from tests.host_inputs import HostWeights

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

SAMPLE_ROWS = 4
DECODE = 4


def _head_layer_local(g, w, h_out, ref64, refb):
    """Final norm + lm_head on the oracle's final residual: a one-block model
    whose block adds exactly 0 (o_proj and down_proj zeroed) passes the rows
    through unchanged."""
    import dataclasses

    import dense_gqa_llama_amd as L
    g1 = dataclasses.replace(g, n_blocks=1, n_loops=1)
    zo = torch.zeros((g.hidden, g.q_dim), dtype=torch.int16, device="cuda")
    zd = torch.zeros((g.hidden, g.ffn), dtype=torch.int16, device="cuda")
    wt = {f"b0.{k}": w[f"b0.{k}"] for k in ("attn_norm", "q", "k", "v", "mlp_norm", "gate", "up")}
    wt.update({"b0.o": zo, "b0.down": zd, "embed": w["embed"], "final_norm": w["final_norm"],
               "lm_head": w["lm_head"]})
    m = L.Model(g1, wt, max_positions=16, max_chunk_rows=16, max_seqs=1)
    s = m.new_sequence(16)
    out = m.prefill(s, hidden=to_dev(h_out), all_rows=True)
    l32 = out["logits32"].cpu().numpy()
    lb = u16(out["logits"])
    err = float(np.abs(l32 - ref64).max())
    kl = parity.mean_kl(ref64, l32)
    counts, _ = parity.judge(parity.bf16_bits_to_f64(refb), parity.bf16_bits_to_f64(lb))
    assert out["next"].cpu().tolist() == [oracle.argmax(x) for x in lb]
    return err, kl, counts


def _run(cfg, sampled_execs):
    import dense_gqa_llama_amd as L
    from synth import device as sd
    g = config(cfg)
    P = g.prompt_len
    prompt = sd.tokens(P, g.prompt_seeds[0], 0, g.vocab)
    ptoks = prompt.cpu().numpy()
    log(f"config {cfg}: oracle over {g.n_exec} executions, {SAMPLE_ROWS} rows + {DECODE} steps")
    W = HostWeights(g, keep_blocks=1)
    om = OracleModel(g, W)
    oseq = om.new_sequence(SAMPLE_ROWS + DECODE)
    r = om.forward(oseq, tokens=ptoks[:SAMPLE_ROWS], logits="all", capture=True)
    ref64, refb, caps, h_out = r["logits64"], r["logits"], r["capture"], r["h_out"]
    log(f"config {cfg}: oracle prompt rows done")
    gen = [int(r["tokens"][-1])]
    dec64, decb = [], []
    for i in range(DECODE):
        rr = om.forward(oseq, tokens=np.array([gen[-1]], dtype=np.int32), logits="all")
        dec64.append(rr["logits64"][0])
        decb.append(rr["logits"][0])
        gen.append(int(rr["tokens"][-1]))
        log(f"config {cfg}: oracle decode step {i + 1}/{DECODE} done")
    log(f"config {cfg}: oracle greedy {gen}")
    # the model's own noise floor: the same rows with every element of the
    # first row's embedding moved by one bf16 step (a rounding-scale change)
    class Nudged:
        def __call__(self, name):
            a = W(name)
            if name == "embed":
                a = a.copy()
                a[ptoks[0], :] += np.uint16(1)
            return a
    om2 = OracleModel(g, Nudged())
    s2o = om2.new_sequence(SAMPLE_ROWS + DECODE)
    n64 = [om2.forward(s2o, tokens=ptoks[:SAMPLE_ROWS], logits="all")["logits64"]]
    log(f"config {cfg}: nudged oracle prompt rows done")
    for i, t in enumerate(gen[:DECODE]):
        n64.append(om2.forward(s2o, tokens=np.array([t], dtype=np.int32), logits="all")["logits64"])
        log(f"config {cfg}: nudged oracle step {i + 1}/{DECODE} done")
    n64 = np.concatenate(n64)
    w = sd.weights(g)
    torch.cuda.synchronize()

    # 1. sampled executions, layer-local per half, as prompt chunks
    runner = HalfRunner(g, w, 64, 64)
    ins = exec_inputs(g, oracle.embed(W("embed"), ptoks[:SAMPLE_ROWS]), caps, W("final_norm"))
    empty = np.zeros((1, g.n_kv_heads, g.head_dim), dtype=np.uint16)
    for e in sampled_execs:
        b = e % g.n_blocks
        mid, outr = caps[e]
        got_mid, _ = runner.run(b, ins[e], empty, empty, 0, "attn", chunk=True)
        got_out, _ = runner.run(b, mid, empty, empty, 0, "mlp", chunk=True)
        assert half_report(f"config {cfg} exec {e} attention half", got_mid, mid, ins[e]) >= 0.999
        assert half_report(f"config {cfg} exec {e} MLP half", got_out, outr, mid) >= 0.999

    # 2. the head, layer-local
    err, kl, counts = _head_layer_local(g, w, h_out, ref64, refb)
    log(f"config {cfg} head from the oracle's residual: max|d| {err:.3e} KL {kl:.2e} {counts}")
    assert err <= 0.05 and kl <= 1e-3 and parity.top1_gate(counts, SAMPLE_ROWS)

    # 3. end to end in the benchmark's chunk: all P rows, first rows compared
    model = L.Model(g, w, max_positions=P + DECODE, max_chunk_rows=P, max_window_rows=16,
                    max_seqs=1)
    seq = model.new_sequence(P + DECODE)
    lg = torch.empty((P, g.vocab), dtype=torch.int16, device="cuda")
    l32 = torch.empty((P, g.vocab), dtype=torch.float32, device="cuda")
    nxt = torch.empty(P, dtype=torch.int32, device="cuda")
    L.binding.llama_prefill_chunk(model.handle, seq.handle, prompt.data_ptr(), None, P, 0, None,
                                  lg.data_ptr(), l32.data_ptr(), 1, nxt.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    got32 = l32[:SAMPLE_ROWS].cpu().numpy()
    gotb = u16(lg[:SAMPLE_ROWS])
    assert nxt[:SAMPLE_ROWS].cpu().tolist() == [oracle.argmax(x) for x in gotb]
    del lg, l32
    # then greedy decode after the same rows, teacher-forced on the oracle's ids
    s2 = model.new_sequence(P + DECODE)
    model.prefill(s2, tokens=prompt[:SAMPLE_ROWS])
    d32, dbf = [], []
    for t in gen[:DECODE]:
        o = model.decode([s2], tokens=to_dev(np.array([t], dtype=np.int32)))
        d32.append(o["logits32"][0].cpu().numpy())
        dbf.append(u16(o["logits"])[0])
    model.check_finite()
    all64 = np.concatenate([ref64, np.stack(dec64)])
    allb = np.concatenate([refb, np.stack(decb)])
    got = np.concatenate([got32, np.stack(d32)])
    gotbf = np.concatenate([gotb, np.stack(dbf)])
    err = float(np.abs(got - all64).max())
    kl = parity.mean_kl(all64, got)
    floors = np.abs(n64 - all64).max(axis=1)
    counts, detail = parity.judge_with_floor(parity.bf16_bits_to_f64(allb),
                                             parity.bf16_bits_to_f64(gotbf), floors)
    log(f"config {cfg} end to end: logits max|d| {err:.3e} KL {kl:.2e} (reported); the oracle "
        f"nudged by one step moves by up to {floors.max():.3e} (KL "
        f"{parity.mean_kl(all64, n64):.2e}); judge {counts} {detail}")
    assert parity.top1_gate(counts, all64.shape[0])


def test_33b_full_model_sampled():
    _run(3, (0, 25, 51))


def test_looped_full_model_sampled():
    _run(4, (0, 21, 22, 43))
