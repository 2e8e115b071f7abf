"""GPU parity of prompt chunks (matrix-core projections and attention)
against the CPU oracle: ragged chunks spanning several 128-row tiles, a second
chunk continuing at pos0 > 0 (continuity across chunk boundaries, as the
NInfer card's "Validation" section checks), and a 33B-shaped layer over a
4096-slot cache.  Same gates as the decode tests (layer-local halves within 2
bf16 steps at the addend on >= 99.9% of elements; logits max-abs 0.05 on the
fp32 sums, KL <= 1e-3, top-1 >= 99% with near-ties only)."""
import numpy as np
import pytest

import oracle
from oracle.model import OracleModel
from synth.workloads import TensorIds, config
from tests import parity
from tests.gpu_util import HalfRunner, exec_inputs, gpu_model, half_report, log, to_dev, u16
from tests.host_inputs import HostWeights

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

CHUNKS = (137, 63)  # 200 rows: a ragged 2-tile chunk, then a chunk at pos0 = 137


@pytest.fixture(scope="module")
def tiny200():
    import synth
    g = config(1)
    W = HostWeights(g)
    toks = synth.tokens(sum(CHUNKS), 7001, 0, g.vocab)
    om = OracleModel(g, W)
    seq = om.new_sequence(256)
    steps = []
    p = 0
    for n in CHUNKS:
        r = om.forward(seq, tokens=toks[p:p + n], logits="all", capture=True)
        steps.append(dict(tokens=toks[p:p + n], pos0=p, caps=r["capture"], logits64=r["logits64"],
                          logits=r["logits"]))
        p += n
    log(f"tiny200: oracle {CHUNKS}")
    return dict(g=g, W=W, toks=toks, steps=steps, kc=seq.kc, vc=seq.vc)


def test_chunked_prompt_logits(tiny200):
    g = tiny200["g"]
    model = gpu_model(g, 256, max_chunk_rows=256, max_seqs=1)
    seq = model.new_sequence(256)
    l32, lbf = [], []
    p = 0
    for n in CHUNKS:
        out = model.prefill(seq, tokens=to_dev(tiny200["toks"][p:p + n]), all_rows=True)
        l32.append(out["logits32"].cpu().numpy())
        lbf.append(u16(out["logits"]))
        nxt = out["next"].cpu().numpy()
        assert nxt.tolist() == [oracle.argmax(r) for r in lbf[-1]]
        p += n
    model.check_finite()
    ref64 = np.concatenate([s["logits64"] for s in tiny200["steps"]])
    refb = np.concatenate([s["logits"] for s in tiny200["steps"]])
    l32, lbf = np.concatenate(l32), np.concatenate(lbf)
    err = float(np.abs(l32 - ref64).max())
    kl = parity.mean_kl(ref64, l32)
    counts, detail = parity.judge(parity.bf16_bits_to_f64(refb), parity.bf16_bits_to_f64(lbf))
    log(f"tiny200 chunks: max|dlogit| {err:.3e} KL {kl:.2e} judge {counts} {detail[:5]}")
    assert err <= 0.05 and kl <= 1e-3 and counts["red"] == 0
    assert counts["near-tie"] <= max(1, int(0.01 * ref64.shape[0]))
    assert seq.length == sum(CHUNKS)


@pytest.mark.parametrize("chunk", [0, 1])
def test_chunk_layer_local(tiny200, chunk):
    from synth import device as sd
    g, W = tiny200["g"], tiny200["W"]
    st = tiny200["steps"][chunk]
    runner = HalfRunner(g, sd.weights(g), 256, 256)
    ins = exec_inputs(g, oracle.embed(W("embed"), st["tokens"]), st["caps"], W("final_norm"))
    for e in range(g.n_exec):
        mid, outr = st["caps"][e]
        kc0, vc0 = tiny200["kc"][e], tiny200["vc"][e]
        got_mid, (kc, vc) = runner.run(e % g.n_blocks, ins[e], kc0, vc0, st["pos0"], "attn")
        got_out, _ = runner.run(e % g.n_blocks, mid, kc0, vc0, st["pos0"], "mlp")
        tag = f"tiny chunk {chunk} exec {e}"
        assert half_report(tag + " attention half", got_mid, mid, ins[e]) >= 0.999
        assert half_report(tag + " MLP half", got_out, outr, mid) >= 0.999
        n = st["pos0"] + len(st["tokens"])
        for c, ref in ((kc, kc0), (vc, vc0)):
            frac, worst = parity.within_ulps(c[st["pos0"]:n], ref[st["pos0"]:n])
            assert frac >= 0.999, (tag, frac, worst)


def test_layer33_chunk_vs_oracle():
    """A 144-row chunk (two 128-row tiles, ragged) of one 33B-shaped layer at
    positions 4096..4239 over the N(0,1) cache."""
    import synth
    from synth import device as sd
    g = config(2)
    T, R = g.extra["cache_positions"], 144
    kvd = g.kv_dim
    W = HostWeights(g)
    kc = np.zeros((T + R, g.n_kv_heads, g.head_dim), dtype=np.uint16)
    vc = np.zeros_like(kc)
    kc[:T] = synth.normal_bf16(T * kvd, g.extra["kv_seed"], TensorIds.K_CACHE).reshape(
        T, g.n_kv_heads, g.head_dim)
    vc[:T] = synth.normal_bf16(T * kvd, g.extra["kv_seed"], TensorIds.V_CACHE).reshape(
        T, g.n_kv_heads, g.head_dim)
    rows = synth.normal_bf16(R * g.hidden, g.extra["input_seed"] + 1, TensorIds.INPUT_ROWS).reshape(
        R, g.hidden)
    log("layer33 chunk: oracle 144 rows")
    kco, vco = kc.copy(), vc.copy()
    h, mid = oracle.block(g, {k: W(f"b0.{k}") for k in
                              ("attn_norm", "q", "k", "v", "o", "mlp_norm", "gate", "up", "down")},
                          kco, vco, np.arange(T, T + R, dtype=np.int32), rows, want_mid=True)
    runner = HalfRunner(g, sd.weights(g), T + R, R)
    got_mid, (kcg, vcg) = runner.run(0, rows, kc, vc, T, "attn")
    got_out, _ = runner.run(0, mid, kc, vc, T, "mlp")
    a = half_report("layer33 chunk attention half", got_mid, mid, rows)
    b = half_report("layer33 chunk MLP half", got_out, h, mid)
    fk, _ = parity.within_ulps(kcg[T:], kco[T:])
    fv, _ = parity.within_ulps(vcg[T:], vco[T:])
    log(f"layer33 chunk cache slots: k {fk:.5f} v {fv:.5f}")
    assert a >= 0.999 and b >= 0.999 and fk >= 0.999 and fv >= 0.999


@pytest.mark.parametrize("cfg,n,bad", [(1, 200, 150), (2, 300, 211)])
def test_nonfinite_row_reaches_only_later_rows(cfg, n, bad):
    """A non-finite input row poisons its own key and value; rows before it
    never attend to that slot (causal), so they must equal a clean run bit for
    bit -- the masked slot's value must not leak through a zero weight
    (0 * NaN) -- while rows from it on read NaN.  Tiny model (d = 64) and a
    33B-shaped layer (d = 128), the bad row inside a later 64-slot tile."""
    import synth
    from synth.workloads import TensorIds
    g = config(cfg)
    model = gpu_model(g, 320, max_chunk_rows=320, max_seqs=1)
    rows = synth.normal_bf16(n * g.hidden, 3120 + cfg, TensorIds.INPUT_ROWS).reshape(n, g.hidden)
    clean = model.new_sequence(320)
    hc = u16(model.prefill(clean, hidden=to_dev(rows), want_hidden=True)["hidden"])
    poisoned = rows.copy()
    poisoned[bad, 7] = 0x7FC0  # bf16 NaN
    sq = model.new_sequence(320)
    hp = u16(model.prefill(sq, hidden=to_dev(poisoned), want_hidden=True)["hidden"])
    assert np.array_equal(hp[:bad], hc[:bad])
    isnan = ((hp[bad:] & 0x7F80) == 0x7F80) & ((hp[bad:] & 0x007F) != 0)
    assert isnan.any(axis=1).all()
    log(f"config {cfg}: NaN input row {bad} of {n}: earlier rows bit-equal to the clean run, later rows NaN")
