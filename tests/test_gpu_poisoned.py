"""Reads of unwritten memory: every byte of the workspace and of the caches
is set to 0xFF (a NaN in bf16 and in fp32) before the first step, and the
results must equal, bit for bit, those of the same steps on zero-filled
memory -- prompt chunks (ragged, continued at pos0 > 0), one-row steps,
decode windows and two batched sequences, on the tiny model and on one
33B-shaped layer.  A kernel that read a cache slot past the written length,
a partial sum it had not written, or padding of a tile would carry the NaN
into some output."""
import numpy as np
import pytest

from synth.workloads import TensorIds, config
from tests.gpu_util import gpu_model, log, to_dev, u16

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _run(g, fill, hidden_rows=None):
    model = gpu_model(g, 320, max_chunk_rows=256, max_window_rows=16, max_seqs=2)
    model.workspace.fill_(fill)
    seqs = [model.new_sequence(320) for _ in range(2)]
    for s in seqs:
        s.buf.fill_(fill)
    torch.cuda.synchronize()
    outs = []
    if hidden_rows is None:
        import synth
        toks = synth.tokens(300, 7300, 0, g.vocab)
        o = model.prefill(seqs[0], tokens=to_dev(toks[:137]), all_rows=True)
        outs += [u16(o["logits"]), o["next"].cpu().numpy()]
        o = model.prefill(seqs[0], tokens=to_dev(toks[137:200]), all_rows=True)
        outs += [u16(o["logits"])]
        o = model.prefill(seqs[1], tokens=to_dev(toks[:64]), all_rows=True)
        outs += [u16(o["logits"])]
        for i in range(3):
            o = model.decode([seqs[0]], tokens=to_dev(toks[200 + i:201 + i]))
            outs += [u16(o["logits"])]
        o = model.decode([seqs[0]], tokens=to_dev(toks[203:219]), rows=16)
        outs += [u16(o["logits"])]
        o = model.decode(seqs, tokens=to_dev(toks[219:227]), rows=4)
        outs += [u16(o["logits"]), o["next"].cpu().numpy()]
        model.check_finite()
    else:
        h = to_dev(hidden_rows)
        o = model.prefill(seqs[0], hidden=h[:200], want_hidden=True)
        outs += [u16(o["hidden"])]
        o = model.prefill(seqs[0], hidden=h[200:250], want_hidden=True)
        outs += [u16(o["hidden"])]
        o = model.prefill(seqs[1], hidden=h[:30], want_hidden=True)
        outs += [u16(o["hidden"])]
        o = model.decode([seqs[0]], hidden=h[250:251], want_hidden=True)
        outs += [u16(o["hidden"])]
        o = model.decode([seqs[0]], hidden=h[251:267], rows=16, want_hidden=True)
        outs += [u16(o["hidden"])]
        o = model.decode(seqs, hidden=h[267:275], rows=4, want_hidden=True)
        outs += [u16(o["hidden"])]
    lens = [s.length for s in seqs]
    caches = [u16(s.view())[:, :, :n] for s, n in zip(seqs, lens)]
    return outs, caches


@pytest.mark.parametrize("cfg", [1, 2])
def test_poisoned_memory_equals_zeroed(cfg):
    g = config(cfg)
    rows = None
    if cfg == 2:
        import synth
        rows = synth.normal_bf16(280 * g.hidden, 3130, TensorIds.INPUT_ROWS).reshape(280, g.hidden)
    a, ca = _run(g, 0, rows)
    b, cb = _run(g, 0xFF, rows)
    for i, (x, y) in enumerate(zip(a, b)):
        assert np.array_equal(x, y), f"output {i} differs on poisoned memory"
    for x, y in zip(ca, cb):
        assert np.array_equal(x, y)
    log(f"config {cfg}: {len(a)} outputs and both caches equal on 0xFF-filled and zeroed memory")
