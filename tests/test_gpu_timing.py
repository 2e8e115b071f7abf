"""The measurement hook (llama_set_timing / llama_timing_read) on the GPU:
while a kernel class is timed, its kernels go through the event-timed launch,
and the step's results must not change; the hook must count the launches the
class makes and report positive kernel time.  Covers the path bench.py uses
for its per-kernel figures."""
import numpy as np
import pytest

from synth.workloads import config
from tests.gpu_util import gpu_model, log, to_dev, u16
from tests.host_inputs import prompt

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import dense_gqa_llama_amd.binding as B  # noqa: E402

STEPS = 6


def _request(model, toks):
    """A prompt chunk and STEPS one-row decode steps; returns every logit row
    (bf16 bits) and the generated ids."""
    s = model.new_sequence(len(toks) + STEPS + 1)
    out = model.prefill(s, tokens=to_dev(toks), all_rows=True)
    rows = [u16(out["logits"])]
    nxt = out["next"][-1:].clone()
    ids = [int(nxt.item())]
    for _ in range(STEPS):
        out = model.decode([s], tokens=nxt, rows=1)
        rows.append(u16(out["logits"]))
        nxt = out["next"][-1:].clone()
        ids.append(int(nxt.item()))
    return np.concatenate(rows), ids


def test_timed_kernels_give_the_same_bits_and_count_their_launches():
    g = config(1)
    toks = prompt(g)
    model = gpu_model(g, len(toks) + STEPS + 1, max_chunk_rows=len(toks), max_window_rows=1,
                      max_seqs=1)
    ref_rows, ref_ids = _request(model, toks)
    # launches per request: the decode classes once per execution and step
    # (attention twice: the split pass and the merge); the head and the prompt
    # classes once or more per request or execution
    expect = {"gate_up": g.n_exec * STEPS, "down": g.n_exec * STEPS, "qkv": g.n_exec * STEPS,
              "o": g.n_exec * STEPS, "attn": 2 * g.n_exec * STEPS}
    for kind in ("gate_up", "down", "qkv", "o", "attn", "lm_head", "prefill_gemm", "prefill_attn"):
        B.llama_set_timing(model.handle, kind, 1000)
        rows, ids = _request(model, toks)
        torch.cuda.synchronize()
        ms, n = B.llama_timing_read(model.handle)
        B.llama_set_timing(model.handle, "off")
        log(f"timed {kind}: {n} launches, {ms * 1e3:.1f} us in all")
        assert np.array_equal(rows, ref_rows), kind
        assert ids == ref_ids, kind
        assert ms > 0.0, kind
        if kind in expect:
            assert n == expect[kind], (kind, n)
        elif kind == "prefill_attn":
            assert n == g.n_exec, (kind, n)
        elif kind == "lm_head":  # the prompt's rows may take more than one launch
            assert n >= STEPS + 1, (kind, n)
        else:
            assert n >= 4 * g.n_exec, (kind, n)
    # a pool smaller than the launches records the first ones only
    B.llama_set_timing(model.handle, "gate_up", 3)
    _request(model, toks)
    torch.cuda.synchronize()
    ms, n = B.llama_timing_read(model.handle)
    B.llama_set_timing(model.handle, "off")
    assert n == 3 and ms > 0.0
