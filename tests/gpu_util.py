"""Helpers for the GPU parity tests: building a model of a workload on the GPU
from the synthetic generator, running single block executions on the
oracle's own inputs, and moving bf16 bits between torch and numpy."""
import dataclasses
import os
import sys

import numpy as np

import oracle
from tests import parity

KINDS = ("attn_norm", "q", "k", "v", "o", "mlp_norm", "gate", "up", "down")


_PROGRESS = []


def log(msg):
    """Prints a progress line and, when the environment names a directory in
    GPU_TESTS_PROGRESS_DIR, appends it to gpu_tests_progress.log there (pytest
    holds a test's own output until it ends; the file shows a long test
    advancing while it runs)."""
    print(msg, flush=True)
    sys.stdout.flush()
    d = os.environ.get("GPU_TESTS_PROGRESS_DIR")
    if not d:
        return
    try:
        if not _PROGRESS:
            os.makedirs(d, exist_ok=True)
            _PROGRESS.append(open(os.path.join(d, "gpu_tests_progress.log"), "a"))
        _PROGRESS[0].write(msg + "\n")
        _PROGRESS[0].flush()
    except OSError:
        pass


def u16(t):
    """Device int16 tensor of bf16 bits -> host uint16 array."""
    return t.detach().cpu().numpy().view(np.uint16)


def to_dev(a):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).cuda()
    return torch.from_numpy(a.copy()).cuda()


def gpu_model(g, max_positions, max_chunk_rows=2048, max_window_rows=16, max_seqs=2, weights=None,
              prompt_exact=False):
    import torch

    import dense_gqa_llama_amd as L
    from synth import device as sd
    w = weights if weights is not None else sd.weights(g)
    torch.cuda.synchronize()
    return L.Model(g, w, max_positions=max_positions, max_chunk_rows=max_chunk_rows,
                   max_window_rows=max_window_rows, max_seqs=max_seqs, prompt_exact=prompt_exact)


class HalfRunner:
    """Runs one block execution on the GPU from the oracle's inputs, through
    the C ABI with a one-block, blocks-only model.  Zeroing o_proj makes the
    attention half add exactly 0 (bf16(h + 0) = h), which isolates the MLP
    half; zeroing down_proj isolates the attention half."""

    def __init__(self, g, dev_weights, max_positions, max_rows, prompt_exact=False):
        import torch
        self.prompt_exact = prompt_exact
        self.g1 = dataclasses.replace(g, n_blocks=1, n_loops=1, vocab=0)
        self.dev = dev_weights
        self.maxp = max_positions
        self.max_rows = max_rows
        self.zero_o = torch.zeros((g.hidden, g.q_dim), dtype=torch.int16, device="cuda")
        self.zero_down = torch.zeros((g.hidden, g.ffn), dtype=torch.int16, device="cuda")

    def run(self, block, h_in, kc, vc, pos0, mode, chunk=None):
        """mode: 'layer', 'attn' (down zeroed) or 'mlp' (o zeroed).  kc, vc:
        the oracle's cache of this execution (positions [0, pos0) are used).
        chunk: run as a prompt chunk (default: when rows > 16) or a window.
        Returns (h_out bits, cache after the step as (k, v) host arrays)."""
        import dense_gqa_llama_amd as L
        w = {f"b0.{k}": self.dev[f"b{block}.{k}"] for k in KINDS}
        if mode == "attn":
            w["b0.down"] = self.zero_down
        elif mode == "mlp":
            w["b0.o"] = self.zero_o
        rows = h_in.shape[0]
        m = L.Model(self.g1, w, max_positions=self.maxp, max_chunk_rows=self.max_rows,
                    max_window_rows=16, max_seqs=1, prompt_exact=self.prompt_exact)
        s = m.new_sequence(self.maxp)
        if pos0:
            v = s.view()
            v[0, 0, :pos0] = to_dev(np.ascontiguousarray(kc[:pos0]))
            v[0, 1, :pos0] = to_dev(np.ascontiguousarray(vc[:pos0]))
            s.declare(pos0)
        hin = to_dev(np.ascontiguousarray(h_in))
        if chunk is None:
            chunk = rows > 16
        if chunk:
            out = m.prefill(s, hidden=hin)
        else:
            out = m.decode([s], hidden=hin, rows=rows)
        h = u16(out["hidden"])
        cache = u16(s.view())
        return h, (cache[0, 0], cache[0, 1])


def half_report(tag, got, ref, h_in, gate="literal"):
    """Logs the agreement of a half's residual output with the oracle's:
    exact, within 2 bf16 steps at max(|got|, |ref|), and within 2 steps at the
    larger addend of the residual add (the distance a rounding-scale change of
    the added term can make).  Returns the first (gate "literal"), or the
    second (gate "addend": the prompt chunks' fast form, whose matrix-unit
    sums are measured per kernel; its literal figure is logged beside)."""
    plain, pw = parity.within_ulps(got, ref)
    frac, worst = parity.within_addend_ulps(got, ref, h_in)
    exact = float((got == ref).mean())
    log(f"{tag}: exact {exact:.5f}  within 2 steps {plain:.5f} (worst {pw:g})  "
        f"at the addend {frac:.5f} (worst {worst:g})")
    return plain if gate == "literal" else frac


def exec_inputs(g, embed_rows, caps, final_norm):
    """The oracle's input rows of every execution, from its captures
    [(mid, out)] of one step: the embedding for the first, the previous
    output otherwise, and at a loop boundary the final-normed previous output
    (the normed state replaces the residual)."""
    ins = []
    for e in range(g.n_exec):
        if e == 0:
            ins.append(embed_rows)
        elif e % g.n_blocks == 0:
            ins.append(oracle.rmsnorm(caps[e - 1][1], final_norm, g.rms_eps))
        else:
            ins.append(caps[e - 1][1])
    return ins
