"""The oracle's forward pass, composed from the steps in ``oracle.c``.

TEST INFRASTRUCTURE (see the package docstring).

Per row at absolute position p, one execution of block b runs the steps of the
pull request "llama: Nanbeige4.3-33B on Metal, the bf16 release served as
published", section "How", in modeling_llama's order: RMSNorm, q/k/v
projections, RoPE on q and k, keys and values stored at slot p of this
execution's position-major cache, causal grouped-query attention, o
projection and residual add, RMSNorm, gate/up projections, SwiGLU, down
projection and residual add.

Looped models (Nanbeige4.2-3B card, section "About the architecture") run the
whole block stack ``n_loops`` times over the same weights; execution
``loop * n_blocks + b`` keeps its own cache, and the final norm is applied at
the end of every loop, its output replacing the residual.  lm_head then reads
the normed state after the last loop.  A model without a vocabulary (one
block, hidden rows in and out) has no final norm.
"""
import numpy as np

from . import (argmax, attention, block, embed, f64, linear, residual_add, rmsnorm, rope,
               swiglu)

BLOCK_KINDS = ("attn_norm", "q", "k", "v", "o", "mlp_norm", "gate", "up", "down")


class OracleSequence:
    """One sequence's caches and length over a model's executions."""

    def __init__(self, geom, max_positions):
        shape = (geom.n_blocks * geom.n_loops, max_positions, geom.n_kv_heads, geom.head_dim)
        self.kc = np.zeros(shape, dtype=np.uint16)
        self.vc = np.zeros(shape, dtype=np.uint16)
        self.length = 0
        self.max_positions = max_positions


class OracleModel:
    """``weights(name)`` returns the uint16 array of a stored tensor, names as
    in ``embed``, ``b{i}.q`` ..., ``final_norm``, ``lm_head``; it may generate
    blocks on demand so that only one block is held at a time."""

    def __init__(self, geom, weights):
        self.g = geom
        self.weights = weights

    def new_sequence(self, max_positions):
        return OracleSequence(self.g, max_positions)

    def _block(self, b):
        return {k: self.weights(f"b{b}.{k}") for k in BLOCK_KINDS}

    def forward(self, seq, tokens=None, hidden=None, logits="all", capture=False):
        """Runs rows at positions [seq.length, seq.length + rows) and appends
        them to the sequence.  Returns a dict with ``h_out`` (the residual after
        the last execution, before the final norm), ``logits`` (bf16 bits) and
        ``logits64`` (the binary64 sums) for all rows or the last, greedy
        ``tokens``, and with ``capture`` the per-execution residuals after each
        half as a list of (mid, out)."""
        g = self.g
        if tokens is not None:
            tokens = np.asarray(tokens, dtype=np.int32).reshape(-1)
            h = embed(self.weights("embed"), tokens)
        else:
            h = np.ascontiguousarray(hidden, dtype=np.uint16).reshape(-1, g.hidden)
        rows = h.shape[0]
        if seq.length + rows > seq.max_positions:
            raise ValueError("capacity")
        pos = np.arange(seq.length, seq.length + rows, dtype=np.int32)
        caps = []
        h_out = None
        for loop in range(g.n_loops):
            for b in range(g.n_blocks):
                e = loop * g.n_blocks + b
                h, mid = block(g, self._block(b), seq.kc[e], seq.vc[e], pos, h, want_mid=True)
                if capture:
                    caps.append((mid, h.copy()))
            h_out = h.copy()
            if g.vocab:
                h = rmsnorm(h, self.weights("final_norm"), g.rms_eps)
        seq.length += rows
        out = {"h_out": h_out, "capture": caps}
        if g.vocab and logits:
            x = h if logits == "all" else h[-1:]
            lg, lg64 = linear(x, self.weights("lm_head"), want64=True)
            out["logits"] = lg
            out["logits64"] = lg64
            out["tokens"] = np.array([argmax(r) for r in lg], dtype=np.int32)
        return out

    def generate(self, seq, prompt, steps, chunk_rows=None):
        """Greedy continuation: the prompt's last row gives the first token,
        then ``steps - 1`` one-row steps each consume the previous token.
        Returns the ``steps`` generated ids."""
        prompt = np.asarray(prompt, dtype=np.int32)
        chunk = chunk_rows or prompt.size
        for s in range(0, prompt.size, chunk):
            r = self.forward(seq, tokens=prompt[s:s + chunk], logits="last")
        out = [int(r["tokens"][-1])]
        for _ in range(steps - 1):
            r = self.forward(seq, tokens=np.array([out[-1]], dtype=np.int32), logits="last")
            out.append(int(r["tokens"][-1]))
        return np.array(out, dtype=np.int32)


def logits_f64(bits):
    return f64(bits)


def block_rows(geom, w, kc, vc, pos, h, rows):
    """One block execution over rows at positions ``pos`` whose outputs are
    needed only for the rows ``rows`` (indexes into h): every row's key and
    value are stored at its slot (as orc_block stores them, before any row
    attends), then the selected rows run the rest of the block.  Returns
    (mid, out) of the selected rows: the residual after the attention half
    and after the MLP half.  The same steps in the same order as orc_block,
    so the selected rows' bits equal a full block's."""
    g = geom
    pos = np.asarray(pos, dtype=np.int32)
    rows = np.asarray(rows)
    x = rmsnorm(h, w["attn_norm"], g.rms_eps)
    k = rope(linear(x, w["k"]), pos, g.n_kv_heads, g.head_dim, g.rope_theta)
    v = linear(x, w["v"])
    kc[pos] = k.reshape(-1, g.n_kv_heads, g.head_dim)
    vc[pos] = v.reshape(-1, g.n_kv_heads, g.head_dim)
    xs = np.ascontiguousarray(x[rows])
    q = rope(linear(xs, w["q"]), pos[rows], g.n_q_heads, g.head_dim, g.rope_theta)
    a = attention(q, kc, vc, pos[rows], g.n_q_heads, g.n_kv_heads, g.head_dim)
    mid = residual_add(np.ascontiguousarray(h[rows]), linear(a, w["o"]))
    return mid, mlp_half(geom, w, mid)


def mlp_half(geom, w, mid):
    """The MLP half of a block on residual rows: RMSNorm, gate/up, SwiGLU,
    down projection, residual add."""
    x = rmsnorm(mid, w["mlp_norm"], geom.rms_eps)
    m = swiglu(linear(x, w["gate"]), linear(x, w["up"]))
    return residual_add(mid, linear(m, w["down"]))
