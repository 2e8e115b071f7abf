"""PyTorch-side handles: device memory for the workspace and caches, and
calls into the C ABI on the current stream.  Marshalling only."""
import torch

from . import binding as B


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


class Model:
    """Wraps llama_load_weights.  ``weights`` maps names to bf16 device
    tensors: ``embed``, ``final_norm``, ``lm_head`` (absent for a blocks-only
    model) and ``b{i}.{attn_norm,q,k,v,o,mlp_norm,gate,up,down}``."""

    def __init__(self, geom, weights, max_positions, max_chunk_rows=2048, max_window_rows=16,
                 max_seqs=2, prompt_exact=False, device="cuda"):
        self.g = geom
        self.cfg = B.make_config(geom.n_blocks, geom.n_loops, geom.hidden, geom.n_q_heads,
                                 geom.n_kv_heads, geom.head_dim, geom.ffn, geom.vocab,
                                 geom.rope_theta, geom.rms_eps, max_chunk_rows, max_window_rows,
                                 max_seqs, prompt_exact)
        self.max_positions = max_positions
        nbytes = B.llama_workspace_bytes(self.cfg, max_positions)
        if nbytes == 0:
            raise B.LlamaError(B.LLAMA_E_GEOMETRY, B.last_error())
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.weights = weights
        blocks = [{f: weights[f"b{i}.{f}"].data_ptr() for f in B.BLOCK_FIELDS}
                  for i in range(geom.n_blocks)]
        get = lambda k: weights[k].data_ptr() if k in weights else None  # noqa: E731
        self.handle = B.llama_load_weights(self.cfg, blocks, get("embed"), get("final_norm"),
                                           get("lm_head"), self.workspace.data_ptr(), nbytes,
                                           max_positions)
        self.capture = None

    def set_probe(self, exec_index, rows, fields=None):
        """Allocates and installs parity-probe buffers of ``rows`` rows for
        execution ``exec_index`` (all fields, or those named); returns the
        dict of device tensors (bf16 fields as int16).  ``rows=0`` clears the
        hook."""
        if not rows:
            B.llama_set_probe(self.handle, 0, None, 0)
            self.probe = None
            return None
        g = self.g
        qd, kvd = g.n_q_heads * g.head_dim, g.n_kv_heads * g.head_dim
        shapes = {"h_in": (g.hidden, torch.int16), "x_attn": (g.hidden, torch.int16),
                  "qkv32": (qd + 2 * kvd, torch.float32), "q_rope": (qd, torch.int16),
                  "attn": (qd, torch.int16), "attn32": (qd, torch.float32),
                  "o32": (g.hidden, torch.float32), "x_mlp": (g.hidden, torch.int16),
                  "gate_up32": (2 * g.ffn, torch.float32), "act": (g.ffn, torch.int16),
                  "down32": (g.hidden, torch.float32)}
        dev = self.workspace.device
        self.probe = {k: torch.full((rows, w), -1, dtype=t, device=dev)
                      for k, (w, t) in shapes.items() if fields is None or k in fields}
        B.llama_set_probe(self.handle, exec_index,
                          {k: v.data_ptr() for k, v in self.probe.items()}, rows)
        return self.probe

    def new_sequence(self, max_positions=None):
        return Sequence(self, max_positions or self.max_positions)

    def set_capture(self, rows):
        """Allocates and installs a capture buffer for steps of ``rows`` rows
        (bf16 [executions][2][rows][hidden]); ``rows=0`` clears it."""
        if not rows:
            B.llama_set_capture(self.handle, None, 0)
            self.capture = None
            return None
        g = self.g
        self.capture = torch.empty((g.n_blocks * g.n_loops, 2, rows, g.hidden), dtype=torch.int16,
                                   device=self.workspace.device)
        B.llama_set_capture(self.handle, self.capture.data_ptr(),
                            self.capture.numel() * 2)
        return self.capture

    def prefill(self, seq, tokens=None, hidden=None, all_rows=False, want_logits=True,
                want_hidden=False):
        """One prompt chunk.  Returns dict of device tensors: ``next`` (int32),
        and when asked ``logits`` (bf16 bits as int16), ``logits32``, ``hidden``."""
        g = self.g
        n = (tokens if tokens is not None else hidden).shape[0]
        dev = self.workspace.device
        nl = n if all_rows else 1
        out = {}
        if g.vocab:
            out["next"] = torch.empty(nl, dtype=torch.int32, device=dev)
            if want_logits:
                out["logits"] = torch.empty((nl, g.vocab), dtype=torch.int16, device=dev)
                out["logits32"] = torch.empty((nl, g.vocab), dtype=torch.float32, device=dev)
        if want_hidden or not g.vocab:
            out["hidden"] = torch.empty((n, g.hidden), dtype=torch.int16, device=dev)
        B.llama_prefill_chunk(self.handle, seq.handle, _ptr(tokens), _ptr(hidden), n, seq.length,
                              _ptr(out.get("hidden")), _ptr(out.get("logits")),
                              _ptr(out.get("logits32")), int(all_rows), _ptr(out.get("next")),
                              _stream())
        return out

    def decode(self, seqs, tokens=None, hidden=None, rows=1, want_logits=True, want_hidden=False,
               next_out=None):
        """One decode window for each sequence in ``seqs`` (batched).
        tokens: int32 [n_seq*rows]; returns dict as :meth:`prefill`."""
        g = self.g
        total = len(seqs) * rows
        dev = self.workspace.device
        out = {}
        if g.vocab:
            out["next"] = next_out if next_out is not None else torch.empty(
                total, dtype=torch.int32, device=dev)
            if want_logits:
                out["logits"] = torch.empty((total, g.vocab), dtype=torch.int16, device=dev)
                out["logits32"] = torch.empty((total, g.vocab), dtype=torch.float32, device=dev)
        if want_hidden or not g.vocab:
            out["hidden"] = torch.empty((total, g.hidden), dtype=torch.int16, device=dev)
        B.llama_decode_step(self.handle, [s.handle for s in seqs], _ptr(tokens), _ptr(hidden),
                            rows, _ptr(out.get("hidden")), _ptr(out.get("logits")),
                            _ptr(out.get("logits32")), _ptr(out.get("next")), _stream())
        return out

    def sample(self, logits, u, temperature, top_k, top_p, out=None):
        """Seeded top-k / top-p draw for each row of ``logits`` (bf16 bits as
        int16 [rows][>= vocab]) against the uniforms ``u`` (float32 [rows]);
        returns int32 token ids (-1 for a non-finite row)."""
        rows = logits.shape[0]
        if out is None:
            out = torch.empty(rows, dtype=torch.int32, device=logits.device)
        B.llama_sample(self.handle, logits.data_ptr(), rows, logits.stride(0), float(temperature),
                       int(top_k), float(top_p), u.data_ptr(), out.data_ptr(), _stream())
        return out

    def draft_round(self, seq, draft, draft_seq, n_draft, last_token, out=None):
        """One drafted greedy round (``llama_draft_round``): ``draft`` (a Model
        on the same vocabulary) proposes ``n_draft`` tokens after
        ``last_token`` (int32 [1] on the device) and this model verifies them
        in one window.  Returns (tokens, n): the round's n tokens are
        tokens[:n]; tokens[n - 1] is the next round's input."""
        if out is None:
            out = torch.empty(n_draft + 1, dtype=torch.int32, device=last_token.device)
        n = B.llama_draft_round(self.handle, seq.handle, draft.handle, draft_seq.handle,
                                int(n_draft), last_token.data_ptr(), out.data_ptr(), _stream())
        return out, n

    def draft_round_sampled(self, seq, draft, draft_seq, n_draft, last_token, u, temperature,
                            top_k, top_p, out=None):
        """As draft_round, with this model's tokens drawn by seeded sampling:
        u (float32 [n_draft + 1] on the device) holds the uniform of each
        window row's draw."""
        if out is None:
            out = torch.empty(n_draft + 1, dtype=torch.int32, device=last_token.device)
        n = B.llama_draft_round_sampled(self.handle, seq.handle, draft.handle, draft_seq.handle,
                                        int(n_draft), last_token.data_ptr(), float(temperature),
                                        int(top_k), float(top_p), u.data_ptr(), out.data_ptr(),
                                        _stream())
        return out, n

    def check_finite(self):
        B.llama_check_finite(self.handle, _stream())

    def close(self):
        if self.handle:
            B.llama_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Sequence:
    """One sequence's cache (every execution), in a caller-owned device buffer."""

    def __init__(self, model, max_positions):
        self.model = model
        nbytes = B.llama_kv_bytes(model.handle, max_positions)
        g = model.g
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=model.workspace.device)
        self.handle = B.llama_kv_alloc(model.handle, max_positions, self.buf.data_ptr(), nbytes)
        self.max_positions = max_positions
        self.shape = (g.n_blocks * g.n_loops, 2, max_positions, g.n_kv_heads, g.head_dim)

    @property
    def length(self):
        return B.llama_kv_length(self.handle)

    def truncate(self, n):
        """Keeps positions [0, n) (a resumed prompt state); shortens only."""
        B.llama_kv_truncate(self.handle, n)

    def declare(self, n):
        """Test hook: positions [0, n) hold keys and values written through
        ``view()``."""
        B.llama_test_kv_declare(self.handle, n)

    def view(self):
        """The cache as int16 [executions][K/V][positions][kv_heads][head_dim]."""
        return self.buf.view(torch.int16).view(self.shape)

    def close(self):
        if self.handle:
            B.llama_kv_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
