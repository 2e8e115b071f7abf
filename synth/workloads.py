"""Geometry, seeds and tensor ids of the five synthetic workloads.

Each workload is a dense grouped-query Llama decoder served from bf16 weights
with a bf16 position-major key/value cache:

1. tiny: 2 blocks, hidden 512, 8 query / 2 KV heads of 64, SwiGLU FFN 1408,
   vocabulary 4096, RoPE theta 1e4, eps 1e-5; a 64-token prompt, then 16
   greedy one-row steps.
2. one Nanbeige4.3-33B-shaped block (hidden 7168, 56/8 heads of 128, FFN
   22016, theta 1.2e8) decoding 1-row and 16-row windows over a 4096-position
   cache filled with N(0,1) keys and values; its input rows are N(0,1).
3. the full 33B shape: 52 blocks, vocabulary 166,912, untied lm_head; a
   2,048-token prompt in one chunk, then 128 greedy steps.
4. a looped model: 22 blocks run twice (44 executions, each with its own cache,
   the final norm applied after each loop), hidden 3072, 48 query heads of 128,
   8 KV heads, FFN 8192, vocabulary 166,912; a 512-token prompt, then 256 steps.
5. the 33B shape at long context: two sequences, 131,072-token prompts in
   2,048-row chunks, then 64 greedy steps per sequence.

Architecture facts (layer count, widths, head counts, vocabulary, theta) are
those of the Nanbeige4.3-33B model card ("Provenance and representation") and
of the looped Nanbeige4.2-3B card ("About the architecture").  Projection and
embedding weights are ~N(0, 0.02); RMSNorm weights are 1 + N(0, 0.02).
"""
from dataclasses import dataclass, field


@dataclass(frozen=True)
class LlamaGeometry:
    name: str
    n_blocks: int
    n_loops: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    rope_theta: float
    rms_eps: float = 1e-5
    # workload
    weight_seed: int = 0
    prompt_seeds: tuple = ()
    prompt_len: int = 0
    chunk_rows: int = 2048
    decode_steps: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def n_exec(self):
        return self.n_blocks * self.n_loops

    @property
    def q_dim(self):
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self):
        return self.n_kv_heads * self.head_dim

    def block_params(self):
        H, F = self.hidden, self.ffn
        return 2 * H + H * self.q_dim + 2 * H * self.kv_dim + self.q_dim * H + 3 * H * F

    def params(self):
        """Stored parameters: embedding, blocks, final norm, untied lm_head."""
        p = self.n_blocks * self.block_params()
        if self.vocab:
            p += 2 * self.vocab * self.hidden + self.hidden
        return p

    def kv_bytes_per_position(self):
        """bf16 keys and values for every execution (loops keep their own caches)."""
        return self.n_exec * self.kv_dim * 2 * 2

    def decode_weight_bytes(self):
        """Weight bytes one decode token streams: every block's projections and
        norms (once per execution), the final norm (once per loop), lm_head,
        and one embedding row."""
        H = self.hidden
        b = self.n_exec * self.block_params() * 2
        if self.vocab:
            b += self.n_loops * H * 2 + self.vocab * H * 2 + H * 2
        return b


class TensorIds:
    """Stream ids of the synthetic tensors (one SplitMix64 stream each)."""
    EMBED = 1
    FINAL_NORM = 2
    LM_HEAD = 3
    # per block: 1000 + 16*b + kind
    ATTN_NORM, Q, K, V, O, MLP_NORM, GATE, UP, DOWN = range(9)
    KIND_NAMES = ("attn_norm", "q", "k", "v", "o", "mlp_norm", "gate", "up", "down")
    # cache / input fills
    K_CACHE = 10
    V_CACHE = 11
    INPUT_ROWS = 20
    # sampling: the uniform drawn for step s of a sequence, and synthetic logits
    SAMPLE_UNIFORM = 30
    SAMPLE_LOGITS = 31

    @staticmethod
    def block(b, kind):
        return 1000 + 16 * b + kind


CONFIGS = {
    1: LlamaGeometry("tiny", 2, 1, 512, 8, 2, 64, 1408, 4096, 1e4, 1e-5,
                     weight_seed=1001, prompt_seeds=(2001,), prompt_len=64, chunk_rows=64,
                     decode_steps=16),
    2: LlamaGeometry("33b-layer", 1, 1, 7168, 56, 8, 128, 22016, 0, 1.2e8, 1e-5,
                     weight_seed=1002, prompt_seeds=(), prompt_len=0, chunk_rows=2048,
                     decode_steps=1,
                     extra={"cache_positions": 4096, "kv_seed": 3002, "input_seed": 3102,
                            "windows": (1, 16)}),
    3: LlamaGeometry("33b", 52, 1, 7168, 56, 8, 128, 22016, 166912, 1.2e8, 1e-5,
                     weight_seed=1003, prompt_seeds=(2003,), prompt_len=2048, chunk_rows=2048,
                     decode_steps=128),
    4: LlamaGeometry("looped", 22, 2, 3072, 48, 8, 128, 8192, 166912, 1.2e8, 1e-5,
                     weight_seed=1004, prompt_seeds=(2004,), prompt_len=512, chunk_rows=512,
                     decode_steps=256),
    5: LlamaGeometry("33b-long", 52, 1, 7168, 56, 8, 128, 22016, 166912, 1.2e8, 1e-5,
                     weight_seed=1005, prompt_seeds=(2005, 2006), prompt_len=131072,
                     chunk_rows=2048, decode_steps=64),
}


def config(i):
    return CONFIGS[i]


def weight_spec(g: LlamaGeometry):
    """(name, tensor id, shape, mean, std) of every stored weight, in load order.

    Shapes are [out][in] row-major, as the projections are stored."""
    H, F = g.hidden, g.ffn
    spec = []
    if g.vocab:
        spec.append(("embed", TensorIds.EMBED, (g.vocab, H), 0.0, 0.02))
    for b in range(g.n_blocks):
        t = TensorIds
        spec += [
            (f"b{b}.attn_norm", t.block(b, t.ATTN_NORM), (H,), 1.0, 0.02),
            (f"b{b}.q", t.block(b, t.Q), (g.q_dim, H), 0.0, 0.02),
            (f"b{b}.k", t.block(b, t.K), (g.kv_dim, H), 0.0, 0.02),
            (f"b{b}.v", t.block(b, t.V), (g.kv_dim, H), 0.0, 0.02),
            (f"b{b}.o", t.block(b, t.O), (H, g.q_dim), 0.0, 0.02),
            (f"b{b}.mlp_norm", t.block(b, t.MLP_NORM), (H,), 1.0, 0.02),
            (f"b{b}.gate", t.block(b, t.GATE), (F, H), 0.0, 0.02),
            (f"b{b}.up", t.block(b, t.UP), (F, H), 0.0, 0.02),
            (f"b{b}.down", t.block(b, t.DOWN), (H, F), 0.0, 0.02),
        ]
    if g.vocab:
        spec.append(("final_norm", TensorIds.FINAL_NORM, (H,), 1.0, 0.02))
        spec.append(("lm_head", TensorIds.LM_HEAD, (g.vocab, H), 0.0, 0.02))
    return spec
