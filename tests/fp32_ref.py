"""A second reference of one block execution: the same rounding points as the
oracle (bf16 after every step the spec rounds), with every sum in between in
float32 through numpy's BLAS matrix products instead of the oracle's binary64.

It is the arithmetic of an ordinary fp32 implementation of the spec (what
Hugging Face modeling_llama does on a CPU with fp32 accumulation), so its
distance from the oracle shows how far any in-spec fp32 implementation lands
from the binary64 one: a one-step difference of an intermediate bf16 value
(an fp32 sum on the other side of a rounding boundary) moves every output
that reads it, and where a residual add cancels, a one-step change of an
addend is many steps of the small sum.  Test infrastructure; it shares no
code with the HIP path.  RoPE is taken from the oracle: its products of bf16
values are exact in float32 as in binary64."""
import numpy as np

import oracle


def f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16(x):
    """float32 -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def rmsnorm(h, w, eps):
    x = f32(h)
    var = np.mean(x * x, axis=-1, dtype=np.float32, keepdims=True)
    r = np.float32(1.0) / np.sqrt(var + np.float32(eps))
    return bf16(f32(w)[None, :] * f32(bf16(x * r)))


def linear(x, W):
    return bf16(f32(x) @ f32(W).T)


def attention(q, kc, vc, pos, nq, nkv, d):
    """Causal GQA attention of rows at positions pos over caches [T][nkv][d]:
    float32 scores, softmax and weighted sum, rounded once."""
    rows = q.shape[0]
    G = nq // nkv
    qf = f32(q).reshape(rows, nq, d)
    out = np.empty((rows, nq, d), dtype=np.float32)
    T = int(np.max(pos)) + 1
    K = f32(kc[:T])
    V = f32(vc[:T])
    scale = np.float32(1.0 / np.sqrt(d))
    mask = np.arange(T)[None, :] > np.asarray(pos)[:, None]
    for h in range(nq):
        s = (qf[:, h, :] @ K[:, h // G, :].T) * scale
        s[mask] = -np.inf
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s, dtype=np.float32)
        p /= p.sum(axis=1, dtype=np.float32, keepdims=True)
        out[:, h, :] = p @ V[:, h // G, :]
    return bf16(out.reshape(rows, nq * d))


def swiglu(g, u):
    gf = f32(g)
    s = bf16(gf / (np.float32(1.0) + np.exp(-gf)))
    return bf16(f32(s) * f32(u))


def residual_add(h, y):
    return bf16(f32(h) + f32(y))


def attn_half(geom, w, kc, vc, pos, h, rows):
    """The attention half of one execution over rows at positions pos: every
    row's key and value stored at its slot (into copies of kc, vc), then the
    selected rows (indexes into h) attend.  Returns their residual rows."""
    g = geom
    pos = np.asarray(pos, dtype=np.int32)
    rows = np.asarray(rows)
    kc = kc.copy()
    vc = vc.copy()
    x = rmsnorm(h, w["attn_norm"], g.rms_eps)
    k = oracle.rope(linear(x, w["k"]), pos, g.n_kv_heads, g.head_dim, g.rope_theta)
    kc[pos] = k.reshape(-1, g.n_kv_heads, g.head_dim)
    vc[pos] = linear(x, w["v"]).reshape(-1, g.n_kv_heads, g.head_dim)
    xs = np.ascontiguousarray(x[rows])
    q = oracle.rope(linear(xs, w["q"]), pos[rows], g.n_q_heads, g.head_dim, g.rope_theta)
    a = attention(q, kc, vc, pos[rows], g.n_q_heads, g.n_kv_heads, g.head_dim)
    return residual_add(np.ascontiguousarray(h[rows]), linear(a, w["o"]))


def mlp_half(geom, w, mid):
    x = rmsnorm(mid, w["mlp_norm"], geom.rms_eps)
    m = swiglu(linear(x, w["gate"]), linear(x, w["up"]))
    return residual_add(mid, linear(m, w["down"]))


KINDS = ("attn_norm", "q", "k", "v", "o", "mlp_norm", "gate", "up", "down")


def forward(geom, W, tokens):
    """A whole prompt through the model: every block execution of every loop
    over all rows, the final norm at the end of every loop (its output
    replacing the residual), then lm_head.  Returns (float32 logit sums,
    their bf16 bits).  W: host weights by name."""
    g = geom
    n = len(tokens)
    pos = np.arange(n, dtype=np.int32)
    rows = np.arange(n)
    h = oracle.embed(W("embed"), tokens)
    for _ in range(g.n_loops):
        for b in range(g.n_blocks):
            blk = {k: W(f"b{b}.{k}") for k in KINDS}
            kc = np.zeros((n, g.n_kv_heads, g.head_dim), dtype=np.uint16)
            mid = attn_half(g, blk, kc, kc.copy(), pos, h, rows)
            h = mlp_half(g, blk, mid)
        h = rmsnorm(h, W("final_norm"), g.rms_eps)
    logits = f32(h) @ f32(W("lm_head")).T
    return logits, bf16(logits)
