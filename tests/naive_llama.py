"""An independent, whole-sequence numpy rewrite of the forward pass, used only
to cross-check the C oracle on tiny shapes.

It is organised differently on purpose: all rows at once, dense masked score
matrices per head, numpy BLAS for products in binary64, a vectorised bf16
rounding of its own, and RoPE written as a rotation of (first-half,
second-half) pairs.  Same spec (Hugging Face modeling_llama's bf16 rounding
points), different code.
"""
import numpy as np


def rnd(x):
    """binary64 -> nearest bf16 value (ties to even), as binary64."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(np.abs(x))
    q = np.maximum(e - 8, -133)
    r = np.rint(np.ldexp(np.abs(x), -q))  # rint: ties to even
    return np.copysign(np.ldexp(r, q), x)


def f(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)


def rmsnorm(h, w, eps):
    ms = (h * h).mean(axis=-1, keepdims=True)
    return rnd(w * rnd(h / np.sqrt(ms + float(np.float32(eps)))))


def rope(x, pos, d, theta):
    """x: [rows, heads, d] bf16 values."""
    half = d // 2
    expo = (np.arange(half, dtype=np.float32) * np.float32(2)) / np.float32(d)
    pw = np.power(np.float64(np.float32(theta)), expo.astype(np.float64)).astype(np.float32)
    inv = np.float32(1.0) / pw
    ang = (pos.astype(np.float64)[:, None] * inv.astype(np.float64)[None, :]).astype(np.float32)
    c = rnd(np.cos(ang.astype(np.float64)).astype(np.float32).astype(np.float64))[:, None, :]
    s = rnd(np.sin(ang.astype(np.float64)).astype(np.float32).astype(np.float64))[:, None, :]
    a, b = x[..., :half], x[..., half:]
    first = rnd(rnd(a * c) + rnd(-b * s))
    second = rnd(rnd(b * c) + rnd(a * s))
    return np.concatenate([first, second], axis=-1)


def forward(g, W, tokens):
    """Prefill of ``tokens`` from an empty cache; returns (logits64 [rows][V],
    per-execution outputs)."""
    rows = len(tokens)
    H, d, nq, nkv = g.hidden, g.head_dim, g.n_q_heads, g.n_kv_heads
    pos = np.arange(rows)
    h = f(W["embed"])[np.asarray(tokens)]
    outs = []
    for loop in range(g.n_loops):
        for b in range(g.n_blocks):
            p = lambda k: f(W[f"b{b}.{k}"])  # noqa: E731
            x = rmsnorm(h, p("attn_norm"), g.rms_eps)
            q = rnd(x @ p("q").T).reshape(rows, nq, d)
            k = rnd(x @ p("k").T).reshape(rows, nkv, d)
            v = rnd(x @ p("v").T).reshape(rows, nkv, d)
            q = rope(q, pos, d, g.rope_theta)
            k = rope(k, pos, d, g.rope_theta)
            att = np.empty((rows, nq, d))
            causal = np.triu(np.ones((rows, rows), dtype=bool), 1)
            for hh in range(nq):
                kv = hh * nkv // nq
                S = q[:, hh, :] @ k[:, kv, :].T / np.sqrt(d)
                S[causal] = -np.inf
                P = np.exp(S - S.max(axis=1, keepdims=True))
                P = P / P.sum(axis=1, keepdims=True)
                att[:, hh, :] = rnd(P @ v[:, kv, :])
            h = rnd(h + rnd(att.reshape(rows, nq * d) @ p("o").T))
            x = rmsnorm(h, p("mlp_norm"), g.rms_eps)
            gt = rnd(x @ p("gate").T)
            up = rnd(x @ p("up").T)
            m = rnd(rnd(gt / (1.0 + np.exp(-gt))) * up)
            h = rnd(h + rnd(m @ p("down").T))
            outs.append(h.copy())
        h = rmsnorm(h, f(W["final_norm"]), g.rms_eps)
    return h @ f(W["lm_head"]).T, outs
