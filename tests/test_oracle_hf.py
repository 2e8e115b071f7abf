"""The oracle's step functions against Hugging Face transformers' own Llama
modules in bf16 on the CPU: the pull request "llama: Nanbeige4.3-33B on
Metal, the bf16 release served as published" (section "Measured") measures
against HF's own code in bf16 on the CPU, and its section "How" lists HF's
rounding points as the spec.  LlamaRMSNorm, LlamaRotaryEmbedding with
apply_rotary_pos_emb, and LlamaMLP are run on the tiny geometry's weights and
on seeded inputs; the oracle must return the same bf16 values except where
HF's fp32 sums (an order the spec leaves open) and the oracle's binary64 sums
round to neighbouring bf16 values, i.e. within one bf16 step, on nearly every
element.  The agreement rates are printed.
"""
import numpy as np
import pytest

import oracle
from synth.workloads import TensorIds, config
from tests import parity
from tests.host_inputs import HostWeights

torch = pytest.importorskip("torch")
ml = pytest.importorskip("transformers.models.llama.modeling_llama")
LlamaConfig = pytest.importorskip("transformers").LlamaConfig


def _t(bits):
    """uint16 bf16 bits -> torch bf16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).view(torch.bfloat16)


def _bits(t):
    return t.detach().contiguous().view(torch.int16).numpy().view(np.uint16)


def _hf_config(g):
    return LlamaConfig(hidden_size=g.hidden, intermediate_size=g.ffn,
                       num_attention_heads=g.n_q_heads, num_key_value_heads=g.n_kv_heads,
                       head_dim=g.head_dim, vocab_size=g.vocab, rms_norm_eps=g.rms_eps,
                       rope_theta=g.rope_theta, max_position_embeddings=4096,
                       hidden_act="silu", attention_bias=False, mlp_bias=False)


def _agreement(tag, got, ref):
    d = parity.ulp_distance(got, ref)
    exact = float((got == ref).mean())
    print(f"{tag}: {exact:.5f} equal to the oracle, worst {d.max():g} bf16 steps")
    return exact, float(d.max())


@pytest.fixture(scope="module")
def tiny():
    import synth
    g = config(1)
    W = HostWeights(g)
    rows = 64
    x = synth.normal_bf16(rows * g.hidden, 3400, TensorIds.INPUT_ROWS).reshape(rows, g.hidden)
    return g, W, x


def test_rmsnorm_equals_hf(tiny):
    g, W, x = tiny
    m = ml.LlamaRMSNorm(g.hidden, eps=g.rms_eps).to(torch.bfloat16)
    with torch.no_grad():
        m.weight.copy_(_t(W("b0.attn_norm")))
        got = _bits(m(_t(x)))
    exact, worst = _agreement("RMSNorm", oracle.rmsnorm(x, W("b0.attn_norm"), g.rms_eps), got)
    assert worst <= 1 and exact >= 0.999


def test_rope_equals_hf(tiny):
    """Positions up to 4,000 (angles to 4,000 rad in the fastest pair)."""
    g, W, x = tiny
    hc = _hf_config(g)
    rot = ml.LlamaRotaryEmbedding(hc)
    q = oracle.linear(x, W("b0.q"))  # bf16 q rows
    k = oracle.linear(x, W("b0.k"))
    pos = np.linspace(0, 4000, x.shape[0]).astype(np.int32)
    qt = _t(q).view(1, -1, g.n_q_heads, g.head_dim).transpose(1, 2)
    kt = _t(k).view(1, -1, g.n_kv_heads, g.head_dim).transpose(1, 2)
    with torch.no_grad():
        cos, sin = rot(qt, torch.from_numpy(pos.astype(np.int64))[None, :])
        qe, ke = ml.apply_rotary_pos_emb(qt, kt, cos, sin)
    hq = _bits(qe.transpose(1, 2).reshape(x.shape[0], -1))
    hk = _bits(ke.transpose(1, 2).reshape(x.shape[0], -1))
    oq = oracle.rope(q, pos, g.n_q_heads, g.head_dim, g.rope_theta)
    ok = oracle.rope(k, pos, g.n_kv_heads, g.head_dim, g.rope_theta)
    eq, wq = _agreement("RoPE q", oq, hq)
    ek, wk = _agreement("RoPE k", ok, hk)
    assert max(wq, wk) <= 1 and min(eq, ek) >= 0.999


def test_mlp_equals_hf(tiny):
    """gate/up projections, SwiGLU and the down projection, each rounded to
    bf16 where modeling_llama rounds: each projection within one step of the
    oracle's (one rounding of a sum whose order the spec leaves open), SwiGLU
    on the same bf16 inputs bit for bit, and the composed MLP (reported: one
    SwiGLU value a step apart moves its whole output row by a fraction of a
    step) within two steps on >= 99.9% of elements."""
    g, W, x = tiny
    m = ml.LlamaMLP(_hf_config(g)).to(torch.bfloat16)
    with torch.no_grad():
        m.gate_proj.weight.copy_(_t(W("b0.gate")))
        m.up_proj.weight.copy_(_t(W("b0.up")))
        m.down_proj.weight.copy_(_t(W("b0.down")))
        xt = _t(x)
        hg, hu = m.gate_proj(xt), m.up_proj(xt)
        hact = m.act_fn(hg) * hu
        got = _bits(m.down_proj(hact))
        hdown = _bits(m.down_proj(hact))
    og, ou = oracle.linear(x, W("b0.gate")), oracle.linear(x, W("b0.up"))
    for tag, xin, wname, o, h in (
            ("gate projection", x, "b0.gate", og, _bits(hg)),
            ("up projection", x, "b0.up", ou, _bits(hu)),
            ("down projection (HF's own SwiGLU rows)", _bits(hact), "b0.down",
             oracle.linear(_bits(hact), W("b0.down")), hdown)):
        exact, worst = _agreement(tag, o, h)
        absum = np.abs(oracle.f64(xin)) @ np.abs(oracle.f64(W(wname))).T
        assert parity.sum_bound_ok(h, o, absum, xin.shape[1]).all()
        assert exact >= 0.999
    exact, worst = _agreement("SwiGLU (HF's own gate/up rows)", oracle.swiglu(_bits(hg), _bits(hu)),
                              _bits(hact))
    assert worst == 0
    ref = oracle.linear(oracle.swiglu(og, ou), W("b0.down"))
    exact, worst = _agreement("MLP", ref, got)
    within2, _ = parity.within_ulps(ref, got)
    print(f"MLP: {within2:.5f} within two bf16 steps")
    assert exact >= 0.99 and within2 >= 0.999
