"""Pins of the CPU oracle to facts outside itself: closed forms, library
routines, brute force on tiny inputs, the pages' printed numbers, and planted
mistakes that must be caught.  CPU only.

Passages cited are on the pull request "llama: Nanbeige4.3-33B on Metal, the
bf16 release served as published" (the rounding points, section "How"), the
NInfer model card "Nanbeige4.3-33B IQ3_XXS - NInfer v3" (architecture, section
"Provenance and representation"; FP64 checks, section "Validation") and the
Nanbeige4.2-3B MLX card (inv_freq pitfall, section "Verification").
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests.parity import bf16_round_f64

rng = np.random.default_rng(12345)


def bits(x):
    return oracle.bf16(np.asarray(x, dtype=np.float64))


def val(b):
    return oracle.f64(b)


def rand_bf16(shape, scale=1.0, gen=rng):
    return bits(gen.standard_normal(shape) * scale)


# ------------------------------------------------------------------ bf16 ----

def test_bf16_matches_torch_for_binary32_inputs():
    """Rounding of binary32 values agrees with PyTorch's float->bfloat16
    conversion (round to nearest even), the conversion the reference uses."""
    g = np.random.default_rng(1)
    f = np.concatenate([
        g.standard_normal(200000).astype(np.float32) * np.float32(37.0),
        (g.standard_normal(20000) * 1e-39).astype(np.float32),  # binary32 subnormals
        np.array([float.fromhex('0x1.FEp127'), float.fromhex('0x1.FFp127'),
                  -float.fromhex('0x1.FF8p127'), 3.0e38, 1e-45], dtype=np.float32),
    ])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (bits(f.astype(np.float64)) == ref).all()


def test_bf16_ties_and_specials():
    one = 1.0
    assert val(bits(one + 2.0 ** -8)) == 1.0                        # tie -> even (down)
    assert val(bits(one + 3 * 2.0 ** -8)) == 1.0 + 2.0 ** -6        # tie -> even (up)
    assert val(bits(one + 2.0 ** -8 + 2.0 ** -40)) == 1.0 + 2.0 ** -7  # above the tie
    assert val(bits(2.0 ** -133)) == 2.0 ** -133                    # smallest subnormal
    assert val(bits(2.0 ** -134)) == 0.0                            # tie with zero -> even
    assert val(bits(3 * 2.0 ** -134)) == 2.0 ** -132
    assert bits(float("inf")) == 0x7F80 and bits(-float("inf")) == 0xFF80
    assert bits(float.fromhex('0x1.FFp127')) == 0x7F80                               # rounds past max -> inf
    assert bits(float("nan")) == 0x7FC0
    assert bits(-0.0) == 0x8000


def test_bf16_row_1370_rounded_once(root):
    """The float64 logits printed for position 1370 round once to the printed
    bf16 values, and 38.1266 lies 0.0016 above the midpoint 38.125."""
    import csv
    with open(f"{root}/tests/golden/row1370.tsv") as fh:
        rows = list(csv.DictReader(fh, delimiter="\t"))
    for r in rows:
        assert val(bits(float(r["float64"]))) == float(r["rounded_once"])
    assert abs(38.1266 - 38.125 - 0.0016) < 1e-9


def test_bf16_step_sizes_from_the_pages():
    """One bf16 step is 0.125 below 32 and 0.25 from 32 to 64."""
    assert val(bits(31.9)) in (31.875, 32.0) and val(bits(20.70)) == 20.75
    assert val(bits(20.6)) == 20.625
    assert np.nextafter(np.float32(20.0), np.float32(99)) > 0  # keep numpy honest
    for v, step in ((20.75, 0.125), (31.875, 0.125), (38.25, 0.25), (63.75, 0.25)):
        b = bits(v)
        nxt = val(np.uint16(int(b.item()) + 1))
        assert nxt - v == step


# --------------------------------------------------------------- RMSNorm ----

@pytest.mark.parametrize("c", [1.0, 2.0 ** -8, 3.0, -0.375, 100.0])
@pytest.mark.parametrize("H", [512, 7168])
def test_rmsnorm_constant_vector_closed_form(c, H):
    """For h = c*1 and w = 1, mean(h^2) = c^2, so every output is
    bf16(c / sqrt(c^2 + eps))."""
    eps = np.float32(1e-5)
    h = np.full((1, H), bits(c), dtype=np.uint16)
    w = np.full(H, bits(1.0), dtype=np.uint16)
    out = oracle.rmsnorm(h, w, eps)
    expect = bf16_round_f64(c / math.sqrt(c * c + float(eps)))
    assert (val(out) == expect).all()


def test_rmsnorm_scale_and_weight():
    """Scaling h by a power of two leaves the output unchanged when eps = 0;
    a weight of 2 doubles it exactly; the output's mean square is 1 within
    bf16 rounding."""
    H = 1024
    h = rand_bf16((3, H), 0.7)
    w1 = np.full(H, bits(1.0), dtype=np.uint16)
    w2 = np.full(H, bits(2.0), dtype=np.uint16)
    a = oracle.rmsnorm(h, w1, 0.0)
    b = oracle.rmsnorm(bits(val(h) * 8.0), w1, 0.0)
    assert (a == b).all()
    assert (val(oracle.rmsnorm(h, w2, 0.0)) == 2 * val(a)).all()
    ms = (val(a) ** 2).mean(axis=1)
    assert np.allclose(ms, 1.0, atol=2 * 2.0 ** -8)


def test_rmsnorm_uses_each_weight_elementwise():
    H = 256
    h = np.full((1, H), bits(1.0), dtype=np.uint16)
    wv = np.arange(H) / 64.0 - 2.0
    out = oracle.rmsnorm(h, bits(wv), 1e-5)
    n = bf16_round_f64(1.0 / math.sqrt(1.0 + float(np.float32(1e-5))))
    assert (val(out[0]) == [bf16_round_f64(float(x) * n) for x in val(bits(wv))]).all()


# ------------------------------------------------------------ projection ----

def test_linear_identity_returns_x():
    K = 64
    x = rand_bf16((5, K))
    eye = bits(np.eye(K))
    assert (oracle.linear(x, eye) == x).all()


def test_linear_brute_force_exact_rational():
    """Each output is the exact sum of the bf16 products (computed with
    rationals) rounded once; the binary64 sums agree to 1e-12."""
    g = np.random.default_rng(7)
    rows, N, K = 3, 9, 40  # N != K so a transposed operand cannot pass
    x = rand_bf16((rows, K), 1.0, g)
    W = rand_bf16((N, K), 0.5, g)
    y, y64 = oracle.linear(x, W, want64=True)
    xf, Wf = val(x), val(W)
    for r in range(rows):
        for n in range(N):
            exact = sum(Fraction(float(Wf[n, k])) * Fraction(float(xf[r, k])) for k in range(K))
            e = float(exact)
            assert abs(y64[r, n] - e) <= 1e-12 * max(1.0, abs(e))
            assert val(y[r, n]) == bf16_round_f64(e)


# ------------------------------------------------------------------ RoPE ----

def test_rope_position_zero_is_identity():
    x = rand_bf16((2, 4 * 64))
    out = oracle.rope(x, [0, 0], 4, 64, 1e4)
    assert (out == x).all()


def test_rope_inverse_frequencies():
    """inv_0 = 1 exactly; at i = d/4 the power theta^(1/2) is sqrt(theta):
    100 for theta = 1e4 (d = 64), sqrt(1.2e8) for the 33B (d = 128)."""
    inv = oracle.rope_inv_freq(64, 1e4)
    assert inv[0] == 1.0
    assert inv[16] == np.float32(1.0) / np.float32(100.0)
    inv = oracle.rope_inv_freq(128, 1.2e8)
    assert inv[0] == 1.0
    assert inv[32] == np.float32(1.0) / np.float32(math.sqrt(1.2e8))
    # decreasing geometric sequence with ratio theta^(-2/d)
    r = inv[1:].astype(np.float64) / inv[:-1]
    assert np.allclose(r, 1.2e8 ** (-2 / 128), rtol=1e-6)


@pytest.mark.parametrize("p", [1, 7, 100, 4095, 131071])
def test_rope_rotates_pairs_counterclockwise(p):
    """A unit vector on the first element of pair i rotates to
    (cos a, sin a); one on the second to (-sin a, cos a), a = p * inv_i in
    binary32, cos/sin rounded to binary32 then bf16."""
    d, heads, theta = 128, 1, 1.2e8
    # closed-form frequencies: theta^0 = 1 and theta^(1/2) = sqrt(theta)
    inv = {0: np.float32(1.0), d // 4: np.float32(1.0) / np.float32(math.sqrt(theta))}
    for i in (0, d // 4):
        a = float(np.float32(np.float64(p) * np.float64(inv[i])))
        c = bf16_round_f64(float(np.float32(math.cos(a))))
        s = bf16_round_f64(float(np.float32(math.sin(a))))
        x = np.zeros((1, d))
        x[0, i] = 1.0
        out = val(oracle.rope(bits(x), [p], heads, d, theta))[0]
        assert out[i] == c and out[i + d // 2] == s
        assert np.count_nonzero(out) <= 2
        x = np.zeros((1, d))
        x[0, i + d // 2] = 1.0
        out = val(oracle.rope(bits(x), [p], heads, d, theta))[0]
        assert out[i] == -s and out[i + d // 2] == c


def test_rope_norm_preserved_within_rounding():
    d, heads = 128, 4
    x = rand_bf16((6, heads * d))
    pos = [3, 50, 999, 4096, 70000, 131071]
    out = val(oracle.rope(x, pos, heads, d, 1.2e8)).reshape(6, heads, 2, d // 2)
    xin = val(x).reshape(6, heads, 2, d // 2)
    n_in = np.hypot(xin[:, :, 0], xin[:, :, 1])
    n_out = np.hypot(out[:, :, 0], out[:, :, 1])
    # cos/sin (2^-9 each), two products and the sum (2^-9 each) -> well under 2^-6
    assert np.all(np.abs(n_out - n_in) <= 2.0 ** -6 * n_in + 1e-30)


def _relative_dot(pos_q, pos_k, d=64, theta=1e4, seed=3):
    g = np.random.default_rng(seed)
    q = rand_bf16((1, d), 1.0, g)
    k = rand_bf16((1, d), 1.0, g)
    rq = val(oracle.rope(q, [pos_q], 1, d, theta))[0]
    rk = val(oracle.rope(k, [pos_k], 1, d, theta))[0]
    return float(rq @ rk), float(np.abs(val(q)).sum() * np.abs(val(k)).max())


def test_rope_relative_position_invariance():
    """<R_m q, R_n k> depends only on m - n (within the bf16 rounding bound)
    and changes with m - n."""
    for shift in (1, 17, 1000):
        a, bound = _relative_dot(40, 30)
        b, _ = _relative_dot(40 + shift, 30 + shift)
        assert abs(a - b) <= 2.0 ** -6 * bound
    # for q = k = e_0 (frequency 1 rad per position) the product is cos(m - n)
    e0 = np.zeros((1, 64)); e0[0, 0] = 1.0
    for m, n in ((40, 30), (40, 10), (7, 7)):
        rq = val(oracle.rope(bits(e0), [m], 1, 64, 1e4))[0]
        rk = val(oracle.rope(bits(e0), [n], 1, 64, 1e4))[0]
        assert abs(float(rq @ rk) - math.cos(m - n)) <= 2.0 ** -7


def test_planted_zero_inv_freq_is_caught():
    """Leaving inv_freq at zero (the non-persistent buffer pitfall) makes RoPE
    a no-op; the rotation pin must then fail."""
    oracle.plant(1)
    try:
        with pytest.raises(AssertionError):
            test_rope_rotates_pairs_counterclockwise(7)
    finally:
        oracle.plant(0)
    test_rope_rotates_pairs_counterclockwise(7)


# ------------------------------------------------------------- attention ----

def test_attention_values_of_one_give_one():
    """Softmax weights sum to 1: with every value 1 the output is exactly 1."""
    nq, nkv, d, T = 4, 2, 16, 37
    q = rand_bf16((3, nq * d))
    kc = rand_bf16((T, nkv, d))
    vc = np.full((T, nkv, d), bits(1.0), dtype=np.uint16)
    out = oracle.attention(q, kc, vc, [0, 20, 36], nq, nkv, d)
    assert (val(out) == 1.0).all()


def test_attention_single_key_returns_its_value():
    nq, nkv, d = 2, 1, 8
    q = rand_bf16((1, nq * d))
    kc = rand_bf16((4, nkv, d))
    vc = rand_bf16((4, nkv, d))
    out = oracle.attention(q, kc, vc, [0], nq, nkv, d)
    assert (out.reshape(nq, d) == vc[0, 0]).all()


def test_attention_two_keys_sigmoid_closed_form():
    """Two keys whose scores differ by 1 after the 1/sqrt(d) scale: the
    weight on the second is e/(1+e), so with values 0 and 1 the output is
    bf16(e/(1+e)).  A wrong scale (1/d, none) would move it."""
    d = 64
    q = np.zeros((1, d)); q[0, 0] = 1.0
    kc = np.zeros((2, 1, d)); kc[1, 0, 0] = 8.0  # q.k1 = 8 = sqrt(64)
    vc = np.zeros((2, 1, d)); vc[1, 0, :] = 1.0
    out = val(oracle.attention(bits(q), bits(kc), bits(vc), [1], 1, 1, d))
    expect = bf16_round_f64(math.e / (1.0 + math.e))
    assert (out == expect).all()


def test_attention_brute_force_masked_matrix():
    """Against a dense masked score matrix (numpy, -inf above the diagonal)
    on tiny shapes: the binary64 outputs agree to 1e-12 and the bf16 outputs
    match except at rounding midpoints."""
    g = np.random.default_rng(11)
    nq, nkv, d, T = 6, 2, 16, 24
    rows = 5
    pos = np.array([3, 9, 10, 17, 23], dtype=np.int32)
    q = rand_bf16((rows, nq * d), 1.0, g)
    kc = rand_bf16((T, nkv, d), 1.0, g)
    vc = rand_bf16((T, nkv, d), 1.0, g)
    out, o64 = oracle.attention(q, kc, vc, pos, nq, nkv, d, want64=True)
    Q = val(q).reshape(rows, nq, d)
    K = val(kc)
    V = val(vc)
    rep = nq // nkv
    for h in range(nq):
        Kh = K[:, h // rep, :]
        Vh = V[:, h // rep, :]
        S = Q[:, h, :] @ Kh.T / math.sqrt(d)
        mask = np.arange(T)[None, :] > pos[:, None]
        S = np.where(mask, -np.inf, S)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        P /= P.sum(axis=1, keepdims=True)
        O = P @ Vh
        assert np.allclose(o64.reshape(rows, nq, d)[:, h, :], O, rtol=1e-12, atol=1e-14)
        got = val(out).reshape(rows, nq, d)[:, h, :]
        want = np.vectorize(bf16_round_f64)(O)
        assert (got == want).mean() > 0.999


def test_attention_gqa_head_mapping():
    """Query head h reads KV head h // (nq/nkv): give KV head g values g+1."""
    nq, nkv, d, T = 56, 8, 16, 5
    q = rand_bf16((1, nq * d))
    kc = rand_bf16((T, nkv, d))
    vc = np.zeros((T, nkv, d))
    for gi in range(nkv):
        vc[:, gi, :] = gi + 1
    out = val(oracle.attention(q, kc, bits(vc), [T - 1], nq, nkv, d)).reshape(nq, d)
    for h in range(nq):
        assert (out[h] == h // 7 + 1).all()


def test_attention_is_causal():
    nq, nkv, d, T = 4, 2, 16, 30
    q = rand_bf16((1, nq * d))
    kc = rand_bf16((T, nkv, d))
    vc = rand_bf16((T, nkv, d))
    a = oracle.attention(q, kc, vc, [12], nq, nkv, d)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[13:] = rand_bf16((T - 13, nkv, d))
    vc2[13:] = rand_bf16((T - 13, nkv, d))
    assert (oracle.attention(q, kc2, vc2, [12], nq, nkv, d) == a).all()
    kc2[12] = rand_bf16((nkv, d))
    assert (oracle.attention(q, kc2, vc, [12], nq, nkv, d) != a).any()


# ----------------------------------------------------------------- SwiGLU ---

def test_swiglu_closed_forms():
    g = bits([0.0, 1.0, 100.0, -100.0, 2.0])
    u = bits([5.0, 1.0, 1.0, 1.0, 2.0])
    out = val(oracle.swiglu(g, u))
    assert out[0] == 0.0                                    # silu(0) = 0
    assert out[1] == bf16_round_f64(1.0 / (1.0 + math.exp(-1.0)))   # sigma(1)
    assert out[2] == 100.0                                  # silu(x) -> x
    assert out[3] == 0.0 or abs(out[3]) < 1e-40             # silu(-100) ~ -3.7e-42
    s2 = bf16_round_f64(2.0 / (1.0 + math.exp(-2.0)))
    assert out[4] == bf16_round_f64(s2 * 2.0)               # silu rounded before the product


def test_swiglu_odd_part_identity():
    """silu(g) - silu(-g) = g exactly in real arithmetic; with bf16 rounding of
    each silu the gap stays within two steps."""
    g = rand_bf16(2000, 3.0)
    one = np.full(2000, bits(1.0), dtype=np.uint16)
    a = val(oracle.swiglu(g, one))
    b = val(oracle.swiglu(bits(-val(g)), one))
    gv = val(g)
    step = np.exp2(np.floor(np.log2(np.maximum(np.abs(gv), 1e-30))) - 7)
    assert np.all(np.abs(a - b - gv) <= 2 * step + 1e-30)


def test_residual_add_rounds_once():
    h = bits([1.0, 1.0, 256.0, -3.0])
    y = bits([2.0 ** -8, 3 * 2.0 ** -8, 1.0, 3.0])
    out = val(oracle.residual_add(h, y))
    assert list(out) == [1.0, 1.0 + 2.0 ** -6, 256.0, 0.0]


# ---------------------------------------------------------------- argmax ----

def test_argmax_ties_to_lowest_and_refuses_non_finite():
    assert oracle.argmax(bits([1.0, 3.0, 3.0, 2.0])) == 1
    assert oracle.argmax(bits([5.0, 5.0])) == 0
    assert oracle.argmax(bits([-1.0, -0.5, -2.0])) == 1
    for bad in (float("nan"), float("inf"), -float("inf")):
        assert oracle.argmax(bits([bad, 0.0, 1.0])) == -1
        assert oracle.argmax(bits([0.0, 1.0, bad])) == -1


def test_embed_gathers_rows():
    E = rand_bf16((10, 8))
    out = oracle.embed(E, [3, 0, 9, 3])
    assert (out == E[[3, 0, 9, 3]]).all()


def test_uniform_generator_range_and_moments():
    """The shared 24-bit uniform generator: values k * 2^-24 in [0, 1), mean
    1/2 and variance 1/12 to within sampling error, independent of offset."""
    import synth
    u = synth.uniform_f32(200000, 4500, 30)
    assert u.min() >= 0.0 and u.max() < 1.0
    assert np.all(u * 16777216.0 == np.floor(u * 16777216.0))
    assert abs(u.mean() - 0.5) < 0.005 and abs(u.var() - 1.0 / 12) < 0.002
    assert np.array_equal(synth.uniform_f32(100, 4500, 30, offset=1000), u[1000:1100])
