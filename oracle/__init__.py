"""Plain CPU oracle of the dense grouped-query Llama forward step.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  It shares no
code with the HIP path (``dense_gqa_llama_amd``) and neither imports the
other.

``liboracle.so`` (``oracle.c``) holds the arithmetic, in binary64 between the
bf16 rounding points of Hugging Face modeling_llama; this module only marshals
numpy arrays of bf16 bit patterns (``uint16``) into it.  ``model.py`` composes
the steps into a forward pass.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int64


class Geom(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int64), ("n_q_heads", ctypes.c_int64),
                ("n_kv_heads", ctypes.c_int64), ("head_dim", ctypes.c_int64),
                ("ffn", ctypes.c_int64), ("rope_theta", ctypes.c_double),
                ("rms_eps", ctypes.c_float)]


class BlockWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "q", "k", "v", "o", "mlp_norm", "gate", "up", "down")]


def lib():
    global _lib
    if _lib is None:
        path = os.path.join(_HERE, "liboracle.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(path)
        L.orc_bf16.argtypes = [ctypes.c_double]
        L.orc_bf16.restype = ctypes.c_uint16
        L.orc_f64.argtypes = [ctypes.c_uint16]
        L.orc_f64.restype = ctypes.c_double
        L.orc_bf16_array.argtypes = [_P, _I, _P]
        L.orc_plant.argtypes = [ctypes.c_int]
        L.orc_embed.argtypes = [_P, _I, _I, _P, _I, _P]
        L.orc_rmsnorm.argtypes = [_P, _P, _I, _I, ctypes.c_float, _P]
        L.orc_linear.argtypes = [_P, _P, _I, _I, _I, _P, _P]
        L.orc_rope_inv_freq.argtypes = [_I, ctypes.c_double, _P]
        L.orc_rope.argtypes = [_P, _P, _I, _I, _I, ctypes.c_double]
        L.orc_attention.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _P, _P]
        L.orc_swiglu.argtypes = [_P, _P, _I, _P]
        L.orc_residual_add.argtypes = [_P, _P, _I]
        L.orc_argmax.argtypes = [_P, _I]
        L.orc_argmax.restype = ctypes.c_int32
        L.orc_sample.argtypes = [_P, _I, ctypes.c_double, ctypes.c_int32, ctypes.c_double,
                                 ctypes.c_double, _P]
        L.orc_sample.restype = ctypes.c_int32
        L.orc_block.argtypes = [ctypes.POINTER(Geom), ctypes.POINTER(BlockWeights), _P, _P, _I,
                                _P, _I, _P, _P]
        L.orc_block.restype = ctypes.c_int
        for name in ("orc_bf16_array", "orc_plant", "orc_embed", "orc_rmsnorm", "orc_linear",
                     "orc_rope_inv_freq", "orc_rope", "orc_attention", "orc_swiglu",
                     "orc_residual_add"):
            getattr(L, name).restype = None
        _lib = L
    return _lib


def _u16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, a.dtype
    return a


def _ptr(a):
    return a.ctypes.data if a is not None else None


# ------------------------------------------------------------- conversions --

def bf16(x):
    """binary64 values -> bf16 bit patterns (round to nearest, ties to even)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    lib().orc_bf16_array(x.ctypes.data, x.size, out.ctypes.data)
    return out


def f64(b):
    """bf16 bit patterns -> binary64 values (exact)."""
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def plant(code):
    lib().orc_plant(int(code))


# ------------------------------------------------------------------- steps --

def embed(E, tokens):
    E = _u16(E)
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    V, H = E.shape
    out = np.empty((tok.size, H), dtype=np.uint16)
    lib().orc_embed(E.ctypes.data, V, H, tok.ctypes.data, tok.size, out.ctypes.data)
    return out


def rmsnorm(h, w, eps):
    h, w = _u16(h), _u16(w)
    rows, H = h.reshape(-1, w.size).shape
    out = np.empty_like(h)
    lib().orc_rmsnorm(h.ctypes.data, w.ctypes.data, rows, H, float(eps), out.ctypes.data)
    return out


def linear(x, W, want64=False):
    x, W = _u16(x), _u16(W)
    N, K = W.shape
    rows = x.size // K
    y = np.empty((rows, N), dtype=np.uint16)
    y64 = np.empty((rows, N), dtype=np.float64) if want64 else None
    lib().orc_linear(x.ctypes.data, W.ctypes.data, rows, N, K, y.ctypes.data, _ptr(y64))
    return (y, y64) if want64 else y


def rope_inv_freq(d, theta):
    inv = np.empty(d // 2, dtype=np.float32)
    lib().orc_rope_inv_freq(d, float(theta), inv.ctypes.data)
    return inv


def rope(x, pos, heads, d, theta):
    """Returns a rotated copy of x [rows][heads*d]."""
    x = _u16(x).copy()
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    lib().orc_rope(x.ctypes.data, pos.ctypes.data, pos.size, heads, d, float(theta))
    return x


def attention(q, kc, vc, pos, nq, nkv, d, want64=False):
    q, kc, vc = _u16(q), _u16(kc), _u16(vc)
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    rows = pos.size
    out = np.empty((rows, nq * d), dtype=np.uint16)
    o64 = np.empty((rows, nq * d), dtype=np.float64) if want64 else None
    lib().orc_attention(q.ctypes.data, kc.ctypes.data, vc.ctypes.data, pos.ctypes.data, rows, nq,
                        nkv, d, out.ctypes.data, _ptr(o64))
    return (out, o64) if want64 else out


def swiglu(g, u):
    g, u = _u16(g), _u16(u)
    out = np.empty_like(g)
    lib().orc_swiglu(g.ctypes.data, u.ctypes.data, g.size, out.ctypes.data)
    return out


def residual_add(h, y):
    h = _u16(h).copy()
    lib().orc_residual_add(h.ctypes.data, _u16(y).ctypes.data, h.size)
    return h


def argmax(logits):
    """Greedy id of one bf16 logit row; -1 when the row holds NaN or +-Inf."""
    return int(lib().orc_argmax(_u16(logits).ctypes.data, logits.size))


def sample(logits, temperature, top_k, top_p, u):
    """Seeded top-k / top-p draw from one row of bf16 logits against the
    uniform ``u``; returns (token id or -1, decision margin)."""
    logits = _u16(logits)
    m = np.zeros(1, dtype=np.float64)
    t = lib().orc_sample(logits.ctypes.data, logits.size, float(temperature), int(top_k),
                         float(top_p), float(u), m.ctypes.data)
    return int(t), float(m[0])


def block(geom, w, kc, vc, pos, h, want_mid=False):
    """One block execution; kc/vc ([T][nkv][d] uint16) are updated in place,
    a new h is returned (and the mid-block residual when asked)."""
    g = Geom(geom.hidden, geom.n_q_heads, geom.n_kv_heads, geom.head_dim, geom.ffn,
             float(geom.rope_theta), float(geom.rms_eps))
    names = [f[0] for f in BlockWeights._fields_]
    arrs = {k: _u16(w[k]) for k in names}
    bw = BlockWeights(*[arrs[k].ctypes.data for k in names])
    assert kc.dtype == np.uint16 and kc.flags.c_contiguous
    assert vc.dtype == np.uint16 and vc.flags.c_contiguous
    pos = np.ascontiguousarray(pos, dtype=np.int32)
    h = _u16(h).copy()
    mid = np.empty_like(h) if want_mid else None
    T = kc.shape[0]
    rc = lib().orc_block(ctypes.byref(g), ctypes.byref(bw), kc.ctypes.data, vc.ctypes.data, T,
                         pos.ctypes.data, pos.size, h.ctypes.data, _ptr(mid))
    if rc != 0:
        raise ValueError("position outside the cache")
    return (h, mid) if want_mid else h
