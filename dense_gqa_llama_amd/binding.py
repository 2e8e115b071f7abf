"""ctypes binding of libllama_mi355x.so, with the C-ABI's own names.

Argument marshalling only: every step of the forward pass runs in the HIP
library.  Pointers are passed as integers (device addresses, e.g.
``tensor.data_ptr()``); streams as hipStream_t handles
(``torch.cuda.current_stream().cuda_stream``).  A negative return code raises
:class:`LlamaError` carrying the library's reason.  If the library is not
built this module raises at import: there is no fallback.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libllama_mi355x.so")

LLAMA_OK = 0
LLAMA_E_ARG = -1
LLAMA_E_GEOMETRY = -2
LLAMA_E_CAPACITY = -3
LLAMA_E_POSITION = -4
LLAMA_E_DEVICE = -5
LLAMA_E_NONFINITE = -6
LLAMA_E_WORKSPACE = -7
_NAMES = {0: "LLAMA_OK", -1: "LLAMA_E_ARG", -2: "LLAMA_E_GEOMETRY", -3: "LLAMA_E_CAPACITY",
          -4: "LLAMA_E_POSITION", -5: "LLAMA_E_DEVICE", -6: "LLAMA_E_NONFINITE",
          -7: "LLAMA_E_WORKSPACE"}


class LlamaError(RuntimeError):
    def __init__(self, code, reason):
        super().__init__(f"{_NAMES.get(code, code)}: {reason}")
        self.code = code
        self.reason = reason


class llama_config(ctypes.Structure):
    _fields_ = [("n_blocks", ctypes.c_int32), ("n_loops", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("rope_theta", ctypes.c_double), ("rms_eps", ctypes.c_float),
                ("max_chunk_rows", ctypes.c_int32), ("max_window_rows", ctypes.c_int32),
                ("max_seqs", ctypes.c_int32), ("prompt_exact", ctypes.c_int32)]


BLOCK_FIELDS = ("attn_norm", "q", "k", "v", "o", "mlp_norm", "gate", "up", "down")


class llama_block_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BLOCK_FIELDS]


_P = ctypes.c_void_p
_SIGS = {
    "llama_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(llama_config), ctypes.c_int32]),
    "llama_load_weights": (ctypes.c_int, [ctypes.POINTER(llama_config),
                                          ctypes.POINTER(llama_block_weights), _P, _P, _P, _P,
                                          ctypes.c_size_t, ctypes.c_int32,
                                          ctypes.POINTER(_P)]),
    "llama_kv_bytes": (ctypes.c_size_t, [_P, ctypes.c_int32]),
    "llama_kv_alloc": (ctypes.c_int, [_P, ctypes.c_int32, _P, ctypes.c_size_t,
                                      ctypes.POINTER(_P)]),
    "llama_kv_length": (ctypes.c_int32, [_P]),
    "llama_kv_truncate": (ctypes.c_int, [_P, ctypes.c_int32]),
    "llama_test_kv_declare": (ctypes.c_int, [_P, ctypes.c_int32]),
    "llama_kv_slab": (_P, [_P, ctypes.c_int32, ctypes.c_int32]),
    "llama_prefill_chunk": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P,
                                           _P, ctypes.c_int32, _P, _P]),
    "llama_decode_step": (ctypes.c_int, [_P, ctypes.POINTER(_P), ctypes.c_int32, _P, _P,
                                         ctypes.c_int32, _P, _P, _P, _P, _P]),
    "llama_set_capture": (ctypes.c_int, [_P, _P, ctypes.c_size_t]),
    "llama_set_probe": (ctypes.c_int, [_P, ctypes.c_int32, _P, ctypes.c_int32]),
    "llama_test_linear": (ctypes.c_int, [_P, ctypes.c_int32, _P, ctypes.c_int32, _P,
                                         ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "llama_test_attention": (ctypes.c_int, [_P, ctypes.c_int32, _P, ctypes.c_int32, _P,
                                            ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "llama_check_finite": (ctypes.c_int, [_P, _P]),
    "llama_sample": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                    ctypes.c_int32, ctypes.c_float, _P, _P, _P]),
    "llama_sample_noalloc": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64,
                                            ctypes.c_float, ctypes.c_int32, ctypes.c_float, _P,
                                            _P, _P]),
    "llama_draft_round": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int32, _P, _P,
                                          ctypes.POINTER(ctypes.c_int32), _P]),
    "llama_draft_round_sampled": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int32, _P,
                                                  ctypes.c_float, ctypes.c_int32, ctypes.c_float,
                                                  _P, _P, ctypes.POINTER(ctypes.c_int32), _P]),
    "llama_set_timing": (ctypes.c_int, [_P, ctypes.c_int32, ctypes.c_int32]),
    "llama_timing_read": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_double),
                                         ctypes.POINTER(ctypes.c_int64)]),
    "llama_kv_free": (None, [_P]),
    "llama_free": (None, [_P]),
    "llama_last_error": (ctypes.c_char_p, []),
}

EXPORTS = tuple(_SIGS)


def _share_torch_runtime():
    """PyTorch ships its own HIP runtime (same SONAME, libamdhip64.so.7).  If
    this library were loaded first it would pull in the system copy and torch
    would later load a second runtime instance, which then owns the device.
    Importing torch first makes the dynamic loader bind this library to the
    runtime torch uses, so device memory and streams are shared."""
    try:
        import torch  # noqa: F401
    except ImportError:
        pass


def _load():
    _share_torch_runtime()
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def last_error():
    return (lib.llama_last_error() or b"").decode()


def _check(rc):
    if rc != LLAMA_OK:
        raise LlamaError(rc, last_error())
    return rc


def make_config(n_blocks, n_loops, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab,
                rope_theta, rms_eps, max_chunk_rows=2048, max_window_rows=16, max_seqs=2,
                prompt_exact=0):
    return llama_config(n_blocks, n_loops, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab,
                        float(rope_theta), float(rms_eps), max_chunk_rows, max_window_rows,
                        max_seqs, int(prompt_exact))


def llama_workspace_bytes(cfg, max_positions):
    return lib.llama_workspace_bytes(ctypes.byref(cfg), max_positions)


def llama_load_weights(cfg, blocks, embed, final_norm, lm_head, workspace, workspace_bytes,
                       max_positions):
    """blocks: sequence of dicts (field -> device address).  Returns the model
    handle (an integer)."""
    arr = (llama_block_weights * len(blocks))()
    for i, b in enumerate(blocks):
        for f in BLOCK_FIELDS:
            setattr(arr[i], f, b[f])
    out = _P()
    _check(lib.llama_load_weights(ctypes.byref(cfg), arr, embed, final_norm, lm_head, workspace,
                                  workspace_bytes, max_positions, ctypes.byref(out)))
    return out.value


def llama_kv_bytes(model, max_positions):
    return lib.llama_kv_bytes(model, max_positions)


def llama_kv_alloc(model, max_positions, buf, nbytes):
    out = _P()
    _check(lib.llama_kv_alloc(model, max_positions, buf, nbytes, ctypes.byref(out)))
    return out.value


def llama_kv_length(kv):
    return lib.llama_kv_length(kv)


def llama_kv_truncate(kv, n):
    return _check(lib.llama_kv_truncate(kv, n))


def llama_test_kv_declare(kv, n):
    return _check(lib.llama_test_kv_declare(kv, n))


def llama_kv_slab(kv, exec_index, which):
    return lib.llama_kv_slab(kv, exec_index, which)


def llama_prefill_chunk(model, kv, tokens, hidden_in, n_rows, pos0, hidden_out=None,
                        logits_bf16=None, logits_f32=None, all_rows=0, next_token=None,
                        stream=None):
    return _check(lib.llama_prefill_chunk(model, kv, tokens, hidden_in, n_rows, pos0, hidden_out,
                                          logits_bf16, logits_f32, all_rows, next_token, stream))


def llama_decode_step(model, kvs, tokens, hidden_in, rows, hidden_out=None, logits_bf16=None,
                      logits_f32=None, next_tokens=None, stream=None):
    arr = (_P * len(kvs))(*kvs)
    return _check(lib.llama_decode_step(model, arr, len(kvs), tokens, hidden_in, rows,
                                        hidden_out, logits_bf16, logits_f32, next_tokens, stream))


def llama_set_capture(model, buf, nbytes):
    return _check(lib.llama_set_capture(model, buf, nbytes))


PROBE_FIELDS = ("h_in", "x_attn", "qkv32", "q_rope", "attn", "attn32", "o32", "x_mlp",
                "gate_up32", "act", "down32")


class llama_probe(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in PROBE_FIELDS]


def llama_set_probe(model, exec_index, buffers, max_rows):
    """buffers: dict field -> device address (missing fields are NULL), or
    None to clear the hook."""
    if buffers is None:
        return _check(lib.llama_set_probe(model, 0, None, 0))
    pr = llama_probe(*[buffers.get(f) for f in PROBE_FIELDS])
    return _check(lib.llama_set_probe(model, exec_index, ctypes.byref(pr), max_rows))


def llama_test_linear(model, prompt_kernel, x, rows, w, n, k, y, y32, stream=None):
    return _check(lib.llama_test_linear(model, int(prompt_kernel), x, rows, w, n, k, y, y32,
                                        stream))


def llama_test_attention(model, prompt_kernel, kv, exec_index, q, rows, pos0, out, out32=None,
                         stream=None):
    return _check(lib.llama_test_attention(model, int(prompt_kernel), kv, exec_index, q, rows,
                                           pos0, out, out32, stream))


def llama_check_finite(model, stream=None):
    return _check(lib.llama_check_finite(model, stream))


def llama_sample(model, logits_bf16, rows, ld, temperature, top_k, top_p, u, tokens, stream=None):
    return _check(lib.llama_sample(model, logits_bf16, rows, ld, temperature, top_k, top_p, u,
                                   tokens, stream))


def llama_sample_noalloc(logits_bf16, vocab, rows, ld, temperature, top_k, top_p, u, tokens,
                         stream=None):
    return _check(lib.llama_sample_noalloc(logits_bf16, vocab, rows, ld, temperature, top_k, top_p,
                                           u, tokens, stream))


def llama_draft_round(target, target_kv, draft, draft_kv, n_draft, last_token, tokens_out,
                      stream=None):
    """Returns the number of tokens the round wrote to tokens_out."""
    n = ctypes.c_int32(0)
    _check(lib.llama_draft_round(target, target_kv, draft, draft_kv, n_draft, last_token,
                                 tokens_out, ctypes.byref(n), stream))
    return n.value


def llama_draft_round_sampled(target, target_kv, draft, draft_kv, n_draft, last_token,
                              temperature, top_k, top_p, u, tokens_out, stream=None):
    """Returns the number of tokens the round wrote to tokens_out."""
    n = ctypes.c_int32(0)
    _check(lib.llama_draft_round_sampled(target, target_kv, draft, draft_kv, n_draft, last_token,
                                         temperature, top_k, top_p, u, tokens_out,
                                         ctypes.byref(n), stream))
    return n.value


TIMING = {"off": 0, "gate_up": 1, "down": 2, "qkv": 3, "o": 4, "lm_head": 5, "attn": 6,
          "prefill_gemm": 7, "prefill_attn": 8}


def llama_set_timing(model, kernel, max_launches=0):
    return _check(lib.llama_set_timing(model, TIMING.get(kernel, kernel), max_launches))


def llama_timing_read(model):
    """Returns (summed milliseconds, launches) since the previous read."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(lib.llama_timing_read(model, ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def llama_kv_free(kv):
    lib.llama_kv_free(kv)


def llama_free(model):
    lib.llama_free(model)
