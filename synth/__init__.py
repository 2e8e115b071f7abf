"""Seeded synthetic inputs: weights, caches and prompt tokens.

Both the CPU oracle's tests and the HIP path's tests and benchmark take their
inputs from here; the module holds none of the forward step's arithmetic.  The
generator (SplitMix64 streams, Irwin-Hall normal deviates, multiply-shift token
ids) is defined in ``synth_core.h``; ``libsynth.so`` runs it on the host and
``libsynth_dev.so`` on the GPU, bit-identically.
"""
import ctypes
import os

import numpy as np

from .workloads import (  # noqa: F401  (re-exported)
    CONFIGS,
    LlamaGeometry,
    TensorIds,
    config,
)

_HERE = os.path.dirname(os.path.abspath(__file__))
_host = None
_dev = None


def _load_host():
    global _host
    if _host is None:
        path = os.path.join(_HERE, "libsynth.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.synth_normal_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_int64, ctypes.c_double,
                                          ctypes.c_double]
        lib.synth_normal_bf16.restype = None
        lib.synth_tokens.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                     ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32]
        lib.synth_tokens.restype = None
        lib.synth_uniform_f32.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_int64]
        lib.synth_uniform_f32.restype = None
        _host = lib
    return _host


def _load_dev():
    global _dev
    if _dev is None:
        # bind to the HIP runtime PyTorch already loaded (see
        # dense_gqa_llama_amd.binding) rather than a second system copy
        import torch  # noqa: F401
        path = os.path.join(_HERE, "libsynth_dev.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        lib.synth_normal_bf16_dev.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                              ctypes.c_uint64, ctypes.c_int64, ctypes.c_double,
                                              ctypes.c_double, ctypes.c_void_p]
        lib.synth_normal_bf16_dev.restype = ctypes.c_int
        lib.synth_tokens_dev.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                         ctypes.c_uint64, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_void_p]
        lib.synth_tokens_dev.restype = ctypes.c_int
        lib.synth_uniform_f32_dev.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64,
                                              ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p]
        lib.synth_uniform_f32_dev.restype = ctypes.c_int
        _dev = lib
    return _dev


def normal_bf16(n, seed, tensor_id, mean=0.0, std=1.0, offset=0):
    """Host array of ``n`` bf16 bit patterns (uint16) ~ mean + std * N(0,1)."""
    out = np.empty(int(n), dtype=np.uint16)
    if n:
        _load_host().synth_normal_bf16(out.ctypes.data, int(n), seed, tensor_id, int(offset),
                                       float(mean), float(std))
    return out


def tokens(n, seed, stream_id, vocab, offset=0):
    """Host int32 array of ``n`` token ids uniform over [0, vocab)."""
    out = np.empty(int(n), dtype=np.int32)
    if n:
        _load_host().synth_tokens(out.ctypes.data, int(n), seed, stream_id, int(offset), int(vocab))
    return out


def uniform_f32(n, seed, stream_id, offset=0):
    """Host float32 array of ``n`` values uniform over [0, 1) (24-bit)."""
    out = np.empty(int(n), dtype=np.float32)
    if n:
        _load_host().synth_uniform_f32(out.ctypes.data, int(n), seed, stream_id, int(offset))
    return out


def normal_bf16_dev(ptr, n, seed, tensor_id, mean=0.0, std=1.0, offset=0, stream=0):
    """Fill ``n`` bf16 elements at device address ``ptr`` with the same bits as
    :func:`normal_bf16`.  Asynchronous on ``stream`` (a hipStream_t handle)."""
    rc = _load_dev().synth_normal_bf16_dev(ptr, int(n), seed, tensor_id, int(offset), float(mean),
                                           float(std), stream)
    if rc != 0:
        raise RuntimeError(f"synth_normal_bf16_dev failed ({rc})")


def tokens_dev(ptr, n, seed, stream_id, vocab, offset=0, stream=0):
    rc = _load_dev().synth_tokens_dev(ptr, int(n), seed, stream_id, int(offset), int(vocab), stream)
    if rc != 0:
        raise RuntimeError(f"synth_tokens_dev failed ({rc})")


def uniform_f32_dev(ptr, n, seed, stream_id, offset=0, stream=0):
    rc = _load_dev().synth_uniform_f32_dev(ptr, int(n), seed, stream_id, int(offset), stream)
    if rc != 0:
        raise RuntimeError(f"synth_uniform_f32_dev failed ({rc})")
