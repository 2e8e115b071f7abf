"""Helpers for the GPU parity tests: building a model of a workload on the GPU
from the synthetic generator, and moving bf16 bits between torch and numpy."""
import sys

import numpy as np


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def u16(t):
    """Device int16 tensor of bf16 bits -> host uint16 array."""
    return t.detach().cpu().numpy().view(np.uint16)


def to_dev(a, dtype=None):
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(a).cuda()


def gpu_model(g, max_positions, max_chunk_rows=2048, max_window_rows=16, max_seqs=2):
    import torch

    import dense_gqa_llama_amd as L
    from synth import device as sd
    w = sd.weights(g)
    torch.cuda.synchronize()
    return L.Model(g, w, max_positions=max_positions, max_chunk_rows=max_chunk_rows,
                   max_window_rows=max_window_rows, max_seqs=max_seqs)
