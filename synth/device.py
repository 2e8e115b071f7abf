"""Synthetic weights and inputs generated directly in device memory (PyTorch
tensors), bit-identical to the host generator."""
import numpy as np
import torch

from . import normal_bf16_dev, tokens_dev, uniform_f32_dev
from .workloads import weight_spec


def _stream():
    return torch.cuda.current_stream().cuda_stream


def weights(g, device="cuda"):
    """dict name -> bf16 bit tensor (int16) of every stored weight of ``g``."""
    out = {}
    for name, tid, shape, mean, std in weight_spec(g):
        t = torch.empty(shape, dtype=torch.int16, device=device)
        normal_bf16_dev(t.data_ptr(), t.numel(), g.weight_seed, tid, mean, std, stream=_stream())
        out[name] = t
    return out


def normal(shape, seed, tensor_id, mean=0.0, std=1.0, device="cuda", offset=0):
    t = torch.empty(shape, dtype=torch.int16, device=device)
    normal_bf16_dev(t.data_ptr(), t.numel(), seed, tensor_id, mean, std, offset=offset,
                    stream=_stream())
    return t


def tokens(n, seed, stream_id, vocab, device="cuda", offset=0):
    t = torch.empty(int(n), dtype=torch.int32, device=device)
    tokens_dev(t.data_ptr(), int(n), seed, stream_id, vocab, offset=offset, stream=_stream())
    return t


def uniform(n, seed, stream_id, device="cuda", offset=0):
    t = torch.empty(int(n), dtype=torch.float32, device=device)
    uniform_f32_dev(t.data_ptr(), int(n), seed, stream_id, offset=offset, stream=_stream())
    return t


def to_host_u16(t):
    return t.cpu().numpy().view(np.uint16)
