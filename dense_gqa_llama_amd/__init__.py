"""MI355X (gfx950) forward step of a dense grouped-query Llama decoder.

The compute lives in ``libllama_mi355x.so`` (hand-written HIP kernels behind
the C ABI of ``include/llama_mi355x.h``); ``binding`` exposes that ABI with
the same names and ``runtime`` wraps it with PyTorch device memory and
streams.  Importing fails if the library is not built.
"""
from . import binding  # noqa: F401
from .binding import LlamaError  # noqa: F401
from .runtime import Model, Sequence  # noqa: F401
