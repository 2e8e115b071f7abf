"""The sampling entry point that allocates nothing (llama_sample_noalloc,
for callers that cannot allocate: its candidates live in a fixed per-device
scratch array) against llama_sample, which keeps them in a model's
workspace: the same tokens for the same logits, parameters and uniforms, on
two calls in a row, the second with fewer rows and a smaller vocabulary, so a
stale candidate left in the shared scratch by the first call would show."""
import numpy as np
import pytest

from synth.workloads import TensorIds, config
from tests.gpu_util import gpu_model, log

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)


def _draw_both(model, V, rows, seed, temperature, top_k, top_p, nonfinite_row=None):
    import dense_gqa_llama_amd.binding as B
    from synth import device as sd
    logits = sd.normal((rows, V), seed, TensorIds.SAMPLE_LOGITS, 0.0, 2.0)
    if nonfinite_row is not None:
        logits[nonfinite_row, V // 3] = 0x7F80  # +Inf
    u = sd.uniform(rows, seed, TensorIds.SAMPLE_UNIFORM)
    ref = model.sample(logits, u, temperature, top_k, top_p)
    got = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    B.llama_sample_noalloc(logits.data_ptr(), V, rows, logits.stride(0), temperature, top_k, top_p,
                           u.data_ptr(), got.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return ref.cpu().numpy(), got.cpu().numpy()


def test_noalloc_sampling_equals_workspace_sampling():
    import dataclasses
    g = config(3)  # vocabulary 166,912: 41 chunks of 4,096 logits
    small = config(1)  # vocabulary 4,096: one chunk
    gh = dataclasses.replace(small, vocab=g.vocab)  # the tiny model with the 33B vocabulary
    m_big = gpu_model(gh, 16, max_chunk_rows=16, max_seqs=1)
    m_small = gpu_model(small, 16, max_chunk_rows=16, max_seqs=1)
    cases = [(m_big, g.vocab, 64, 4501, 0.6, 64, 0.95, 5),   # largest rows and top_k
             (m_small, small.vocab, 3, 4502, 1.0, 20, 0.9, None)]  # then fewer rows, one chunk
    for model, V, rows, seed, T, K, P, bad in cases:
        ref, got = _draw_both(model, V, rows, seed, T, K, P, bad)
        log(f"no-alloc sampling, V={V} rows={rows} top_k={K}: {got[:6].tolist()} ... "
            f"equal to the workspace draw: {np.array_equal(ref, got)}")
        assert np.array_equal(ref, got)
        if bad is not None:
            assert got[bad] == -1
        assert (got[np.arange(rows) != (bad if bad is not None else -1)] >= 0).all()
