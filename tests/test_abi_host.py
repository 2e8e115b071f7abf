"""The C-ABI library on the host: it loads, exports every entry point the
header declares, sizes its buffers, and refuses bad arguments before it
enqueues anything (so no GPU is needed).  Refusals follow the pull request
"llama: Nanbeige4.3-33B on Metal, the bf16 release served as published"
(tied heads and other geometries refused at load, section "Checks") and the
NInfer card's capacity check (the position past the cache is rejected,
section "Validation")."""
import os
import re

import pytest

from synth.workloads import CONFIGS

B = pytest.importorskip("dense_gqa_llama_amd.binding")

FAKE = 0x10000  # host-side stand-in address; the refusal paths never touch it


def header_functions(root):
    text = open(os.path.join(root, "include", "llama_mi355x.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(llama_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(root):
    import ctypes
    lib = ctypes.CDLL(B.LIB_PATH)
    names = header_functions(root)
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTS) == names


def test_no_undefined_thread_local_init_reference():
    """A hidden thread-local declared in one file and defined in another makes
    the compiler test a weak, hidden init function (_ZTH...) by its address;
    left undefined in a shared library, that address reads as the load base,
    not zero, and the first use calls into the ELF header.  The library's
    thread-locals that cross files are __thread, which has no such function."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not found")
    out = subprocess.run([nm, B.LIB_PATH], capture_output=True, text=True, check=True).stdout
    bad = [l for l in out.splitlines() if " U _ZTH" in l or " w _ZTH" in l]
    assert not bad, bad


def cfg_of(g, **kw):
    base = dict(n_blocks=g.n_blocks, n_loops=g.n_loops, hidden=g.hidden, n_q_heads=g.n_q_heads,
                n_kv_heads=g.n_kv_heads, head_dim=g.head_dim, ffn=g.ffn, vocab=g.vocab,
                rope_theta=g.rope_theta, rms_eps=g.rms_eps)
    base.update(kw)
    extra = {k: base.pop(k) for k in ("max_chunk_rows", "max_window_rows", "max_seqs",
                                      "prompt_exact") if k in base}
    return B.make_config(**base, **extra)


@pytest.mark.parametrize("i", sorted(CONFIGS))
def test_served_configs_are_sized(i):
    g = CONFIGS[i]
    assert B.llama_workspace_bytes(cfg_of(g), 4096) > 0


@pytest.mark.parametrize("change", [
    dict(head_dim=96), dict(hidden=7000), dict(n_q_heads=50), dict(n_q_heads=72, n_kv_heads=8),
    dict(vocab=166913), dict(rope_theta=0.0), dict(max_chunk_rows=4096), dict(max_window_rows=17),
    dict(max_seqs=0), dict(ffn=22000), dict(n_loops=0), dict(rms_eps=-1.0),
    dict(prompt_exact=2), dict(prompt_exact=-1),
])
def test_refused_geometries(change):
    g = CONFIGS[3]
    assert B.llama_workspace_bytes(cfg_of(g, **change), 4096) == 0
    assert B.last_error()


def blocks(n):
    return [{f: FAKE for f in B.BLOCK_FIELDS} for _ in range(n)]


def load(g, **kw):
    cfg = cfg_of(g, **kw)
    ws = B.llama_workspace_bytes(cfg, 512)
    emb = (FAKE, FAKE + 0x100, FAKE + 0x200) if g.vocab else (None, None, None)
    return B.llama_load_weights(cfg, blocks(g.n_blocks), *emb, FAKE, ws, 512), cfg


def expect(code, fn, *a, **k):
    with pytest.raises(B.LlamaError) as e:
        fn(*a, **k)
    assert e.value.code == code, str(e.value)
    assert B.last_error()


def test_load_refusals():
    g = CONFIGS[1]
    cfg = cfg_of(g)
    ws = B.llama_workspace_bytes(cfg, 512)
    expect(B.LLAMA_E_GEOMETRY, B.llama_load_weights, cfg, blocks(2), FAKE, FAKE, FAKE, FAKE, ws,
           512)  # tied head
    expect(B.LLAMA_E_ARG, B.llama_load_weights, cfg, blocks(2), FAKE, FAKE, None, FAKE, ws, 512)
    expect(B.LLAMA_E_WORKSPACE, B.llama_load_weights, cfg, blocks(2), FAKE, FAKE + 2, FAKE + 4,
           FAKE, ws - 1, 512)
    bad = blocks(2)
    bad[1]["down"] = None
    expect(B.LLAMA_E_ARG, B.llama_load_weights, cfg, bad, FAKE, FAKE + 2, FAKE + 4, FAKE, ws, 512)
    g2 = CONFIGS[2]
    cfg2 = cfg_of(g2)
    ws2 = B.llama_workspace_bytes(cfg2, 512)
    expect(B.LLAMA_E_ARG, B.llama_load_weights, cfg2, blocks(1), FAKE, None, None, FAKE, ws2, 512)


def test_step_refusals_before_any_launch():
    g = CONFIGS[1]
    m, cfg = load(g, max_chunk_rows=64, max_window_rows=16, max_seqs=2)
    try:
        kvb = B.llama_kv_bytes(m, 128)
        assert kvb == g.n_exec * 128 * g.kv_dim * 2 * 2
        expect(B.LLAMA_E_CAPACITY, B.llama_kv_alloc, m, 513, FAKE, 10 ** 9)
        expect(B.LLAMA_E_WORKSPACE, B.llama_kv_alloc, m, 128, FAKE, kvb - 1)
        kv = B.llama_kv_alloc(m, 128, FAKE, kvb)
        kv2 = B.llama_kv_alloc(m, 128, FAKE + kvb, kvb)
        assert B.llama_kv_length(kv) == 0
        slab = B.llama_kv_slab(kv, 1, 1)
        assert slab == FAKE + (2 * 1 + 1) * 128 * g.kv_dim * 2
        assert B.llama_kv_slab(kv, 2, 0) is None
        # windows and batches
        expect(B.LLAMA_E_ARG, B.llama_decode_step, m, [kv], FAKE, None, 17)
        expect(B.LLAMA_E_ARG, B.llama_decode_step, m, [kv], FAKE, None, 0)
        expect(B.LLAMA_E_ARG, B.llama_decode_step, m, [kv, kv], FAKE, None, 1)
        expect(B.LLAMA_E_ARG, B.llama_decode_step, m, [kv, kv2, kv], FAKE, None, 1)
        expect(B.LLAMA_E_ARG, B.llama_decode_step, m, [kv], FAKE, FAKE, 1)  # both inputs
        expect(B.LLAMA_E_ARG, B.llama_decode_step, m, [kv], None, None, 1)  # neither
        # capacity: the last legal position is usable, the next is refused
        B.llama_test_kv_declare(kv, 127)
        expect(B.LLAMA_E_CAPACITY, B.llama_decode_step, m, [kv], FAKE, None, 2)
        B.llama_test_kv_declare(kv, 128)
        expect(B.LLAMA_E_CAPACITY, B.llama_decode_step, m, [kv], FAKE, None, 1)
        expect(B.LLAMA_E_CAPACITY, B.llama_test_kv_declare, kv, 129)
        assert B.llama_kv_length(kv) == 128  # refusal changed nothing
        # truncation only shortens: it cannot declare positions nobody wrote
        B.llama_kv_truncate(kv, 100)
        expect(B.LLAMA_E_POSITION, B.llama_kv_truncate, kv, 101)
        expect(B.LLAMA_E_POSITION, B.llama_kv_truncate, kv, -1)
        assert B.llama_kv_length(kv) == 100
        B.llama_kv_truncate(kv, 0)
        # prompt chunks
        expect(B.LLAMA_E_POSITION, B.llama_prefill_chunk, m, kv, FAKE, None, 8, 3)
        expect(B.LLAMA_E_ARG, B.llama_prefill_chunk, m, kv, FAKE, None, 65, 0)
        expect(B.LLAMA_E_ARG, B.llama_prefill_chunk, m, kv, None, None, 8, 0)
        B.llama_test_kv_declare(kv, 100)
        expect(B.LLAMA_E_CAPACITY, B.llama_prefill_chunk, m, kv, FAKE, None, 64, 100)
        # capture too small for the step
        B.llama_set_capture(m, FAKE, 16)
        B.llama_kv_truncate(kv, 0)
        expect(B.LLAMA_E_WORKSPACE, B.llama_decode_step, m, [kv], FAKE, None, 1)
        B.llama_set_capture(m, None, 0)
        # parity probe: execution in range, rows bounded
        expect(B.LLAMA_E_ARG, B.llama_set_probe, m, g.n_exec, {"attn": FAKE}, 4)
        expect(B.LLAMA_E_ARG, B.llama_set_probe, m, -1, {"attn": FAKE}, 4)
        expect(B.LLAMA_E_ARG, B.llama_set_probe, m, 0, {"attn": FAKE}, 0)
        B.llama_set_probe(m, 1, {"attn": FAKE}, 4)
        expect(B.LLAMA_E_WORKSPACE, B.llama_decode_step, m, [kv, kv2], FAKE, None, 3)
        expect(B.LLAMA_E_WORKSPACE, B.llama_prefill_chunk, m, kv, FAKE, None, 5, 0)
        B.llama_set_probe(m, 0, None, 0)
        assert B.llama_kv_length(kv) == 0
        # single-kernel test entries: kernel kind, shapes, rows, positions
        st = None
        expect(B.LLAMA_E_ARG, B.llama_test_linear, m, 3, FAKE, 4, FAKE, 128, 128, FAKE, FAKE, st)
        expect(B.LLAMA_E_ARG, B.llama_test_linear, m, 1, FAKE, 4, FAKE, 100, 128, FAKE, FAKE, st)
        expect(B.LLAMA_E_ARG, B.llama_test_linear, m, 0, FAKE, 17, FAKE, 128, 128, FAKE, FAKE, st)
        expect(B.LLAMA_E_ARG, B.llama_test_linear, m, 1, FAKE, 2049, FAKE, 128, 128, FAKE, FAKE,
               st)
        expect(B.LLAMA_E_ARG, B.llama_test_attention, m, 1, kv, g.n_exec, FAKE, 4, 0, FAKE)
        expect(B.LLAMA_E_POSITION, B.llama_test_attention, m, 1, kv, 0, FAKE, 4, 0, FAKE)
        B.llama_test_kv_declare(kv, 10)
        expect(B.LLAMA_E_POSITION, B.llama_test_attention, m, 2, kv, 0, FAKE, 4, 7, FAKE)
        expect(B.LLAMA_E_ARG, B.llama_test_attention, m, 0, kv, 0, FAKE, 33, 0, FAKE)
        B.llama_kv_truncate(kv, 0)
        # another model's cache
        m2, _ = load(g, max_chunk_rows=64)
        expect(B.LLAMA_E_ARG, B.llama_decode_step, m2, [kv], FAKE, None, 1)
        B.llama_free(m2)
        B.llama_kv_free(kv)
        B.llama_kv_free(kv2)
    finally:
        B.llama_free(m)


def test_blocks_only_model_refuses_tokens_and_logits():
    g = CONFIGS[2]
    m, cfg = load(g, max_chunk_rows=16, max_window_rows=16, max_seqs=1)
    try:
        kv = B.llama_kv_alloc(m, 64, FAKE, B.llama_kv_bytes(m, 64))
        expect(B.LLAMA_E_ARG, B.llama_decode_step, m, [kv], FAKE, None, 1)
        expect(B.LLAMA_E_ARG, B.llama_decode_step, m, [kv], None, FAKE, 1, logits_bf16=FAKE)
        expect(B.LLAMA_E_ARG, B.llama_prefill_chunk, m, kv, None, FAKE, 4, 0, next_token=FAKE)
        B.llama_kv_free(kv)
    finally:
        B.llama_free(m)


def test_sampling_refusals():
    g = CONFIGS[1]
    m, cfg = load(g, max_chunk_rows=64)
    try:
        V = g.vocab
        ok = dict(rows=4, ld=V, temperature=0.6, top_k=20, top_p=0.95)

        def call(**kw):
            a = dict(ok)
            a.update(kw)
            return B.llama_sample(m, kw.get("logits", FAKE), a["rows"], a["ld"], a["temperature"],
                                  a["top_k"], a["top_p"], kw.get("u", FAKE), kw.get("tok", FAKE))
        for kw in (dict(rows=0), dict(rows=65), dict(ld=V - 1), dict(temperature=0.0),
                   dict(temperature=-1.0), dict(temperature=float("inf")),
                   dict(temperature=float("nan")), dict(top_k=0), dict(top_k=65),
                   dict(top_p=0.0), dict(top_p=1.5), dict(top_p=float("nan")),
                   dict(logits=None), dict(u=None), dict(tok=None)):
            expect(B.LLAMA_E_ARG, call, **kw)
    finally:
        B.llama_free(m)
    g2 = CONFIGS[2]
    m2, _ = load(g2, max_chunk_rows=16)
    try:
        expect(B.LLAMA_E_ARG, B.llama_sample, m2, FAKE, 1, 128, 1.0, 1, 1.0, FAKE, FAKE)
    finally:
        B.llama_free(m2)


def test_draft_round_refusals():
    """llama_draft_round (and its seeded variant) checks both models and
    caches before it enqueues anything: same vocabulary, a window that fits,
    caches of equal length with room for the round, sampling arguments, and
    refusals leave the lengths as they were."""
    g = CONFIGS[1]
    t, _ = load(g, max_chunk_rows=64, max_window_rows=8)
    d, _ = load(g, max_chunk_rows=64, max_window_rows=1)
    g4 = CONFIGS[4]
    other, _ = load(g4, max_chunk_rows=16, max_window_rows=1)
    try:
        tkv = B.llama_kv_alloc(t, 64, FAKE, B.llama_kv_bytes(t, 64))
        dkv = B.llama_kv_alloc(d, 32, FAKE, B.llama_kv_bytes(d, 32))
        okv = B.llama_kv_alloc(other, 64, FAKE, B.llama_kv_bytes(other, 64))

        def call(target=t, target_kv=tkv, draft=d, draft_kv=dkv, n=4, last=FAKE, out=FAKE):
            return B.llama_draft_round(target, target_kv, draft, draft_kv, n, last, out)
        for kw in (dict(n=0), dict(n=8), dict(last=None), dict(out=None), dict(target=None),
                   dict(draft=t, draft_kv=tkv), dict(draft_kv=tkv), dict(target_kv=dkv),
                   dict(draft=other, draft_kv=okv)):
            expect(B.LLAMA_E_ARG, call, **kw)
        B.llama_test_kv_declare(dkv, 3)
        expect(B.LLAMA_E_POSITION, call)
        B.llama_test_kv_declare(tkv, 27)
        B.llama_test_kv_declare(dkv, 27)
        expect(B.LLAMA_E_CAPACITY, call, n=5)  # the draft cache ends at 32
        # the seeded variant also checks its sampling arguments
        assert B.llama_kv_length(dkv) == 27 and B.llama_kv_length(tkv) == 27

        def sampled(T=0.6, K=20, P=0.95, u=FAKE, n=4):
            return B.llama_draft_round_sampled(t, tkv, d, dkv, n, FAKE, T, K, P, u, FAKE)
        for kw in (dict(T=0.0), dict(T=float("inf")), dict(K=0), dict(K=65), dict(P=0.0),
                   dict(P=1.5), dict(u=None), dict(n=8)):
            expect(B.LLAMA_E_ARG, sampled, **kw)
        expect(B.LLAMA_E_CAPACITY, sampled, n=5)
        dkv2 = B.llama_kv_alloc(d, 128, FAKE, B.llama_kv_bytes(d, 128))
        B.llama_test_kv_declare(tkv, 60)
        B.llama_test_kv_declare(dkv2, 60)
        expect(B.LLAMA_E_CAPACITY, call, draft_kv=dkv2, n=4)  # the target cache ends at 64
        assert B.llama_kv_length(tkv) == 60 and B.llama_kv_length(dkv2) == 60
        assert B.llama_kv_length(dkv) == 27
        for kv in (tkv, dkv, dkv2, okv):
            B.llama_kv_free(kv)
    finally:
        for m in (t, d, other):
            B.llama_free(m)
