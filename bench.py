"""Benchmark of the forward step on one MI355X.

Workload: the full 33B shape (52 blocks, hidden 7168, 56/8 heads of 128, FFN
22016, vocabulary 166,912, 61.69 GiB of bf16 weights, seeded random init),
batch 1: a 2,048-token uniform-random prompt prefilled as one chunk, then 128
greedy decode steps whose tokens stay on the GPU.  One benchmark step is that
whole request.  Reported value: decode tokens per second over the timed steps
(HIP events on the stream the library runs on); beside it prefill tokens per
second, the decode HBM rate against the 8 TB/s peak, the dominant kernel's
roofline fraction, and the CPU oracle timed on a bounded sample.

    python bench.py [--steps K] [--warmup W] [--no-cpu-baseline]
    python bench.py --copy-probe-mib N    # a plain device copy of N MiB, for
                                          # calibrating HBM byte counters
    python bench.py --request-only        # one headline request (prompt chunk +
                                          # decode steps) and nothing else, for
                                          # counter runs under a profiler
    python bench.py --vendor-gemm         # the 33B projections at 2,048 rows:
                                          # this library's prompt GEMM beside the
                                          # vendor library's (torch bf16 linear)
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
STREAMS = (2, 12)      # concurrent sequences sharing every decode round
WINDOWS = (1, 7, 16)    # decode window widths timed
WINDOW_STEPS = 8
DRAFT_K = 7             # proposals per drafted round
DRAFT_ROUNDS = 8
LONG_T = 131072         # prompt tokens of the long-context sequences (64 chunks)
LONG_ROUNDS = 8
STREAM_ROUNDS = 32
MFMA_BF16_PEAK_TFLOPS = 2500.0
# HBM bytes of the dominant kernel from rocprofv3 counters, with the digest of
# the sources they were taken on (a changed kernel reports no traffic)
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemv_gate_up_33b_decode_pmc.md")
KERNEL_SOURCES = [os.path.join(ROOT, "dense_gqa_llama_amd", "csrc", f)
                  for f in ("k_gemv.hip", "common.h")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def ensure_built():
    need = [os.path.join(ROOT, "dense_gqa_llama_amd", "libllama_mi355x.so"),
            os.path.join(ROOT, "synth", "libsynth_dev.so"), os.path.join(ROOT, "synth", "libsynth.so"),
            os.path.join(ROOT, "oracle", "liboracle.so")]
    if not all(os.path.exists(p) for p in need):
        import __graft_entry__
        __graft_entry__.build()


def gate_up_bytes(g, rows=1):
    """Algorithmic bytes of one decode gate/up launch: both weight matrices
    once, the normed input rows, the SwiGLU output rows."""
    return 2 * g.ffn * g.hidden * 2 + rows * g.hidden * 2 + rows * g.ffn * 2


def decode_bytes(g, T):
    """Algorithmic bytes of one decode token at context T (positions 0..T-1
    before the new row): every weight once (one embedding row), the cache's
    keys and values read for T+1 positions, the new row's keys and values
    written."""
    kvp = g.kv_bytes_per_position()
    return g.decode_weight_bytes() + (T + 1) * kvp + kvp


def prefill_gemm_flops(g, rows):
    """Algorithmic flops of the projections of one prompt chunk (2 per
    multiply-add; every execution's q/k/v, o, gate/up and down)."""
    per_exec = g.hidden * (g.q_dim + 2 * g.kv_dim) + g.q_dim * g.hidden + 3 * g.hidden * g.ffn
    return 2.0 * rows * per_exec * g.n_exec


def prefill_attn_flops(g, rows, pos0=0):
    """Algorithmic flops of causal attention for a chunk at pos0: each row
    scores and sums its positions (4 d per query head and position)."""
    pairs = rows * pos0 + rows * (rows + 1) / 2
    return 4.0 * g.head_dim * g.n_q_heads * pairs * g.n_exec


def sources_digest():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic():
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when it is absent or was taken on other sources."""
    try:
        fields = {}
        with open(TRAFFIC_SUMMARY) as fh:
            for line in fh:
                if ":" in line and line.startswith("- "):
                    k, v = line[2:].split(":", 1)
                    fields[k.strip()] = v.strip().strip("`")
        if fields.get("sources_sha256") != sources_digest():
            return None
        return int(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def copy_probe(mib):
    """A plain device-to-device copy of mib MiB, three times: its counters
    read a known number of bytes."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy probe: 3 copies of {n} bytes")


def cpu_baseline(g, T, reps=3):
    """The oracle, as it stands, on a bounded sample of the same workload:
    one decode row through one 33B block at context T (cache drawn N(0,1)) and
    one lm_head row; a token costs 52 block rows plus the head row."""
    import numpy as np

    import oracle
    import synth
    from synth.workloads import TensorIds
    from tests.host_inputs import HostWeights

    W = HostWeights(g)
    blk = {k: W(f"b0.{k}") for k in ("attn_norm", "q", "k", "v", "o", "mlp_norm", "gate", "up",
                                      "down")}
    kc = synth.normal_bf16((T + 1) * g.kv_dim, 9001, TensorIds.K_CACHE).reshape(
        T + 1, g.n_kv_heads, g.head_dim)
    vc = synth.normal_bf16((T + 1) * g.kv_dim, 9001, TensorIds.V_CACHE).reshape(
        T + 1, g.n_kv_heads, g.head_dim)
    row = synth.normal_bf16(g.hidden, 9002, TensorIds.INPUT_ROWS).reshape(1, g.hidden)
    t0 = time.perf_counter()
    for _ in range(reps):
        oracle.block(g, blk, kc, vc, np.array([T], dtype=np.int32), row)
    t_block = (time.perf_counter() - t0) / reps
    lm = W("lm_head")
    t0 = time.perf_counter()
    oracle.linear(row, lm)
    t_head = time.perf_counter() - t0
    t_tok = g.n_exec * t_block + t_head
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": 1.0 / t_tok, "unit": "tok/s", "cores": cores, "kind": "oracle",
            "cpu": cpu_model(),
            "sample": (f"{reps} decode rows through one 33B block at context {T} "
                       f"({t_block:.3f} s each) + one lm_head row ({t_head:.3f} s); "
                       f"a token = {g.n_exec} block rows + 1 head row")}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_cores():
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def timed(stream, fn, reps=1):
    """HIP-event milliseconds of reps calls of fn on the current stream."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b)


def bench_tiny(stream, cpu):
    """The tiny workload: a 64-token prompt in one chunk, then 15 one-row
    greedy steps (16 generated tokens); the oracle runs the same request."""
    import numpy as np
    import torch

    import dense_gqa_llama_amd as L
    from synth import device as sd
    from synth.workloads import config
    g = config(1)
    P, D = g.prompt_len, g.decode_steps
    model = L.Model(g, sd.weights(g), max_positions=P + D, max_chunk_rows=P, max_seqs=1)
    prompt = sd.tokens(P, g.prompt_seeds[0], 0, g.vocab)
    seq = model.new_sequence(P + D)
    buf = torch.empty(D, dtype=torch.int32, device="cuda")

    def req():
        seq.truncate(0)
        buf[0:1].copy_(model.prefill(seq, tokens=prompt, want_logits=False)["next"])
        for i in range(1, D):
            model.decode([seq], tokens=buf[i - 1:i], want_logits=False, next_out=buf[i:i + 1])
    req()
    torch.cuda.synchronize()
    pre_ms = timed(stream, lambda: (seq.truncate(0),
                                    model.prefill(seq, tokens=prompt, want_logits=False)), 20) / 20
    req_ms = timed(stream, req, 20) / 20
    dec_ms = (req_ms - pre_ms) / (D - 1)
    wbytes = g.decode_weight_bytes()
    out = {"workload": "tiny dense GQA Llama (2 blocks, hidden 512, 8/2 heads of 64, FFN 1408, "
                       "vocab 4096): 64-token prompt + 16 greedy tokens",
           "prefill_tok_s": round(P / (pre_ms / 1e3), 1),
           "decode_tok_s": round(1e3 / dec_ms, 1), "decode_ms_per_token": round(dec_ms, 4),
           "decode_hbm_gbs": round(decode_bytes(g, P + D / 2) / (dec_ms / 1e3) / 1e9, 1),
           "decode_hbm_frac": round(decode_bytes(g, P + D / 2) / (dec_ms / 1e3) / 1e9
                                    / HBM_PEAK_GBS, 5),
           "note": f"{wbytes / 1e6:.1f} MB of weights per token: bound by launch latency, "
                   "not by HBM"}
    if cpu:
        from oracle.model import OracleModel
        from tests.host_inputs import HostWeights
        om = OracleModel(g, HostWeights(g))
        t0 = time.perf_counter()
        om.generate(om.new_sequence(P + D), prompt.cpu().numpy(), D)
        t = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round((P + D) / t, 2), "unit": "tok/s (prompt + generated)",
                               "cores": oracle_cores(), "kind": "oracle", "cpu": cpu_model(),
                               "sample": "the whole request (64 prompt rows + 15 steps)"}
    return out


def bench_layer33(stream, cpu):
    """One 33B-shaped layer decoding 1- and 16-row windows at 4,096 cache
    positions of N(0,1) keys and values.  Four copies of the layer with
    their own weights run in turn (4.7 GB, far past the 256 MB cache in front
    of HBM), so each layer's weights come from HBM."""
    import dataclasses

    import numpy as np
    import torch

    import dense_gqa_llama_amd as L
    from synth import device as sd
    from synth import normal_bf16_dev
    from synth.workloads import config
    g1 = config(2)
    NC = 4
    g = dataclasses.replace(g1, n_blocks=NC)
    T = g.extra["cache_positions"]
    model = L.Model(g, sd.weights(g), max_positions=T + 64, max_chunk_rows=16, max_seqs=1)
    seq = model.new_sequence(T + 64)
    normal_bf16_dev(seq.buf.data_ptr(), seq.buf.numel() // 2, g.extra["kv_seed"], 0,
                    stream=stream.cuda_stream)
    rows = sd.normal((16, g.hidden), g.extra["input_seed"], 20)
    out = {"workload": "one 33B-shaped layer (hidden 7168, 56/8 heads of 128, FFN 22016), "
                       "decode windows at 4,096 cache positions of N(0,1) keys and values",
           "windows": []}
    layer_w = g1.decode_weight_bytes()
    for R in (1, 16):
        seq.declare(T)
        model.decode([seq], hidden=rows[:R], rows=R, want_hidden=True)  # warm
        torch.cuda.synchronize()
        reps = 10

        def step():
            seq.truncate(T)
            model.decode([seq], hidden=rows[:R], rows=R, want_hidden=True)
        ms = timed(stream, step, reps) / reps / NC
        kvp = g1.kv_bytes_per_position()
        byts = layer_w + (T + R) * kvp + R * kvp
        out["windows"].append({"rows": R, "us_per_layer": round(ms * 1e3, 2),
                               "hbm_gbs": round(byts / (ms / 1e3) / 1e9, 1),
                               "hbm_frac": round(byts / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)})
    if cpu:
        import oracle
        import synth
        from synth.workloads import TensorIds
        from tests.host_inputs import HostWeights
        W = HostWeights(g1)
        blk = {k: W(f"b0.{k}") for k in ("attn_norm", "q", "k", "v", "o", "mlp_norm", "gate",
                                          "up", "down")}
        kc = synth.normal_bf16((T + 1) * g1.kv_dim, g1.extra["kv_seed"], TensorIds.K_CACHE).reshape(
            T + 1, g1.n_kv_heads, g1.head_dim)
        vc = synth.normal_bf16((T + 1) * g1.kv_dim, g1.extra["kv_seed"], TensorIds.V_CACHE).reshape(
            T + 1, g1.n_kv_heads, g1.head_dim)
        row = synth.normal_bf16(g1.hidden, g1.extra["input_seed"], TensorIds.INPUT_ROWS).reshape(
            1, g1.hidden)
        t0 = time.perf_counter()
        for _ in range(3):
            oracle.block(g1, blk, kc, vc, np.array([T], dtype=np.int32), row)
        t = (time.perf_counter() - t0) / 3
        out["cpu_baseline"] = {"value": round(1e6 * t, 1), "unit": "us per layer row",
                               "cores": oracle_cores(), "kind": "oracle", "cpu": cpu_model(),
                               "sample": f"3 one-row decode steps of the layer at position {T}"}
    return out


def bench_looped(stream, cpu):
    """The looped model: a 512-token prompt in one chunk, then 255 one-row
    greedy steps (256 generated tokens); 44 executions over 22 blocks."""
    import numpy as np
    import torch

    import dense_gqa_llama_amd as L
    from synth import device as sd
    from synth.workloads import config
    g = config(4)
    P, D = g.prompt_len, g.decode_steps
    model = L.Model(g, sd.weights(g), max_positions=P + D, max_chunk_rows=P, max_seqs=1)
    prompt = sd.tokens(P, g.prompt_seeds[0], 0, g.vocab)
    seq = model.new_sequence(P + D)
    buf = torch.empty(D, dtype=torch.int32, device="cuda")
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(3)]

    def req(ev=None):
        seq.truncate(0)
        if ev:
            ev[0].record(stream)
        buf[0:1].copy_(model.prefill(seq, tokens=prompt, want_logits=False)["next"])
        if ev:
            ev[1].record(stream)
        for i in range(1, D):
            model.decode([seq], tokens=buf[i - 1:i], want_logits=False, next_out=buf[i:i + 1])
        if ev:
            ev[2].record(stream)
    req()
    req(marks)
    torch.cuda.synchronize()
    pre_ms = marks[0].elapsed_time(marks[1])
    dec_ms = marks[1].elapsed_time(marks[2]) / (D - 1)
    byts = decode_bytes(g, P + D / 2)
    out = {"workload": "looped model (22 blocks x 2 loops, hidden 3072, 48/8 heads of 128, "
                       "FFN 8192, vocab 166912): 512-token prompt + 256 greedy tokens",
           "prefill_tok_s": round(P / (pre_ms / 1e3), 1),
           "prefill_gemm_tflops": round(prefill_gemm_flops(g, P) / (pre_ms / 1e3) / 1e12, 1),
           "decode_tok_s": round(1e3 / dec_ms, 2), "decode_ms_per_token": round(dec_ms, 4),
           "decode_hbm_gbs": round(byts / (dec_ms / 1e3) / 1e9, 1),
           "decode_hbm_frac": round(byts / (dec_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4)}
    if cpu:
        import oracle
        import synth
        from synth.workloads import TensorIds
        from tests.host_inputs import HostWeights
        W = HostWeights(g)
        blk = {k: W(f"b0.{k}") for k in ("attn_norm", "q", "k", "v", "o", "mlp_norm", "gate",
                                          "up", "down")}
        T = P + D // 2
        kc = synth.normal_bf16((T + 1) * g.kv_dim, 9004, TensorIds.K_CACHE).reshape(
            T + 1, g.n_kv_heads, g.head_dim)
        vc = synth.normal_bf16((T + 1) * g.kv_dim, 9004, TensorIds.V_CACHE).reshape(
            T + 1, g.n_kv_heads, g.head_dim)
        row = synth.normal_bf16(g.hidden, 9005, TensorIds.INPUT_ROWS).reshape(1, g.hidden)
        t0 = time.perf_counter()
        for _ in range(3):
            oracle.block(g, blk, kc, vc, np.array([T], dtype=np.int32), row)
        tb = (time.perf_counter() - t0) / 3
        t0 = time.perf_counter()
        oracle.linear(row, W("lm_head"))
        th = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(1.0 / (g.n_exec * tb + th), 3), "unit": "tok/s",
                               "cores": oracle_cores(), "kind": "oracle", "cpu": cpu_model(),
                               "sample": (f"3 decode rows through one block at context {T} "
                                          f"({tb:.3f} s each) + one lm_head row ({th:.3f} s); a "
                                          f"token = {g.n_exec} block rows + 1 head row")}
    return out


def vendor_gemm(reps=20):
    """The four projections of one 33B block at 2,048 rows, each as one
    STORE launch of this library's prompt GEMM (llama_test_linear; q/k/v as
    one 9,216-column matrix, gate/up as one 44,032-column matrix) and as
    torch's bf16 linear (the vendor BLAS), on the same operands, alternating,
    best of two rounds of `reps` launches each.  Prints one JSON line."""
    import torch
    import dense_gqa_llama_amd as L
    from dense_gqa_llama_amd import binding as B
    from synth import device as sd
    from synth.workloads import config
    g = config(2)
    w = sd.weights(g)
    m = L.Model(g, w, max_positions=64, max_chunk_rows=2048, max_seqs=1)
    st = torch.cuda.current_stream()
    M = 2048
    mats = {"qkv": torch.cat([w["b0.q"], w["b0.k"], w["b0.v"]]).contiguous(), "o": w["b0.o"],
            "gate_up": torch.cat([w["b0.gate"], w["b0.up"]]).contiguous(), "down": w["b0.down"]}

    def timed(call):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(reps):
            call()
        b.record(st)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    rows, tot = {}, {"this": 0.0, "vendor": 0.0, "gflop": 0.0}
    for name, Wd in mats.items():
        n, k = Wd.shape
        x = sd.normal((M, k), 3200, 0).view(torch.bfloat16)
        y = torch.empty((M, n), dtype=torch.int16, device="cuda")
        y32 = torch.empty((M, n), dtype=torch.float32, device="cuda")
        ours = lambda: B.llama_test_linear(m.handle, 1, x.data_ptr(), M, Wd.data_ptr(), n, k,
                                           y.data_ptr(), y32.data_ptr(), st.cuda_stream)
        Wb = Wd.view(torch.bfloat16)
        vendor = lambda: torch.nn.functional.linear(x, Wb)
        ours(); vendor(); torch.cuda.synchronize()
        t = {"this": 9e9, "vendor": 9e9}
        for _ in range(2):
            t["this"] = min(t["this"], timed(ours))
            t["vendor"] = min(t["vendor"], timed(vendor))
        gf = 2.0 * M * n * k / 1e9
        rows[name] = {"n": n, "k": k, "gflop": round(gf, 1),
                      "this_us": round(t["this"] * 1e3, 1), "vendor_us": round(t["vendor"] * 1e3, 1),
                      "this_tflops": round(gf / t["this"], 1), "vendor_tflops": round(gf / t["vendor"], 1)}
        tot["this"] += t["this"]
        tot["vendor"] += t["vendor"]
        tot["gflop"] += gf
        log(f"{name}: {rows[name]}")
    print(json.dumps({"workload": "33B projections at 2,048 rows, one STORE launch each",
                      "rows": rows, "this_tflops": round(tot["gflop"] / tot["this"], 1),
                      "vendor_tflops": round(tot["gflop"] / tot["vendor"], 1),
                      "vendor": "torch.nn.functional.linear, bf16 (hipBLASLt)"}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe-mib", type=int, default=0)
    ap.add_argument("--request-only", action="store_true")
    ap.add_argument("--vendor-gemm", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU: the forward step has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(2)

    ensure_built()
    import torch
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.vendor_gemm:
        vendor_gemm()
        return

    import dense_gqa_llama_amd as L
    from dense_gqa_llama_amd import binding as B
    from synth import device as sd
    from synth.workloads import config

    g = config(3)
    P, D = g.prompt_len, g.decode_steps
    cap = P + D
    torch.cuda.set_device(0)
    log(f"generating {g.params() * 2 / 2**30:.2f} GiB of weights on the GPU")
    w = sd.weights(g)
    torch.cuda.synchronize()
    model = L.Model(g, w, max_positions=max(cap, LONG_T + LONG_ROUNDS + 1), max_chunk_rows=P, max_window_rows=16,
                    max_seqs=STREAMS[-1])
    seq = model.new_sequence(cap)
    prompt = sd.tokens(P, g.prompt_seeds[0], 0, g.vocab)
    stream = torch.cuda.current_stream()

    def request(before_decode=None):
        """One request: prefill + D greedy steps; returns its events and tokens."""
        seq.truncate(0)
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        out = model.prefill(seq, tokens=prompt, want_logits=False)
        e1.record(stream)
        if before_decode:
            before_decode()
        nxt = out["next"]
        buf = torch.empty(D, dtype=torch.int32, device="cuda")
        buf[0:1].copy_(nxt)
        for i in range(1, D):
            model.decode([seq], tokens=buf[i - 1:i], want_logits=False, next_out=buf[i:i + 1])
        e2.record(stream)
        return e0, e1, e2, buf

    if args.request_only:
        request()
        torch.cuda.synchronize()
        model.check_finite()
        log("one request done")
        return
    for i in range(args.warmup):
        log(f"warmup step {i}")
        request()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    evs = [request() for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    model.check_finite()
    pre_ms = sum(a.elapsed_time(b) for a, b, _, _ in evs)
    dec_ms = sum(b.elapsed_time(c) for _, b, c, _ in evs)
    # the first generated token comes from the prefill; D - 1 decode steps follow
    dec_tokens = args.steps * (D - 1)
    dec_tps = dec_tokens / (dec_ms / 1e3)
    pre_tps = args.steps * P / (pre_ms / 1e3)
    avg_T = P + (D - 1) / 2.0
    dec_gbs = decode_bytes(g, avg_T) * dec_tokens / (dec_ms / 1e3) / 1e9
    toks = evs[-1][3].cpu().tolist()
    log(f"decode {dec_tps:.2f} tok/s ({dec_gbs:.0f} GB/s), prefill {pre_tps:.0f} tok/s, "
        f"first tokens {toks[:8]}")

    # dominant kernel: the decode gate/up projection (53% of a token's bytes)
    # each decode launch's own execution time (the prompt chunk is excluded)
    request(before_decode=lambda: B.llama_set_timing(model.handle, "gate_up", g.n_exec * D))
    torch.cuda.synchronize()
    ms, n = B.llama_timing_read(model.handle)
    B.llama_set_timing(model.handle, "off")
    per_launch_ms = ms / max(n, 1)
    achieved = gate_up_bytes(g) / (per_launch_ms / 1e3) / 1e9
    log(f"gate/up projection: {n} launches, {per_launch_ms * 1e3:.1f} us each, "
        f"{achieved:.0f} GB/s")

    # prompt-chunk projections and attention, each class timed on its own
    def timed_prefill(kind, launches):
        B.llama_set_timing(model.handle, kind, launches)
        request()
        torch.cuda.synchronize()
        t, k = B.llama_timing_read(model.handle)
        B.llama_set_timing(model.handle, "off")
        return t, k
    gemm_ms, _ = timed_prefill("prefill_gemm", 6 * g.n_exec)
    attn_ms, _ = timed_prefill("prefill_attn", g.n_exec)
    gemm_tf = prefill_gemm_flops(g, P) / (gemm_ms / 1e3) / 1e12
    attn_tf = prefill_attn_flops(g, P) / (attn_ms / 1e3) / 1e12
    log(f"prefill projections {gemm_ms:.1f} ms ({gemm_tf:.0f} TFLOP/s), attention "
        f"{attn_ms:.1f} ms ({attn_tf:.0f} TFLOP/s)")
    traffic = stored_traffic()

    # the exact prompt form (sums restarted every 128 terms, three-part
    # attention weights) on the same chunk, in a second model over the same
    # weights
    mx = L.Model(g, w, max_positions=P, max_chunk_rows=P, max_window_rows=1, max_seqs=1,
                 prompt_exact=True)
    sx = mx.new_sequence(P)

    def exact_chunk(kind=None, launches=0):
        sx.truncate(0)
        if kind:
            B.llama_set_timing(mx.handle, kind, launches)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        mx.prefill(sx, tokens=prompt, want_logits=False)
        b.record(stream)
        torch.cuda.synchronize()
        t = B.llama_timing_read(mx.handle)[0] if kind else 0.0
        if kind:
            B.llama_set_timing(mx.handle, "off")
        return a.elapsed_time(b), t
    exact_chunk()  # warm
    xms = min(exact_chunk()[0] for _ in range(args.steps))
    xg = exact_chunk("prefill_gemm", 6 * g.n_exec)[1]
    xa = exact_chunk("prefill_attn", g.n_exec)[1]
    prefill_exact = {"tok_s": round(P / (xms / 1e3), 1), "ms_per_chunk": round(xms, 2),
                     "gemm_ms": round(xg, 2),
                     "gemm_tflops": round(prefill_gemm_flops(g, P) / (xg / 1e3) / 1e12, 1),
                     "attention_ms": round(xa, 2),
                     "attention_tflops": round(prefill_attn_flops(g, P) / (xa / 1e3) / 1e12, 1)}
    log(f"exact prompt form: {prefill_exact}")
    del sx, mx
    torch.cuda.empty_cache()

    # concurrent streams: n sequences, each with the prompt, share every decode
    # round (one row per sequence); aggregate tokens per second
    streams = [{"n": 1, "tok_s": round(dec_tps, 2)}]
    for n in STREAMS:
        seqs = [model.new_sequence(P + STREAM_ROUNDS + 1) for _ in range(n)]
        firsts = [model.prefill(sq, tokens=prompt, want_logits=False)["next"] for sq in seqs]
        tok = torch.cat(firsts)
        model.decode(seqs, tokens=tok, want_logits=False, next_out=tok)  # warm
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(STREAM_ROUNDS):
            model.decode(seqs, tokens=tok, want_logits=False, next_out=tok)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b)
        streams.append({"n": n, "tok_s": round(n * STREAM_ROUNDS / (ms / 1e3), 2)})
        log(f"{n} streams: {streams[-1]['tok_s']:.1f} tok/s together ({ms / STREAM_ROUNDS:.2f} ms a round)")
        del seqs
    torch.cuda.empty_cache()

    # decode windows (teacher-forced rows after the prompt): one window of
    # `rows` rows per step, the verification step of drafted decoding
    windows = []
    wseq = model.new_sequence(cap)  # P + 16 * WINDOW_STEPS positions fit
    for rows in WINDOWS:
        wseq.truncate(0)
        model.prefill(wseq, tokens=prompt, want_logits=False)
        toks = sd.tokens(rows * WINDOW_STEPS, 4700 + rows, 0, g.vocab)
        model.decode([wseq], tokens=toks[:rows], rows=rows, want_logits=False)  # warm
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for i in range(1, WINDOW_STEPS):
            model.decode([wseq], tokens=toks[i * rows:(i + 1) * rows], rows=rows,
                         want_logits=False)
        b.record(stream)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / (WINDOW_STEPS - 1)
        windows.append({"rows": rows, "ms_per_window": round(ms, 3)})
        log(f"{rows}-row windows: {ms:.2f} ms each")
    del wseq

    # drafted greedy rounds with the looped 3B-shaped model (same vocabulary)
    # drafting; with random weights its proposals are rarely taken, so this
    # measures the rounds' cost, not a drafted speed-up
    gd = config(4)
    wd = sd.weights(gd)
    torch.cuda.synchronize()
    dmodel = L.Model(gd, wd, max_positions=cap, max_chunk_rows=P, max_window_rows=1, max_seqs=1)
    tseq, dseq = model.new_sequence(cap), dmodel.new_sequence(cap)
    last = model.prefill(tseq, tokens=prompt, want_logits=False)["next"]
    dmodel.prefill(dseq, tokens=prompt, want_logits=False)
    model.draft_round(tseq, dmodel, dseq, DRAFT_K, last)  # warm
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ntok = taken = 0
    for _ in range(DRAFT_ROUNDS):
        toks, m = model.draft_round(tseq, dmodel, dseq, DRAFT_K, last)
        ntok += m
        taken += m - 1
        last = toks[m - 1:m].clone()
    torch.cuda.synchronize()
    draft_s = time.perf_counter() - t0
    drafting = {"draft": "looped model, 22 blocks x 2 loops, hidden 3072, vocab 166912 "
                         "(random weights)",
                "n_draft": DRAFT_K, "rounds": DRAFT_ROUNDS, "tokens": ntok,
                "proposals_taken": round(taken / (DRAFT_K * DRAFT_ROUNDS), 4),
                "ms_per_round": round(draft_s * 1e3 / DRAFT_ROUNDS, 3),
                "tok_s": round(ntok / draft_s, 2)}
    log(f"drafted rounds: {drafting}")
    del dmodel, wd, tseq, dseq
    torch.cuda.empty_cache()

    # the long-context workload: sequence 0 prefills its 131,072-token prompt
    # in 64 chunks of 2,048 rows (timed whole; the last chunk's attention also
    # on its own); sequence 1's cache is planted with N(0,1) keys and values
    # (a second 131k prefill would add half a minute); then both share every
    # decode round
    gl = config(5)
    lseqs = [model.new_sequence(LONG_T + LONG_ROUNDS + 1) for _ in range(2)]
    from synth import normal_bf16_dev
    normal_bf16_dev(lseqs[1].buf.data_ptr(), lseqs[1].buf.numel() // 2, 3006, 0,
                    stream=stream.cuda_stream)
    lseqs[1].declare(LONG_T)
    lprompt = sd.tokens(LONG_T, gl.prompt_seeds[0], 0, g.vocab)
    nch = LONG_T // P
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nch + 1)]
    B.llama_set_timing(model.handle, "prefill_attn", g.n_exec * nch)
    ev[0].record(stream)
    for c in range(nch):
        if c == nch - 1:
            lam_before, _ = B.llama_timing_read(model.handle)
        model.prefill(lseqs[0], tokens=lprompt[c * P:(c + 1) * P], want_logits=False)
        ev[c + 1].record(stream)
        if c % 16 == 15:
            log(f"131k prompt: chunk {c + 1}/{nch}")
    torch.cuda.synchronize()
    lams, _ = B.llama_timing_read(model.handle)  # the last chunk's attention
    B.llama_set_timing(model.handle, "off")
    whole_ms = ev[0].elapsed_time(ev[nch])
    cms = ev[nch - 1].elapsed_time(ev[nch])
    lp0 = LONG_T - P
    all_attn = sum(prefill_attn_flops(g, P, c * P) for c in range(nch))
    lchunk = {"rows": P, "pos0": lp0, "ms": round(cms, 2), "tok_s": round(P / (cms / 1e3), 1),
              "attention_ms": round(lams, 2),
              "attention_tflops": round(prefill_attn_flops(g, P, lp0) / (lams / 1e3) / 1e12, 1)}
    lprefill = {"tokens": LONG_T, "chunks": nch, "ms": round(whole_ms, 1),
                "tok_s": round(LONG_T / (whole_ms / 1e3), 1),
                "tflops": round((prefill_gemm_flops(g, LONG_T) + all_attn) / (whole_ms / 1e3) / 1e12, 1),
                "attention_ms_before_last_chunk": round(lam_before, 1)}
    log(f"131k prompt prefill: {lprefill}; last chunk: {lchunk}")
    ltok = sd.tokens(2, gl.prompt_seeds[0], 1, g.vocab)
    model.decode(lseqs, tokens=ltok, want_logits=False, next_out=ltok)  # warm
    torch.cuda.synchronize()
    B.llama_set_timing(model.handle, "attn", 2 * g.n_exec * LONG_ROUNDS)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(LONG_ROUNDS):
        model.decode(lseqs, tokens=ltok, want_logits=False, next_out=ltok)
    b.record(stream)
    torch.cuda.synchronize()
    ams, _ = B.llama_timing_read(model.handle)
    B.llama_set_timing(model.handle, "off")
    lms = a.elapsed_time(b) / LONG_ROUNDS
    T_avg = LONG_T + (LONG_ROUNDS - 1) / 2.0  # positions before each round's rows
    kvp = g.kv_bytes_per_position()
    lbytes = decode_bytes(g, T_avg) + (T_avg + 2) * kvp  # weights once, both caches
    long_ctx = {"positions": LONG_T, "sequences": 2, "ms_per_round": round(lms, 3),
                "tok_s": round(2 / (lms / 1e3), 2),
                "hbm_gbs": round(lbytes / (lms / 1e3) / 1e9, 1),
                "attention_us_per_block": round(ams * 1e3 / (g.n_exec * LONG_ROUNDS), 2),
                "attention_gbs": round(2 * (T_avg + 2) * kvp / g.n_exec
                                       / (ams / (g.n_exec * LONG_ROUNDS) / 1e3) / 1e9, 1),
                "prompt_chunk": lchunk, "prompt_prefill": lprefill}
    log(f"long context: {long_ctx}")
    del lseqs
    torch.cuda.empty_cache()

    # seeded sampling of one logit row (temperature 0.6, top_k 20, top_p 0.95)
    sq = model.new_sequence(cap)
    lg = model.prefill(sq, tokens=prompt)["logits"]
    u = sd.uniform(256, 4600, 30)
    out = torch.empty(1, dtype=torch.int32, device="cuda")
    model.sample(lg, u[:1], 0.6, 20, 0.95, out=out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(256):
        model.sample(lg, u[i:i + 1], 0.6, 20, 0.95, out=out)
    b.record(stream)
    torch.cuda.synchronize()
    sample_us = a.elapsed_time(b) * 1e3 / 256
    log(f"sampling: {sample_us:.1f} us per row")
    del sq

    # the other workloads, each in its own model (the 33B's memory is released
    # first: its weights and caches are no longer needed)
    del model, w, seq
    torch.cuda.empty_cache()
    cpu = not args.no_cpu_baseline
    configs = {}
    for name, fn in (("tiny", bench_tiny), ("layer33", bench_layer33), ("looped", bench_looped)):
        log(f"workload {name}")
        configs[name] = fn(stream, cpu)
        log(f"{name}: {configs[name]}")
        torch.cuda.empty_cache()

    result = {
        "metric": "decode tok/s + HBM GB/s (% peak), 33B bf16 batch 1; prefill tok/s",
        "value": round(dec_tps, 3),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded random-init weights ~N(0,0.02) (norms 1+N(0,0.02)), "
                "uniform random prompt tokens",
        "config": {"workload": "33B-shaped dense GQA Llama (52 blocks, hidden 7168, 56/8 heads "
                               "of 128, FFN 22016, vocab 166912), 2048-token prompt in one "
                               "chunk + 128 greedy decode steps, batch 1",
                   "prompt_tokens": P, "decode_steps": D, "batch": 1, "parallelism": "none"},
        "decode_ms_per_token": round(dec_ms / dec_tokens, 4),
        "decode_hbm_gbs": round(dec_gbs, 1),
        "decode_hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
        "prefill_tok_s": round(pre_tps, 1),
        "prefill_gemm": {"bound": "mfma", "achieved": round(gemm_tf, 1),
                         "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                         "frac": round(gemm_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                         "ms_per_chunk": round(gemm_ms, 3)},
        "prefill_exact_form": prefill_exact,
        "prefill_attention": {"bound": "mfma", "achieved": round(attn_tf, 1),
                              "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(attn_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                              "ms_per_chunk": round(attn_ms, 3)},
        "streams": streams,
        "windows": windows,
        "long_context": long_ctx,
        "drafting": drafting,
        "sampling": {"us_per_row": round(sample_us, 2), "temperature": 0.6, "top_k": 20,
                     "top_p": 0.95},
        "configs": configs,
        "roofline": {"bound": "hbm", "kernel": "decode gate/up projection + SwiGLU (R=1)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "launch_us": round(per_launch_ms * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle sample)")
        result["cpu_baseline"] = cpu_baseline(g, int(avg_T))
        log("cpu baseline at the long context (oracle sample)")
        result["long_context"]["cpu_baseline"] = cpu_baseline(g, LONG_T + LONG_ROUNDS // 2, reps=2)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
