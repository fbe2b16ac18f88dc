#!/usr/bin/env python3
"""Benchmark of the QSA decode step on one MI355X.

Workload (default): 12 QSA layers with independent seeded caches at 255,181
tokens of context (the 256k input size of the source post), 4 x 128 f16
indexer keys, 16 q / 2 KV heads x 256 f16 K/V, indexer top-k 2048 tokens.  One
benchmark step = one decode step of every layer in turn (12 layer-steps; the
12 pooled caches, 784 MB together, do not fit the 256 MB Infinity Cache, so
every step streams from HBM).  Every layer-step runs the whole path: append +
incremental pool, score of every cached block, top-k, gather + attention.

Prints ONE JSON line.  `value` is QSA-layer decode steps per second.
`roofline` is for the dominant kernel (the block-score stream), timed with HIP
events around passes of back-to-back launches on the stream it runs on.  `cpu_baseline` times
the CPU oracle on a bounded sample of the same workload (rank 0, N = 1 only);
the other legs carry the oracle's time beside theirs (`cpu_oracle`), also on
bounded samples.
`multi_decode` (after the headline, outside its timed region): speculative
verify, one call of 4 tokens per layer on the same 12 caches.
`ablations` (after that): the page's comparisons timed on the same caches -- pooled-key cache
off, cell-level top-k, gather off -- beside the calls they stand for.
`context_sweep` (after that): the same 12-layer decode at 61,789 and 126,253 tokens beside the
256k headline, each split into the score kernel's time and the rest of the step.
`batch_and_chunk` (after that, also outside the headline's timed region): batched
decode of 8 sequences of mixed context in one call per step, and one prefill
chunk of 1024 tokens at 126,253 tokens of context, on the same layer shapes.
"""
import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QSA-layer decode steps/s at 256k ctx + achieved HBM GB/s (% of peak)"
# The whole decode step's share of HBM peak that the method's context-
# independent design aims at (the pooled-key stream dominating the step).
STEP_TARGET_FRAC = 0.60
# Correlation of consecutive chunk queries in the grouped-union comparison.
CHUNK_RHO = 0.95
HBM_PEAK_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def layer_step_bytes(w, n):
    """Algorithmic HBM bytes of one layer-step at n tokens (current one included)."""
    nb = n // 4
    idx_row = w.idx_heads * w.idx_dim * (2 if w.idx_f16 else 4)
    kv_row = w.kv_heads * w.head_dim * 2
    n_sel = 4 * min(w.k_blocks, nb) + n % 4
    pooled = idx_row * nb                         # score stream
    gathered = 2 * kv_row * n_sel                 # K and V rows of the chosen cells
    append = idx_row + 2 * kv_row                 # new raw key, K and V rows
    pool = 4 * idx_row + idx_row if n % 4 == 0 else 0   # a completed block: 4 rows in, 1 out
    queries = 4 * (w.idx_heads * w.idx_dim + w.idx_heads + 2 * w.q_heads * w.head_dim)
    return pooled + gathered + append + pool + queries


def score_kernel_bytes(w, nb):
    idx_row = w.idx_heads * w.idx_dim * (2 if w.idx_f16 else 4)
    return idx_row * nb + 4 * (w.idx_heads * w.idx_dim + w.idx_heads) + 4 * nb


def source_code(text):
    """C / HIP source with its comments dropped and its whitespace collapsed:
    what a change to the kernel has to touch."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_hash(*paths):
    """Hash of the code of the given sources (comments and layout aside)."""
    h = hashlib.sha256()
    for path in paths:
        with open(path, encoding="utf-8") as f:
            h.update(source_code(f.read()).encode())
    return h.hexdigest()[:16]


# The score kernel's sources (its epilogue's histogram insertion included).
SCORE_SOURCES = tuple(os.path.join(ROOT, "sparse_attention_decode_cache_amd", "csrc", f)
                      for f in ("k_score.hip", "qsa_hist.h"))


def traffic_record(w, nb):
    """HBM bytes per score launch from committed rocprofv3 counter runs, if the
    kernel source has not changed since they were taken."""
    p = os.path.join(ROOT, "profiles", "score_kernel_traffic.json")
    try:
        rec = json.load(open(p))
    except (OSError, ValueError):
        return None
    if rec.get("k_score_sha256_16") != source_hash(*SCORE_SOURCES) or rec.get("workload") != w.name:
        return None
    return rec.get("bytes_per_launch")


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, n_steps, n_serial=3):
    """The CPU oracle on one layer of the same workload: `n_steps` decode
    steps with its OpenMP loops on every thread it is given, then `n_serial`
    more on one thread."""
    import numpy as np
    import oracle
    from qsagen import workloads as W
    t0 = time.time()
    cap = w.n0 + n_steps + n_serial
    dt = np.float16 if w.idx_f16 else np.float32
    raw = np.zeros((cap,) + w.idx_row, dt)
    K = np.zeros((cap,) + w.kv_row, np.float16)
    V = np.zeros_like(K)
    rows = np.arange(w.n0)
    raw[:w.n0] = W.host_raw_rows(w, rows, 0)
    K[:w.n0], V[:w.n0] = W.host_kv_rows(w, rows, 0)
    L = oracle.OracleLayer(raw, K, V, W.host_gamma(w, 0), w.rms_eps, w.rope_theta, w.n0, w.k_blocks)
    L.rebuild()
    log(f"cpu baseline: oracle cache built in {time.time() - t0:.1f}s")

    def run(s0, n):
        out = []
        for s in range(s0, s0 + n):
            pos = w.n0 + s
            rr = W.host_raw_rows(w, [pos], 0)[0]
            kr, vr = (x[0] for x in W.host_kv_rows(w, [pos], 0))
            qi, wt, q = W.host_step_inputs(w, 0, s)
            t = time.perf_counter()
            L.step(rr, kr, vr, qi, wt, q)
            out.append(time.perf_counter() - t)
        return out

    threads = oracle.threads()
    steps = run(0, n_steps)
    oracle.set_threads(1)
    serial = run(n_steps, n_serial)
    oracle.set_threads(threads)
    affinity = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None
    return {"value": round(len(steps) / sum(steps), 3), "unit": "QSA-layer decode steps/s",
            "cores": threads, "kind": "oracle",
            "cpu": cpu_model(), "nproc": os.cpu_count(), "affinity_cpus": affinity,
            "single_thread": {"value": round(len(serial) / sum(serial), 3),
                              "median_step_ms": round(1e3 * statistics.median(serial), 1), "steps": n_serial},
            "sample": f"{n_steps} decode steps of layer 0 of {w.name} (n0={w.n0}), fp64 C oracle "
                      f"with OpenMP over blocks (pooling, scores) and heads (attention) on {threads} "
                      f"threads, top-k serial; cache build excluded; median step "
                      f"{1e3 * statistics.median(steps):.1f} ms"}


def oracle_step_ms(w, n0, n_steps, seq=0):
    """Median time (ms) of the CPU oracle's decode step on one layer of
    workload w at n0 tokens (seeded rows of stream `seq`), over n_steps
    steps; the oracle's cache build is not timed."""
    import numpy as np
    import oracle
    from qsagen import workloads as W
    cap = n0 + n_steps
    dt = np.float16 if w.idx_f16 else np.float32
    raw = np.zeros((cap,) + w.idx_row, dt)
    K = np.zeros((cap,) + w.kv_row, np.float16)
    V = np.zeros_like(K)
    rows = np.arange(n0)
    raw[:n0] = W.host_raw_rows(w, rows, 0, seq)
    K[:n0], V[:n0] = W.host_kv_rows(w, rows, 0, seq)
    L = oracle.OracleLayer(raw, K, V, W.host_gamma(w, 0), w.rms_eps, w.rope_theta, n0, w.k_blocks)
    L.rebuild()
    times = []
    for s in range(n_steps):
        pos = n0 + s
        rr = W.host_raw_rows(w, [pos], 0, seq)[0]
        kr, vr = (x[0] for x in W.host_kv_rows(w, [pos], 0, seq))
        qi, wt, q = W.host_step_inputs(w, 0, s, seq)
        t = time.perf_counter()
        L.step(rr, kr, vr, qi, wt, q)
        times.append(time.perf_counter() - t)
    return 1e3 * statistics.median(times)


def oracle_beside_legs(result, w256, cpu_step_ms):
    """The CPU oracle beside the other legs, on bounded samples: a verify call
    is n_q oracle decode steps; a batched step is one oracle step per
    sequence (one step each, timed on that sequence's own context); a chunk
    is n_q oracle steps, estimated from 4 steps at the chunk's context; the
    q8_0 leg's quantisation is timed on 8,192 rows and scaled, its attention
    timed once on the 256k selection's cells."""
    import oracle
    from qsagen import workloads as W
    threads = oracle.threads()          # the OpenMP threads the oracle runs on
    cpu = cpu_model()
    md = result.get("multi_decode")
    if md:
        md["cpu_oracle"] = {"ms_per_call": round(md["n_q"] * cpu_step_ms, 1), "cores": threads, "cpu": cpu,
                            "sample": f"{md['n_q']} x the median oracle decode step at n0={w256.n0} "
                                      f"({cpu_step_ms:.1f} ms, cpu_baseline's sample)"}
    bc = result.get("batch_and_chunk")
    if bc:
        b = W.BATCH
        per = [oracle_step_ms(b, n0, 1, seq=i) for i, n0 in enumerate(W.BATCH_CONTEXTS)]
        bc["batch_decode"]["cpu_oracle"] = {
            "ms_per_batched_step": round(sum(per), 1), "cores": threads, "cpu": cpu,
            "sample": "one oracle decode step per sequence, each at its own context"}
        c = W.CHUNK128K
        ms = oracle_step_ms(c, c.n0, 4)
        bc["chunk"]["cpu_oracle"] = {
            "ms_per_chunk": round(ms * c.steps, 1), "cores": threads, "cpu": cpu,
            "sample": f"{c.steps} x the median of 4 oracle decode steps at n0={c.n0} ({ms:.1f} ms)"}
    q8 = result.get("q8_0_kv")
    if q8:
        import numpy as np
        import oracle
        import qsagen
        rows = 8192
        k, v = W.host_kv_rows(w256, np.arange(rows), 0)
        t0 = time.perf_counter()
        oracle.q8_0_quantize(k)
        oracle.q8_0_quantize(v)
        quant_ms = (time.perf_counter() - t0) * 1e3 * w256.n0 / rows
        rng = np.random.default_rng(0)
        sel = np.sort(rng.choice(w256.n0 // 4, w256.k_blocks, replace=False)).astype(np.int32)
        cells = oracle.cells(sel, w256.n0)
        k, v = W.host_kv_rows(w256, cells, 0)
        kc, kd = oracle.q8_0_quantize(k)
        vc, vd = oracle.q8_0_quantize(v)
        q = qsagen.host_normal((w256.q_heads, w256.head_dim), w256.seed, 7)
        t0 = time.perf_counter()
        oracle.attend_q8_0(q, kc, kd, vc, vd, np.arange(len(cells), dtype=np.int32))
        att_ms = (time.perf_counter() - t0) * 1e3
        q8["cpu_oracle"] = {
            "quantize_ms_per_layer": round(quant_ms, 1), "gather_attend_q8_0_ms": round(att_ms, 2),
            "cores": 1, "cpu": cpu,
            "sample": f"q8_0 of {rows} K and V rows scaled to {w256.n0}; one attention over "
                      f"{len(cells)} cells (single-threaded C)"}


TRAFFIC_COPY_MB = 256
MULTI_Q = 4                        # tokens per speculative-verify call (the token + 3 drafts)
MFMA_F16_PEAK_TFLOPS = 2500.0      # MI355X dense f16 matrix-core peak


def chunk_bytes(w, n_q):
    """Algorithmic HBM bytes of a prefill chunk: appended rows, the blocks it
    pools, one read of every summary, and each query's gathered K/V rows."""
    idx_row = w.idx_heads * w.idx_dim * (2 if w.idx_f16 else 4)
    kv_row = w.kv_heads * w.head_dim * 2
    nb_last = (w.n0 + n_q) // 4
    new_blocks = nb_last - w.n0 // 4
    gathered = 0
    for i in range(n_q):
        n = w.n0 + i + 1
        gathered += 2 * kv_row * (4 * min(w.k_blocks, n // 4) + n % 4)
    queries = 4 * n_q * (w.idx_heads * w.idx_dim + w.idx_heads + 2 * w.q_heads * w.head_dim)
    return n_q * (idx_row + 2 * kv_row) + 5 * idx_row * new_blocks + idx_row * nb_last + gathered + queries


def chunk_flops(w, n_q):
    """The method's flops of the chunk's score GEMM: every query against every
    block (the causal mask is applied in the epilogue), one multiply-add per
    element (the kernel issues it twice, the query as two f16 halves)."""
    nb_last = (w.n0 + n_q) // 4
    return 2 * n_q * nb_last * w.idx_heads * w.idx_dim


def multi_call_bytes(w, n0, n_q):
    """Algorithmic HBM bytes of one multi-query call of n_q tokens at n0: one
    read of every summary for all queries, each query's gathered K/V rows, the
    appended rows, the blocks pooled and the queries."""
    idx_row = w.idx_heads * w.idx_dim * (2 if w.idx_f16 else 4)
    kv_row = w.kv_heads * w.head_dim * 2
    nb_last = (n0 + n_q) // 4
    new_blocks = nb_last - n0 // 4
    gathered = sum(2 * kv_row * (4 * min(w.k_blocks, (n0 + i + 1) // 4) + (n0 + i + 1) % 4)
                   for i in range(n_q))
    queries = 4 * n_q * (w.idx_heads * w.idx_dim + w.idx_heads + 2 * w.q_heads * w.head_dim)
    return idx_row * nb_last + gathered + n_q * (idx_row + 2 * kv_row) + 5 * idx_row * new_blocks + queries


def graph_kernel_us(torch, stream, launch_pass, per_pass, reps):
    """Mean duration of one launch of a kernel: `reps` passes of `per_pass`
    back-to-back launches (launch_pass(st) enqueues one pass on st) captured
    in one HIP graph, replayed once untimed and once between HIP events on
    the stream.  A graph keeps the host's per-call cost (the Python binding,
    several microseconds a call) out of the figure, so short launches are not
    timed at the host's rate."""
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream()
        for _ in range(reps):
            launch_pass(cs)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del g
    return 1e3 * e0.elapsed_time(e1) / (reps * per_pass)


def time_decode(torch, qsa, W, w, desc, stream, dev, steps, warmup, kernel_reps, n_layers=None):
    """n_layers layers of workload w (independent caches, round-robin; default
    w.layers): the mean layer-step time of `steps` decode steps captured in a
    HIP graph (after `warmup` eager steps; one untimed replay, one timed), and
    the score kernel's own time (passes of back-to-back qsa_index_score
    launches over the same caches, graph-replayed)."""
    import dataclasses
    n_layers = n_layers or w.layers
    w = dataclasses.replace(w, steps=warmup + steps)
    cap = w.capacity()
    layers = []
    for li in range(n_layers):
        buf = qsa.LayerBuffers(desc, cap)
        W.dev_fill_layer_(w, buf, li, w.n0)
        gamma = W.dev_gamma(w, li)
        qsa.qsa_cache_update(desc, buf.cache, gamma, 0, w.n0 // 4)
        layers.append((buf, gamma, W.dev_step_inputs(w, li, 0, w.steps),
                       qsa.qsa_seq_state(w.n0, w.n0 // 4)))
    ws = qsa.workspace(desc, cap)
    out = torch.empty((w.q_heads, w.head_dim), dtype=torch.float32, device=dev)

    def step(s, st):
        for buf, gamma, inp, state in layers:
            qsa.qsa_decode_step(desc, buf.cache, state, inp.raw[s], inp.k[s], inp.v[s], gamma,
                                inp.q_idx[s], inp.w[s], inp.q[s], out, None, None, ws, st)

    for s in range(warmup):
        step(s, stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cs = torch.cuda.current_stream()
        for i in range(steps):
            step(warmup + i, cs)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    graph.replay()
    b.record(stream)
    torch.cuda.synchronize()
    step_us = 1e3 * a.elapsed_time(b) / (steps * n_layers)
    del graph
    nb = layers[0][3].n_tokens // 4
    scores = torch.empty(nb, dtype=torch.float32, device=dev)

    def score_pass(st):
        for buf, gamma, inp, state in layers:
            qsa.qsa_index_score(desc, buf.cache, nb, inp.q_idx[0], inp.w[0], scores, st)

    score_us = graph_kernel_us(torch, stream, score_pass, len(layers), kernel_reps)
    del layers, ws
    torch.cuda.empty_cache()
    return step_us, score_us, nb


# Context points of the sweep: (tokens in the cache, layers).  Below 256k more
# layer replicas than the headline's 12, so that every point's pooled keys
# (1 KB per block per layer) exceed twice the 256 MB last-level cache and each
# step streams them from HBM.
SWEEP_POINTS = ((61789, 36), (126253, 18), (300000, 12), (524000, 12))


def bench_context_sweep(args, torch, qsa, W, w256, desc, stream, dev, head):
    """The decode step at 61,789 / 126,253 / 300,000 / 524,000 tokens beside
    the 255,181-token headline, every point streaming its pooled keys from
    HBM: the score pass grows with the context (one read of every summary),
    the rest of the step (selection, gather + attention of at most 2,051
    cells, merge) should not.  A least-squares line t = a + c N_b over the
    points gives the per-block cost c and the context-independent part a."""
    import dataclasses
    res = {}
    for n0, nl in SWEEP_POINTS:
        w = dataclasses.replace(w256, n0=n0)
        step_us, score_us, nb = time_decode(torch, qsa, W, w, desc, stream, dev, args.sweep_steps, 4,
                                            args.kernel_reps, n_layers=nl)
        res[str(n0)] = {"layers": nl, "n_blocks": nb, "layer_step_us": round(step_us, 2),
                        "score_us": round(score_us, 2), "rest_us": round(step_us - score_us, 2)}
        log(f"context {n0} x {nl} layers: {res[str(n0)]}")
    res[str(w256.n0)] = {"layers": w256.layers, "n_blocks": head["nb"],
                         "layer_step_us": head["layer_step_us"]["mean"],
                         "score_us": head["roofline"]["scores_only_us"],
                         "rest_us": round(head["layer_step_us"]["mean"] - head["roofline"]["scores_only_us"], 2)}
    pts = sorted(res.values(), key=lambda r: r["n_blocks"])
    xs = [float(r["n_blocks"]) for r in pts]
    ys = [float(r["layer_step_us"]) for r in pts]
    mx, my = sum(xs) / len(xs), sum(ys) / len(ys)
    c = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sum((x - mx) ** 2 for x in xs)
    a = my - c * mx
    fit = {"a_us": round(a, 3), "c_ns_per_block": round(1e3 * c, 4),
           "implied_GBs_per_block_stream": round(1024 / (1e3 * c), 1) if c > 0 else None,
           "max_residual_us": round(max(abs(y - (a + c * x)) for x, y in zip(xs, ys)), 3)}
    log(f"context sweep fit: {fit}")
    return {"workload": "decode step at 61,789 (36 layers) / 126,253 (18) / 255,181 (12) / "
                        "300,000 (12) / 524,000 (12) tokens, headline layer shapes, HIP graph",
            "by_context": res, "fit_t_eq_a_plus_c_Nb": fit,
            "note": "rest_us = layer step - score kernel (the score kernel's own time, scores only)"}


def bench_multi(args, torch, qsa, w, desc, layers, stream, dev, decode_us):
    """Speculative verify on the headline caches: one qsa_decode_step_multi
    call of MULTI_Q tokens (the token and its drafts) per layer, the 12 layers
    round-robin; after each call the drafts are dropped (qsa_state_truncate
    back to the original context), so every call appends, pools one block,
    streams every summary once for all queries, selects and attends per query."""
    n_q = MULTI_Q
    n0 = w.n0
    ws = qsa.multi_workspace(desc, layers[0]["buf"].capacity, n_q)
    outs = torch.empty((n_q, w.q_heads, w.head_dim), dtype=torch.float32, device=dev)

    def call(L):
        inp = L["inp"]
        qsa.qsa_decode_step_multi(desc, L["buf"].cache, L["state"], n_q, inp.raw[:n_q], inp.k[:n_q],
                                  inp.v[:n_q], L["gamma"], inp.q_idx[:n_q], inp.w[:n_q],
                                  inp.q[:n_q], outs, None, None, ws, stream)
        qsa.qsa_state_truncate(L["state"], n0)

    for L in layers:
        qsa.qsa_state_truncate(L["state"], n0)
    for _ in range(2):
        for L in layers:
            call(L)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.multi_reps):
        for L in layers:
            call(L)
    e1.record(stream)
    torch.cuda.synchronize()
    calls = args.multi_reps * len(layers)
    us = 1e3 * e0.elapsed_time(e1) / calls
    nbytes = multi_call_bytes(w, n0, n_q)
    gbs = nbytes / (us / 1e6) / 1e9
    log(f"multi-query decode: {us:.1f} us per call of {n_q} tokens at n0={n0}, {gbs:.0f} GB/s")
    return {"workload": f"qsa-verify{n_q}-256k-12layers", "n0": n0, "n_q": n_q, "calls": calls,
            "us_per_call": round(us, 2), "tokens_per_s": round(n_q / (us / 1e6), 1),
            "vs_decode_steps": round(n_q * decode_us / us, 3),
            "hbm": {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_call": nbytes}}


def bench_ablations(args, torch, qsa, w, desc, layers, ws, stream, dev, decode_us):
    """The page's own comparisons on the headline caches (12 layers at 256k,
    round-robin so every pass reads HBM), each pair timed A, B, B, A with HIP
    events on the library's stream:
      pooled-key cache off: qsa_state_invalidate(st, 0) before a decode step,
        so every block is pooled again (the step then drops its token);
      cell-level top-k: qsa_topk_cells (scores expanded to cells, top-k over
        cells) against qsa_topk_blocks on the same scores;
      gather off: qsa_attend_masked (every cached row read, the selection as a
        mask) against qsa_gather_attend with the same ids."""
    n0 = w.n0
    nb = n0 // 4
    K = w.k_blocks
    aws = qsa.ablation_workspace(desc, layers[0]["buf"].capacity)
    scores = [torch.empty(nb, dtype=torch.float32, device=dev) for _ in layers]
    sels = [torch.empty(K, dtype=torch.int32, device=dev) for _ in layers]
    cells = torch.empty(w.top_k_tokens + 4, dtype=torch.int32, device=dev)
    out = torch.empty((w.q_heads, w.head_dim), dtype=torch.float32, device=dev)
    for L in layers:
        qsa.qsa_state_truncate(L["state"], n0)
    for i, L in enumerate(layers):
        inp = L["inp"]
        qsa.qsa_index_score(desc, L["buf"].cache, nb, inp.q_idx[0], inp.w[0], scores[i], stream)
        qsa.qsa_topk_blocks(scores[i], nb, K, sels[i], ws, stream)

    def timed(fn, reps):
        for i, L in enumerate(layers):      # warm
            fn(i, L)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            for i, L in enumerate(layers):
                fn(i, L)
        b.record(stream)
        torch.cuda.synchronize()
        return 1e3 * a.elapsed_time(b) / (reps * len(layers))

    def cache_off(i, L):
        inp = L["inp"]
        qsa.qsa_state_invalidate(L["state"], 0)
        qsa.qsa_decode_step(desc, L["buf"].cache, L["state"], inp.raw[0], inp.k[0], inp.v[0],
                            L["gamma"], inp.q_idx[0], inp.w[0], inp.q[0], L["out"], None, None, ws,
                            stream)
        qsa.qsa_state_truncate(L["state"], n0)

    def topk_blocks(i, L):
        qsa.qsa_topk_blocks(scores[i], nb, K, sels[i], ws, stream)

    def topk_cells(i, L):
        qsa.qsa_topk_cells(scores[i], n0, w.top_k_tokens, cells, aws, stream)

    def gathered(i, L):
        qsa.qsa_gather_attend(desc, L["buf"].cache, n0, sels[i], K, L["inp"].q[0], out, ws, stream)

    def masked(i, L):
        qsa.qsa_attend_masked(desc, L["buf"].cache, n0, sels[i], K, L["inp"].q[0], out, aws, stream)

    def cache_on(i, L):
        inp = L["inp"]
        qsa.qsa_decode_step(desc, L["buf"].cache, L["state"], inp.raw[0], inp.k[0], inp.v[0],
                            L["gamma"], inp.q_idx[0], inp.w[0], inp.q[0], L["out"], None, None, ws,
                            stream)
        qsa.qsa_state_truncate(L["state"], n0)

    def abba(fa, fb, reps):
        """A, B, B, A: each side's mean of its two passes (and the passes)."""
        a1 = timed(fa, reps)
        b1 = timed(fb, reps)
        b2 = timed(fb, reps)
        a2 = timed(fa, reps)
        return (round((a1 + a2) / 2, 2), round((b1 + b2) / 2, 2),
                [round(a1, 2), round(b1, 2), round(b2, 2), round(a2, 2)])

    r = args.ablation_reps
    on, off, p_cache = abba(cache_on, cache_off, max(1, r // 4))
    blk, cel, p_topk = abba(topk_blocks, topk_cells, r)
    gat, msk, p_attn = abba(gathered, masked, r)
    res = {"workload": f"{w.name} (n0={n0}, {len(layers)} layers round-robin)",
           "order": "ABBA per comparison (A, B, B, A; each side the mean of its two passes)",
           "cache_on_layer_step_us": on, "cache_off_layer_step_us": off, "cache_passes_us": p_cache,
           "topk_blocks_us": blk, "topk_cells_us": cel, "topk_passes_us": p_topk,
           "gather_attend_us": gat, "masked_attend_us": msk, "attend_passes_us": p_attn}
    kv_all = 2 * w.kv_heads * w.head_dim * 2 * n0
    res["masked_attend_gbs"] = round(kv_all / (res["masked_attend_us"] / 1e6) / 1e9, 1)
    log(f"ablations: {res}")
    return res


def bench_q8(args, torch, qsa, w, desc, layers, ws, stream, dev):
    """q8_0 K/V (the 8-bit cache type of the runtime-tuning post) on the
    headline caches: every layer's K and V quantised (qsa_q8_0_quantize over
    the n0 rows), then the gathered attention over the q8_0 planes against the
    f16 one with the same ids (12 layers round-robin, HIP events on the
    library's stream)."""
    n0 = w.n0
    nb = n0 // 4
    K = w.k_blocks
    Hkv, Dh = w.kv_heads, w.head_dim
    cap = layers[0]["buf"].capacity
    scores = torch.empty(nb, dtype=torch.float32, device=dev)
    sels = [torch.empty(K, dtype=torch.int32, device=dev) for _ in layers]
    for L in layers:
        qsa.qsa_state_truncate(L["state"], n0)
    for i, L in enumerate(layers):
        inp = L["inp"]
        qsa.qsa_index_score(desc, L["buf"].cache, nb, inp.q_idx[0], inp.w[0], scores, stream)
        qsa.qsa_topk_blocks(scores, nb, K, sels[i], ws, stream)
    planes = [[(torch.empty((cap, Hkv, Dh), dtype=torch.int8, device=dev),
                torch.empty((cap, Hkv, Dh // 32), dtype=torch.int16, device=dev)) for _ in range(2)]
              for _ in layers]
    out = torch.empty((w.q_heads, Dh), dtype=torch.float32, device=dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def quantize_all():
        for L, pl in zip(layers, planes):
            for X, (c, s) in zip((L["buf"].k, L["buf"].v), pl):
                qsa.qsa_q8_0_quantize(X, c, s, n_values=n0 * Hkv * Dh, stream=stream)

    quantize_all()
    a.record(stream)
    quantize_all()
    b.record(stream)
    torch.cuda.synchronize()
    quant_us = 1e3 * a.elapsed_time(b) / len(layers)
    kvs = [qsa.kv_q8_0(pl[0][0], pl[0][1], pl[1][0], pl[1][1]) for pl in planes]

    def timed(fn, reps):
        for i, L in enumerate(layers):
            fn(i, L)
        a.record(stream)
        for _ in range(reps):
            for i, L in enumerate(layers):
                fn(i, L)
        b.record(stream)
        torch.cuda.synchronize()
        return 1e3 * a.elapsed_time(b) / (reps * len(layers))

    def f16(i, L):
        qsa.qsa_gather_attend(desc, L["buf"].cache, n0, sels[i], K, L["inp"].q[0], out, ws, stream)

    def q8(i, L):
        qsa.qsa_gather_attend_q8_0(desc, kvs[i], n0, sels[i], K, L["inp"].q[0], out, ws, stream)

    r = args.ablation_reps
    n_cells = 4 * K + n0 % 4
    res = {"workload": f"{w.name} (n0={n0}, {len(layers)} layers round-robin, {n_cells} cells)",
           "quantize_us_per_layer": round(quant_us, 2),
           "gather_attend_f16_us": round(timed(f16, r), 2),
           "gather_attend_q8_0_us": round(timed(q8, r), 2),
           "gathered_bytes_f16": n_cells * Hkv * Dh * 2 * 2,
           "gathered_bytes_q8_0": n_cells * Hkv * (Dh + Dh // 16) * 2}
    q_bytes = 2 * n0 * Hkv * (2 * Dh + Dh + Dh // 16)      # K and V: f16 in, codes + scales out
    res["quantize_gbs"] = round(q_bytes / (quant_us / 1e6) / 1e9, 1)
    log(f"q8_0: {res}")
    return res


def bench_batch_and_chunk(args, torch, qsa, W, stream, dev):
    """Batched decode of 8 mixed-context sequences, and one 1024-token prefill
    chunk at 128k, on the headline layer shapes."""
    import ctypes
    import dataclasses
    lib = qsa.lib()
    res = {}

    # ---- batched decode
    base = W.BATCH
    total = args.batch_warmup + args.batch_steps
    desc = qsa.make_desc(base.idx_heads, base.idx_dim, qsa.QSA_F16, base.q_heads, base.kv_heads,
                         base.head_dim, base.top_k_tokens, base.rms_eps, base.rope_theta)
    seqs = []
    gamma = W.dev_gamma(base, 0)
    for i, n0 in enumerate(W.BATCH_CONTEXTS):
        w = dataclasses.replace(base, n0=n0, steps=total)
        buf = qsa.LayerBuffers(desc, w.capacity())
        W.dev_fill_layer_(w, buf, 0, n0, seq=i)
        qsa.qsa_cache_update(desc, buf.cache, gamma, 0, n0 // 4)
        seqs.append({"w": w, "buf": buf, "inp": W.dev_step_inputs(w, 0, 0, total, seq=i),
                     "out": torch.empty((w.q_heads, w.head_dim), dtype=torch.float32, device=dev)})
    n = len(seqs)
    ws = qsa.batch_workspace(desc, [x["w"].capacity() for x in seqs])
    c_arr = (qsa.qsa_layer_cache * n)(*[x["buf"].cache for x in seqs])
    s_arr = (qsa.qsa_seq_state * n)(*[qsa.qsa_seq_state(x["w"].n0, x["w"].n0 // 4) for x in seqs])
    io = []
    for st in range(total):      # marshalled ahead: the timed loop only calls the library
        io.append((qsa.qsa_seq_io * n)(*[qsa.qsa_seq_io(
            x["inp"].raw[st].data_ptr(), x["inp"].k[st].data_ptr(), x["inp"].v[st].data_ptr(),
            x["inp"].q_idx[st].data_ptr(), x["inp"].w[st].data_ptr(), x["inp"].q[st].data_ptr(),
            x["out"].data_ptr(), None) for x in seqs]))
    D = ctypes.byref(desc)
    g = ctypes.c_void_p(gamma.data_ptr())
    wp, wn = ctypes.c_void_p(ws.data_ptr()), ws.numel()
    sp = ctypes.c_void_p(stream.cuda_stream)

    def bstep(st):
        r = lib.qsa_decode_step_batch(D, n, c_arr, s_arr, io[st], g, wp, wn, sp)
        if r != 0:
            raise qsa.QSAError(r, lib.qsa_last_error().decode())

    torch.cuda.synchronize()
    for st in range(args.batch_warmup):
        bstep(st)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    nbytes = 0
    e0.record(stream)
    for i in range(args.batch_steps):
        for j, x in enumerate(seqs):
            nbytes += layer_step_bytes(x["w"], s_arr[j].n_tokens + 1)
        bstep(args.batch_warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    per = ms / args.batch_steps
    gbs = nbytes / (ms / 1e3) / 1e9
    log(f"batched decode: {per * 1e3:.1f} us per step of {n} sequences, {gbs:.0f} GB/s")
    res["batch_decode"] = {
        "workload": base.name, "contexts": list(W.BATCH_CONTEXTS), "steps": args.batch_steps,
        "warmup": args.batch_warmup, "us_per_batched_step": round(1e3 * per, 2),
        "tokens_per_s": round(n / (per / 1e3), 1),
        "hbm": {"achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_step": round(nbytes / args.batch_steps)}}
    del seqs, ws, io
    torch.cuda.empty_cache()

    # ---- prefill chunk
    w = W.CHUNK128K
    n_q = w.steps
    cdesc = qsa.make_desc(w.idx_heads, w.idx_dim, qsa.QSA_F16, w.q_heads, w.kv_heads, w.head_dim,
                          w.top_k_tokens, w.rms_eps, w.rope_theta)
    buf = qsa.LayerBuffers(cdesc, w.capacity())
    W.dev_fill_layer_(w, buf, 0, w.n0)
    cg = W.dev_gamma(w, 0)
    qsa.qsa_cache_update(cdesc, buf.cache, cg, 0, w.n0 // 4)
    inp = W.dev_step_inputs(w, 0, 0, n_q)
    out = torch.empty((n_q, w.q_heads, w.head_dim), dtype=torch.float32, device=dev)
    cws = qsa.chunk_workspace(cdesc, w.capacity(), n_q)
    state = qsa.qsa_seq_state(w.n0, w.n0 // 4)
    q_iid = inp.q_idx.clone()
    q_corr = torch.from_numpy(W.host_correlated_q_idx(w, 0, 0, n_q, CHUNK_RHO)).to(dev)

    def chunk_ms(fn, q_idx):
        times = []
        for rep in range(args.chunk_reps + 1):
            qsa.qsa_state_truncate(state, w.n0)      # the same chunk again: re-append, re-pool
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn(cdesc, buf.cache, state, n_q, inp.raw, inp.k, inp.v, cg, q_idx, inp.w, inp.q, out, None, None,
               cws, stream)
            b.record(stream)
            times.append((a, b))
        torch.cuda.synchronize()
        return statistics.median([a.elapsed_time(b) for a, b in times[1:]])

    def abba(q_idx):
        a1 = chunk_ms(qsa.qsa_chunk_step, q_idx)
        b1 = chunk_ms(qsa.qsa_chunk_step_grouped, q_idx)
        b2 = chunk_ms(qsa.qsa_chunk_step_grouped, q_idx)
        a2 = chunk_ms(qsa.qsa_chunk_step, q_idx)
        return (a1 + a2) / 2, (b1 + b2) / 2, [round(x, 4) for x in (a1, b1, b2, a2)]

    c_ms, g_ms, passes = abba(q_iid)
    cc_ms, gc_ms, passes_c = abba(q_corr)
    cb = chunk_bytes(w, n_q)
    flops = chunk_flops(w, n_q)
    log(f"prefill chunk: {c_ms:.3f} ms for {n_q} tokens at n0={w.n0} (grouped-union {g_ms:.3f} ms); "
        f"correlated queries: {cc_ms:.3f} ms (grouped-union {gc_ms:.3f} ms)")
    res["chunk"] = {
        "workload": w.name, "n0": w.n0, "n_q": n_q, "reps": args.chunk_reps,
        "ms": round(c_ms, 4), "tokens_per_s": round(n_q / (c_ms / 1e3), 1),
        "algorithmic_gbs": round(cb / (c_ms / 1e3) / 1e9, 1), "bytes": cb,
        "score_gemm_flops": flops, "score_gemm_flops_issued": 2 * flops,
        "score_gemm_note": "flops are the method's (2 n_q nb H D); the kernel issues twice that "
                           "(the query as two f16 halves); the GEMM kernel's own time is in profiles/",
        "whole_call_tflops": round(flops / (c_ms / 1e3) / 1e12, 2),
        "mfma_f16_peak_tflops": MFMA_F16_PEAK_TFLOPS,
        "grouped_union": {"order": "ABBA (per-query, grouped, grouped, per-query)",
                          "iid_ms": round(g_ms, 4), "iid_per_query_ms": round(c_ms, 4), "iid_passes": passes,
                          "correlated_rho": CHUNK_RHO, "correlated_ms": round(gc_ms, 4),
                          "correlated_per_query_ms": round(cc_ms, 4), "correlated_passes": passes_c}}
    return res


def traffic_run(args):
    """Short program for the rocprofv3 counter passes: `kernel_reps` score
    launches at the bench workload as the decode step runs them (layer 0,
    qsa_decode_score: the kernel, grid and outputs of the roofline timing),
    then as many plain copies of TRAFFIC_COPY_MB MiB (the reference of known
    size that scales the counters)."""
    import torch
    import sparse_attention_decode_cache_amd as qsa
    from qsagen import workloads as W
    w = W.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    desc = qsa.make_desc(w.idx_heads, w.idx_dim, qsa.QSA_F16 if w.idx_f16 else qsa.QSA_F32,
                         w.q_heads, w.kv_heads, w.head_dim, w.top_k_tokens, w.rms_eps, w.rope_theta)
    buf = qsa.LayerBuffers(desc, w.capacity())
    W.dev_fill_layer_(w, buf, 0, w.n0)
    gamma = W.dev_gamma(w, 0)
    qsa.qsa_cache_update(desc, buf.cache, gamma, 0, w.n0 // 4)
    inp = W.dev_step_inputs(w, 0, 0, 1)
    nb = w.n0 // 4
    state = qsa.qsa_seq_state(w.n0, nb)
    ws = qsa.workspace(desc, w.capacity())
    stream = torch.cuda.current_stream()
    src = torch.empty(TRAFFIC_COPY_MB << 20, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    for _ in range(args.kernel_reps):
        qsa.qsa_decode_score(desc, buf.cache, state, gamma, inp.q_idx[0], inp.w[0], None, ws, stream)
    for _ in range(args.kernel_reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"traffic run: {args.kernel_reps} score launches ({nb} blocks), "
        f"{args.kernel_reps} copies of {TRAFFIC_COPY_MB} MiB")


def traffic_summarize(args):
    """Turn the two counter passes (FETCH_SIZE, WRITE_SIZE; KiB per dispatch)
    into bytes per score launch, each scaled by what the same counter reads
    for the plain copy (TRAFFIC_COPY_MB MiB read and written)."""
    import csv
    from qsagen import workloads as W
    w = W.WORKLOADS[args.workload]
    fetch_dir, write_dir = args.traffic_summarize

    def per_dispatch(d, counter):
        vals = {"score": [], "copy": []}
        for root, _, files in os.walk(d):
            for f in files:
                if not f.endswith("counter_collection.csv"):
                    continue
                for r in csv.DictReader(open(os.path.join(root, f))):
                    if r.get("Counter_Name") != counter:
                        continue
                    name = r.get("Kernel_Name", "")
                    key = "score" if "k_score" in name else ("copy" if "copy" in name.lower() else None)
                    if key:
                        vals[key].append(float(r["Counter_Value"]))
        return {k: statistics.mean(v) if v else None for k, v in vals.items()}

    fetch = per_dispatch(fetch_dir, "FETCH_SIZE")
    write = per_dispatch(write_dir, "WRITE_SIZE")
    copy_bytes = float(TRAFFIC_COPY_MB << 20)
    f_scale = copy_bytes / (fetch["copy"] * 1024.0)
    w_scale = copy_bytes / (write["copy"] * 1024.0)
    f_bytes = fetch["score"] * 1024.0 * f_scale
    w_bytes = write["score"] * 1024.0 * w_scale
    nb = w.n0 // 4
    rec = {"workload": w.name, "k_score_sha256_16": source_hash(*SCORE_SOURCES), "n_blocks": nb,
           "variant": "as the decode step runs it (qsa_decode_score)",
           "algorithmic_bytes": score_kernel_bytes(w, nb),
           "fetch_kib_per_dispatch": round(fetch["score"], 1),
           "write_kib_per_dispatch": round(write["score"], 1),
           "copy_fetch_kib": round(fetch["copy"], 1), "copy_write_kib": round(write["copy"], 1),
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
           "bytes_per_launch": round(f_bytes + w_bytes)}
    out = os.path.join(ROOT, "profiles", "score_kernel_traffic.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="qsa-256k-12layers")
    ap.add_argument("--cpu-steps", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=8, help="score-kernel timing passes")
    ap.add_argument("--no-batch", action="store_true", help="skip the batched-decode / chunk leg")
    ap.add_argument("--batch-steps", type=int, default=48)
    ap.add_argument("--batch-warmup", type=int, default=4)
    ap.add_argument("--chunk-reps", type=int, default=5)
    ap.add_argument("--multi-reps", type=int, default=8, help="rounds of multi-query calls")
    ap.add_argument("--no-multi", action="store_true", help="skip the multi-query decode leg")
    ap.add_argument("--ablation-reps", type=int, default=8)
    ap.add_argument("--sweep-steps", type=int, default=16, help="decode steps per context of the sweep")
    ap.add_argument("--no-sweep", action="store_true", help="skip the 64k / 128k context sweep")
    ap.add_argument("--no-ablations", action="store_true", help="skip the ablation leg")
    ap.add_argument("--no-q8", action="store_true", help="skip the q8_0 K/V leg")
    ap.add_argument("--batch-only", action="store_true", help="only the batched-decode / chunk leg")
    ap.add_argument("--traffic-run", action="store_true",
                    help="only launch the score kernel and a plain copy (for rocprofv3 --pmc)")
    ap.add_argument("--traffic-summarize", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/score_kernel_traffic.json from two counter passes")
    args = ap.parse_args()
    if args.traffic_summarize:
        traffic_summarize(args)
        return
    if args.traffic_run:
        traffic_run(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_attention_decode_cache_amd as qsa
    from qsagen import workloads as W

    if args.batch_only:
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        print(json.dumps(bench_batch_and_chunk(args, torch, qsa, W, torch.cuda.current_stream(), dev)),
              flush=True)
        return

    w0 = W.WORKLOADS[args.workload]
    # eager warmup, eager timed steps, then the same number of steps again
    # captured in a HIP graph (replayed once untimed, once timed)
    total = args.warmup + 2 * args.steps
    import dataclasses
    w = dataclasses.replace(w0, steps=total)
    cap = w.capacity()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    desc = qsa.make_desc(w.idx_heads, w.idx_dim, qsa.QSA_F16 if w.idx_f16 else qsa.QSA_F32,
                         w.q_heads, w.kv_heads, w.head_dim, w.top_k_tokens, w.rms_eps, w.rope_theta)
    t0 = time.time()
    layers = []
    for li in range(w.layers):
        buf = qsa.LayerBuffers(desc, cap)
        W.dev_fill_layer_(w, buf, li, w.n0)
        gamma = W.dev_gamma(w, li)
        qsa.qsa_cache_update(desc, buf.cache, gamma, 0, w.n0 // 4)
        inp = W.dev_step_inputs(w, li, 0, total)
        layers.append({"buf": buf, "gamma": gamma, "inp": inp,
                       "state": qsa.qsa_seq_state(w.n0, w.n0 // 4),
                       "out": torch.empty((w.q_heads, w.head_dim), dtype=torch.float32, device=dev)})
    ws = qsa.workspace(desc, cap)
    torch.cuda.synchronize()
    log(f"{w.name}: {w.layers} layers, capacity {cap}, set up in {time.time() - t0:.1f}s")

    def layer_step(L, s, st=stream):
        inp = L["inp"]
        qsa.qsa_decode_step(desc, L["buf"].cache, L["state"], inp.raw[s], inp.k[s], inp.v[s],
                            L["gamma"], inp.q_idx[s], inp.w[s], inp.q[s], L["out"], None, None, ws,
                            st)

    for s in range(args.warmup):
        for L in layers:
            layer_step(L, s)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # eager: every call launched from the host as it comes
    events = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    events[0].record(stream)
    for i in range(args.steps):
        s = args.warmup + i
        for L in layers:
            layer_step(L, s)
        events[i + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = [events[i].elapsed_time(events[i + 1]) for i in range(args.steps)]
    eager_ms = events[0].elapsed_time(events[-1])
    layer_steps = args.steps * w.layers
    eager_value = layer_steps / (eager_ms / 1e3)
    log(f"eager: {args.steps} steps in {eager_ms:.3f} ms, {eager_value:.0f} layer-steps/s")

    # graph: the next `steps` steps of every layer captured once (each call's
    # arguments fixed at capture, as the host computed them), replayed as one
    # launch; a replay repeats exactly those steps (same rows, same queries)
    nbytes = 0
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cs = torch.cuda.current_stream()
        for i in range(args.steps):
            s = args.warmup + args.steps + i
            for L in layers:
                nbytes += layer_step_bytes(w, L["state"].n_tokens + 1)
                layer_step(L, s, cs)
    torch.cuda.synchronize()
    graph.replay()                      # untimed: first replay
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    total_ms = g0.elapsed_time(g1)
    value = layer_steps / (total_ms / 1e3)
    step_gbs = nbytes / (total_ms / 1e3) / 1e9
    log(f"graph: {args.steps} steps in {total_ms:.3f} ms, {value:.0f} layer-steps/s, {step_gbs:.0f} GB/s")
    del graph

    # Dominant kernel: the block-score stream, as the decode step runs it
    # (keys, tile lists and the score histogram besides the scores),
    # launched alone through qsa_decode_score on the same stream over the same
    # 12 caches (round-robin, so HBM-resident); `kernel_reps` passes of 12
    # back-to-back launches are captured in a HIP graph and one replay is
    # bracketed by HIP events on the stream, so the average is the kernel's
    # own duration plus the graph's short dispatch gap, as rocprofv3 reports
    # it.  The scores-only variant (qsa_index_score) is timed beside it.
    nb = layers[0]["state"].n_tokens // 4
    scores = torch.empty(nb, dtype=torch.float32, device=dev)

    def kernel_us(fn):
        def one_pass(st):
            for L in layers:
                fn(L, st)
        return graph_kernel_us(torch, stream, one_pass, len(layers), args.kernel_reps)

    k_avg_s = 1e-6 * kernel_us(lambda L, st: qsa.qsa_decode_score(
        desc, L["buf"].cache, L["state"], L["gamma"], L["inp"].q_idx[0], L["inp"].w[0], None, ws, st))
    scores_only_us = kernel_us(lambda L, st: qsa.qsa_index_score(
        desc, L["buf"].cache, nb, L["inp"].q_idx[0], L["inp"].w[0], scores, st))
    kbytes = score_kernel_bytes(w, nb)
    achieved = kbytes / k_avg_s / 1e9
    traffic = traffic_record(w, nb)

    # Which selection path the decode steps take (untimed): two more rounds of
    # the 12 layers, each step read back and then dropped again
    # (qsa_state_truncate), so the caches end as they were.  The status word
    # in the workspace names the path: the score histogram + tile lists, or
    # the full top-k over every key.  The first step follows the score-only
    # passes above (their histogram is not this step's) and is not counted.
    paths = {"hist": 0, "full": 0}
    status = ws[qsa.QSA_DECODE_STATUS_OFFSET:qsa.QSA_DECODE_STATUS_OFFSET + 8]
    for rnd in range(2):
        for li, L in enumerate(layers):
            n_before = L["state"].n_tokens
            layer_step(L, 0)
            p = int(status.cpu().view(torch.int64).item()) & 0xFF
            qsa.qsa_state_truncate(L["state"], n_before)
            if rnd or li:
                paths["hist" if p == qsa.QSA_PATH_HIST else "full"] += 1
    log(f"selection paths over {sum(paths.values())} decode steps: {paths}")
    log(f"score kernel (in-step variant): {1e6 * k_avg_s:.2f} us avg over {args.kernel_reps * len(layers)} launches, "
        f"{achieved:.0f} GB/s; scores only {scores_only_us:.2f} us")

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "QSA-layer decode steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": w.layers, "context_tokens": w0.n0,
                   "layer_steps_per_step": w.layers, "idx": f"{w.idx_heads}x{w.idx_dim} "
                   f"{'f16' if w.idx_f16 else 'f32'}", "attn": f"{w.q_heads}/{w.kv_heads}x{w.head_dim} f16",
                   "top_k_tokens": w.top_k_tokens, "storage": "f16", "accumulate": "f32"},
        "launch": "hip graph (the timed steps captured once, replayed)",
        "layer_step_us": {"mean": round(1e3 * total_ms / layer_steps, 3)},
        "eager": {"value": round(eager_value, 1), "ms_per_step": round(eager_ms / args.steps, 4),
                  "layer_step_us": {
                      "median": round(1e3 * statistics.median(step_ms) / w.layers, 3),
                      "p10": round(1e3 * sorted(step_ms)[len(step_ms) // 10] / w.layers, 3),
                      "p90": round(1e3 * sorted(step_ms)[(9 * len(step_ms)) // 10] / w.layers, 3)}},
        "step_hbm": {"achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                     "bytes_per_layer_step": round(nbytes / layer_steps),
                     "target_frac": STEP_TARGET_FRAC,
                     "target_met": step_gbs / HBM_PEAK_GBS >= STEP_TARGET_FRAC},
        "roofline": {"bound": "hbm", "kernel": "k_score (block-score stream, as the decode step runs it)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": kbytes,
                     "avg_launch_us": round(1e6 * k_avg_s, 3),
                     "scores_only_us": round(scores_only_us, 3)},
        "nb": nb,
        "selection_paths": {**paths, "note": "untimed decode steps after the timed ones, one per layer twice "
                                             "around, read back one by one"},
        "cpu_baseline": None,
        "batch_and_chunk": None,
        "context_sweep": None,
    }
    if not args.no_multi:
        result["multi_decode"] = bench_multi(args, torch, qsa, w, desc, layers, stream, dev,
                                             result["eager"]["layer_step_us"]["median"])
    if not args.no_ablations:
        result["ablations"] = bench_ablations(args, torch, qsa, w, desc, layers, ws, stream, dev,
                                              result["eager"]["layer_step_us"]["median"])
    if not args.no_q8:
        result["q8_0_kv"] = bench_q8(args, torch, qsa, w, desc, layers, ws, stream, dev)
    del layers, ws                      # the 256k caches: the legs below allocate their own
    torch.cuda.empty_cache()
    if not args.no_sweep:
        result["context_sweep"] = bench_context_sweep(args, torch, qsa, W, w0, desc, stream, dev, result)
    if not args.no_batch:
        result["batch_and_chunk"] = bench_batch_and_chunk(args, torch, qsa, W, stream, dev)
    if not args.no_cpu_baseline:
        log("cpu baseline ...")
        result["cpu_baseline"] = cpu_baseline(w0, args.cpu_steps)
        step_ms = float(result["cpu_baseline"]["sample"].split("median step ")[1].split(" ms")[0])
        oracle_beside_legs(result, w0, step_ms)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
