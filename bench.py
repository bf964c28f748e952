"""Decode-attention benchmark of the quantized KV cache on one MI355X.

A step is one pass of the hot path over every layer of the workload, with inputs already in HBM:
per layer, append one token per sequence (tail-ring write), evict the oldest tail token (requantize
into the qN_0 body) and run decode attention over the whole cache; sparse workloads append and then
run sparse decode over the step's position list.

Default workload (the largest single-GPU one): 16 layers, batch 1, context 262,144, 16 query / 2 KV heads
x 256, K 6-bit / V 5-bit body with a 2,048-position 8-bit (q8_0) recent-token ring, a decode step at full
length (synthetic Gaussian K/V with 4 outlier K channels x20). --config 1..5 selects the other workloads.

Prints one JSON line. `value` is the effective GB/s of decode attention over the whole step (algorithmic
bytes of the decode calls / step time; a call's algorithmic bytes are the K and V rows it attends, the KVarN
scales, the bf16 query rows it reads and the fp32 output rows it writes). `roofline` is the decode kernel's
rate: algorithmic bytes per launch / average kernel time, from HIP events that the kernel dispatches stamp
with their start and end (library launch timing, measured on a second run of the same number of steps),
against 8 TB/s HBM3E. `traffic` is the HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE
counters (scaled by the copy-kernel calibration stored with them), used only while the kernel source still
matches the one that was measured. `cpu_baseline` is the CPU oracle timed on a bounded sample of the same
workload, one layer per worker process over the host's cores (measured before the GPU is touched). Also
reported: `graph` (the same steps with each step's launches captured into one HIP graph beforehand and
replayed back to back), `cold` (single-layer workloads: decode time after a 512 MiB write has evicted L2 and
the MALL), `copy_ceiling_gbs` (a plain 1 GiB device copy, bytes read + written per second) and
`read_ceiling` (a plain read-only pass over 1 GiB, and over the decode call's own byte count, by the
streaming-read probe). With --verify-queries T, `multi_query` times multi-query decode of the last T
positions of every sequence (verification of T - 1 drafted tokens) over every layer. With --prefill, `prefill`
times chunked prefill attention (append + causal attention of each 4096-token chunk) of layer 0 of the first
sequence over its whole context. With --dense-rows (sparse workload), `dense_rows` times dense decode of its
row-layout cache over every position (the gather kernel).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak (AMD specification)
BLOCK = 32
PROFILES = os.path.join(ROOT, "profiles")
DECODE_SRC = os.path.join(ROOT, "quantized_decode_attention_append_amd", "csrc", "kvq_decode.hip")
GATHER_SRC = os.path.join(ROOT, "quantized_decode_attention_append_amd", "csrc", "kvq_gather.hip")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def row_bytes(n_bits: int, d: int) -> int:
    return d // BLOCK * (4 * n_bits + 2)


def ring_row_bytes(cfg: dict) -> int:
    if cfg["tail_len"] == 0:
        return 0
    return 2 * cfg["head_dim"] if cfg["tail_dtype"] in (1, 3) else row_bytes(8, cfg["head_dim"])   # bf16 / f16, or q8_0


def decode_kv_bytes(cfg: dict, lens, bodies) -> int:
    """Cache bytes of one dense decode call: every attended body row and ring row, K and V, plus the KVarN
    scales of each sequence."""
    hk, d = cfg["n_kv_heads"], cfg["head_dim"]
    body = hk * (row_bytes(cfg["k_bits"], d) + row_bytes(cfg["v_bits"], d))
    ring = hk * 2 * ring_row_bytes(cfg)
    total = 0
    for ln, bl in zip(lens, bodies):
        total += bl * body + (ln - bl) * ring
        if cfg["kvarn"]:
            total += hk * 2 * d * 2
    return total


def query_out_bytes(cfg: dict, n: int) -> int:
    """bf16 query rows read and fp32 output rows written for n query vectors."""
    return n * cfg["n_q_heads"] * cfg["head_dim"] * (2 + 4)


def decode_call_bytes(cfg: dict, lens, bodies) -> int:
    """Algorithmic bytes of one dense decode call (one query per sequence)."""
    return decode_kv_bytes(cfg, lens, bodies) + query_out_bytes(cfg, len(lens))


def sparse_kv_bytes(cfg: dict, budget: int, n_seqs: int) -> int:
    """Cache bytes of one sparse decode call over a body-only cache: budget K and V rows per sequence."""
    hk, d = cfg["n_kv_heads"], cfg["head_dim"]
    return n_seqs * budget * hk * (row_bytes(cfg["k_bits"], d) + row_bytes(cfg["v_bits"], d))


def sparse_call_bytes(cfg: dict, budget: int, n_seqs: int) -> int:
    """Algorithmic bytes of one sparse decode call over a body-only cache."""
    return sparse_kv_bytes(cfg, budget, n_seqs) + query_out_bytes(cfg, n_seqs)


SHARED_HEADERS = ("kvq_kernels.h", "kvq_mfma.h", "kvq_write.h", "kvq_format.h")


def source_digest(path: str) -> str:
    """SHA-256 of a kernel source together with the device headers every kernel source includes."""
    h = hashlib.sha256()
    for p in (path, *(os.path.join(os.path.dirname(path), n) for n in SHARED_HEADERS)):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str, kernel: str, src: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it covers this workload and
    kernel source; else None."""
    path = os.path.join(PROFILES, "traffic.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line.startswith("{"):
                continue
            rec = json.loads(line)
            if rec.get("workload") == workload and rec.get("kernel") == kernel \
                    and rec.get("source_sha256") == source_digest(src):
                kib = rec["fetch_kib_per_launch"] * rec["fetch_factor"] + rec["write_kib_per_launch"] * rec["write_factor"]
                return int(round(kib * 1024))
    return None


# ---------------------------------------------------------------------------------------------- CPU baseline

def _blas_one_thread():
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        return contextlib.nullcontext()


def _oracle_dense_layer(job) -> dict:
    """One worker of the CPU baseline: layer `layer` of a dense workload in the oracle (one BLAS thread). The
    prefill appends are timed as the oracle's append rate; then decode steps as the GPU runs them (append one
    token per sequence, evict, fp64 attention over the dequantized cache) until `budget_s` of step time or the
    workload's steps are done."""
    cfg_id, layer, budget_s = job
    import oracle
    import workloads as W
    wl = W.workload(cfg_id)
    seqs = list(range(wl.batch))
    cfg1 = dict(wl.cache_config(), n_layers=1)
    with _blas_one_thread():
        o = oracle.OracleCache(cfg1)
        t_app, n_app = 0.0, 0
        for seq, n in enumerate(wl.contexts):
            for s0 in range(0, n, W.CHUNK):
                k, v = W.kv_tokens(wl.cfg, layer, seq, s0, min(W.CHUNK, n - s0))
                t0 = time.perf_counter()
                o.append(0, [seq], [k.shape[0]], k, v)
                t_app += time.perf_counter() - t0
                n_app += k.shape[0]
        t0 = time.perf_counter()
        o.tail_evict(0, seqs)
        t_app += time.perf_counter() - t0
        t_write, t_total, nbytes, steps, attended = 0.0, 0.0, 0, 0, 0
        while steps < max(wl.decode_steps, 1) and (steps == 0 or t_total < budget_s):
            q = np.stack([W.query(wl.cfg, layer, s, steps) for s in seqs])
            toks = [W.decode_token(wl.cfg, layer, s, steps) for s in seqs] if wl.decode_steps else []
            t0 = time.perf_counter()
            if toks:
                o.append(0, seqs, [1] * len(seqs), np.concatenate([t[0] for t in toks]),
                         np.concatenate([t[1] for t in toks]))
                o.tail_evict(0, seqs)
            t1 = time.perf_counter()
            oracle.decode_reference(o, 0, seqs, q)
            t2 = time.perf_counter()
            t_write += t1 - t0
            t_total += t2 - t0
            lens = [o.lengths(0, s) for s in seqs]
            nbytes += decode_call_bytes(cfg1, [x[0] for x in lens], [x[1] for x in lens])
            attended += sum(x[0] for x in lens)
            steps += 1
    return {"layer": layer, "steps": steps, "seconds": t_total, "write_seconds": t_write, "bytes": nbytes,
            "attended": attended, "append_seconds": t_app, "appended": n_app}


def _oracle_sparse_layer(job) -> dict:
    """One worker of the CPU baseline on the sparse workload: body-only rows depend on their own token only, so
    a cache holding just the step's listed tokens attends over the same rows as the full cache; each step
    quantizes the listed tokens (timed as append) and runs fp64 attention over them."""
    cfg_id, layer, budget_s = job
    import oracle
    import workloads as W
    wl = W.workload(cfg_id)
    ctx = wl.contexts[0]
    cfg1 = dict(wl.cache_config(), n_layers=1, max_seqs=1, capacity=wl.budget)
    t_total, t_app, nbytes, steps = 0.0, 0.0, 0, 0
    with _blas_one_thread():
        while steps < wl.decode_steps and (steps == 0 or t_total < budget_s):
            n = ctx + steps + 1
            pos = W.sparse_positions(wl.cfg, layer, 0, steps, n, wl.budget, wl.recent)
            k = np.zeros((wl.budget, wl.n_kv_heads, wl.head_dim), dtype=np.uint16)
            v = np.zeros_like(k)
            chunks = {}
            for i, p in enumerate(pos):
                p = int(p)
                if p >= ctx:
                    kk, vv = W.decode_token(wl.cfg, layer, 0, p - ctx)
                    k[i], v[i] = kk[0], vv[0]
                else:
                    c0 = (p // W.CHUNK) * W.CHUNK
                    if c0 not in chunks:
                        chunks[c0] = W.kv_tokens(wl.cfg, layer, 0, c0, min(W.CHUNK, ctx - c0))
                    k[i], v[i] = chunks[c0][0][p - c0], chunks[c0][1][p - c0]
            q = W.query(wl.cfg, layer, 0, steps)[None]
            t0 = time.perf_counter()
            o = oracle.OracleCache(cfg1)
            o.append(0, [0], [wl.budget], k, v)
            t1 = time.perf_counter()
            oracle.decode_reference(o, 0, [0], q)
            t_total += time.perf_counter() - t0
            t_app += t1 - t0
            nbytes += sparse_call_bytes(cfg1, wl.budget, 1)
            steps += 1
    return {"layer": layer, "steps": steps, "seconds": t_total, "write_seconds": t_app, "bytes": nbytes,
            "attended": steps * wl.budget, "append_seconds": t_app, "appended": steps * wl.budget}


def _single_core_cfg1(budget_s: float = 4.0) -> dict:
    """The oracle's decode of the 4k single-layer q8_0 workload on one core (one BLAS thread)."""
    import oracle
    import workloads as W
    wl = W.workload(1)
    cfg1 = wl.cache_config()
    with _blas_one_thread():
        o = oracle.OracleCache(cfg1)
        k, v = W.kv_tokens(wl.cfg, 0, 0, 0, wl.contexts[0])
        t0 = time.perf_counter()
        o.append(0, [0], [k.shape[0]], k, v)
        t_app = time.perf_counter() - t0
        q = W.query(wl.cfg, 0, 0, 0)[None]
        t_total, calls = 0.0, 0
        while calls == 0 or t_total < budget_s:
            t0 = time.perf_counter()
            oracle.decode_reference(o, 0, [0], q)
            t_total += time.perf_counter() - t0
            calls += 1
    nb = decode_call_bytes(cfg1, [wl.contexts[0]], [wl.contexts[0]])
    return {"value": round(nb * calls / t_total / 1e9, 4), "unit": "GB/s", "cores": 1,
            "ms_per_call": round(t_total * 1e3 / calls, 2),
            "append_tok_per_s": round(k.shape[0] / t_app, 1),
            "sample": f"q8_0 single layer, context 4096: {calls} decode calls (fp64 attention), one core"}


def cpu_pool_size() -> int:
    """Worker processes of the CPU baseline: the host's cores, at most 16 (the CPU share of one GPU on the
    measurement boxes)."""
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n, os.cpu_count() or 1))


def cpu_baseline(wl, budget_s: float = 10.0) -> dict:
    """The oracle (plain NumPy, fp64 attention) timed on the host's cores: one worker process per layer (up to
    the pool size), each with one BLAS thread, running the workload's decode steps on its layer for a bounded
    time. Aggregate rate = bytes of all workers / the longest worker's step time (they run at the same time).
    Run before the GPU is initialized (the workers are started with 'spawn')."""
    import multiprocessing as mp
    P = cpu_pool_size()
    layers = list(range(min(wl.n_layers, P)))
    fn = _oracle_sparse_layer if wl.budget else _oracle_dense_layer
    log(f"cpu baseline: oracle on layers 0..{layers[-1]} in {len(layers)} worker processes")
    t0 = time.time()
    with mp.get_context("spawn").Pool(len(layers)) as pool:
        res = pool.map(fn, [(wl.cfg, layer, budget_s) for layer in layers])
    wall = time.time() - t0
    longest = max(r["seconds"] for r in res)
    nbytes = sum(r["bytes"] for r in res)
    attended = sum(r["attended"] for r in res)
    steps = sum(r["steps"] for r in res)
    single = _single_core_cfg1()
    log(f"cpu baseline done in {wall:.1f} s")
    return {"value": round(nbytes / longest / 1e9, 4), "unit": "GB/s", "cores": len(layers), "kind": "oracle",
            "sample": f"layers 0..{layers[-1]} of the workload, one worker process per layer with one BLAS thread "
                      f"({len(layers)} of {os.cpu_count()} host cores): {steps} layer-steps in all "
                      f"({'quantize the listed tokens, fp64 attention' if wl.budget else 'append 1, evict, fp64 attention over the dequantized cache'}), "
                      f"longest worker {longest:.1f} s of step time",
            "tok_per_s_per_layer": round(attended / longest / len(layers), 1),
            "append_evict_ms_per_step": round(1e3 * sum(r["write_seconds"] for r in res) / max(steps, 1), 3),
            "append_tok_per_s_per_core": round(sum(r["appended"] for r in res)
                                               / max(sum(r["append_seconds"] for r in res), 1e-9), 1),
            "single_core_cfg1": single}


def graph_steps(torch, step, first: int, n: int, n_layers: int) -> float:
    """Seconds per step with each step's launches (all layers) captured into one HIP graph beforehand.

    Capturing runs no kernel but advances the cache's host state, so steps first .. first+n-1 are captured
    in order and their graphs replayed in the same order: the device work is that of n ordinary steps, without
    the per-launch host overhead."""
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(n):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side, capture_error_mode="thread_local"):
                step(first + i)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / n
    log(f"graph: {n} steps of {n_layers} layers, {dt * 1e3:.4f} ms per step")
    return dt


def copy_ceiling(torch, mib: int = 1024, reps: int = 5) -> float:
    """Device-to-device copy rate (GB/s of bytes read + written) of a plain 1 GiB torch copy: the streaming
    ceiling measured on this GPU, beside the 8 TB/s specification."""
    src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    best = float("inf")
    for _ in range(reps):
        e0.record()
        dst.copy_(src)
        e1.record()
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1) / 1e3)
    del src, dst
    return 2.0 * (mib << 20) / best / 1e9


def read_ceiling(torch, call_bytes: int, mib: int = 1024) -> dict:
    """Read-only streaming rate of this GPU, by the probe library (a plain pass of 16-byte loads XOR-reduced to
    one word per work-group): the best over launch shapes of one pass over 1 GiB, and the best time of a pass over
    `call_bytes` (the decode call's algorithmic bytes), both with the buffer cold in L2 and the 256 MB MALL (the
    1 GiB pass exceeds them; the call-sized passes rotate over 5 regions of the buffer)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "quantized_decode_attention_append_amd", "libkvq_probe.so"))
    lib.kvq_probe_read.restype = ctypes.c_int
    lib.kvq_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    nbytes = mib << 20
    call16 = (call_bytes + 15) // 16 * 16
    region = (call16 + 4095) // 4096 * 4096
    buf = torch.zeros(max(nbytes, 5 * region), dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run(off, size, shape):
        grid, block, unroll, nt = shape
        rc = lib.kvq_probe_read(ctypes.c_void_p(buf.data_ptr() + off), size, ctypes.c_void_p(sink.data_ptr()),
                                grid, block, unroll, nt, ctypes.c_void_p(stream))
        if rc != 0:
            raise RuntimeError(f"read probe launch failed ({rc})")

    def timed(off, size, shape, reps):
        best = float("inf")
        for r in range(reps):
            o = off[r % len(off)] if isinstance(off, list) else off
            e0.record()
            run(o, size, shape)
            e1.record()
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1) / 1e3)
        return best

    shapes = [(g * n_cu, b, u, nt) for g in (1, 2, 4, 8) for b in (256, 512, 1024) for u in (2, 4, 8) for nt in (0, 1)
              if g * b <= 2048]
    res = []
    for sh in shapes:
        run(0, nbytes, sh)
        res.append((nbytes / timed(0, nbytes, sh, 3) / 1e9, sh))
    res.sort(reverse=True)
    offs = [i * region for i in range(5)]
    call = []
    for gbs, sh in res[:6]:
        t = timed(offs, call16, sh, 10)
        call.append((t, sh))
    call.sort()
    del buf, sink
    best = res[0]
    return {"gbs_1gib": round(best[0], 1), "shape_1gib": {"grid": best[1][0], "block": best[1][1],
                                                          "unroll": best[1][2], "nontemporal": best[1][3]},
            "call_bytes": int(call16), "call_us": round(call[0][0] * 1e6, 2),
            "call_gbs": round(call16 / call[0][0] / 1e9, 1),
            "how": "plain read-only pass (16-byte loads), best over launch shapes; the call-sized pass is timed "
                   "with HIP events on the launch stream, cold in L2 and MALL"}


def cold_calls(torch, cache, seqs, q, out, ws, n: int) -> dict:
    """Decode call time with the cache's lines evicted from L2 and the 256 MB MALL first (a 512 MiB write
    before every call), from the library's launch timing."""
    scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cache.timing(True)
    for i in range(n):
        scratch.fill_(i & 0xFF)
        cache.decode_attn(0, seqs, q, out=out, workspace=ws)
    torch.cuda.synchronize()
    t = {k: cache.timing_read(k) for k in ("decode", "combine")}
    cache.timing(False)
    del scratch
    return {"kernel_us": {k: round(v[0] * 1e3 / v[1], 3) for k, v in t.items() if v[1]},
            "how": "each decode call after a 512 MiB device write (L2 and MALL evicted)"}


def dense_rows_leg(torch, cache, cfg, L, seqs, q, out, ws, reps):
    """Dense decode of a row-layout cache (the sparse workload's): one kvq_decode_attn per layer over every
    position, which runs the gather kernel with the whole cache as its list; reps passes over the layers. Reports
    the wall time per pass and the gather kernel's rate in algorithmic bytes (every K and V row once)."""
    lens = [cache.lengths(0, s) for s in seqs]
    call_bytes = decode_call_bytes(cfg, [x[0] for x in lens], [x[1] for x in lens])

    def run():
        for layer in range(L):
            cache.decode_attn(layer, seqs, q[layer], out=out[layer], workspace=ws)

    run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    cache.timing(True)
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    ms, n = cache.timing_read("gather")
    cms, cn = cache.timing_read("combine")
    cache.timing(False)
    kernel_s = ms / 1e3 / max(n, 1)
    achieved = call_bytes / kernel_s / 1e9
    return {"ms_per_pass": round(elapsed * 1e3 / reps, 4), "kernel": "gather",
            "kernel_us": round(kernel_s * 1e6, 3), "combine_us": round(cms * 1e3 / max(cn, 1), 3),
            "bytes_per_call": int(call_bytes), "achieved_GBs": round(achieved, 2),
            "frac": round(achieved / HBM_PEAK_GBS, 4), "value_GBs": round(call_bytes * L * reps / elapsed / 1e9, 2),
            "how": "per layer one kvq_decode_attn over all positions of the row-layout cache (gather kernel "
                   "with every position as its list); no append"}


def multi_query_leg(torch, cache, cfg, L, seqs, qin, n_q, reps, dev):
    """Multi-query decode (the last n_q cached positions of every sequence, causal among them) over every layer,
    reps times: wall time per pass over the layers, the split kernel's dispatch-stamped average, and that kernel's
    rate in unique cache bytes (each row counted once, however many queries read it)."""
    B = len(seqs)
    hq, d = qin.shape[-2], qin.shape[-1]
    qm = [torch.from_numpy(np.ascontiguousarray(qin[np.arange(n_q) % qin.shape[0], layer].transpose(1, 0, 2, 3))
                           .view(np.int16)).to(dev) for layer in range(L)]
    lens = [cache.lengths(0, s) for s in seqs]
    ws = cache.workspace(min(B * n_q, 64), max(x[0] for x in lens))
    out = torch.empty((B, n_q, hq, d), dtype=torch.float32, device=dev)

    def run():
        for layer in range(L):
            cache.decode_attn_multi(layer, seqs, qm[layer], out=out, workspace=ws)

    run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kind = "gather" if cfg.get("layout", 0) == 1 else ("mq" if n_q > 1 else "decode")
    cache.timing(True)
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    ms, n = cache.timing_read(kind)
    cms, cn = cache.timing_read("combine")
    cache.timing(False)
    unique = decode_kv_bytes(cfg, [x[0] for x in lens], [x[1] for x in lens]) + query_out_bytes(cfg, B * n_q)
    k_us = ms * 1e3 / max(n, 1)
    log(f"multi-query decode, {n_q} queries per sequence: {k_us:.2f} us per {kind} launch")
    return {"queries": n_q, "ms_per_pass": round(elapsed * 1e3 / reps, 4), "kernel": kind,
            "kernel_us": round(k_us, 3), "combine_us": round(cms * 1e3 / max(cn, 1), 3),
            "unique_bytes_per_call": int(unique),
            "unique_GBs": round(unique / (k_us * 1e-6) / 1e9, 2),
            "frac": round(unique / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def prefill_leg(torch, kvq, W, wl, cfg, dev, reps: int = 2) -> dict:
    """Chunked prefill of layer 0 of the workload's first sequence through kvq_prefill_attn: 4096-token chunks,
    each appended and then attended causally by its own queries over the cache as it then stands. The chunk
    inputs (K, V, queries) are generated and copied to HBM first; the sequence is reset between passes. Reports
    prompt tokens per second (wall clock over the whole context), the multi-query and append kernels'
    dispatch-stamped totals, and the attention rate in useful FLOP/s (QK and PV: 4 x Hq x D per query and
    attended position) against the fp16 dense MFMA peak."""
    from concurrent.futures import ThreadPoolExecutor
    n = wl.contexts[0]
    pcfg = dict(cfg, n_layers=1, max_seqs=1, capacity=((n + 31) // 32) * 32)
    pcfg.pop("index_dim", None)
    pcfg.pop("index_pool", None)
    cache = kvq.Cache(pcfg)
    starts = list(range(0, n, W.CHUNK))

    def gen(s):
        m = min(W.CHUNK, n - s)
        k, v = W.kv_tokens(wl.cfg, 0, 0, s, m)
        q = W.prefill_queries(wl.cfg, 0, 0, s, m, wl.n_q_heads, wl.head_dim)
        return [torch.from_numpy(x.view(np.int16)).to(dev) for x in (k, v, q)]

    with ThreadPoolExecutor(max_workers=cpu_pool_size()) as ex:
        inputs = list(ex.map(gen, starts))
    out = torch.empty((W.CHUNK, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    ws = torch.empty(max(cache.prefill_workspace_bytes(1, W.CHUNK, n), 256), dtype=torch.uint8, device=dev)

    def run():
        cache.seq_reset(0, [0])
        for s, (k, v, q) in zip(starts, inputs):
            m = k.shape[0]
            cache.prefill_attn(0, [0], [m], k, v, q, out=out[:m], workspace=ws)

    run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / reps
    cache.timing(True)
    run()
    torch.cuda.synchronize()
    kt = {k: cache.timing_read(k) for k in ("mq", "combine", "append")}
    cache.timing(False)
    pairs = n * (n + 1) // 2                      # (query, attended position) pairs of the causal prefill
    flops = 4.0 * wl.n_q_heads * wl.head_dim * pairs
    mq_s = kt["mq"][0] / 1e3
    log(f"prefill of {n} tokens (layer 0): {wall * 1e3:.1f} ms, multi-query kernels {mq_s * 1e3:.1f} ms")
    del inputs, cache
    return {"tokens": n, "chunk": W.CHUNK, "ms": round(wall * 1e3, 3), "tok_per_s": round(n / wall, 1),
            "kernel_ms": {k: round(v[0], 3) for k, v in kt.items()},
            "launches": {k: v[1] for k, v in kt.items()},
            "attn_useful_TFLOPs": round(flops / mq_s / 1e12, 2),
            "frac_fp16_mfma_peak": round(flops / mq_s / 1e12 / 2500.0, 4)}


def indexer_leg(torch, cache, cfg, wl, L, seqs, first_step, n_steps, ws, dev):
    """Sparse steps whose positions the QSA indexer chooses: per layer, append one token, write its index key,
    choose the budget (the `recent` newest forced, the rest by score) and run sparse decode over the choice.
    Reports the step time and the indexer's and the gather kernel's dispatch-stamped times."""
    import workloads as W
    B = len(seqs)
    steps = list(range(first_step, first_step + 2 * n_steps))
    kin, vin, ikin, iq, qin = {}, {}, {}, {}, {}
    for st in steps:
        for layer in range(L):
            ks, vs, iks, iqs, qs = [], [], [], [], []
            for s in seqs:
                k, v = W.decode_token(wl.cfg, layer, s, st)
                ks.append(k)
                vs.append(v)
                iks.append(W.index_keys(wl.cfg, layer, s, 0, 1, chunk_id=W.DECODE_BASE + st))
                iqs.append(W.index_query(wl.cfg, layer, s, st))
                qs.append(W.query(wl.cfg, layer, s, st))
            key = (st, layer)
            kin[key] = torch.from_numpy(np.concatenate(ks).view(np.int16)).to(dev)
            vin[key] = torch.from_numpy(np.concatenate(vs).view(np.int16)).to(dev)
            ikin[key] = torch.from_numpy(np.concatenate(iks).view(np.int16)).to(dev)
            iq[key] = torch.from_numpy(np.stack(iqs).view(np.int16)).to(dev)
            qin[key] = torch.from_numpy(np.stack(qs).view(np.int16)).to(dev)
    max_len = max(cache.lengths(0, s)[0] for s in seqs) + len(steps) + 1
    iws = torch.empty(max(cache.index_workspace_bytes(B, max_len), 256), dtype=torch.uint8, device=dev)
    pos = torch.empty((L, B, wl.budget), dtype=torch.int32, device=dev)
    out = torch.empty((L, B, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    ones = [1] * B

    def step(st):
        for layer in range(L):
            key = (st, layer)
            cache.append(layer, seqs, ones, kin[key], vin[key])
            cache.index_write(layer, seqs, ones, ikin[key])
            cache.index_select(layer, seqs, iq[key], wl.budget, wl.recent, out=pos[layer], workspace=iws)
            cache.sparse_decode_attn(layer, seqs, qin[key], pos[layer], out=out[layer], workspace=ws)

    step(steps[0])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for st in steps[1:n_steps]:
        step(st)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / max(n_steps - 1, 1)
    cache.timing(True)
    for st in steps[n_steps:]:
        step(st)
    torch.cuda.synchronize()
    t = {k: cache.timing_read(k) for k in ("index", "gather", "combine", "append")}
    cache.timing(False)
    us = {k: round(v[0] * 1e3 / v[1], 3) for k, v in t.items() if v[1]}
    log(f"indexer steps: {dt * 1e3:.4f} ms per step")
    index_bytes = sum(cache.lengths(0, s)[0] for s in seqs) * 64
    return {"ms_per_step": round(dt * 1e3, 4), "kernel_us": us, "launches": {k: v[1] for k, v in t.items() if v[1]},
            "index_key_bytes_per_layer": int(index_bytes),
            "how": f"per layer: append 1 token, write its pooled index key, index select {wl.budget} positions "
                   f"({wl.recent} newest forced), sparse decode over them; 'index' spans the select's scoring and "
                   f"picking launches, 'append' covers the row and index key writes"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--config", type=int, default=4, choices=[1, 2, 3, 4, 5],
                    help="1: q8_0 4k single layer; 2: K6/V5 + bf16 tail, 64k, 16 layers; 3: KVarN K4/V4, 8 streams; "
                         "4: K6/V5 + q8_0 ring, 262k, 16 layers (default: the largest single-GPU workload); "
                         "5: sparse q8_0, budget 2048 of 262k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--verify-queries", type=int, default=0,
                    help="also time multi-query decode of the last T positions per sequence (T = 1 + drafts, <= 8) "
                         "on dense workloads, reported as the line's multi_query object")
    ap.add_argument("--indexer", action="store_true",
                    help="sparse workload: also time steps whose positions the QSA indexer chooses (append, index key "
                         "write, index select of the budget with the newest `recent` forced, sparse decode), reported "
                         "as the line's indexer object")
    ap.add_argument("--prefill", action="store_true",
                    help="dense workloads: also time chunked prefill attention of layer 0 of the first sequence over "
                         "its whole context (append + causal attention of each 4096-token chunk), reported as the "
                         "line's prefill object")
    ap.add_argument("--dense-rows", action="store_true",
                    help="sparse workload: also time dense decode of its row-layout cache over every position "
                         "(the gather kernel), reported as the line's dense_rows object")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB (for HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2

    import workloads as W
    wl = W.workload(args.config)
    # the CPU baseline first: its worker processes start before anything touches the GPU
    cpu = None if args.no_cpu_baseline else cpu_baseline(wl)

    import torch
    from quantized_decode_attention_append_amd import kvq

    # warmup, timed steps, as many steps with kernel timing, then as many captured as HIP graphs
    total_steps = args.warmup + 3 * args.steps
    ctx = list(wl.contexts)
    use_index = bool(args.indexer and wl.budget)
    index_steps = args.steps if use_index else 0
    cfg = wl.cache_config(capacity=((max(ctx) + total_steps + 2 * index_steps + 8 + 31) // 32) * 32)
    if use_index:   # offload page: indexer_head_dim 128, compress ratio 4
        cfg.update(index_dim=128, index_pool=4)
    L, B = wl.n_layers, wl.batch
    sparse = wl.budget > 0
    appends = wl.decode_steps > 0
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"workload {wl.name}; arena {kvq.cache_bytes(cfg) / 2**30:.2f} GiB")
    cache = kvq.Cache(cfg)

    # ---- prefill (set-up, not timed): 4096-token chunks per (layer, sequence), then drain the ring to W
    # the seeded chunks are drawn by a thread pool (numpy's generator releases the GIL), one layer ahead of the
    # appends
    from concurrent.futures import ThreadPoolExecutor
    gen = ThreadPoolExecutor(max_workers=cpu_pool_size())

    def chunk(layer, seq, s):
        n = min(W.CHUNK, ctx[seq] - s)
        k, v = W.kv_tokens(wl.cfg, layer, seq, s, n)
        return k, v, (W.index_keys(wl.cfg, layer, seq, s, n) if use_index else None)

    def submit_layer(layer):
        return [(seq, gen.submit(chunk, layer, seq, s)) for seq in range(B) for s in range(0, ctx[seq], W.CHUNK)]

    t0 = time.time()
    pending = submit_layer(0)
    for layer in range(L):
        chunks = pending
        pending = submit_layer(layer + 1) if layer + 1 < L else []
        for seq, fut in chunks:
            k, v, ik = fut.result()
            cache.append(layer, [seq], [k.shape[0]], torch.from_numpy(k.view(np.int16)).to(dev),
                         torch.from_numpy(v.view(np.int16)).to(dev))
            if ik is not None:
                cache.index_write(layer, [seq], [k.shape[0]], torch.from_numpy(ik.view(np.int16)).to(dev))
        del chunks
        cache.tail_evict(layer, list(range(B)))
        if layer % 4 == 3 or layer == L - 1:
            torch.cuda.synchronize()
            log(f"prefill layers 0..{layer} done ({time.time() - t0:.1f} s)")
    gen.shutdown()

    # ---- step inputs resident in HBM before timing
    kin = np.zeros((total_steps, L, B, wl.n_kv_heads, wl.head_dim), dtype=np.uint16)
    vin = np.zeros_like(kin)
    qin = np.zeros((total_steps, L, B, wl.n_q_heads, wl.head_dim), dtype=np.uint16)
    pin = np.zeros((total_steps, L, B, max(wl.budget, 1)), dtype=np.int32)
    for st in range(total_steps):
        for layer in range(L):
            for seq in range(B):
                if appends:
                    k, v = W.decode_token(wl.cfg, layer, seq, st)
                    kin[st, layer, seq], vin[st, layer, seq] = k[0], v[0]
                qin[st, layer, seq] = W.query(wl.cfg, layer, seq, st)
                if sparse:
                    pin[st, layer, seq] = W.sparse_positions(wl.cfg, layer, seq, st, ctx[seq] + st + 1,
                                                             wl.budget, wl.recent)
    kin_d = torch.from_numpy(kin.view(np.int16)).to(dev)
    vin_d = torch.from_numpy(vin.view(np.int16)).to(dev)
    qin_d = torch.from_numpy(qin.view(np.int16)).to(dev)
    pin_d = torch.from_numpy(pin).to(dev)
    seqs = list(range(B))
    ws = cache.workspace(B, max(max(ctx) + total_steps + 1, wl.budget))
    out = torch.empty((L, B, wl.n_q_heads, wl.head_dim), dtype=torch.float32, device=dev)
    ones = [1] * B

    if args.copy_calibration_mib:
        nb = args.copy_calibration_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: one device copy of {nb} bytes")
        del src, dst

    fused = appends and not sparse and wl.tail_len > 0 and cfg.get("layout", 0) == 0

    def step(st, nbytes=None):
        for layer in range(L):
            if fused:   # append one token, requantize the one leaving the window and attend: one call
                if nbytes is not None:
                    lens = [cache.lengths(layer, s) for s in seqs]
                    W_ = wl.tail_len
                    nbytes.append(decode_call_bytes(cfg, [x[0] + 1 for x in lens],
                                                    [max(x[1], x[0] + 1 - W_) for x in lens]))
                cache.decode_step(layer, seqs, kin_d[st, layer], vin_d[st, layer], qin_d[st, layer], out=out[layer],
                                  workspace=ws)
                continue
            if sparse and appends and wl.tail_len == 0:   # append one token and attend: one call
                if nbytes is not None:
                    nbytes.append(sparse_call_bytes(cfg, wl.budget, B))
                cache.sparse_decode_step(layer, seqs, kin_d[st, layer], vin_d[st, layer], qin_d[st, layer],
                                         pin_d[st, layer], out=out[layer], workspace=ws)
                continue
            if appends:   # append one token and requantize the one leaving the window: one launch
                cache.append_evict(layer, seqs, ones, kin_d[st, layer], vin_d[st, layer])
            if sparse:
                if nbytes is not None:
                    nbytes.append(sparse_call_bytes(cfg, wl.budget, B))
                cache.sparse_decode_attn(layer, seqs, qin_d[st, layer], pin_d[st, layer], out=out[layer],
                                         workspace=ws)
            else:
                if nbytes is not None:
                    lens = [cache.lengths(layer, s) for s in seqs]
                    nbytes.append(decode_call_bytes(cfg, [x[0] for x in lens], [x[1] for x in lens]))
                cache.decode_attn(layer, seqs, qin_d[st, layer], out=out[layer], workspace=ws)

    for st in range(args.warmup):
        step(st)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    nbytes = []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, nbytes)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    log(f"timed {args.steps} steps in {elapsed:.3f} s")
    # kernel durations: the same number of further steps with every launch stamped by its dispatch
    kbytes = []
    cache.timing(True)
    for i in range(args.steps):
        step(args.warmup + args.steps + i, kbytes)
    torch.cuda.synchronize()
    times = {k: cache.timing_read(k) for k in ("decode", "gather", "combine", "append", "evict", "append_evict")}
    cache.timing(False)
    graph = graph_steps(torch, step, args.warmup + 2 * args.steps, args.steps, L)
    cold = cold_calls(torch, cache, seqs, qin_d[0, 0], out[0], ws, args.steps) if (L == 1 and not appends) else None

    indexed = indexer_leg(torch, cache, cfg, wl, L, seqs, total_steps, index_steps, ws, dev) if use_index else None
    dense_rows = None
    if args.dense_rows and cfg.get("layout", 0) == 1:
        dense_rows = dense_rows_leg(torch, cache, cfg, L, seqs, qin_d[0], out, ws, max(2, args.steps // 4))
    multi = None
    if args.verify_queries and not sparse:
        multi = multi_query_leg(torch, cache, cfg, L, seqs, qin, args.verify_queries, args.steps, dev)
    pre = None
    if args.prefill and not sparse and cfg.get("layout", 0) == 0:
        pre = prefill_leg(torch, kvq, W, wl, cfg, dev)
    main_kernel = "gather" if (sparse or cfg.get("layout", 0) == 1) else "decode"
    ms, n = times[main_kernel]
    avg_s = ms / 1e3 / max(n, 1)
    total_bytes = float(sum(nbytes))
    bytes_per_launch = float(sum(kbytes)) / max(len(kbytes), 1)
    achieved = bytes_per_launch / avg_s / 1e9
    value = total_bytes / elapsed / 1e9
    ms_per_step = elapsed * 1e3 / args.steps
    attended = wl.budget * B if sparse else sum(cache.lengths(0, s)[0] for s in seqs)
    kname = (f"gather_kernel<{wl.k_bits},{wl.v_bits}>" if main_kernel == "gather"
             else f"decode_kernel<{wl.k_bits},{wl.v_bits}>")
    traffic = measured_traffic(wl.name, kname, GATHER_SRC if main_kernel == "gather" else DECODE_SRC)
    res = {
        "metric": "decode-attn effective KV GB/s (and % of HBM peak; attended tok/s per layer)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "batch": B, "context": ctx if B > 1 else ctx[0],
                   "q_heads": wl.n_q_heads, "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim,
                   "k_bits": wl.k_bits, "v_bits": wl.v_bits, "kvarn": wl.kvarn, "tail": wl.tail_len,
                   "tail_dtype": ["none", "bf16", "q8_0", "f16"][wl.tail_dtype], "budget": wl.budget,
                   "layout": ["tiles", "rows"][cfg.get("layout", 0)],
                   "step": ("per layer: append 1 token, sparse decode over the step's position list (one call)" if sparse
                            else "per layer: append 1 token, evict 1 tail token, decode attention (one call)"
                            if fused else "per layer: append 1 token, evict 1 tail token, decode attention" if appends
                            else "per layer: decode attention")},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "attended_tok_per_s_per_layer": round(attended * args.steps / elapsed, 1),
        "kernel_us": {k: round(v[0] * 1e3 / v[1], 3) for k, v in times.items() if v[1]},
        "launches": {k: v[1] for k, v in times.items() if v[1]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": kname, "bytes_per_launch": int(bytes_per_launch)},
    }
    if multi is not None:
        res["multi_query"] = multi
    if dense_rows is not None:
        res["dense_rows"] = dense_rows
    if indexed is not None:
        res["indexer"] = indexed
    if pre is not None:
        res["prefill"] = pre
    gbytes = float(sum(nbytes)) / args.steps   # the graph steps read the same bytes per step (to a few rows)
    res["graph"] = {"ms_per_step": round(graph * 1e3, 4), "value": round(gbytes / graph / 1e9, 2), "unit": "GB/s",
                    "how": f"one HIP graph per step ({L} layers), all {args.steps} captured before timing, "
                           "replayed back to back"}
    if cold is not None:
        res["cold"] = cold
    res["copy_ceiling_gbs"] = round(copy_ceiling(torch), 1)
    if not sparse:
        res["read_ceiling"] = read_ceiling(torch, int(bytes_per_launch))
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
