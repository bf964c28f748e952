"""Decode-attention benchmark of the quantized KV cache on one MI355X.

A step is one pass of the hot path over every layer of the workload, with inputs already in HBM:
per layer, append one token per sequence (tail-ring write), evict the oldest tail token (requantize
into the qN_0 body) and run decode attention over the whole cache; sparse workloads append and then
run sparse decode over the step's position list.

Default workload: 16 layers, batch 1, context 65,536, 16 query / 2 KV heads x 256, K 6-bit / V 5-bit
body with a 2,048-token bf16 precision tail, 64 decode steps (synthetic Gaussian K/V with per-channel
standard deviations log-uniform in [0.1, 10]).

Prints one JSON line. `value` is the effective KV GB/s of decode attention over the whole step
(algorithmic KV bytes read by the decode calls / step time). `roofline` is the decode kernel's rate:
algorithmic bytes per launch / average kernel time, from HIP events that the kernel dispatches stamp
with their start and end (library launch timing, measured on a second run of the same number of steps),
against 8 TB/s HBM3E. `traffic` is the HBM bytes per launch measured with
rocprofv3 FETCH_SIZE / WRITE_SIZE counters (scaled by the copy-kernel calibration stored with them),
used only while the kernel source still matches the one that was measured. `cpu_baseline` is the CPU
oracle timed on a bounded sample of the same workload. Also reported: `graph` (the same steps with each step's
launches captured into one HIP graph beforehand and replayed back to back), `cold` (single-layer workloads:
decode time after a 512 MiB write has evicted L2 and the MALL) and `copy_ceiling_gbs` (a plain 1 GiB device
copy, bytes read + written per second). With --verify-queries T, `multi_query` times multi-query decode of the
last T positions of every sequence (verification of T - 1 drafted tokens) over every layer.
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


def decode_call_bytes(cfg: dict, lens, bodies) -> int:
    """Algorithmic KV bytes of one dense decode call: every attended body row and ring row, K and V,
    plus the KVarN scales."""
    hk, d = cfg["n_kv_heads"], cfg["head_dim"]
    body = hk * (row_bytes(cfg["k_bits"], d) + row_bytes(cfg["v_bits"], d))
    ring = hk * 2 * ring_row_bytes(cfg)
    total = 0
    for ln, bl in zip(lens, bodies):
        total += bl * body + (ln - bl) * ring
        if cfg["kvarn"]:
            total += hk * 2 * d * 2
    return total


def sparse_call_bytes(cfg: dict, budget: int, n_seqs: int) -> int:
    """Algorithmic KV bytes of one sparse decode call over a body-only cache: budget K and V rows."""
    hk, d = cfg["n_kv_heads"], cfg["head_dim"]
    return n_seqs * budget * hk * (row_bytes(cfg["k_bits"], d) + row_bytes(cfg["v_bits"], d))


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


def cpu_baseline(wl, budget_s: float = 15.0) -> dict:
    """The oracle (plain NumPy, fp64 attention) on layer 0 of the workload, one BLAS thread."""
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        limit = contextlib.nullcontext()
    import oracle
    import workloads as W
    cfg1 = dict(wl.cache_config(), n_layers=1, max_seqs=1)
    ctx = wl.contexts[0]
    if wl.budget:
        # body-only rows depend on their own token only: a cache holding just the step's listed tokens
        # attends over the same rows as the full cache
        t_total, nbytes, steps = 0.0, 0, 0
        with limit:
            while t_total < budget_s and steps < wl.decode_steps:
                n = ctx + steps + 1
                pos = W.sparse_positions(wl.cfg, 0, 0, steps, n, wl.budget, wl.recent)
                k = np.zeros((wl.budget, wl.n_kv_heads, wl.head_dim), dtype=np.uint16)
                v = np.zeros_like(k)
                chunks = {}
                for i, p in enumerate(pos):
                    p = int(p)
                    if p >= ctx:
                        kk, vv = W.decode_token(wl.cfg, 0, 0, p - ctx)
                        k[i], v[i] = kk[0], vv[0]
                    else:
                        c0 = (p // W.CHUNK) * W.CHUNK
                        if c0 not in chunks:
                            chunks[c0] = W.kv_tokens(wl.cfg, 0, 0, c0, min(W.CHUNK, ctx - c0))
                        k[i], v[i] = chunks[c0][0][p - c0], chunks[c0][1][p - c0]
                q = W.query(wl.cfg, 0, 0, steps)[None]
                cfg_s = dict(cfg1, capacity=wl.budget)
                t0 = time.perf_counter()
                o = oracle.OracleCache(cfg_s)
                o.append(0, [0], [wl.budget], k, v)
                oracle.decode_reference(o, 0, [0], q)
                t_total += time.perf_counter() - t0
                nbytes += sparse_call_bytes(cfg1, wl.budget, 1)
                steps += 1
        return {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"layer 0: {steps} sparse decode steps over {wl.budget} listed positions (quantize the "
                          f"listed tokens, fp64 attention), {t_total:.1f} s, one BLAS thread",
                "tok_per_s_per_layer": round(steps * wl.budget / t_total, 1)}
    log(f"cpu baseline: oracle prefill of {ctx} tokens (not timed)")
    o = oracle.OracleCache(cfg1)
    for s in range(0, ctx, W.CHUNK):
        k, v = W.kv_tokens(wl.cfg, 0, 0, s, min(W.CHUNK, ctx - s))
        o.append(0, [0], [k.shape[0]], k, v)
    o.tail_evict(0, [0])
    t_total, t_write, nbytes, steps = 0.0, 0.0, 0, 0
    with limit:
        while t_total < budget_s and steps < max(wl.decode_steps, 1):
            q = W.query(wl.cfg, 0, 0, steps)[None]
            t0 = time.perf_counter()
            if wl.decode_steps:
                k, v = W.decode_token(wl.cfg, 0, 0, steps)
                o.append(0, [0], [1], k, v)
                o.tail_evict(0, [0])
            t_write += time.perf_counter() - t0
            oracle.decode_reference(o, 0, [0], q)
            t_total += time.perf_counter() - t0
            ln, bl = o.lengths(0, 0)
            nbytes += decode_call_bytes(cfg1, [ln], [bl])
            steps += 1
    return {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"layer 0 of the workload at context {ctx}: {steps} decode steps (append 1, evict, "
                      f"fp64 attention over the dequantized cache), {t_total:.1f} s, one BLAS thread",
            "tok_per_s_per_layer": round(steps * (ctx + steps / 2) / t_total, 1),
            "append_evict_ms_per_step": round(t_write * 1e3 / max(steps, 1), 3)}


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
    kind = "gather" if cfg.get("layout", 0) == 1 else "decode"
    cache.timing(True)
    for _ in range(reps):
        run()
    torch.cuda.synchronize()
    ms, n = cache.timing_read(kind)
    cms, cn = cache.timing_read("combine")
    cache.timing(False)
    unique = decode_call_bytes(cfg, [x[0] for x in lens], [x[1] for x in lens])
    k_us = ms * 1e3 / max(n, 1)
    log(f"multi-query decode, {n_q} queries per sequence: {k_us:.2f} us per {kind} launch")
    return {"queries": n_q, "ms_per_pass": round(elapsed * 1e3 / reps, 4), "kernel": kind,
            "kernel_us": round(k_us, 3), "combine_us": round(cms * 1e3 / max(cn, 1), 3),
            "unique_bytes_per_call": int(unique),
            "unique_GBs": round(unique / (k_us * 1e-6) / 1e9, 2),
            "frac": round(unique / (k_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5],
                    help="1: q8_0 4k single layer; 2: K6/V5 + bf16 tail, 64k, 16 layers (default); 3: KVarN "
                         "K4/V4, 8 streams; 4: K6/V5 + q8_0 ring, 262k; 5: sparse q8_0, budget 2048 of 262k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--verify-queries", type=int, default=0,
                    help="also time multi-query decode of the last T positions per sequence (T = 1 + drafts, <= 8) "
                         "on dense workloads, reported as the line's multi_query object")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB (for HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import workloads as W
    from quantized_decode_attention_append_amd import kvq

    wl = W.workload(args.config)
    # warmup, timed steps, as many steps with kernel timing, then as many captured as HIP graphs
    total_steps = args.warmup + 3 * args.steps
    ctx = list(wl.contexts)
    cfg = wl.cache_config(capacity=((max(ctx) + total_steps + 8 + 31) // 32) * 32)
    L, B = wl.n_layers, wl.batch
    sparse = wl.budget > 0
    appends = wl.decode_steps > 0
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"workload {wl.name}; arena {kvq.cache_bytes(cfg) / 2**30:.2f} GiB")
    cache = kvq.Cache(cfg)

    # ---- prefill (set-up, not timed): 4096-token chunks per (layer, sequence), then drain the ring to W
    t0 = time.time()
    for layer in range(L):
        for seq in range(B):
            n = ctx[seq]
            for s in range(0, n, W.CHUNK):
                k, v = W.kv_tokens(wl.cfg, layer, seq, s, min(W.CHUNK, n - s))
                cache.append(layer, [seq], [k.shape[0]], torch.from_numpy(k.view(np.int16)).to(dev),
                             torch.from_numpy(v.view(np.int16)).to(dev))
        cache.tail_evict(layer, list(range(B)))
        if layer % 4 == 3 or layer == L - 1:
            torch.cuda.synchronize()
            log(f"prefill layers 0..{layer} done ({time.time() - t0:.1f} s)")

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

    multi = None
    if args.verify_queries and not sparse:
        multi = multi_query_leg(torch, cache, cfg, L, seqs, qin, args.verify_queries, args.steps, dev)
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
                   "tail_dtype": ["none", "bf16", "q8_0"][wl.tail_dtype], "budget": wl.budget,
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
    gbytes = float(sum(nbytes)) / args.steps   # the graph steps read the same bytes per step (to a few rows)
    res["graph"] = {"ms_per_step": round(graph * 1e3, 4), "value": round(gbytes / graph / 1e9, 2), "unit": "GB/s",
                    "how": f"one HIP graph per step ({L} layers), all {args.steps} captured before timing, "
                           "replayed back to back"}
    if cold is not None:
        res["cold"] = cold
    res["copy_ceiling_gbs"] = round(copy_ceiling(torch), 1)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
