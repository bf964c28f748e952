"""Decode-attention benchmark of the quantized KV cache on one MI355X.

A step is one pass of the hot path over every layer of the workload: append one token (tail-ring write),
evict the oldest tail token (requantize into the qN_0 body) and run decode attention over the whole
cache. Inputs (decode tokens, queries) are resident in HBM before the timed region starts.

Default workload: 16 layers, batch 1, context 65,536, 16 query / 2 KV heads x 256, K 6-bit / V 5-bit
body with a 2,048-token bf16 precision tail, 64 decode steps (synthetic Gaussian K/V with per-channel
standard deviations log-uniform in [0.1, 10]).

Prints one JSON line: effective KV GB/s of decode attention over the step (algorithmic KV bytes read by
the decode calls / step time), attended tokens/s per layer, the roofline of the decode kernel (bytes per
launch / average launch time from HIP events on the launch stream, against 8 TB/s HBM3E) and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak (AMD specification)
BLOCK = 32


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def row_bytes(n_bits: int, d: int) -> int:
    return d // BLOCK * (4 * n_bits + 2)


def decode_call_bytes(cfg: dict, lens, bodies) -> int:
    """Algorithmic KV bytes one decode call reads: every attended body row and ring row, K and V."""
    hk, d = cfg["n_kv_heads"], cfg["head_dim"]
    body = hk * (row_bytes(cfg["k_bits"], d) + row_bytes(cfg["v_bits"], d))
    if cfg["tail_len"] > 0:
        ring = hk * 2 * (2 * d if cfg["tail_dtype"] == 1 else row_bytes(8, d))
    else:
        ring = 0
    total = 0
    for ln, bl in zip(lens, bodies):
        total += bl * body + (ln - bl) * ring
        if cfg["kvarn"]:
            total += hk * 2 * d * 2
    return total


def cpu_baseline(wl, budget_s: float = 15.0) -> dict:
    """The oracle (plain NumPy, fp64 attention) on layer 0 of the workload, single BLAS thread."""
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    import oracle
    import workloads as W
    cfg1 = dict(wl.cache_config(), n_layers=1, max_seqs=1)
    ctx = wl.contexts[0]
    log(f"cpu baseline: oracle prefill of {ctx} tokens (not timed)")
    o = oracle.OracleCache(cfg1)
    for s in range(0, ctx, W.CHUNK):
        k, v = W.kv_tokens(wl.cfg, 0, 0, s, min(W.CHUNK, ctx - s))
        o.append(0, [0], [k.shape[0]], k, v)
    o.tail_evict(0, [0])
    import contextlib
    limit = threadpool_limits(limits=1) if threadpool_limits else contextlib.nullcontext()
    t_total, nbytes, steps = 0.0, 0, 0
    with limit:
        while t_total < budget_s and steps < wl.decode_steps:
            k, v = W.decode_token(wl.cfg, 0, 0, steps)
            q = W.query(wl.cfg, 0, 0, steps)[None]
            t0 = time.perf_counter()
            o.append(0, [0], [1], k, v)
            o.tail_evict(0, [0])
            oracle.decode_reference(o, 0, [0], q)
            t_total += time.perf_counter() - t0
            ln, bl = o.lengths(0, 0)
            nbytes += decode_call_bytes(cfg1, [ln], [bl])
            steps += 1
    return {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"layer 0 of the workload at context {ctx}: {steps} decode steps (append 1, evict, "
                      f"fp64 attention over the dequantized cache), {t_total:.1f} s, single BLAS thread",
            "tok_per_s_per_layer": round(steps * (ctx + steps / 2) / t_total, 1)}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=60)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB (for HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2

    import torch
    import workloads as W
    from quantized_decode_attention_append_amd import kvq

    wl = W.workload(args.config)
    total_steps = args.warmup + args.steps
    ctx = list(wl.contexts)
    cfg = wl.cache_config(capacity=((max(ctx) + total_steps + 8 + 31) // 32) * 32)
    L, B = wl.n_layers, wl.batch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"workload {wl.name}; arena {kvq.cache_bytes(cfg) / 2**30:.2f} GiB")
    cache = kvq.Cache(cfg)

    # ---- prefill (setup, not timed): 4096-token chunks per (layer, sequence), then drain the ring to W
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

    # ---- decode inputs resident in HBM before timing
    kin = np.zeros((total_steps, L, B, 2, 256), dtype=np.uint16)
    vin = np.zeros_like(kin)
    qin = np.zeros((total_steps, L, B, wl.n_q_heads, 256), dtype=np.uint16)
    for st in range(total_steps):
        for layer in range(L):
            for seq in range(B):
                k, v = W.decode_token(wl.cfg, layer, seq, st)
                kin[st, layer, seq], vin[st, layer, seq] = k[0], v[0]
                qin[st, layer, seq] = W.query(wl.cfg, layer, seq, st)
    kin_d = torch.from_numpy(kin.view(np.int16)).to(dev)
    vin_d = torch.from_numpy(vin.view(np.int16)).to(dev)
    qin_d = torch.from_numpy(qin.view(np.int16)).to(dev)
    seqs = list(range(B))
    ws = cache.workspace(B, max(ctx) + total_steps + 1)
    out = torch.empty((L, B, wl.n_q_heads, 256), dtype=torch.float32, device=dev)
    ones = [1] * B

    if args.copy_calibration_mib:
        nb = args.copy_calibration_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: one device copy of {nb} bytes")
        del src, dst

    def step(st, events=None, nbytes=None):
        for layer in range(L):
            cache.append(layer, seqs, ones, kin_d[st, layer], vin_d[st, layer])
            cache.tail_evict(layer, seqs)
            if nbytes is not None:
                lens = [cache.lengths(layer, s) for s in seqs]
                nbytes.append(decode_call_bytes(cfg, [x[0] for x in lens], [x[1] for x in lens]))
            if events is not None:
                events[layer][0].record()
            cache.decode_attn(layer, seqs, qin_d[st, layer], out=out[layer], workspace=ws)
            if events is not None:
                events[layer][1].record()

    for st in range(args.warmup):
        step(st)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    ev = [[[torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)] for _ in range(L)]
          for _ in range(args.steps)]
    nbytes = []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, ev[i], nbytes)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    call_ms = [ev[i][layer][0].elapsed_time(ev[i][layer][1]) for i in range(args.steps) for layer in range(L)]
    log(f"timed {args.steps} steps in {elapsed:.3f} s")

    total_bytes = float(sum(nbytes))
    ms_per_step = elapsed * 1e3 / args.steps
    value = total_bytes / elapsed / 1e9
    avg_call_s = float(np.mean(call_ms)) / 1e3
    bytes_per_call = total_bytes / len(nbytes)
    achieved = bytes_per_call / avg_call_s / 1e9
    attended = sum(cache.lengths(0, s)[0] for s in seqs)
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
        "config": {"workload": wl.name, "layers": L, "batch": B,
                   "context": ctx if B > 1 else ctx[0], "q_heads": wl.n_q_heads, "kv_heads": wl.n_kv_heads,
                   "head_dim": wl.head_dim, "k_bits": wl.k_bits, "v_bits": wl.v_bits, "kvarn": wl.kvarn,
                   "tail": wl.tail_len, "tail_dtype": ["none", "bf16", "q8_0"][wl.tail_dtype],
                   "step": "per layer: append 1 token, evict 1 tail token, decode attention"},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "attended_tok_per_s_per_layer": round(attended * args.steps / elapsed, 1),
        "decode_call_us": round(avg_call_s * 1e6, 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "decode_kernel (one launch per decode call)",
                     "bytes_per_launch": int(bytes_per_call)},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
