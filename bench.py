"""Throughput of one paged-attention step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--eager] [--no-cpu-baseline]

A step is the whole hot path over one synthetic batch: slot mapping, cache write and
attention over the mixed decode + chunked-prefill super-sequence, on one stream. By
default the step is recorded once as a HIP graph and each timed step is one replay
(--eager: separate launches); per-kernel durations come from a second pass of eager
steps with HIP events around every launch. The
default workload is the mixed chunked-prefill step (1664 decode rows plus three
2048-row prefill chunks with 0 / 2048 / 6144 tokens of cached context; 32 query heads
over 8 kv heads, head dim 128, bf16, 16-token blocks): the one workload that exercises
every kernel of the path. Inputs are seeded synthetic draws, resident in HBM before the
timed region starts.

Prints one JSON line with the whole-step rate (tokens/s), the decode kernel's HBM
roofline figures, the prefill kernel's MFMA utilisation, and the CPU oracle's rate on a
bounded sample of the same step.
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

METRIC = "paged-attn decode KV GB/s (% HBM peak); mixed-step tokens/s; prefill MFMA util"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16 matrix peak, TFLOP/s


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def step_work(step):
    """Algorithmic work of one step: decode KV bytes, prefill flops, scatter bytes."""
    ctx, qlen, L = step.lengths()
    e = 2 if step.dtype == "bf16" else 4
    hkv, hq, d = step.num_kv_heads, step.num_q_heads, step.head_dim
    dec = qlen == 1
    kv_bytes = int((L[dec] * hkv * d * 2 * e).sum())
    ch = qlen >= 2
    pairs = int((qlen[ch] * ctx[ch] + qlen[ch] * (qlen[ch] + 1) // 2).sum())
    prefill_flops = 4 * d * hq * pairs
    scatter_bytes = int(qlen.sum()) * hkv * d * 2 * e * 2  # read + write, K and V
    return {"decode_kv_bytes": kv_bytes, "decode_rows": int(dec.sum()), "prefill_flops": prefill_flops,
            "prefill_causal_pairs_per_head": pairs, "scatter_bytes": scatter_bytes}


def profiled_traffic(workload_name):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary, or None.

    The summary records a sha256 over the kernel's sources; the figure is used only while
    those sources are unchanged (a changed kernel has not been measured yet).
    """
    import hashlib

    path = os.path.join(ROOT, "profiles", f"pa_kernels_{workload_name}_hbm_bytes.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        key, sep, val = line.strip().partition(": ")
        if sep and key.startswith("traffic_"):
            fields[key] = val
    try:
        h = hashlib.sha256()
        for src in fields["traffic_sources"].split():
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != fields["traffic_sources_sha256"]:
            return None
        return float(fields["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def cpu_baseline(step, frac):
    """The CPU oracle, as it stands, on every k-th row of the same step."""
    import oracle
    import workload
    from threadpoolctl import threadpool_info

    T = step.num_tokens
    stride = max(1, int(round(1.0 / frac)))
    rows = np.arange(0, T, stride)
    qsl = step.query_start_loc.cpu().numpy()
    seq_of = np.searchsorted(qsl, rows, side="right") - 1
    seqs = np.unique(seq_of)
    sub = workload.subset_sequences(step, seqs, compact_pool=True)
    a = workload.host_arrays(sub)
    sub_qsl = a["query_start_loc"]
    pos_in_sub = {int(s): j for j, s in enumerate(seqs)}
    sub_rows = np.array([sub_qsl[pos_in_sub[int(s)]] + (r - qsl[s]) for r, s in zip(rows, seq_of)])
    t0 = time.perf_counter()
    _, slots = oracle.slot_mapping(a["block_tables"], a["query_start_loc"], a["context_lens"])
    kc, vc = oracle.reshape_and_cache(a["k"], a["v"], a["k_cache"], a["v_cache"], slots)
    oracle.attention(a["q"], kc, vc, a["block_tables"], a["seq_lens"], a["query_start_loc"], a["context_lens"],
                     a["scale"], rows=sub_rows)
    secs = time.perf_counter() - t0
    pools = threadpool_info()
    threads = max([p.get("num_threads", 1) for p in pools] + [1])
    blas = ", ".join(sorted({f"{p.get('internal_api', '?')} {p.get('version', '')}".strip() for p in pools})) or "unknown"
    cpu_model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": len(rows) / secs,
        "unit": "tokens/s",
        "cores": int(threads),
        "cpu_model": cpu_model,
        "blas": blas,
        "kind": "oracle",
        "sample": f"every {stride}th row of the step ({len(rows)} of {T} rows, {len(seqs)} sequences), "
                  f"fp64 numpy; cache write + attention for those rows; {secs:.1f} s",
        "seconds": secs,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixed_step_bf16")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time the step as separate launches instead of one HIP-graph replay")
    ap.add_argument("--cpu-sample-frac", type=float, default=1.0 / 3)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the timed steps, run one plain device-to-device copy of this many MiB "
                         "(a known-size reference for HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "bench.py measures one GPU: --gpus must be 1 (the path does not shard across GPUs)"}), flush=True)
        sys.exit(2)

    import torch

    import paged_kv_cache_460_amd as pa
    import workload

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    pa.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    log(f"[bench] building workload {args.workload} (seed {args.seed}) on {dev}")
    step = workload.make_config(args.workload, seed=args.seed, device=dev)
    work = step_work(step)
    T = step.num_tokens
    ws = torch.empty(max(1, pa.attention_workspace_size(step.num_seqs, step.max_blocks_per_seq, T, step.num_q_heads,
                                                        step.num_kv_heads, step.head_dim, step.q.dtype)),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(step.q)
    slots = torch.empty(T, dtype=torch.int64, device=dev)

    def run_step():
        _, sm = pa.build_slot_mapping(step.block_tables, step.query_start_loc, step.context_lens, num_tokens=T,
                                      with_positions=False)
        pa.reshape_and_cache(step.k, step.v, step.k_cache, step.v_cache, sm)
        pa.attention(step.q, step.k_cache, step.v_cache, step.block_tables, step.seq_lens, step.query_start_loc,
                     step.context_lens, step.scale, out=out, workspace=ws)

    # The step recorded once as a HIP graph (slot mapping, cache write, attention; the
    # same kernels with the same arguments) and replayed with one launch per step.
    graph = None if args.eager else pa.StepGraph(step.q, step.k, step.v, step.k_cache, step.v_cache,
                                                  step.block_tables, step.seq_lens, step.query_start_loc,
                                                  step.context_lens, step.scale, out, slots, ws)
    headline = run_step if graph is None else graph.replay
    mode = "eager" if graph is None else "hip_graph"

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        run_step()
        if graph is not None:
            graph.replay()
    torch.cuda.synchronize()

    log(f"[bench] timing {args.steps} steps ({mode})")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        headline()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    value = T / (ms_per_step / 1e3)
    log(f"[bench] {ms_per_step:.3f} ms/step")
    # The spread of single steps: K more steps, each between two events on the stream.
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    marks[0].record()
    for k in range(args.steps):
        headline()
        marks[k + 1].record()
    torch.cuda.synchronize()
    per_step = sorted(marks[k].elapsed_time(marks[k + 1]) for k in range(args.steps))
    step_median, step_min = per_step[len(per_step) // 2], per_step[0]
    if graph is not None:
        graph.close()

    # Per-kernel durations: K eager steps with every launch bracketed by HIP events on its
    # own stream (libpa's timing); a graph replay runs these same kernels.
    log(f"[bench] timing {args.steps} eager steps with per-kernel events")
    with pa.KernelTimer() as timer:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            run_step()
        torch.cuda.synchronize()
        eager_ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
        kernels = {k: timer.read(k) for k in ("slot_mapping", "scatter", "plan", "prefix", "decode", "reduce",
                                              "prefill", "attn_f32")}
    avg_ms = {k: (v[0] / v[1] if v[1] else 0.0) for k, v in kernels.items()}
    log(f"[bench] eager {eager_ms_per_step:.3f} ms/step; kernel averages (ms): "
        + ", ".join(f"{k}={v:.4f}" for k, v in avg_ms.items() if v))

    dec_ms = avg_ms["decode"]
    dec_gbps = work["decode_kv_bytes"] / (dec_ms * 1e-3) / 1e9 if dec_ms else None
    pre_ms = avg_ms["prefill"]
    pre_tflops = work["prefill_flops"] / (pre_ms * 1e-3) / 1e12 if pre_ms and work["prefill_flops"] else None

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if step.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "num_seqs": step.num_seqs,
            "tokens_per_step": T,
            "decode_rows": work["decode_rows"],
            "num_q_heads": step.num_q_heads,
            "num_kv_heads": step.num_kv_heads,
            "head_dim": step.head_dim,
            "block_size": 16,
            "num_blocks": step.num_blocks,
            "seed": args.seed,
            "execution": mode,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode",
            "achieved": dec_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": dec_gbps / HBM_PEAK_GBPS if dec_gbps else None,
            "traffic": profiled_traffic(args.workload),
            "algorithmic_bytes_per_launch": work["decode_kv_bytes"],
            "avg_launch_ms": dec_ms,
        },
        "breakdown": {
            "kernel_avg_ms": avg_ms,
            "decode_kv_gbps": dec_gbps,
            "decode_hbm_frac": dec_gbps / HBM_PEAK_GBPS if dec_gbps else None,
            "prefill_tflops": pre_tflops,
            "prefill_mfma_util": pre_tflops / BF16_MFMA_PEAK_TFLOPS if pre_tflops else None,
            "prefill_flops_per_launch": work["prefill_flops"],
            "scatter_bytes_per_launch": work["scatter_bytes"],
            "execution": mode,
            "ms_per_step_median": step_median,
            "ms_per_step_min": step_min,
            "eager_ms_per_step_with_kernel_events": eager_ms_per_step,
        },
    }
    if args.copy_probe_mib > 0:
        n = (args.copy_probe_mib << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)  # one elementwise kernel: reads n*4 bytes, writes n*4 bytes
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {args.copy_probe_mib} MiB read + {args.copy_probe_mib} MiB written")
        del src, dst
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on a sample of the step)")
        result["cpu_baseline"] = cpu_baseline(step, args.cpu_sample_frac)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
