"""Throughput of the multi-row sparse-attention decode core on one MI355X.

One step = the whole path for every row of the workload: indexer score ->
top-512 -> gather of the selected KV rows -> sparse attention with sinks.
The headline runs it as one C-ABI call, ds_rows_indexer_topk_attn: the
indexer with the first selection stage in its epilogue, then the final
selection level inside the attention's workgroups (gather fused), then the
attention's combine. The two-call form (ds_rows_indexer_topk, then
ds_rows_sparse_attn_direct), the three-call form (separate
ds_rows_indexer_score and ds_rows_topk) and the four-call form
(ds_rows_gather, then ds_rows_sparse_attn) compute the same outputs and are
timed beside it.
Default workload: 8 rows x 32768 cached keys (64 heads x 128 indexer, top-512,
64 heads x 512 attention), seeded synthetic inputs resident in HBM.

Cache policy: `--copies` independent device copies of the inputs are used in
rotation (default 8 x ~330 MB), so each step's 64 MiB of indexer keys was
last touched 7 steps earlier, after ~2.3 GB of other traffic: the keys come
from HBM, not from the 256 MB last-level cache. `--copies 1` measures the
warm-cache case.

Prints one JSON line (rank 0, N=1) with the headline value, per-call
durations from HIP events on the launch stream, the roofline of the dominant
kernel (the indexer, in its fused form) and the CPU oracle timed on a bounded
sample.
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

METRIC = "decode rows/s (indexer+top-k+sparse attn), 8 rows×32k KV; % MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", type=int, default=2)
    p.add_argument("--copies", type=int, default=8)
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--leg", choices=("all", "multi_query", "compressor"), default="all",
                   help="run only the multi-query indexer or the compressor leg and print its JSON object")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 64 MiB device-to-device copy 5 times (reference for the "
                        "FETCH_SIZE / WRITE_SIZE counter scale) and exit")
    return p.parse_args()


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "indexer_fused_traffic_8x32768.md")
INDEXER_SOURCES = [os.path.join(ROOT, "sparse_attention_decode_04_amd", "csrc", f)
                   for f in ("indexer_score.hip", "device_common.hpp", "select_common.hpp", "ds_rows_internal.hpp")]


def indexer_source_hash():
    """SHA-256 of the indexer kernel's code: its source file, the shared device
    helpers and the indexer section of the internal header."""
    import hashlib
    h = hashlib.sha256()
    for f in INDEXER_SOURCES:
        with open(f, "rb") as fh:
            text = fh.read()
        if f.endswith("ds_rows_internal.hpp"):
            start = text.index(b"// ---------------------------------------------------------------- indexer")
            end = text.index(b"// ----", start + 10)
            text = text[start:end]
        h.update(text)
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per indexer launch from the committed counter summary, or
    None when there is none or the kernel's sources changed since it was taken."""
    try:
        fields = {}
        with open(TRAFFIC_PROFILE) as fh:
            for line in fh:
                if line.startswith("- `") and "`: " in line:
                    k, v = line[3:].split("`: ", 1)
                    fields[k] = v.strip()
        if fields.get("kernel_source_sha256") != indexer_source_hash():
            return None
        return {"fetch": float(fields["fetch_bytes_per_launch"]), "write": float(fields["write_bytes_per_launch"])}
    except (OSError, KeyError, ValueError):
        return None


def indexer_bytes_flops(inp, fused=False):
    """Algorithmic HBM bytes and MFMA flops of one indexer launch: per key
    256 B of keys read + 4 B of score written and 64*128*2 flops; per row
    16 KiB of query and 256 B of weights read; in the fused form also, per
    1024-key block, 128 candidate keys of 8 B and four 4 B floors written."""
    keys = sum(inp.kv_len)
    b = keys * (256 + 4) + inp.rows * (64 * 128 * 2 + 64 * 4)
    if fused:
        b += sum(-(-n // 1024) for n in inp.kv_len) * (128 * 8 + 4 * 4)
    return b, keys * 64 * 128 * 2


def step_bytes(inp):
    """Algorithmic bytes of one headline step: the fused indexer, the top-k
    levels over its candidates (read, plus the indices written), and the
    attention reading its selected KV rows through the indices."""
    w = [min(n, 512) for n in inp.kv_len]
    blocks = sum(-(-n // 1024) for n in inp.kv_len)
    idx_b, _ = indexer_bytes_flops(inp, fused=True)
    topk_b = blocks * (128 * 8 + 4 * 4) + inp.rows * 512 * 4
    attn_b = sum(64 * 512 * 2 + wi * (1024 + 4) + 64 * 512 * 4 for wi in w) + 256
    return idx_b + topk_b + attn_b


def compressor_bytes(inp):
    """Algorithmic HBM bytes of one ds_rows_compressor call: per row, the
    token's value and score and its position-embedding row (f32, P each),
    the state row the token lands in (written, both states), the output
    (bf16) and, for a token that ends a block, the window (head_dim features
    of each window row, both states) plus, with overlap, the shift (the
    current block's other half read, ratio rows of both states written);
    the RMS scale once per call."""
    coff = 2 if inp.ratio == 4 else 1
    P, hd, ratio = coff * inp.head_dim, inp.head_dim, inp.ratio
    total = 4 * hd
    for pos in inp.start_pos:
        b = 3 * 4 * P + 2 * 4 * P + 2 * hd
        if (pos + 1) % ratio == 0:
            window = 2 * ratio if coff == 2 else ratio
            b += window * hd * 4 * 2
            if coff == 2:
                b += ratio * hd * 4 * 2 + ratio * P * 4 * 2
        total += b
    return total


def compressor_bench(torch, n_calls):
    """Each compressor shape at 8 rows (every token ends a block): mean call
    duration, algorithmic bytes and their rate against HBM peak. A call is a
    few microseconds of GPU work, less than the Python binding needs to
    enqueue one, so 16 calls (one per state set) are captured once in a HIP
    graph and the graph is replayed; the duration is HIP-event time over the
    replays divided by the calls."""
    from sparse_attention_decode_04_amd import inputs as I
    from sparse_attention_decode_04_amd.runner import DeviceCompressor
    res = {}
    stream = torch.cuda.current_stream()
    for ratio, hd in I.COMPRESSOR_SHAPES:
        inp = I.compressor_workload(ratio, hd)
        dev = DeviceCompressor(inp, copies=16)
        for c in range(16):
            dev.run(c)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for c in range(16):
                dev.run(c)
        reps = max(1, n_calls // 16)
        graph.replay()
        torch.cuda.synchronize()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for _ in range(reps):
            graph.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / (16 * reps)
        nbytes = compressor_bytes(inp)
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[f"ratio{ratio}_dim{hd}"] = {
            "rows": inp.rows, "us_per_call": ms * 1e3, "rows_per_s": inp.rows / (ms * 1e-3),
            "bytes_per_call": nbytes, "achieved_gb_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "bound": "latency (< 5 MB per call)"}
    return res


def mq_bytes_flops(inp):
    """Algorithmic bytes and MFMA flops of one ds_rows_indexer_score_mq call:
    per key 256 B read and 4 B per query written, 2*64*128 flops per query;
    per row its queries and weights (16 KiB + 256 B each)."""
    Q, keys = inp.query_len, sum(inp.kv_len)
    nbytes = keys * (256 + 4 * Q) + inp.rows * Q * (64 * 128 * 2 + 64 * 4)
    return nbytes, 2 * 64 * 128 * Q * keys


def mq_bench(torch, n_calls, query_len=8, copies=4):
    """The multi-query indexer on 8 rows x 32768 keys x `query_len` queries:
    mean call duration from HIP events around back-to-back calls over
    `copies` rotating key copies, against the bf16 MFMA and HBM peaks."""
    from sparse_attention_decode_04_amd import inputs as I
    from sparse_attention_decode_04_amd.runner import DeviceMultiQuery
    inp = I.mq_workload(query_len)
    devs = [DeviceMultiQuery(inp) for _ in range(copies)]
    stream = torch.cuda.current_stream()
    for d in devs:
        d.run()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(n_calls):
        devs[i % copies].run()
    ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / n_calls
    nbytes, flops = mq_bytes_flops(inp)
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"call": "ds_rows_indexer_score_mq", "rows": inp.rows, "kv_len": inp.kv_len[0], "query_len": query_len,
            "timing": f"HIP events around back-to-back calls over {copies} rotating key copies",
            "ms_per_call": ms, "keys_per_s": sum(inp.kv_len) / (ms * 1e-3),
            "mfma_tflops": tflops, "mfma_frac_of_bf16_peak": tflops / BF16_PEAK_TFLOPS,
            "achieved_gb_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "bytes_per_call": nbytes, "flops_per_call": flops}


def cpu_baseline(inp, seconds):
    from threadpoolctl import threadpool_info

    from oracle import ds_oracle as O
    rows = 0
    t0 = time.perf_counter()
    while True:
        O.decode_rows(inp)
        rows += inp.rows
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": rows / el, "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows // inp.rows} full oracle steps ({rows} rows of the same workload) in {el:.1f} s; "
                      f"numpy float64/int64, BLAS threads={threads}, host cpu_count={os.cpu_count()}"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): rows are independent requests and "
              "this build measures one GPU's share; see the sharding notes in the design document.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    # Every launch and event goes to one stream of the bench's own (default
    # priority), as a serving loop would use: work on the legacy null stream
    # measured about 1 us more per step.
    torch.cuda.set_stream(torch.cuda.Stream())

    if args.copy_calibration:
        n = 64 << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 5}), flush=True)
        return

    from sparse_attention_decode_04_amd import ds_rows as ds
    from sparse_attention_decode_04_amd import inputs as I
    from sparse_attention_decode_04_amd.runner import DeviceInputs, DeviceRows

    ds.load()
    if args.leg == "multi_query":
        print(json.dumps(mq_bench(torch, args.steps)), flush=True)
        return
    if args.leg == "compressor":
        print(json.dumps(compressor_bench(torch, args.steps)), flush=True)
        return
    inp = I.make_config(args.config)
    base = DeviceInputs(inp)
    copies = [base]
    for _ in range(args.copies - 1):
        c = DeviceInputs.__new__(DeviceInputs)
        c.inp, c.device = inp, base.device
        c.idx_q, c.idx_w, c.attn_q, c.sinks = (base.idx_q.clone(), base.idx_w.clone(),
                                               base.attn_q.clone(), base.sinks.clone())
        c.keys = [k.clone() for k in base.keys]
        c.kv = [k.clone() for k in base.kv]
        copies.append(c)
    runs = [DeviceRows(c) for c in copies]
    stream = torch.cuda.current_stream()


    def timed(step_name):
        """K whole steps bracketed by device synchronisation; ms per step."""
        for i in range(args.warmup):
            getattr(runs[i % len(runs)], step_name)()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(args.steps):
            getattr(runs[i % len(runs)], step_name)()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / args.steps, time.perf_counter() - t0

    # Headline: the one-call decode core.
    ms_per_step, wall = timed("step_one")
    # Score + top-k in one call, then attention with the gather fused in.
    ms_two, _ = timed("step_fused")
    # Separate score and top-k calls, then the same attention.
    ms_three, _ = timed("step_direct")
    # The four-call path (gather, then attention on the gathered rows).
    ms_four, _ = timed("step")

    def per_call_ms(calls):
        """Mean duration of each call, from HIP events recorded around it on
        the launch stream, over K steps."""
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(args.steps)]
        for i in range(args.steps):
            r = runs[i % len(runs)]
            for k, c in enumerate(calls):
                evs[i][k].record(stream)
                getattr(r, c)()
            evs[i][len(calls)].record(stream)
        torch.cuda.synchronize()
        return {c: float(np.mean([evs[i][k].elapsed_time(evs[i][k + 1]) for i in range(args.steps)]))
                for k, c in enumerate(calls)}

    def back_to_back_ms(call, n):
        """Mean duration of one `call` from HIP events on the launch stream
        around n back-to-back launches over the rotating input copies."""
        for i in range(len(runs)):
            getattr(runs[i], call)()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(n):
            getattr(runs[i % len(runs)], call)()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n

    per_call = per_call_ms(("indexer_topk", "sparse_attn_direct"))
    indexer_ms = back_to_back_ms("indexer_candidates", max(args.steps, 50))
    per_call_three = per_call_ms(("indexer_score", "topk", "sparse_attn_direct"))
    per_call_four = per_call_ms(("indexer_score", "topk", "gather", "sparse_attn"))

    idx_bytes, idx_flops = indexer_bytes_flops(inp, fused=True)
    traffic = measured_traffic() if args.config == 2 else None
    idx_s = indexer_ms * 1e-3
    achieved = idx_bytes / idx_s / 1e9
    rows_per_s = inp.rows / (ms_per_step * 1e-3)
    keys_per_s = sum(inp.kv_len) / (ms_per_step * 1e-3)

    out = {
        "metric": METRIC,
        "value": rows_per_s,
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{I.CONFIG_NAMES[args.config]} (indexer 64x128 bf16 integer-valued, top-512, "
                        f"sparse attention 64x512 bf16 with sinks, f32 out)",
            "rows": inp.rows, "kv_len": inp.kv_len if len(set(inp.kv_len)) > 1 else inp.kv_len[0],
            "top_k": 512, "cache": f"{args.copies} rotating input copies" if args.copies > 1 else "warm",
        },
        "keys_per_s": keys_per_s,
        "step_algorithmic_gb_per_s": step_bytes(inp) / (ms_per_step * 1e-3) / 1e9,
        "pipeline": "ds_rows_indexer_topk_attn (indexer with the first top-k stage; final top-k level inside the "
                    "attention workgroups, gather fused; combine)",
        "two_call_pipeline": {
            "calls": "ds_rows_indexer_topk -> ds_rows_sparse_attn_direct",
            "ms_per_step": ms_two, "rows_per_s": inp.rows / (ms_two * 1e-3), "per_call_ms": per_call},
        "three_call_pipeline": {
            "calls": "ds_rows_indexer_score -> ds_rows_topk -> ds_rows_sparse_attn_direct",
            "ms_per_step": ms_three, "rows_per_s": inp.rows / (ms_three * 1e-3), "per_call_ms": per_call_three},
        "four_call_pipeline": {
            "calls": "ds_rows_indexer_score -> ds_rows_topk -> ds_rows_gather -> ds_rows_sparse_attn",
            "ms_per_step": ms_four, "rows_per_s": inp.rows / (ms_four * 1e-3), "per_call_ms": per_call_four},
        "wall_s_timed_region": wall,
        "roofline": {
            "kernel": "indexer_score_kernel<true> (indexer with the fused top-k candidate stage)",
            "kernel_ms": indexer_ms,
            "timing": "HIP events on the launch stream around back-to-back launches over the rotating input copies",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": (traffic["fetch"] + traffic["write"]) if traffic else None,
            "traffic_fetch_write": [traffic["fetch"], traffic["write"]] if traffic else None,
            "bytes_per_launch": idx_bytes,
            "mfma_tflops": idx_flops / idx_s / 1e12,
            "mfma_frac_of_bf16_peak": idx_flops / idx_s / 1e12 / BF16_PEAK_TFLOPS,
        },
    }
    out["multi_query_indexer"] = mq_bench(torch, max(args.steps, 50))
    out["compressor"] = {
        "call": "ds_rows_compressor (one decode token per row: state write, window pooling, RMS norm)",
        "timing": "HIP events around replays of a HIP graph holding 16 calls (16 state sets)",
        "shapes": compressor_bench(torch, max(args.steps, 50)),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
