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
64 heads x 512 attention), seeded synthetic inputs resident in HBM. The other
four workloads (1 x 1024, 8 ragged rows of 600..8192 keys, 8 rows of 1 ..
131072 keys with ternary indexer entries, 1 x 1048576) are timed through the
same one-call entry point and reported under `configs`.

Cache policy: `--copies` independent device copies of the inputs are used in
rotation (default 8 x ~330 MB for the headline), so each step's 64 MiB of
indexer keys was last touched 7 steps earlier, after ~2.3 GB of other
traffic: the keys come from HBM, not from the 256 MB last-level cache.
`--copies 1` measures the warm-cache case.

Prints one JSON line (rank 0, N=1) with the headline value, its per-step
median and spread, per-call durations from HIP events on the launch stream,
the roofline of the dominant kernel (the fused indexer) timed as it runs
inside the step, the attention side's HBM rate, every workload's step time,
and the CPU oracle timed on a bounded sample.
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

METRIC = "decode rows/s (indexer+top-k+sparse attn), 8 rows×32k KV; % MFMA/HBM peak"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
# ds_rows_indexer_topk keeps the first selection stage in the indexer only
# when every row has at least this many visible keys (the library's rule;
# below it the call runs the plain score kernel). With start_pos = 4 kv_len - 1
# every key is visible.
FUSED_MIN_VISIBLE = 16384


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", type=int, default=2)
    p.add_argument("--copies", type=int, default=8)
    p.add_argument("--cpu-seconds", type=float, default=8.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-configs", action="store_true", help="skip the other workloads' step times")
    p.add_argument("--leg", choices=("all", "multi_query", "compressor", "fallback", "stream"), default="all",
                   help="run one leg alone and print its JSON object: the multi-query indexer, the compressor, "
                        "the one-call step on scores that defeat the fused candidates, or plain streaming "
                        "copies of 64 MiB .. 1 GiB (the achievable HBM rate on this GPU)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 64 MiB device-to-device copy 5 times (reference for the "
                        "FETCH_SIZE / WRITE_SIZE counter scale) and exit")
    return p.parse_args()


CSRC = os.path.join(ROOT, "sparse_attention_decode_04_amd", "csrc")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "traffic_8x32768.md")
# Source files of each kernel group whose counter bytes the bench reports;
# the committed counter figures are used only while these hash as recorded.
KERNEL_SOURCES = {
    "indexer": ["indexer_score.hip", "device_common.hpp", "select_common.hpp", "ds_rows_internal.hpp#indexer"],
    "attention": ["topk_attn.hip", "attention.hip", "attn_chunk.hpp", "topk_select.hpp", "select_common.hpp",
                  "device_common.hpp", "ds_rows_internal.hpp"],
}


def source_hash(group):
    """SHA-256 of a kernel group's sources (a `#indexer` suffix takes only the
    indexer section of the internal header)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[group]:
        fname, _, section = name.partition("#")
        with open(os.path.join(CSRC, fname), "rb") as fh:
            text = fh.read()
        if section:
            start = text.index(b"// ---------------------------------------------------------------- " +
                               section.encode())
            end = text.index(b"// ----", start + 10)
            text = text[start:end]
        h.update(text)
    return h.hexdigest()


def profile_fields(path):
    """`- `key`: value` lines of a committed profile summary."""
    fields = {}
    try:
        with open(path) as fh:
            for line in fh:
                if line.startswith("- `") and "`: " in line:
                    k, v = line[3:].split("`: ", 1)
                    fields[k] = v.strip()
    except OSError:
        pass
    return fields


def measured_traffic(group):
    """HBM bytes per launch (fetch, write) of a kernel group from the committed
    counter summary, or None when there is none or its sources changed since."""
    f = profile_fields(TRAFFIC_PROFILE)
    try:
        if f.get(f"{group}_source_sha256") != source_hash(group):
            return None
        return float(f[f"{group}_fetch_bytes_per_launch"]), float(f[f"{group}_write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def fused_route(kv_len):
    return min(kv_len) >= FUSED_MIN_VISIBLE


def fused_wave_cand(kv_len):
    """Candidates per wave of the fused stage: 8 when every row has at least
    262144 visible keys, else 32 (the library's rule; the workloads' rows see
    all of their keys)."""
    return 8 if min(kv_len) >= 262144 else 32


def indexer_kernel_name(kv_len):
    """The indexer kernel a one-call step on rows of these lengths launches
    (the library's rules: fused stage and its budget; for the plain kernel,
    its block size and whether its grid is the compact one)."""
    if fused_route(kv_len):
        return "indexer_score_kernel<%d, false>" % fused_wave_cand(kv_len)
    block = 1024
    while block > 64 and sum(-(-n // block) for n in kv_len) < 256:
        block //= 2
    blocks = sum(-(-n // block) for n in kv_len)
    compact = -(-max(kv_len) // block) * len(kv_len) > 2 * blocks
    return "indexer_score_kernel<0, %s>" % ("true" if compact else "false")


def indexer_bytes_flops(kv_len, fused):
    """Algorithmic HBM bytes and MFMA flops of one indexer launch: per key
    256 B of keys read + 4 B of score written and 64*128*2 flops; per row
    16 KiB of query and 256 B of weights read; in the fused form also, per
    1024-key block, 4 C candidate keys of 8 B (C per wave) and four 8 B floors
    written."""
    keys = sum(kv_len)
    b = keys * (256 + 4) + len(kv_len) * (64 * 128 * 2 + 64 * 4)
    if fused:
        b += sum(-(-n // 1024) for n in kv_len) * (4 * fused_wave_cand(kv_len) * 8 + 4 * 8)
    return b, keys * 64 * 128 * 2


def attention_bytes_flops(kv_len):
    """Algorithmic bytes and flops of the attention over the selected rows,
    read through the indices: per row the query (64 x 512 bf16), width KV rows
    of 1 KiB plus their 4-byte indices, the f32 output (64 x 512); the sinks
    once. Flops: two 64 x 512 x width contractions."""
    w = [min(n, 512) for n in kv_len]
    b = sum(64 * 512 * 2 + wi * (1024 + 4) + 64 * 512 * 4 for wi in w) + 64 * 4
    return b, sum(2 * 2 * 64 * 512 * wi for wi in w)


def gather_bytes(kv_len):
    """Algorithmic bytes of ds_rows_gather: per selected slot the 4-byte index
    and the 1 KiB KV row read, the 1 KiB gathered row and 2-byte mask entry
    written; per row its 4-byte invalid flag."""
    w = [min(n, 512) for n in kv_len]
    return sum(wi * (4 + 1024 + 1024 + 2) + 4 for wi in w)


def step_bytes(kv_len):
    """Algorithmic bytes of one step: the indexer (fused form when taken), the
    selection's reads (candidates or scores) and index writes, and the
    attention reading its selected KV rows through the indices."""
    fused = fused_route(kv_len)
    blocks = sum(-(-n // 1024) for n in kv_len)
    idx_b, _ = indexer_bytes_flops(kv_len, fused)
    sel_b = (blocks * (4 * fused_wave_cand(kv_len) * 8 + 4 * 8) if fused else 4 * sum(kv_len)) + len(kv_len) * 512 * 4
    attn_b, _ = attention_bytes_flops(kv_len)
    return idx_b + sel_b + attn_b


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
    # Untimed calls first: the chip's clocks take a few hundred microseconds
    # of back-to-back matrix work to settle.
    for i in range(2 * n_calls):
        devs[i % copies].run()
    torch.cuda.synchronize()
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
            "timing": f"HIP events around {n_calls} back-to-back calls over {copies} rotating key copies, after {2 * n_calls} untimed ones",
            "ms_per_call": ms, "keys_per_s": sum(inp.kv_len) / (ms * 1e-3),
            "mfma_tflops": tflops, "mfma_frac_of_bf16_peak": tflops / BF16_PEAK_TFLOPS,
            "achieved_gb_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "bytes_per_call": nbytes, "flops_per_call": flops}


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(headline_inp, seconds, config_inputs):
    """The CPU oracle (numpy float64/int64) on the host cores: the headline
    workload for `seconds` with every BLAS thread and for half as long with
    one thread, then one or more steps of every other workload."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import ds_oracle as O

    def run(inp, secs, threads):
        with threadpool_limits(limits=threads):
            steps = 0
            t0 = time.perf_counter()
            while True:
                O.decode_rows(inp)
                steps += 1
                el = time.perf_counter() - t0
                if el >= secs:
                    break
        return steps, el

    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    steps, el = run(headline_inp, seconds, None)
    steps1, el1 = run(headline_inp, seconds / 2, 1)
    R, keys = headline_inp.rows, sum(headline_inp.kv_len)
    out = {"value": steps * R / el, "unit": "rows/s", "cores": threads, "kind": "oracle",
           "sample": f"{steps} full oracle steps of the headline workload ({steps * R} rows) in {el:.1f} s; "
                     f"numpy float64/int64, BLAS threads={threads}, host cpu_count={os.cpu_count()}",
           "keys_per_s": steps * keys / el, "cpu_model": cpu_model(),
           "single_thread": {"rows_per_s": steps1 * R / el1, "keys_per_s": steps1 * keys / el1, "cores": 1,
                             "sample": f"{steps1} steps in {el1:.1f} s"},
           "configs": {}}
    for cid, inp in config_inputs.items():
        n, e = run(inp, 1.0, None)
        out["configs"][str(cid)] = {"rows_per_s": n * inp.rows / e, "keys_per_s": n * sum(inp.kv_len) / e,
                                    "steps": n, "seconds": e}
    return out


def stream_bench(torch):
    """Plain device-to-device copies (torch copy_, the HIP runtime's blit
    kernel) of 64 MiB, 256 MiB and 1 GiB over rotating buffers: the HBM rate
    a simple streaming kernel reaches on this GPU (read + write bytes), the
    practical ceiling next to the 8 TB/s specification."""
    stream = torch.cuda.current_stream()
    res = {}
    for mib in (64, 256, 1024):
        n = mib << 20
        copies = max(2, (2048 // mib))
        src = [torch.ones(n // 4, dtype=torch.float32, device="cuda") for _ in range(copies)]
        dst = [torch.empty_like(x) for x in src]
        for i in range(copies):
            dst[i].copy_(src[i])
        torch.cuda.synchronize()
        reps = 20
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for i in range(reps):
            dst[i % copies].copy_(src[i % copies])
        ev[1].record(stream)
        torch.cuda.synchronize()
        copy_ms = ev[0].elapsed_time(ev[1]) / reps
        res[f"{mib}MiB"] = {"copy_us": copy_ms * 1e3, "copy_gb_s": 2 * n / (copy_ms * 1e-3) / 1e9,
                            "rotating_buffers": copies}
        del src, dst
        torch.cuda.empty_cache()
    return {"timing": "HIP events around 20 back-to-back copies over rotating buffers (2 GiB in total per size)",
            "copy": "torch copy_ (read + write counted)", "sizes": res}


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
    stream = torch.cuda.current_stream()

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
    if args.leg == "stream":
        print(json.dumps(stream_bench(torch)), flush=True)
        return

    def device_copies(inp, n):
        base = DeviceInputs(inp)
        out = [base] + [base.clone() for _ in range(n - 1)]
        return [DeviceRows(c) for c in out]

    def timed(runs, name, steps, warmup):
        """`steps` whole steps bracketed by device synchronisation and one HIP
        event pair: mean ms per step and the wall time of the timed region."""
        for i in range(warmup):
            getattr(runs[i % len(runs)], name)()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(steps):
            getattr(runs[i % len(runs)], name)()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps, time.perf_counter() - t0

    def per_step_us(runs, name, steps):
        """Each of `steps` steps between consecutive HIP events: median and
        spread in microseconds."""
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        evs[0].record(stream)
        for i in range(steps):
            getattr(runs[i % len(runs)], name)()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        d = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(steps)])
        return {"median": float(np.median(d)), "p10": float(np.percentile(d, 10)),
                "p90": float(np.percentile(d, 90)), "min": float(d.min()), "max": float(d.max()),
                "steps": steps}

    def in_step_ms(runs, extra_runs, first_kernel_call, n):
        """Duration of the step's first kernel (the indexer) as it runs inside
        the step: the time of n one-call steps each followed by one more
        launch of that kernel alone, minus the time of n one-call steps, over
        n. Each extra launch starts after a step's attention kernels and is
        followed by the next step's indexer, as in the timed loop; it reads
        input copies of its own (extra_runs, rotating), so that it warms no
        cache for the steps. Both regions are single HIP event pairs on the
        launch stream (a pair around one launch would add the event's own
        dispatch latency)."""
        def region(extra):
            for i in range(len(runs)):
                runs[i].step_one()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(n):
                runs[i % len(runs)].step_one()
                if extra:
                    getattr(extra_runs[i % len(extra_runs)], first_kernel_call)()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1)
        with_extra = region(True)
        without = region(False)
        with_extra2 = region(True)
        return ((with_extra + with_extra2) / 2 - without) / n

    def stamped_ms(runs, call, n):
        """Execution span of the indexer kernel inside `call`, from the
        wall-clock stamps its workgroups write when armed by
        ds_rows_time_next_indexer: smallest workgroup start to largest wave
        end, for each of n calls over the rotating input copies. Each call
        writes to a zeroed buffer of its own, so nothing but the calls runs in
        the loop (the armed launch is an ordinary one plus a few stores per
        workgroup). Mean and median span in ms, and the loop's mean call time."""
        inp_ = runs[0].dev.inp
        per = -(-max(inp_.kv_len) // 64) * inp_.rows * ds.TIMER_STAMPS_PER_WG   # fits any block size
        buf = torch.zeros(n * per, dtype=torch.int64, device="cuda")
        views = [buf[i * per:(i + 1) * per] for i in range(n)]
        khz = ds.wall_clock_khz()
        for i in range(len(runs)):
            getattr(runs[i], call)()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            ds.time_next_indexer(views[i])
            getattr(runs[i % len(runs)], call)()
        e1.record(stream)
        torch.cuda.synchronize()
        host = buf.cpu().numpy().reshape(n, -1)
        d = np.array([ds.indexer_span_ticks(host[i]) for i in range(n)]) / khz   # ms
        return float(d.mean()), float(np.median(d)), e0.elapsed_time(e1) / n

    def back_to_back_ms(runs, call, n):
        """Mean duration of one `call` from HIP events on the launch stream
        around n back-to-back launches over the rotating input copies."""
        for r in runs:
            getattr(r, call)()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        ev0.record(stream)
        for i in range(n):
            getattr(runs[i % len(runs)], call)()
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / n

    def per_call_ms(runs, calls, steps):
        """Mean duration of each call, from HIP events recorded around it on
        the launch stream, over `steps` steps."""
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
        for i in range(steps):
            r = runs[i % len(runs)]
            for k, c in enumerate(calls):
                evs[i][k].record(stream)
                getattr(r, c)()
            evs[i][len(calls)].record(stream)
        torch.cuda.synchronize()
        return {c: float(np.mean([evs[i][k].elapsed_time(evs[i][k + 1]) for i in range(steps)]))
                for k, c in enumerate(calls)}

    if args.leg == "fallback":
        res = {"shape": "8 rows x 32768 keys", "timing": "HIP events around back-to-back one-call steps over "
               f"{args.copies} rotating copies (mean), and per-step events (median)", "kinds": {}}
        base = I.make_config(2)
        runs = device_copies(base, args.copies)
        ms, _ = timed(runs, "step_one", args.steps, args.warmup)
        res["kinds"]["random (headline inputs)"] = {"us_per_step": ms * 1e3,
                                                    "median_us": per_step_us(runs, "step_one", args.steps)["median"]}
        del runs
        for kind in I.FALLBACK_KINDS:
            inp = I.fallback_workload(kind)
            runs = device_copies(inp, args.copies)
            ms, _ = timed(runs, "step_one", args.steps, args.warmup)
            res["kinds"][kind] = {"us_per_step": ms * 1e3,
                                  "median_us": per_step_us(runs, "step_one", args.steps)["median"]}
            del runs
            torch.cuda.empty_cache()
        print(json.dumps(res), flush=True)
        return

    inp = I.make_config(args.config)
    runs = device_copies(inp, args.copies)
    kv_len = inp.kv_len
    fused = fused_route(kv_len)
    first_call = "indexer_candidates" if fused else "indexer_score"

    # Headline: the one-call decode core.
    ms_per_step, wall = timed(runs, "step_one", args.steps, args.warmup)
    step_spread = per_step_us(runs, "step_one", args.steps)
    # Score + top-k in one call, then attention with the gather fused in.
    ms_two, _ = timed(runs, "step_fused", args.steps, args.warmup)
    # Separate score and top-k calls, then the same attention.
    ms_three, _ = timed(runs, "step_direct", args.steps, args.warmup)
    # The four-call path (gather, then attention on the gathered rows).
    ms_four, _ = timed(runs, "step", args.steps, args.warmup)

    n_idx = max(args.steps, 200)
    # The indexer inside the one-call step: its execution span from the
    # workgroups' wall-clock stamps (the roofline figure), and by difference of
    # plain loops (marginal).
    idx_in_mean, idx_in_median, armed_step_ms = stamped_ms(runs, "step_one", n_idx)
    extra_runs = device_copies(inp, args.copies)
    idx_marginal = in_step_ms(runs, extra_runs, first_call, n_idx)
    del extra_runs
    idx_b2b = back_to_back_ms(runs, first_call, n_idx)
    idx_b2b_span, _, _ = stamped_ms(runs, first_call, n_idx)
    per_call = per_call_ms(runs, ("indexer_topk", "sparse_attn_direct"), args.steps)
    per_call_three = per_call_ms(runs, ("indexer_score", "topk", "sparse_attn_direct"), args.steps)
    per_call_four = per_call_ms(runs, ("indexer_score", "topk", "gather", "sparse_attn"), args.steps)

    idx_bytes, idx_flops = indexer_bytes_flops(kv_len, fused)
    idx_traffic = measured_traffic("indexer") if args.config == 2 else None
    achieved = idx_bytes / (idx_in_mean * 1e-3) / 1e9
    rows_per_s = inp.rows / (ms_per_step * 1e-3)
    keys_per_s = sum(kv_len) / (ms_per_step * 1e-3)

    # The attention side of the one-call step: everything after the indexer
    # (final top-k level inside the attention workgroups, attention, combine,
    # and the kernel boundaries between them), and the separate direct
    # attention call (phase 1 + combine) by its own events.
    attn_b, attn_f = attention_bytes_flops(kv_len)
    rest_ms = ms_per_step - idx_marginal
    attn_traffic = measured_traffic("attention") if args.config == 2 else None
    attn_direct_ms = per_call["sparse_attn_direct"]

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
            "rows": inp.rows, "kv_len": kv_len if len(set(kv_len)) > 1 else kv_len[0],
            "top_k": 512, "cache": f"{args.copies} rotating input copies" if args.copies > 1 else "warm",
        },
        "keys_per_s": keys_per_s,
        "step_us": step_spread,
        "step_algorithmic_gb_per_s": step_bytes(kv_len) / (ms_per_step * 1e-3) / 1e9,
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
            "kernel": (indexer_kernel_name(kv_len) + (" (indexer with the fused top-k candidate stage)" if fused
                                                       else " (score kernel)")),
            "kernel_ms": idx_in_mean,
            "kernel_ms_median": idx_in_median,
            "timing": "in step: mean over n = %d one-call steps on the rotating copies of the indexer's execution "
                      "span, smallest workgroup start to largest wave end, from the wall-clock stamps its "
                      "workgroups write (ds_rows_time_next_indexer)" % n_idx,
            "stamped_loop_step_ms": armed_step_ms,
            "marginal_ms": idx_marginal,
            "marginal_timing": "(n one-call steps each followed by one more launch of the indexer alone, on input copies "
                               "of its own) minus (n one-call steps), HIP events on the launch stream; the extra "
                               "launch also puts the next step's indexer behind an indexer, so this measures about "
                               "the back-to-back duration",
            "marginal_frac": idx_bytes / (idx_marginal * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": (idx_traffic[0] + idx_traffic[1]) if idx_traffic else None,
            "traffic_fetch_write": list(idx_traffic) if idx_traffic else None,
            "bytes_per_launch": idx_bytes,
            "back_to_back_ms": idx_b2b,
            "back_to_back_frac": idx_bytes / (idx_b2b * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "back_to_back_span_ms": idx_b2b_span,
            "mfma_tflops": idx_flops / (idx_in_mean * 1e-3) / 1e12,
            "mfma_frac_of_bf16_peak": idx_flops / (idx_in_mean * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
        },
        "attention": {
            "what": "final top-k level + attention (gather fused) + combine of the one-call step",
            "algorithmic_bytes": attn_b,
            "flops": attn_f,
            "in_step_us": rest_ms * 1e3,
            "in_step_timing": "one-call step mean minus the indexer's marginal in-step time (unarmed loops; includes "
                              "the kernel boundaries)",
            "achieved_gb_s": attn_b / (rest_ms * 1e-3) / 1e9,
            "hbm_frac": attn_b / (rest_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "direct_call_us": attn_direct_ms * 1e3,
            "direct_call_gb_s": attn_b / (attn_direct_ms * 1e-3) / 1e9,
            "direct_call_hbm_frac": attn_b / (attn_direct_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": (attn_traffic[0] + attn_traffic[1]) if attn_traffic else None,
            "traffic_fetch_write": list(attn_traffic) if attn_traffic else None,
            "traffic_over_algorithmic": ((attn_traffic[0] + attn_traffic[1]) / attn_b) if attn_traffic else None,
        },
        "gather": {
            "call": "ds_rows_gather (the four-call pipeline's third call)",
            "algorithmic_bytes": gather_bytes(kv_len),
            "us": per_call_four["gather"] * 1e3,
            "timing": "HIP events around the call inside the four-call steps (its flag-clearing kernel included)",
            "achieved_gb_s": gather_bytes(kv_len) / (per_call_four["gather"] * 1e-3) / 1e9,
            "hbm_frac": gather_bytes(kv_len) / (per_call_four["gather"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
        },
    }
    del runs
    torch.cuda.empty_cache()

    config_inputs = {}
    if not args.no_configs:
        out["configs"] = {}
        for cid in range(5):
            if cid == args.config:
                continue
            cinp = I.make_config(cid)
            config_inputs[cid] = cinp
            nbytes = sum(cinp.kv_len) * 1280 + cinp.rows * 96 * 1024
            ncopies = int(max(2, min(args.copies, (2 << 30) // nbytes)))
            cruns = device_copies(cinp, ncopies)
            steps = args.steps if cid != 4 else max(20, args.steps // 4)
            cms, _ = timed(cruns, "step_one", steps, args.warmup)
            spread = per_step_us(cruns, "step_one", steps)
            cfused = fused_route(cinp.kv_len)
            cfirst = "indexer_candidates" if cfused else "indexer_score"
            c_in, _, _ = stamped_ms(cruns, "step_one", max(steps, 20))
            cb, _ = indexer_bytes_flops(cinp.kv_len, cfused)
            out["configs"][str(cid)] = {
                "workload": I.CONFIG_NAMES[cid], "rows": cinp.rows, "keys": sum(cinp.kv_len),
                "us_per_step": cms * 1e3, "step_us_median": spread["median"], "step_us_p10": spread["p10"],
                "step_us_p90": spread["p90"], "rows_per_s": cinp.rows / (cms * 1e-3),
                "keys_per_s": sum(cinp.kv_len) / (cms * 1e-3),
                "step_algorithmic_gb_per_s": step_bytes(cinp.kv_len) / (cms * 1e-3) / 1e9,
                "dominant_kernel": indexer_kernel_name(cinp.kv_len),
                "dominant_kernel_in_step_us": c_in * 1e3,
                "dominant_kernel_hbm_frac": cb / (c_in * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "copies": ncopies, "steps": steps}
            del cruns
            torch.cuda.empty_cache()
        out["configs"][str(args.config)] = {
            "workload": I.CONFIG_NAMES[args.config], "rows": inp.rows, "keys": sum(kv_len),
            "us_per_step": ms_per_step * 1e3, "step_us_median": step_spread["median"],
            "step_us_p10": step_spread["p10"], "step_us_p90": step_spread["p90"], "rows_per_s": rows_per_s,
            "keys_per_s": keys_per_s, "step_algorithmic_gb_per_s": out["step_algorithmic_gb_per_s"],
            "dominant_kernel": indexer_kernel_name(kv_len),
            "dominant_kernel_in_step_us": idx_in_mean * 1e3, "dominant_kernel_hbm_frac": achieved / HBM_PEAK_GBS,
            "copies": args.copies, "steps": args.steps}
        out["configs"] = dict(sorted(out["configs"].items()))

    out["multi_query_indexer"] = mq_bench(torch, max(args.steps, 50))
    out["compressor"] = {
        "call": "ds_rows_compressor (one decode token per row: state write, window pooling, RMS norm)",
        "timing": "HIP events around replays of a HIP graph holding 16 calls (16 state sets)",
        "shapes": compressor_bench(torch, max(args.steps, 50)),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds, config_inputs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
