"""Benchmark of the MLA paged-KV decode hot path on one MI355X.

One step = one pass of the whole path over one batch: build the block table
and plan the splits (one launch), run the split decode, merge the partial
states.  The
workload is the DeepSeek-V3-shaped decode batch: 64 requests, 128 heads,
q_len 1, KV lengths uniform in [1024, 8192], bf16 q and latent cache with
64-token pages scattered in a 2x-oversized pool (synthetic, seeded).

Printed: one JSON line with KV-read GB/s over the whole step (the headline
metric), tokens/s, the decode kernel's roofline position (bytes it must move
per launch / its average launch time, against the 8 TB/s HBM peak) and the
fp64 CPU oracle timed on the host on the same batch.  Beside it: the time of
decode + merge alone and its KV-read rate (the per-layer part of the step,
which a model repeats for every layer while the table and plan are built
once per step), and the time of the table-and-plan launch alone.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload dsv3]
                       [--no-cpu-baseline] [--pools P]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure (no sparsity)
EV_EVERY = 5     # timed steps per decode launch that records its own events
SETTLE_S = 0.3   # default seconds of untimed steps before the warm-up steps


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dsv3")
    ap.add_argument("--pools", type=int, default=3,
                    help="independent copies of the KV pool, rotated per step so that the "
                         "256 MB last-level cache cannot serve a step from the previous one")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed steps before the warm-up steps (clock settling)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured in a HIP graph (measured slower than "
                         "eager launches here: the four launches are not host-bound)")
    ap.add_argument("--cpu-runs", type=int, default=3)
    ap.add_argument("--plan", choices=("balanced", "fixed"), default="balanced",
                    help="balanced: one cost-balanced part per CU (default); fixed: the "
                         "deterministic fixed-tile plan (batch-invariant results)")
    ap.add_argument("--tile-pages", type=int, default=32,
                    help="pages per tile of the fixed plan (32 = 2048 tokens)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before warm-up, run one plain elementwise kernel (bitwise not) that "
                         "reads and writes this many MiB: the known-size reference for HBM "
                         "byte counters")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: turn two rocprofv3 --pmc counter_collection.csv files "
                         "(FETCH_SIZE, then WRITE_SIZE, of a run with --calib-copy-mib) into "
                         "HBM bytes per decode launch and store them under profiles/")
    return ap.parse_args()


def _algorithmic_bytes(w) -> dict:
    """Bytes the method must move for one pass (each latent row read once per
    request, q read once, o and lse written once, one int32 per page of the
    block table), independent of how the kernels split the work."""
    elem = 2 if w.kv_dtype == "bf16" else 1
    L = w.seq_lens.astype(np.int64)
    R = w.rows_per_req
    kv = int(L.sum()) * 576 * elem
    q = w.bs * R * 576 * 2
    o = w.bs * R * 512 * 2
    lse = w.bs * R * 4
    bt = int((-(-L // 64)).sum()) * 4
    return dict(kv=kv, q=q, o=o, lse=lse, bt=bt, total=kv + q + o + lse + bt)


def _algorithmic_flops(w) -> int:
    """Matrix work of one pass: 2 flop per multiply-add of the scores (576
    wide) and of the output (512 wide), per visible (row, key) pair; with
    causal masking row i of q_len n sees L - n + i + 1 keys."""
    L = w.seq_lens.astype(np.int64)
    n = w.q_len
    if w.causal:
        vis = sum(int(np.clip(L - n + i + 1, 0, None).sum()) for i in range(n))
    else:
        vis = int(L.sum()) * n
    return 2 * (576 + 512) * w.heads * vis


def measured_copy_gbs(torch, mib: int = 2048, reps: int = 10) -> float:
    """Copy bandwidth on this machine (bytes read + written per second) of a plain
    elementwise kernel (bitwise not of int32, 2 GiB in, 2 GiB out), the
    practical ceiling an HBM-streaming kernel is compared with.  (torch's
    copy_ goes through the runtime's copy path, which measured slower.)"""
    n = mib << 18
    src = torch.ones(n, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        torch.bitwise_not(src, out=dst)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.bitwise_not(src, out=dst)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return 2 * (mib << 20) / (ms * 1e-3) / 1e9


def _kernel_of(kv_dtype: str):
    """(source file under csrc/, kernel name) of the decode kernel that runs
    for a cache dtype."""
    if kv_dtype == "bf16":
        return "decode.hip", "mla_decode_kernel<false>"
    return "decode.hip", "mla_decode_kernel<true>"


def _kernel_src(root: str, workload: str) -> str:
    from workloads import CONFIGS
    return os.path.join(root, "paged_kv_mla_req_amd", "csrc",
                        _kernel_of(CONFIGS[workload]["kv_dtype"])[0])


def _traffic_path(root: str, workload: str) -> str:
    from workloads import CONFIGS
    tag = "bf16" if CONFIGS[workload]["kv_dtype"] == "bf16" else "fp8"
    return os.path.join(root, "profiles", f"mla_decode_{tag}_{workload}_traffic.json")


def _traffic(root: str, kernel_src: str, workload: str):
    """HBM bytes per decode launch from the committed counter summary, or None
    when that summary is missing or was taken on another version of the
    kernel source (sha256 recorded in the file)."""
    import hashlib
    path = _traffic_path(root, workload)
    try:
        with open(path) as f:
            rec = json.load(f)
        with open(kernel_src, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def traffic_from_counters(fetch_csv: str, write_csv: str, calib_mib: int, root: str,
                          workload: str) -> dict:
    """HBM bytes per decode launch from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by calib_mib MiB over what the same counter read
    for the calibration kernel (bitwise not over calib_mib MiB)."""
    import csv
    import hashlib

    def read(path, counter):
        dec, cal = [], []
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                v = float(r["Counter_Value"]) * 1024.0
                if "mla_decode" in r["Kernel_Name"] and "kernel" in r["Kernel_Name"]:
                    dec.append(v)
                elif "bitwise_not" in r["Kernel_Name"].lower():
                    cal.append(v)
        if not dec or not cal:
            raise SystemExit(f"{path}: no decode or calibration dispatches for {counter}")
        factor = calib_mib * 2.0**20 / max(cal)
        return float(np.mean(dec)) * factor, factor, float(np.mean(dec))

    fetch, f_fac, f_raw = read(fetch_csv, "FETCH_SIZE")
    write, w_fac, w_raw = read(write_csv, "WRITE_SIZE")
    src = _kernel_src(root, workload)
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    return {"hbm_bytes_per_launch": round(fetch + write), "fetch_bytes": round(fetch),
            "write_bytes": round(write), "fetch_raw_bytes": round(f_raw),
            "write_raw_bytes": round(w_raw), "fetch_scale": round(f_fac, 4),
            "write_scale": round(w_fac, 4), "calibration_mib": calib_mib,
            "kernel_source_sha256": sha}


def cpu_baseline(w, runs: int) -> dict:
    """The fp64 oracle (as it stands) on the same batch, all rows, on the host."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()
                       if d.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = os.cpu_count() or 1
    args = (w.q_bits, w.kv, w.kv_dtype, w.kv_descale, w.req_to_token, w.req_pool_indices,
            w.seq_lens, w.softmax_scale, w.causal)
    oracle.paged_decode(*args)  # warm-up
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        oracle.paged_decode(*args)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times))
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": round(w.kv_bytes_read / t / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"whole batch ({w.bs} requests, all {w.rows_per_req} rows each), fp64 numpy, "
                      f"median of {runs} runs after 1 warm-up: {t:.3f} s per pass; "
                      f"host {model or 'unknown CPU'}, os.cpu_count()={os.cpu_count()}",
            "seconds_per_pass": round(t, 4)}


def time_append(mla, torch, w, p, reps: int) -> dict:
    """mla_set_kv_buffer timed with events around `reps` back-to-back launches
    (one at a time, kernel-sized work): the step's new tokens (the last q_len
    of each request) and a 32768-token chunk at random distinct pool slots.
    Bytes per token: the 1152-byte bf16 row read, its 8-byte slot, and the
    1152 (bf16) or 576 (e4m3) bytes written."""
    rng = np.random.default_rng(4242)
    slots_step = np.array([w.req_to_token[int(w.req_pool_indices[b]), int(w.seq_lens[b]) - w.q_len + i]
                           for b in range(w.bs) for i in range(w.q_len)], dtype=np.int64)
    pool_slots = p.kv.shape[0] * 64
    chunk = min(32768, pool_slots)
    slots_chunk = rng.permutation(pool_slots)[:chunk].astype(np.int64)
    res = {}
    scale = None if w.kv_dtype == "bf16" else torch.tensor([1.0 / 64], dtype=torch.float32,
                                                            device="cuda")
    for name, sl in (("step", slots_step), ("chunk", slots_chunk)):
        n = sl.size
        k = torch.randn((n, 576), device="cuda").to(torch.bfloat16)
        loc = torch.from_numpy(sl).cuda()
        for _ in range(3):
            mla.set_kv_buffer(p.kv, loc, k, kv_dtype=w.kv_dtype, kv_scale=scale)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            mla.set_kv_buffer(p.kv, loc, k, kv_dtype=w.kv_dtype, kv_scale=scale)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        per_tok = 1152 + 8 + (1152 if w.kv_dtype == "bf16" else 576)
        res[name] = {"tokens": int(n), "us": round(ms * 1e3, 3),
                     "gbs": round(n * per_tok / (ms * 1e-3) / 1e9, 2)}
    return res


def main() -> int:
    a = _args()
    if a.traffic_from:
        root = os.path.dirname(os.path.abspath(__file__))
        rec = traffic_from_counters(a.traffic_from[0], a.traffic_from[1],
                                    a.calib_copy_mib or 256, root, a.workload)
        rec["workload"] = a.workload
        path = _traffic_path(root, a.workload)
        with open(path, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec))
        return 0
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {a.gpus}); the multi-GPU decode "
              "context-parallel exchange is not part of this build", file=sys.stderr)
        return 2
    import torch

    import paged_kv_mla_req_amd as mla
    from workloads import make_workload
    from workloads.device import to_device

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    print(f"[bench] generating workload {a.workload}", file=sys.stderr, flush=True)
    w = make_workload(a.workload)
    pools = [to_device(w)]
    for i in range(1, a.pools):
        pools.append(to_device(w))  # same bits, different HBM addresses
    d = pools[0]
    R = w.rows_per_req
    width = w.bt_width
    cus = mla.device_num_cus()
    max_len = int(w.seq_lens.max())
    num_parts = cus
    if a.plan == "fixed":
        num_parts = max(1, int(mla._lib.lib().mla_fixed_split_parts_bound(w.bs, max_len,
                                                                         a.tile_pages)))
    bt = torch.empty((w.bs, width), dtype=torch.int32, device="cuda")
    tile_plan = torch.empty((num_parts, 8), dtype=torch.int32, device="cuda")
    split_indptr = torch.empty((w.bs + 1,), dtype=torch.int32, device="cuda")
    po, pl = mla.partial_buffers(w.bs, R, num_parts)
    out = torch.empty((w.bs, w.q_len, w.heads, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.bs, w.q_len, w.heads), dtype=torch.float32, device="cuda")
    # For every EV_EVERY-th timed step, a pair of events that the decode
    # kernel's own launch records at its begin and end
    # (mla_decode_time_next_launch).  An event-recorded launch ends with a
    # release to system scope (an L2 write-back), which costs that step a few
    # microseconds, so only a sample of the timed launches records them.  They
    # are created, and recorded once so that they exist, before timing starts.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range((a.steps + EV_EVERY - 1) // EV_EVERY)]
    for e0, e1 in ev:
        e0.record()
        e1.record()

    def decode(p):
        mla.mla_decode(p.q, p.kv, bt, p.seq_lens, tile_plan, split_indptr, w.softmax_scale,
                       partial_o=po, partial_lse=pl, out=out, lse=lse, kv_dtype=w.kv_dtype,
                       kv_descale=p.kv_descale, causal=w.causal)

    def table_and_plan(p):
        if a.plan == "fixed":
            mla.build_block_table(p.req_to_token, p.req_pool_indices, p.seq_lens, width,
                                  max_seq_len_hint=max_len, out=bt)
            mla.plan_fixed_splits(p.seq_lens, a.tile_pages, num_parts, max_seq_len_hint=max_len,
                                  tile_plan=tile_plan, split_indptr=split_indptr)
            return
        mla.build_table_and_plan(p.req_to_token, p.req_pool_indices, p.seq_lens, width, R,
                                 num_parts, w.kv_dtype, max_seq_len_hint=max_len, out=bt,
                                 tile_plan=tile_plan, split_indptr=split_indptr)

    def step(i: int, timed: int):
        # one pass of the hot path: block table + plan (one launch), split
        # decode, merge
        p = pools[i % len(pools)]
        table_and_plan(p)
        if timed >= 0 and timed % EV_EVERY == 0:
            mla.time_next_decode(*ev[timed // EV_EVERY])
        decode(p)
        mla.merge_states(po, pl, split_indptr, out, lse)

    def timed_loop(fn, n: int) -> float:
        """ms per call of fn(i) over n back-to-back calls."""
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3 / n

    if a.calib_copy_mib > 0:
        n = a.calib_copy_mib << 18  # int32 elements
        src = torch.ones(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.bitwise_not(src, out=dst)  # reads and writes calib_copy_mib MiB
        torch.cuda.synchronize()
        del src, dst
    # The card raises its clocks over the first ~0.1 s of sustained load: steps
    # run untimed for SETTLE_S seconds first, then the W warm-up steps.
    t_settle = time.perf_counter()
    n_settle = 0
    while time.perf_counter() - t_settle < a.settle:
        step(n_settle, -1)
        n_settle += 1
        if n_settle % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    print(f"[bench] clock settling: {n_settle} untimed steps; warmup {a.warmup} steps",
          file=sys.stderr, flush=True)
    for i in range(a.warmup):
        step(i, -1)
    torch.cuda.synchronize()
    graphs = []
    if a.graph:
        # One captured step per KV pool: the three kernels of the step replay
        # without host launch work between them.
        for j in range(len(pools)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(j, -1)
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()

    print(f"[bench] timing {a.steps} steps ({'graph replays' if a.graph else 'eager'})",
          file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(a.steps):
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            step(a.warmup + i, i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / a.steps
    ms_step_eager = None
    if graphs:
        # The decode kernel's own duration comes from eager steps (the launch
        # records the events itself, which a graph replay cannot do).
        t1 = time.perf_counter()
        for i in range(a.steps):
            step(a.warmup + i, i)
        torch.cuda.synchronize()
        ms_step_eager = (time.perf_counter() - t1) * 1e3 / a.steps
    # the decode kernel's average launch duration over the event-timed steps
    dec_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    # The step's parts on their own (the table and plan run once per batch
    # step, decode and merge once per attention layer): same inputs, timed
    # back to back after the main loop.
    ms_dm = timed_loop(lambda i: (decode(pools[i % len(pools)]),
                                  mla.merge_states(po, pl, split_indptr, out, lse)), a.steps)
    ms_tp = timed_loop(lambda i: table_and_plan(pools[i % len(pools)]), a.steps)
    # The KV append that precedes attention (set_kv_buffer): the step's new
    # tokens, then a 32768-token chunk.  It writes into pool 0, so it runs last.
    append = time_append(mla, torch, w, pools[0], a.steps)
    # (skipped in counter runs: their calibration kernel is the only bitwise not)
    copy_gbs = measured_copy_gbs(torch) if a.calib_copy_mib == 0 else None

    b = _algorithmic_bytes(w)
    kv_gbs = b["kv"] / (ms_step * 1e-3) / 1e9
    tokens_s = w.bs * w.q_len / (ms_step * 1e-3)
    achieved = b["total"] / (dec_ms * 1e-3) / 1e9
    flops = _algorithmic_flops(w)
    tflops = flops / (dec_ms * 1e-3) / 1e12
    line = {
        "metric": "MLA decode KV-read GB/s (% of HBM peak; tokens/s) at B=64, 128 heads, "
                  "4k-average context",
        "value": round(kv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.kv_dtype == "bf16" else "fp8_e4m3 kv, bf16 q",
        "data": "synthetic (seeded N(0,1) q and latent cache, scattered 64-token pages)",
        "config": {
            "workload": f"{w.name}: batch {w.bs}, {w.heads} heads, q_len {w.q_len}, "
                        f"KV lengths {int(w.seq_lens.min())}..{int(w.seq_lens.max())} "
                        f"(mean {float(w.seq_lens.mean()):.0f}), latent 576 / value 512, "
                        f"page 64, {w.kv_dtype} cache",
            "global_batch": w.bs,
            "seq_len": int(round(float(w.seq_lens.mean()))),
            "parallelism": "single GPU",
            "num_parts": num_parts,
            "plan": a.plan if a.plan == "balanced" else f"fixed tiles of {a.tile_pages} pages",
            "kv_pools_rotated": len(pools),
        },
        "pct_hbm_peak": round(100.0 * kv_gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(tokens_s, 1),
        "decode_kernel_ms": round(dec_ms, 5),
        "ms_decode_merge": round(ms_dm, 5),
        "kv_read_gbs_decode_merge": round(b["kv"] / (ms_dm * 1e-3) / 1e9, 2),
        "ms_table_and_plan": round(ms_tp, 5),
        "measured_copy_gbs": None if copy_gbs is None else round(copy_gbs, 1),
        "decode_pct_of_measured_copy": None if copy_gbs is None else round(
            100.0 * achieved / copy_gbs, 2),
        "mfma": {"algorithmic_tflop": round(flops / 1e12, 4),
                 "achieved_tflops": round(tflops, 2), "peak_tflops": MFMA_PEAK_TFLOPS,
                 "frac": round(tflops / MFMA_PEAK_TFLOPS, 4),
                 "note": "dense bf16 MFMA peak (the fp8 cache is converted to bf16 in LDS)"},
        "append": append,
        "step_launch": "hip graph replay" if a.graph else "eager",
        "ms_per_step_eager": None if ms_step_eager is None else round(ms_step_eager, 5),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": _traffic(os.path.dirname(os.path.abspath(__file__)),
                                _kernel_src(os.path.dirname(os.path.abspath(__file__)),
                                            a.workload),
                                a.workload),
            "kernel": _kernel_of(w.kv_dtype)[1],
            "bytes_per_launch": b["total"],
        },
    }
    if not a.no_cpu_baseline:
        print("[bench] timing the fp64 CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, a.cpu_runs)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
