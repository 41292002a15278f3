"""Benchmark of the MLA paged-KV decode hot path on one MI355X.

One step = one pass of the whole path over one batch: build the block table,
plan the splits, run the split decode, merge the partial states.  The
workload is the DeepSeek-V3-shaped decode batch: 64 requests, 128 heads,
q_len 1, KV lengths uniform in [1024, 8192], bf16 q and latent cache with
64-token pages scattered in a 2x-oversized pool (synthetic, seeded).

Printed: one JSON line with KV-read GB/s over the whole step (the headline
metric), tokens/s, the decode kernel's roofline position (bytes it must move
per launch / its average launch time, against the 8 TB/s HBM peak) and the
fp64 CPU oracle timed on the host on the same batch.

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
    ap.add_argument("--cpu-runs", type=int, default=3)
    ap.add_argument("--decode-launches", type=int, default=30,
                    help="back-to-back decode launches timed for the kernel's launch duration")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device-to-device copy of this many MiB before warm-up, as the "
                         "known-size reference kernel for HBM byte counters")
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


def _traffic(root: str, kernel_src: str):
    """HBM bytes per decode launch from the committed counter summary, or None
    when that summary is missing or was taken on another version of the
    kernel source (sha256 recorded in the file)."""
    import hashlib
    path = os.path.join(root, "profiles", "mla_decode_bf16_dsv3_traffic.json")
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


def main() -> int:
    a = _args()
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
    num_parts = cus
    bt = torch.empty((w.bs, width), dtype=torch.int32, device="cuda")
    tile_plan = torch.empty((num_parts, 8), dtype=torch.int32, device="cuda")
    split_indptr = torch.empty((w.bs + 1,), dtype=torch.int32, device="cuda")
    po, pl = mla.partial_buffers(w.bs, R, num_parts)
    out = torch.empty((w.bs, w.q_len, w.heads, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.bs, w.q_len, w.heads), dtype=torch.float32, device="cuda")
    max_len = int(w.seq_lens.max())
    ev = []  # (start, end) events around each decode launch of the timed steps

    def decode(p):
        mla.mla_decode(p.q, p.kv, bt, p.seq_lens, tile_plan, split_indptr, w.softmax_scale,
                       partial_o=po, partial_lse=pl, out=out, lse=lse, kv_dtype=w.kv_dtype,
                       kv_descale=p.kv_descale, causal=w.causal)

    def step(i: int, record: bool):
        p = pools[i % len(pools)]
        mla.build_block_table(p.req_to_token, p.req_pool_indices, p.seq_lens, width,
                              max_seq_len_hint=max_len, out=bt)
        mla.plan_splits(p.seq_lens, R, num_parts, w.kv_dtype, tile_plan=tile_plan,
                        split_indptr=split_indptr)
        if record:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
        decode(p)
        if record:
            e1.record()
            ev.append((e0, e1))
        mla.merge_states(po, pl, split_indptr, out, lse)

    if a.calib_copy_mib > 0:
        n = a.calib_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)  # the reference kernel for FETCH_SIZE / WRITE_SIZE: n bytes each way
        torch.cuda.synchronize()
        del src, dst
    print(f"[bench] warmup {a.warmup} steps", file=sys.stderr, flush=True)
    for i in range(a.warmup):
        step(i, False)
    torch.cuda.synchronize()
    print(f"[bench] timing {a.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(a.steps):
        step(a.warmup + i, True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / a.steps
    dec_in_step_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    # The decode kernel's launch duration: events bracketing back-to-back
    # launches on the stream the kernel runs on (the plan and block table of
    # the last step are reused; the pools still rotate, so no launch finds its
    # KV in the caches).  An event pair around a single launch also counts the
    # dispatch and end-of-kernel fences, which this amortises away.
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(a.decode_launches):
        decode(pools[i % len(pools)])
    e1.record(stream)
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1) / a.decode_launches

    b = _algorithmic_bytes(w)
    kv_gbs = b["kv"] / (ms_step * 1e-3) / 1e9
    tokens_s = w.bs * w.q_len / (ms_step * 1e-3)
    achieved = b["total"] / (dec_ms * 1e-3) / 1e9
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
            "kv_pools_rotated": len(pools),
        },
        "pct_hbm_peak": round(100.0 * kv_gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(tokens_s, 1),
        "decode_kernel_ms": round(dec_ms, 5),
        "decode_in_step_event_ms": round(dec_in_step_ms, 5),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": _traffic(os.path.dirname(os.path.abspath(__file__)),
                                os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                             "paged_kv_mla_req_amd", "csrc", "decode.hip")),
            "kernel": "mla_decode_bf16_kernel",
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
