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
MFMA_F8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 MFMA, vendor figure (no sparsity)
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
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other configurations (long, verify, fp8, fp8 with an e4m3 "
                         "query) that are measured after the main line")
    ap.add_argument("--q8", action="store_true",
                    help="fp8-query mode on an fp8 workload: q is quantised with the cache "
                         "scale in the step and decoded by mla_decode_q8")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed steps before the warm-up steps (clock settling)")
    ap.add_argument("--graph", action="store_true",
                    help="time replays of the step captured in a HIP graph (measured slower than "
                         "eager launches here: the four launches are not host-bound)")
    ap.add_argument("--cpu-runs", type=int, default=3)
    ap.add_argument("--plan", choices=("balanced", "fixed", "packed"), default="balanced",
                    help="balanced: one cost-balanced part per CU (default); fixed: the "
                         "deterministic fixed-tile plan, one tile per part; packed: the same "
                         "tiles packed into one cost-balanced part per CU (batch-invariant "
                         "results, like fixed)")
    ap.add_argument("--tile-pages", type=int, default=32,
                    help="pages per tile of the fixed and packed plans (32 = 2048 tokens)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="before warm-up, run one plain elementwise kernel (bitwise not) that "
                         "reads and writes this many MiB: the known-size reference for HBM "
                         "byte counters")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU run: turn two rocprofv3 --pmc counter_collection.csv files "
                         "(FETCH_SIZE, then WRITE_SIZE, of a run with --calib-copy-mib) into "
                         "HBM bytes per decode launch and store them under profiles/")
    return ap.parse_args()


def _algorithmic_bytes(w, q8: bool = False) -> dict:
    """Bytes the method must move for one decode launch (each latent row read
    once per request, q read once -- one byte per value for an e4m3 query --,
    o and lse written once, one int32 per page of the block table),
    independent of how the kernels split the work."""
    elem = 2 if w.kv_dtype == "bf16" else 1
    L = w.seq_lens.astype(np.int64)
    R = w.rows_per_req
    kv = int(L.sum()) * 576 * elem
    q = w.bs * R * 576 * (1 if q8 else 2)
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


def _kernel_of(kv_dtype: str, q8: bool = False):
    """(source files under csrc/, kernel name) of the decode kernel that runs
    for a cache dtype (and an e4m3 query)."""
    if q8:
        return ("decode_q8.hip", "decode_device.h"), "mla_decode_q8_kernel"
    return ("decode.hip", "decode_device.h"), ("mla_decode_kernel<false>" if kv_dtype == "bf16"
                                               else "mla_decode_kernel<true>")


def _kernel_src(root: str, workload: str, q8: bool = False) -> list:
    from workloads import CONFIGS
    return [os.path.join(root, "paged_kv_mla_req_amd", "csrc", f)
            for f in _kernel_of(CONFIGS[workload]["kv_dtype"], q8)[0]]


def _sources_sha(paths) -> str:
    """sha256 over the kernel's source files, in order."""
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def _traffic_path(root: str, workload: str, q8: bool = False) -> str:
    from workloads import CONFIGS
    tag = "bf16" if CONFIGS[workload]["kv_dtype"] == "bf16" else ("q8" if q8 else "fp8")
    return os.path.join(root, "profiles", f"mla_decode_{tag}_{workload}_traffic.json")


def _traffic(root: str, kernel_src, workload: str, q8: bool = False):
    """HBM bytes per decode launch from the committed counter summary, or None
    when that summary is missing or was taken on another version of the
    kernel's sources (sha256 recorded in the file)."""
    path = _traffic_path(root, workload, q8)
    try:
        with open(path) as f:
            rec = json.load(f)
        sha = _sources_sha(kernel_src)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != sha:
        return None
    return rec.get("hbm_bytes_per_launch")


def traffic_from_counters(fetch_csv: str, write_csv: str, calib_mib: int, root: str,
                          workload: str, q8: bool = False) -> dict:
    """HBM bytes per decode launch from FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch), each scaled by calib_mib MiB over what the same counter read
    for the calibration kernel (bitwise not over calib_mib MiB)."""
    import csv

    name = _kernel_of("fp8_e4m3" if q8 else "bf16", q8)[1].split("<")[0]

    def read(path, counter):
        """(scaled bytes per decode dispatch, scale, raw bytes, scaled bytes
        per merge dispatch); counters summed over a dispatch's instances."""
        per = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Dispatch_Id"], r["Kernel_Name"])
                per[key] = per.get(key, 0.0) + float(r["Counter_Value"]) * 1024.0
        dec = [v for (_, k), v in per.items() if name + "(" in k or name + "<" in k]
        mrg = [v for (_, k), v in per.items() if "merge_states_kernel" in k]
        cal = [v for (_, k), v in per.items() if "bitwise_not" in k.lower()]
        if not dec or not cal:
            raise SystemExit(f"{path}: no decode or calibration dispatches for {counter}")
        factor = calib_mib * 2.0**20 / max(cal)
        merge = float(np.mean(mrg)) * factor if mrg else None
        return float(np.mean(dec)) * factor, factor, float(np.mean(dec)), merge

    fetch, f_fac, f_raw, m_fetch = read(fetch_csv, "FETCH_SIZE")
    write, w_fac, w_raw, m_write = read(write_csv, "WRITE_SIZE")
    sha = _sources_sha(_kernel_src(root, workload, q8))
    rec = {"hbm_bytes_per_launch": round(fetch + write), "fetch_bytes": round(fetch),
           "write_bytes": round(write), "fetch_raw_bytes": round(f_raw),
           "write_raw_bytes": round(w_raw), "fetch_scale": round(f_fac, 4),
           "write_scale": round(w_fac, 4), "calibration_mib": calib_mib,
           "kernel_source_sha256": sha}
    if m_fetch is not None and m_write is not None:
        rec["merge"] = {"hbm_bytes_per_launch": round(m_fetch + m_write),
                        "fetch_bytes": round(m_fetch), "write_bytes": round(m_write)}
    return rec


def cpu_baseline(w, runs: int) -> dict:
    """The fp64 oracle (as it stands) on the same batch, all rows, on the host."""
    import oracle
    from threadpoolctl import threadpool_limits

    # every host core this process may use (the machine's CPU share where the
    # environment states one), set explicitly for the BLAS pool
    threads = int(os.environ.get("OMP_NUM_THREADS") or 0) or len(os.sched_getaffinity(0))
    args = (w.q_bits, w.kv, w.kv_dtype, w.kv_descale, w.req_to_token, w.req_pool_indices,
            w.seq_lens, w.softmax_scale, w.causal)
    times = []
    with threadpool_limits(limits=threads, user_api="blas"):
        oracle.paged_decode(*args)  # warm-up
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
                      f"median of {runs} runs after 1 warm-up: {t:.3f} s per pass; BLAS "
                      f"threads set to {threads}; host {model or 'unknown CPU'}, "
                      f"os.cpu_count()={os.cpu_count()}",
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


class Path:
    """Device buffers and launch closures of the hot path for one workload:
    `pools` copies of its KV pool (same bits, different HBM addresses, rotated
    per step), the table / plan / workspace / output buffers, and for the
    fp8-query mode (q8) the query codes' buffer and scale."""

    def __init__(self, mla, torch, w, pools: int, plan: str = "balanced", tile_pages: int = 32,
                 q8: bool = False):
        from workloads.device import to_device

        self.mla, self.torch, self.w, self.q8 = mla, torch, w, q8
        self.plan, self.tile_pages = plan, tile_pages
        self.pools = [to_device(w) for _ in range(pools)]
        self.R = w.rows_per_req
        self.width = w.bt_width
        self.max_len = int(w.seq_lens.max())
        n = mla.device_num_cus()
        tiles = int(mla._lib.lib().mla_fixed_split_parts_bound(w.bs, self.max_len, tile_pages))
        if plan == "fixed":
            n = max(1, tiles)
        self.num_parts = n
        dev = "cuda"
        self.bt = torch.empty((w.bs, self.width), dtype=torch.int32, device=dev)
        self.tile_plan = torch.empty((n, 8), dtype=torch.int32, device=dev)
        self.split_indptr = torch.empty((w.bs + 1,), dtype=torch.int32, device=dev)
        self.po, self.pl = mla.partial_buffers(w.bs, self.R, n,
                                               num_slots=tiles if plan == "packed" else None)
        self.out = torch.empty((w.bs, w.q_len, w.heads, 512), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((w.bs, w.q_len, w.heads), dtype=torch.float32, device=dev)
        if q8:
            # the page's choice: q_scale = descale_q = the cache's k_scale
            self.q_scale = self.pools[0].kv_descale
            self.q_codes = torch.empty(self.pools[0].q.shape, dtype=torch.uint8, device=dev)

    def table_and_plan(self, p):
        mla, w = self.mla, self.w
        if self.plan == "fixed":
            mla.build_block_table(p.req_to_token, p.req_pool_indices, p.seq_lens, self.width,
                                  max_seq_len_hint=self.max_len, out=self.bt)
            mla.plan_fixed_splits(p.seq_lens, self.tile_pages, self.num_parts,
                                  max_seq_len_hint=self.max_len, tile_plan=self.tile_plan,
                                  split_indptr=self.split_indptr)
            return
        if self.plan == "packed":
            mla.build_block_table(p.req_to_token, p.req_pool_indices, p.seq_lens, self.width,
                                  max_seq_len_hint=self.max_len, out=self.bt)
            mla.plan_fixed_packed(p.seq_lens, self.R, self.tile_pages, self.num_parts,
                                  tile_plan=self.tile_plan, split_indptr=self.split_indptr)
            return
        mla.build_table_and_plan(p.req_to_token, p.req_pool_indices, p.seq_lens, self.width,
                                 self.R, self.num_parts, w.kv_dtype, max_seq_len_hint=self.max_len,
                                 out=self.bt, tile_plan=self.tile_plan,
                                 split_indptr=self.split_indptr)

    def decode(self, p):
        """The per-layer attention: (fp8 query: quantise q, then) split decode."""
        mla, w = self.mla, self.w
        if self.q8:
            mla.quantize_q_fp8(p.q, self.q_scale, out=self.q_codes)
            mla.mla_decode_q8(self.q_codes, self.q_scale, p.kv, self.bt, p.seq_lens,
                              self.tile_plan, self.split_indptr, w.softmax_scale,
                              kv_descale=p.kv_descale, partial_o=self.po, partial_lse=self.pl,
                              out=self.out, lse=self.lse, causal=w.causal)
        else:
            mla.mla_decode(p.q, p.kv, self.bt, p.seq_lens, self.tile_plan, self.split_indptr,
                           w.softmax_scale, partial_o=self.po, partial_lse=self.pl,
                           out=self.out, lse=self.lse, kv_dtype=w.kv_dtype,
                           kv_descale=p.kv_descale, causal=w.causal)

    def merge(self):
        self.mla.merge_states(self.po, self.pl, self.split_indptr, self.out, self.lse)

    def step(self, i: int, ev=None):
        """One pass of the hot path: block table + plan (one launch), the
        attention, merge.  ev: a pair of events that the decode kernel's own
        launch records at its begin and end."""
        p = self.pools[i % len(self.pools)]
        self.table_and_plan(p)
        if self.q8:
            self.mla.quantize_q_fp8(p.q, self.q_scale, out=self.q_codes)
        if ev is not None:
            self.mla.time_next_decode(*ev)
        if self.q8:
            w = self.w
            self.mla.mla_decode_q8(self.q_codes, self.q_scale, p.kv, self.bt, p.seq_lens,
                                   self.tile_plan, self.split_indptr, w.softmax_scale,
                                   kv_descale=p.kv_descale, partial_o=self.po,
                                   partial_lse=self.pl, out=self.out, lse=self.lse,
                                   causal=w.causal)
        else:
            self.decode(p)
        self.merge()

    def timed_loop(self, fn, n: int) -> float:
        """ms per call of fn(i) over n back-to-back calls."""
        torch = self.torch
        torch.cuda.synchronize()
        t = time.perf_counter()
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3 / n

    def settle(self, seconds: float) -> int:
        """Untimed steps for `seconds` (the card raises its clocks over the
        first ~0.1 s of sustained load)."""
        t = time.perf_counter()
        n = 0
        while time.perf_counter() - t < seconds:
            self.step(n)
            n += 1
            if n % 16 == 0:
                self.torch.cuda.synchronize()
        self.torch.cuda.synchronize()
        return n

    def events(self, n: int):
        """n event pairs, each recorded once so that it exists."""
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n)]
        for e0, e1 in ev:
            e0.record()
            e1.record()
        return ev


def mfma_floor_ms(w, q8: bool) -> float:
    """Matrix-core time floor of one decode launch at the dense peaks of the
    operand type: everything at the e4m3 peak for an fp8 query (the
    algorithmic flops; the kernel's split of each weight into two e4m3
    numbers doubles its output MFMAs, which this floor does not count), else
    everything at bf16."""
    flops = _algorithmic_flops(w)
    return flops / ((MFMA_F8_PEAK_TFLOPS if q8 else MFMA_PEAK_TFLOPS) * 1e12) * 1e3


def measure_workload(mla, torch, name: str, q8: bool, steps: int, warmup: int,
                     settle: float) -> dict:
    """A second configuration, measured the way the main line is: steps of the
    whole path with rotated pools, the decode kernel's own launch time from
    events it records, decode + merge on its own."""
    from workloads import make_workload

    w = make_workload(name)
    P = Path(mla, torch, w, pools=2, q8=q8)
    P.settle(settle)
    for i in range(warmup):
        P.step(i)
    ev = P.events(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        P.step(warmup + i, ev[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    dec_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    ms_dm = P.timed_loop(lambda i: (P.decode(P.pools[i % 2]), P.merge()), steps)
    b = _algorithmic_bytes(w, q8)
    flops = _algorithmic_flops(w)
    res = {
        "workload": f"{w.name}: batch {w.bs}, {w.heads} heads, q_len {w.q_len}, KV lengths "
                    f"{int(w.seq_lens.min())}..{int(w.seq_lens.max())}, {w.kv_dtype} cache"
                    + (", e4m3 query (quantised in the step)" if q8 else ", bf16 query"),
        "kernel": _kernel_of(w.kv_dtype, q8)[1],
        "num_parts": P.num_parts,
        "ms_per_step": round(ms_step, 5),
        "kv_read_gbs_step": round(b["kv"] / (ms_step * 1e-3) / 1e9, 2),
        "decode_kernel_us": round(dec_ms * 1e3, 2),
        "ms_decode_merge": round(ms_dm, 5),
        "roofline": {"bound": "hbm", "bytes_per_launch": b["total"],
                     "achieved_gbs": round(b["total"] / (dec_ms * 1e-3) / 1e9, 2),
                     "frac": round(b["total"] / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "mfma": {"algorithmic_tflop": round(flops / 1e12, 4),
                 "achieved_tflops": round(flops / (dec_ms * 1e-3) / 1e12, 2),
                 "floor_us": round(mfma_floor_ms(w, q8) * 1e3, 2),
                 "frac": round(mfma_floor_ms(w, q8) / dec_ms, 4),
                 "peaks": "e4m3 5000 TFLOP/s"
                          if q8 else "bf16 2500 TFLOP/s"},
    }
    del P
    torch.cuda.empty_cache()
    return res


EXTRA_WORKLOADS = (("long", False), ("verify", False), ("fp8", False), ("fp8", True))


def main() -> int:
    a = _args()
    if a.traffic_from:
        root = os.path.dirname(os.path.abspath(__file__))
        rec = traffic_from_counters(a.traffic_from[0], a.traffic_from[1],
                                    a.calib_copy_mib or 256, root, a.workload, a.q8)
        rec["workload"] = a.workload + ("_q8" if a.q8 else "")
        path = _traffic_path(root, a.workload, a.q8)
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

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 2
    torch.cuda.set_device(0)
    print(f"[bench] generating workload {a.workload}", file=sys.stderr, flush=True)
    w = make_workload(a.workload)
    if a.q8 and w.kv_dtype != "fp8_e4m3":
        print("--q8 needs a workload with an fp8 cache", file=sys.stderr)
        return 2
    P = Path(mla, torch, w, a.pools, a.plan, a.tile_pages, a.q8)
    # For every EV_EVERY-th timed step, a pair of events that the decode
    # kernel's own launch records at its begin and end
    # (mla_decode_time_next_launch).  An event-recorded launch ends with a
    # release to system scope (an L2 write-back), which costs that step a few
    # microseconds, so only a sample of the timed launches records them.  They
    # are created, and recorded once so that they exist, before timing starts.
    ev = P.events((a.steps + EV_EVERY - 1) // EV_EVERY)

    if a.calib_copy_mib > 0:
        n = a.calib_copy_mib << 18  # int32 elements
        src = torch.ones(n, dtype=torch.int32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.bitwise_not(src, out=dst)  # reads and writes calib_copy_mib MiB
        torch.cuda.synchronize()
        del src, dst
    n_settle = P.settle(a.settle)
    print(f"[bench] clock settling: {n_settle} untimed steps; warmup {a.warmup} steps",
          file=sys.stderr, flush=True)
    for i in range(a.warmup):
        P.step(i)
    torch.cuda.synchronize()
    graphs = []
    if a.graph:
        # One captured step per KV pool: the kernels of the step replay
        # without host launch work between them.
        for j in range(len(P.pools)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                P.step(j)
            graphs.append(g)
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()

    def timed_step(i):
        P.step(a.warmup + i, ev[i // EV_EVERY] if i % EV_EVERY == 0 else None)

    print(f"[bench] timing {a.steps} steps ({'graph replays' if a.graph else 'eager'})",
          file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(a.steps):
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            timed_step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / a.steps
    ms_step_eager = None
    if graphs:
        # The decode kernel's own duration comes from eager steps (the launch
        # records the events itself, which a graph replay cannot do).
        ms_step_eager = P.timed_loop(timed_step, a.steps)
    # the decode kernel's average launch duration over the event-timed steps
    dec_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in ev]))
    # The step's parts on their own (the table and plan run once per batch
    # step, decode and merge once per attention layer): same inputs, timed
    # back to back after the main loop.
    ms_dm = P.timed_loop(lambda i: (P.decode(P.pools[i % len(P.pools)]), P.merge()), a.steps)
    ms_tp = P.timed_loop(lambda i: P.table_and_plan(P.pools[i % len(P.pools)]), a.steps)
    # The KV append that precedes attention (set_kv_buffer): the step's new
    # tokens, then a 32768-token chunk.  It writes into pool 0, so it runs last.
    append = time_append(mla, torch, w, P.pools[0], a.steps)
    # (skipped in counter runs: their calibration kernel is the only bitwise not)
    copy_gbs = measured_copy_gbs(torch) if a.calib_copy_mib == 0 else None

    b = _algorithmic_bytes(w, a.q8)
    kv_gbs = b["kv"] / (ms_step * 1e-3) / 1e9
    tokens_s = w.bs * w.q_len / (ms_step * 1e-3)
    achieved = b["total"] / (dec_ms * 1e-3) / 1e9
    flops = _algorithmic_flops(w)
    tflops = flops / (dec_ms * 1e-3) / 1e12
    root = os.path.dirname(os.path.abspath(__file__))
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
        "dtype": "bf16" if w.kv_dtype == "bf16" else (
            "fp8_e4m3 kv and q" if a.q8 else "fp8_e4m3 kv, bf16 q"),
        "data": "synthetic (seeded N(0,1) q and latent cache, scattered 64-token pages)",
        "config": {
            "workload": f"{w.name}: batch {w.bs}, {w.heads} heads, q_len {w.q_len}, "
                        f"KV lengths {int(w.seq_lens.min())}..{int(w.seq_lens.max())} "
                        f"(mean {float(w.seq_lens.mean()):.0f}), latent 576 / value 512, "
                        f"page 64, {w.kv_dtype} cache" + (", e4m3 query" if a.q8 else ""),
            "global_batch": w.bs,
            "seq_len": int(round(float(w.seq_lens.mean()))),
            "parallelism": "single GPU",
            "num_parts": P.num_parts,
            "plan": (a.plan if a.plan == "balanced" else
                     f"fixed tiles of {a.tile_pages} pages" + (", packed" if a.plan == "packed"
                                                                else "")),
            "kv_pools_rotated": len(P.pools),
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
                 "achieved_tflops": round(tflops, 2),
                 "floor_us": round(mfma_floor_ms(w, a.q8) * 1e3, 2),
                 "frac": round(mfma_floor_ms(w, a.q8) / dec_ms, 4),
                 "peaks": "e4m3 5000 TFLOP/s"
                          if a.q8 else "bf16 2500 TFLOP/s (an e4m3 cache is converted to "
                                       "bf16 in LDS)"},
        "append": append,
        "step_launch": "hip graph replay" if a.graph else "eager",
        "ms_per_step_eager": None if ms_step_eager is None else round(ms_step_eager, 5),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": _traffic(root, _kernel_src(root, a.workload, a.q8), a.workload, a.q8),
            "kernel": _kernel_of(w.kv_dtype, a.q8)[1],
            "bytes_per_launch": b["total"],
        },
    }
    del P, graphs
    torch.cuda.empty_cache()
    if not a.no_extra:
        # the other configurations, each measured on its own (decode kernel
        # time from its own events, decode + merge, roofline and MFMA position)
        extra = {}
        for name, q8 in EXTRA_WORKLOADS:
            key = name + ("_q8" if q8 else "")
            print(f"[bench] workload {key}", file=sys.stderr, flush=True)
            extra[key] = measure_workload(mla, torch, name, q8, steps=min(a.steps, 20),
                                          warmup=3, settle=0.2)
        line["other_workloads"] = extra
    if not a.no_cpu_baseline:
        print("[bench] timing the fp64 CPU oracle", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, a.cpu_runs)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
