"""Benchmark of the OSCAR INT2 decode hot path on one MI355X.

One step = one launch of the fused decode step (oscar_decode_step): each
sequence's new token written to its BF16 slot, the token leaving the recent
window quantized into its INT2 slot, and the paged INT2 decode attention of
one query per sequence, over a cache filled once by the library's kernels.
The timed steps rotate over enough copies of the cache (pools, tables,
rotations, queries) that the 256 MB Infinity Cache cannot serve them, as
consecutive layers of a model would.

Prints ONE JSON line (rank 0):
  value        KV-tokens/s  (sum of context lengths / step time, all KV heads)
  roofline     the fused step kernel: algorithmic bytes (the decode's and the
               update's) / its average launch time (HIP events on the launch
               stream around the K timed launches) vs 8 TB/s
  cpu_baseline the float64 NumPy oracle decoding the same cache on host cores
Context beside it: the decode launch alone, the two-launch step (update, then
decode), the all-BF16 decode, the quantize-append prefill (kernel A), the
chunked-prefill attention and the INT4-cache decode, each timed the same way.

--append-prefill measures quantize-append alone on the large-GQA layer's
prefill (8 sequences x 8192 rows, 96 q / 8 KV heads, d = 128) and prints the
same kind of line for it (rows/s, roofline of the quantize-append kernel, the
oracle quantizing a sample of the rows).
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

HBM_PEAK_GBPS = 8000.0
METRIC = "INT2 paged decode-attn KV-tokens/s + achieved HBM GB/s (% of peak), Qwen3-8B layer"


def blas_threads(n: int):
    """Limit the host BLAS pools to n threads (threadpoolctl) and report the
    count they then hold: the core count a cpu_baseline states is measured,
    not assumed."""
    from threadpoolctl import threadpool_info, threadpool_limits
    lim = threadpool_limits(limits=n, user_api="blas")
    got = [p.get("num_threads") for p in threadpool_info() if p.get("user_api") == "blas"]
    return lim, (max(got) if got else 1)


def algorithmic_bytes(inp, w) -> dict:
    """Unique bytes the decode must move: INT2 middle tokens at 96 B (d=128)
    per KV head (2 x d/4 B codes + 2 x 2 (d/32) f16 scale/zero x 2 B), BF16
    sink/recent tokens at 4 d B per KV head, R_K and R_V (f32), q and out
    (bf16) and the block-table entries read."""
    from int2_rotated_kv_oscar_amd import synth
    d, hkv = w.d, w.n_kv_heads
    per_mid = 2 * (d // 4) + 2 * 2 * (d // 32) * 2
    mid = raw = pages = 0
    seen_mid = set()
    for b, L in enumerate(inp.seq_lens):
        sink, m, rec = synth.regions(int(L), w.n_sink, w.n_recent)
        # shared-prefix middle tokens are stored once
        lo = m[0] if (b == 0 or not w.shared_prefix) else max(m[0], w.shared_prefix)
        mid += max(0, m[1] - lo)
        raw += (sink[1] - sink[0]) + (rec[1] - rec[0]) if (b == 0 or not w.shared_prefix) else (rec[1] - rec[0])
        pages += (int(L) + 15) // 16
    B = len(inp.seq_lens)
    parts = {
        "int2": mid * per_mid * hkv,
        "bf16": raw * 4 * d * hkv,
        "rotations": 2 * d * d * 4 * hkv,
        "q_out": 2 * B * w.n_q_heads * d * 2,
        "tables": pages * 4,
    }
    parts["total"] = sum(parts.values())
    return parts


def step_update_bytes(inp, w) -> int:
    """Unique bytes of the step's cache update beside the decode's: per
    sequence and KV head, the new K/V row read (4 d B) and, when it lands in a
    BF16 region, written to its slot (4 d B); when a token enters the middle
    history, its raw row read from its BF16 slot (4 d B, unless it is the new
    token) and its INT2 slot written (96 B at d = 128)."""
    d, hkv, S, W = w.d, w.n_kv_heads, w.n_sink, w.n_recent
    per_mid = 2 * (d // 4) + 2 * 2 * (d // 32) * 2
    total = 0
    for L in inp.seq_lens:
        L = int(L)
        if L < 1:
            continue
        total += 4 * d
        if W >= 1 or L - 1 < S:
            total += 4 * d
        t = L - 1 - W
        if t >= S:
            total += per_mid + (4 * d if W >= 1 else 0)
    return total * hkv


def decode_kernel_name(w, split_pages: int, all_raw: bool, fused: bool = False) -> str:
    """The decode kernel instance the library launches for this workload
    (template arguments: head dim, all-BF16 cache, balanced slices, MFMA
    column slots per query, fused step update), by the library's rule:
    per-unit items when split_pages is given or the (sequence, KV head) units
    are at most a quarter of the CUs."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    slices = not (split_pages != 0 or 4 * w.batch * w.n_kv_heads <= cus)
    g = w.n_q_heads // w.n_kv_heads
    cs = 1 if all_raw else 4 if g <= 4 else 2 if g <= 8 else 1
    b = lambda x: "true" if x else "false"  # noqa: E731
    return f"decode_kernel<{w.d},{b(all_raw)},{b(slices)},{cs},{b(fused)}>"


DECODE_SOURCES = ["decode.hip", "device_utils.h", "layout.h"]
APPEND_SOURCES = ["quantize_append.hip", "device_utils.h", "layout.h"]


def measured_traffic(workload: str, kernel: str = "decode_kernel", sources=DECODE_SOURCES):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 counter
    summary for this workload (FETCH_SIZE / WRITE_SIZE scaled by a plain-copy
    calibration), or None when there is none or the kernel's sources changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "int2_rotated_kv_oscar_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    digest, traffic = None, None
    with open(path) as fh:
        for line in fh:
            if line.startswith("sources sha256[:16] = ") or line.startswith("decode sources sha256[:16] = "):
                digest = line.split("=")[1].strip()
            if line.startswith("traffic_bytes = "):
                traffic = int(line.split("=")[1].strip())
    return traffic if digest == h.hexdigest()[:16] else None


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--workload", default="qwen3-8b-b1-32k")
    ap.add_argument("--context", type=int, default=0,
                    help="override the context length of a fixed-length workload (the workload is then named <name>-ctx<L>)")
    ap.add_argument("--split-pages", type=int, default=0)
    ap.add_argument("--copies", type=int, default=0, help="cache copies rotated over (0: >= 1 GiB total)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16-baseline", action="store_true")
    ap.add_argument("--no-append", action="store_true",
                    help="leave out the quantize-append prefill line (kernel A) of the default run")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (calibrates HBM byte counters), then exit")
    ap.add_argument("--append-prefill", action="store_true",
                    help="measure quantize-append alone on the large-GQA layer's prefill (8 sequences x 8192 rows)")
    ap.add_argument("--calib-gram", action="store_true",
                    help="measure the GPU calibration target (Q^T Q per KV head) on the Qwen3-8B calibration rows")
    ap.add_argument("--extend", action="store_true",
                    help="measure chunked-prefill attention alone: the 28-sequence Qwen3-8B cache, 512 new rows each")
    ap.add_argument("--int4", action="store_true",
                    help="measure the INT4-cache decode alone on the workload's shape")
    ap.add_argument("--no-extras", action="store_true",
                    help="leave the extend and INT4-decode lines out of the default run")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the decode path shards by KV head "
              f"with no exchange between GPUs)", file=sys.stderr)
        return 2
    from int2_rotated_kv_oscar_amd import synth
    if args.workload not in synth.WORKLOADS:
        print(f"unknown workload {args.workload!r}; known: {', '.join(sorted(synth.WORKLOADS))}", file=sys.stderr)
        return 2
    w = synth.WORKLOADS[args.workload]
    if args.context:
        if w.ctx[0] != "fixed" or args.context <= w.n_sink + w.n_recent:
            print(f"--context needs a fixed-length workload and a length above sink + recent "
                  f"({w.n_sink + w.n_recent}), so that the cache has an INT2 part", file=sys.stderr)
            return 2
        w = synth.Workload(**{**w.__dict__, "name": f"{w.name}-ctx{args.context}",
                              "ctx": ("fixed", args.context, args.context)})

    import torch
    from int2_rotated_kv_oscar_amd import lib

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = "cuda:0"
    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: 5 copies of {n} B")
        return 0
    lib.load()
    if args.append_prefill:
        return run_append_prefill(args, log)
    if args.calib_gram:
        return run_calib_gram(args, log)
    if args.extend:
        print(json.dumps(extend_line(args, log, cpu=not args.no_cpu_baseline)), flush=True)
        return 0
    if args.int4:
        print(json.dumps(int4_decode_line(args, log, w, cpu=not args.no_cpu_baseline)), flush=True)
        return 0
    t0 = time.time()
    inp = synth.decode_inputs(w)
    log(f"inputs {time.time() - t0:.1f}s  B={len(inp.seq_lens)} max_len={inp.max_seq_len}")
    t0 = time.time()
    cal = synth.calibration_set(w)
    rt = lib.build_rotation(cal.q, cal.k, cal.v, w.group_q)
    log(f"calibration (oscar_build_rotation, {w.calib_rows} rows) {time.time() - t0:.1f}s")
    r_k = torch.from_numpy(rt["r_k"].astype(np.float32)).to(dev)
    r_v = torch.from_numpy(rt["r_v"].astype(np.float32)).to(dev)
    tau_k, tau_v = float(np.float32(rt["tau_k"])), float(np.float32(rt["tau_v"]))

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    nbq = lib.int2_page_bytes(w.d, w.n_kv_heads)
    nbh = lib.bf16_page_bytes(w.d, w.n_kv_heads)
    int2 = torch.zeros(inp.n_int2_pages * nbq, dtype=torch.uint8, device=dev)
    B0 = len(inp.seq_lens)
    # one spare BF16 page per sequence: the serving step reads the token that
    # leaves the recent window from its BF16 slot, whose page the current
    # window may no longer hold
    bf16 = torch.zeros((inp.n_bf16_pages + B0) * nbh // 2, dtype=torch.int16, device=dev)
    cache = lib.make_cache(w.d, w.n_kv_heads, w.n_sink, w.n_recent, int2, bf16)
    bt_h_np = inp.bt_h.copy()
    lv_seq, lv_pos, lv_row = [], [], []
    for b, L in enumerate(inp.seq_lens):
        t = int(L) - 1 - w.n_recent
        if w.n_recent >= 1 and t >= w.n_sink:
            if bt_h_np[b, t // 16] < 0:
                bt_h_np[b, t // 16] = inp.n_bf16_pages + b
            lv_seq.append(b); lv_pos.append(t); lv_row.append(inp.row_of[b][t])
    bt_q, bt_h = i32(inp.bt_q), i32(bt_h_np)
    ms, mp, mr = synth.middle_rows(inp)
    lib.quantize_append(cache, bf(inp.k_rows[mr]), bf(inp.v_rows[mr]), i32(ms), i32(mp), bt_q, r_k, r_v, tau_k, tau_v)
    hs, hp, hr = synth.bf16_rows(inp)
    lib.write_bf16(cache, bf(inp.k_rows[hr]), bf(inp.v_rows[hr]), i32(hs), i32(hp), bt_h)
    if lv_seq:  # the leaving tokens' rows, where the previous steps left them
        lib.write_bf16(cache, bf(inp.k_rows[np.array(lv_row)]), bf(inp.v_rows[np.array(lv_row)]), i32(lv_seq),
                       i32(lv_pos), bt_h)
    new_rows = np.array([inp.row_of[b][max(int(L) - 1, 0)] for b, L in enumerate(inp.seq_lens)])
    n_k, n_v = bf(inp.k_rows[new_rows]), bf(inp.v_rows[new_rows])
    torch.cuda.synchronize()

    nbytes = algorithmic_bytes(inp, w)
    footprint = int2.numel() + bf16.numel() * 2 + r_k.numel() * 8
    copies = args.copies or max(1, int(np.ceil((1 << 30) / footprint)))
    pools = [(int2, bf16, r_k, r_v)]
    for _ in range(copies - 1):
        pools.append((int2.clone(), bf16.clone(), r_k.clone(), r_v.clone()))
    caches = [lib.make_cache(w.d, w.n_kv_heads, w.n_sink, w.n_recent, p[0], p[1]) for p in pools]
    q = bf(inp.q)
    qs = [q] + [q.clone() for _ in range(copies - 1)]
    seq_lens = i32(inp.seq_lens)
    B = len(inp.seq_lens)
    ws_bytes = lib.decode_workspace_bytes(B, w.n_kv_heads, w.n_q_heads, w.d, inp.max_seq_len, args.split_pages)
    ws = torch.empty((ws_bytes + 3) // 4, dtype=torch.int32, device=dev)
    lib.decode_workspace_init(ws)
    out = torch.empty(B, w.n_q_heads, w.d, dtype=torch.bfloat16, device=dev)
    log(f"cache footprint {footprint / 1e6:.1f} MB x {copies} copies; workspace {ws_bytes / 1e6:.2f} MB")

    upd_bytes = step_update_bytes(inp, w)

    def step(i):
        c = caches[i % copies]
        _, _, prk, prv = pools[i % copies]
        lib.decode_step(c, n_k, n_v, qs[i % copies], seq_lens, inp.max_seq_len, bt_q, bt_h, prk, prv, tau_k, tau_v,
                        out, ws, split_pages=args.split_pages)

    def timed(fn, n):
        """Average ms of n calls of fn back to back: HIP events on the
        launch stream (torch's current stream, which the binding uses)."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    # throughput: K steps back to back, nothing else on the stream; a step is
    # one launch, so this is also the fused kernel's average launch time
    ms_step = timed(step, K)
    tokens = int(inp.seq_lens.sum())
    value = tokens / (ms_step * 1e-3)
    step_bytes = nbytes["total"] + upd_bytes
    # the library fuses the update into the decode launch with split_pages
    # given or at most as many (sequence, KV head) units as CUs; with more
    # units the step is the update kernel, then the decode
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    fused = args.split_pages != 0 or B * w.n_kv_heads <= cus
    log(f"step ({'one fused launch' if fused else 'update + decode launches'}) {ms_step * 1e3:.1f} us, "
        f"{step_bytes / (ms_step * 1e-3) / 1e9:.0f} GB/s, bytes {nbytes} + update {upd_bytes}")

    # context: the decode launch alone, and the two-launch step (the update
    # kernel, then the decode)
    def decode_only(i):
        lib.paged_decode_attn(caches[i % copies], qs[i % copies], seq_lens, inp.max_seq_len, bt_q, bt_h,
                              pools[i % copies][2], pools[i % copies][3], out, ws, split_pages=args.split_pages)

    def update_only(i):
        lib.decode_step_update(caches[i % copies], n_k, n_v, seq_lens, bt_q, bt_h, pools[i % copies][2],
                               pools[i % copies][3], tau_k, tau_v)

    def two_launch(i):
        update_only(i)
        decode_only(i)

    for i in range(args.warmup):
        two_launch(i)
    dec_avg = timed(decode_only, K)
    upd_ms = timed(update_only, K)
    serve_ms = timed(two_launch, K)
    dec_gbps = nbytes["total"] / (dec_avg * 1e-3) / 1e9
    # the roofline's kernel: the fused launch (it is the step), else the decode
    achieved = step_bytes / (ms_step * 1e-3) / 1e9 if fused else dec_gbps
    log(f"decode launch alone {dec_avg * 1e3:.1f} us ({dec_gbps:.0f} GB/s); two-launch step {serve_ms * 1e3:.1f} us, "
        f"update alone {upd_ms * 1e3:.1f} us")

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "KV-tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "int2 codes x f16 MFMA, f32 accumulate", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "context": inp.max_seq_len, "q_heads": w.n_q_heads,
                   "kv_heads": w.n_kv_heads, "head_dim": w.d, "page_tokens": 16, "sink": w.n_sink,
                   "recent": w.n_recent, "split_pages": args.split_pages or "auto", "cache_copies": copies},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(w.name, "decode_step" if fused else "decode_kernel"),
                     "kernel": decode_kernel_name(w, args.split_pages, False, fused=fused),
                     "algorithmic_bytes_per_launch": step_bytes if fused else nbytes["total"],
                     "avg_launch_us": round((ms_step if fused else dec_avg) * 1e3, 2),
                     "step_launches": 1 if fused else 2},
        "decode_only": {"kernel": decode_kernel_name(w, args.split_pages, False),
                        "avg_launch_us": round(dec_avg * 1e3, 2), "algorithmic_bytes_per_launch": nbytes["total"],
                        "achieved_GBps": round(dec_gbps, 1), "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                        "traffic": measured_traffic(w.name)},
        "two_launch_step": {"kernels": [f"quantize_rows_kernel<{w.d},true,2>", decode_kernel_name(w, args.split_pages, False)],
                            "us_per_step": round(serve_ms * 1e3, 2),
                            "KV_tokens_per_s": round(tokens / (serve_ms * 1e-3), 1),
                            "update_us_per_call": round(upd_ms * 1e3, 2)},
    }

    # attainable bandwidth, as context for the roofline fraction, over 1 GiB
    # (several times the Infinity Cache): a streaming read of the buffer with
    # nothing written back (the library's probe kernel; the decode reads far
    # more than it writes), and torch's vectorized elementwise kernel (read +
    # write bytes)
    pa = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    pb = torch.empty_like(pa)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    for _ in range(3):
        torch.mul(pa, 2.0, out=pb)
        lib.bw_probe_read(pa, sink)
    torch.cuda.synchronize()
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    p0.record()
    for _ in range(20):
        torch.mul(pa, 2.0, out=pb)
    p1.record()
    torch.cuda.synchronize()
    probe = 2 * pa.numel() * 4 / (p0.elapsed_time(p1) / 20 * 1e-3) / 1e9
    p0.record()
    for _ in range(20):
        lib.bw_probe_read(pa, sink)
    p1.record()
    torch.cuda.synchronize()
    rprobe = pa.numel() * 4 / (p0.elapsed_time(p1) / 20 * 1e-3) / 1e9
    del pa, pb
    result["bw_probe"] = {"read_GBps": round(rprobe, 1), "stream_GBps": round(probe, 1),
                          "method": "oscar_bw_probe_read over a 1 GiB buffer (read bytes); torch.mul over a "
                                    "1 GiB float32 buffer (read + write bytes)",
                          "step_frac_of_read_probe": round(achieved / rprobe, 4)}
    log(f"bw probes: read {rprobe:.0f} GB/s, read+write {probe:.0f} GB/s; step at {achieved / rprobe:.1%} of the read probe")

    if not args.no_bf16_baseline:
        # the same decode over an all-BF16 cache (every token in BF16 pages)
        wb = synth.Workload(**{**w.__dict__, "n_sink": 1 << 30, "n_recent": 0})
        inb = synth.DecodeInputs(wb, inp.seq_lens, inp.k_rows, inp.v_rows, inp.row_of, inp.q,
                                 inp.bt_q, *_all_bf16_tables(inp))
        bt_hb = i32(inb.bt_h)
        hb_pool = torch.zeros(inb.n_bf16_pages * nbh // 2, dtype=torch.int16, device=dev)
        cb = lib.make_cache(w.d, w.n_kv_heads, 0, 0, None, hb_pool)
        hs2, hp2, hr2 = synth.bf16_rows(inb)
        lib.write_bf16(cb, bf(inp.k_rows[hr2]), bf(inp.v_rows[hr2]), i32(hs2), i32(hp2), bt_hb)
        ncopy = max(1, int(np.ceil((1 << 30) / (hb_pool.numel() * 2))))
        hpools = [hb_pool] + [hb_pool.clone() for _ in range(ncopy - 1)]
        hcaches = [lib.make_cache(w.d, w.n_kv_heads, 0, 0, None, p) for p in hpools]
        for i in range(args.warmup):
            lib.paged_decode_attn_bf16(hcaches[i % ncopy], q, seq_lens, inp.max_seq_len, bt_hb, out, ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(K):
            lib.paged_decode_attn_bf16(hcaches[i % ncopy], q, seq_lens, inp.max_seq_len, bt_hb, out, ws)
        e1.record()
        torch.cuda.synchronize()
        bms = e0.elapsed_time(e1) / K
        bbytes = tokens * 4 * w.d * w.n_kv_heads + 2 * B * w.n_q_heads * w.d * 2
        result["bf16_baseline"] = {"kernel": decode_kernel_name(w, args.split_pages, True), "us_per_call": round(bms * 1e3, 2),
                                   "KV_tokens_per_s": round(tokens / (bms * 1e-3), 1),
                                   "achieved_GBps": round(bbytes / (bms * 1e-3) / 1e9, 1),
                                   "int2_decode_speedup": round(bms / dec_avg, 3)}
        log(f"bf16 baseline {bms * 1e3:.1f} us/call")
        del hpools, hcaches

    if not args.no_append:
        # kernel A alone on the large-GQA layer's prefill, its own roofline
        result["quantize_append"] = append_prefill_line(args, log, cpu=False)
    if not args.no_extras:
        # the rows beside the decode: chunked prefill over the mixed cache and
        # the INT4-cache decode, each with its own roofline
        result["extend"] = extend_line(args, log, cpu=False)
        result["int4_decode"] = int4_decode_line(args, log, w, cpu=False)

    if not args.no_cpu_baseline:
        cores = len(os.sched_getaffinity(0))
        result["cpu_baseline"] = _cpu_baseline(inp, w, cache, int2, bf16, rt, tokens, log, cores, 10.0)
        result["cpu_baseline_single_core"] = _cpu_baseline(inp, w, cache, int2, bf16, rt, tokens, log, 1, 5.0)
    print(json.dumps(result), flush=True)
    return 0


PREFILL_METRIC = "INT2 quantize-append rows/s + achieved HBM GB/s (% of peak), 96q/8kv layer prefill"


def append_bytes(n_rows: int, n_kv: int, d: int, n_pages: int) -> int:
    """Unique bytes one quantize-append launch must move: per row, KV head and
    tensor the bf16 row in (2d B), its codes (d/4 B) and f16 scale/zero
    (2 x 2 (d/32) B) out; R_K and R_V (f32); row_seq/row_pos; one table entry
    per page written."""
    per = 2 * d + d // 4 + 4 * (d // 32)
    return n_rows * n_kv * 2 * per + 2 * n_kv * d * d * 4 + n_rows * 8 + n_pages * 4


def run_append_prefill(args, log) -> int:
    print(json.dumps(append_prefill_line(args, log, cpu=not args.no_cpu_baseline)), flush=True)
    return 0


def append_prefill_line(args, log, cpu: bool) -> dict:
    """Kernel A alone on the large-GQA layer's prefill: 8 sequences append an
    8192-token chunk each (page-aligned, shuffled pages), 8 KV heads, d = 128.
    The timed launches rotate over input/pool copies totalling >= 1 GiB."""
    import torch
    from int2_rotated_kv_oscar_amd import lib, synth
    dev = "cuda:0"
    w = synth.WORKLOADS["gqa96-b64-ragged"]
    n_seq, chunk = 8, 8192
    t0 = time.time()
    k, v, row_seq, row_pos = synth.prefill_rows(w, n_seq, chunk)
    pages_per = (chunk + 15) // 16
    bt = synth.rng_for(w.cfg_id, 7).permutation(n_seq * pages_per).astype(np.int32).reshape(n_seq, pages_per)
    # the rotation is an input of the kernel; 1024 calibration rows per KV
    # head keep the host calibration short (its size does not change the work)
    cal = synth.calibration_set(w, n_rows=1024)
    rt = lib.build_rotation(cal.q, cal.k, cal.v, w.group_q)
    log(f"prefill rows {k.shape} + calibration {time.time() - t0:.1f}s")
    tau_k, tau_v = float(np.float32(rt["tau_k"])), float(np.float32(rt["tau_v"]))
    n_rows = len(row_seq)
    n_pages = n_seq * pages_per

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    nbq = lib.int2_page_bytes(w.d, w.n_kv_heads)
    per_copy = 2 * k.nbytes + n_pages * nbq
    copies = args.copies or max(1, int(np.ceil((1 << 30) / per_copy)))
    sets = []
    base = (bf(k), bf(v), i32(row_seq), i32(row_pos), i32(bt),
            torch.from_numpy(rt["r_k"].astype(np.float32)).to(dev),
            torch.from_numpy(rt["r_v"].astype(np.float32)).to(dev))
    for c in range(copies):
        t = base if c == 0 else tuple(x.clone() for x in base)
        pool = torch.zeros(n_pages * nbq, dtype=torch.uint8, device=dev)
        sets.append((lib.make_cache(w.d, w.n_kv_heads, w.n_sink, w.n_recent, pool, None), t))
    log(f"{n_rows} rows x {w.n_kv_heads} KV heads; {per_copy / 1e6:.1f} MB x {copies} copies")

    def launch(i):
        c, (kk, vv, rs, rp, bb, rk, rv) = sets[i % copies]
        lib.quantize_append(c, kk, vv, rs, rp, bb, rk, rv, tau_k, tau_v)

    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()
    K = args.steps
    # HIP events on the stream the binding launches on (torch's current one)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        launch(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    nbytes = append_bytes(n_rows, w.n_kv_heads, w.d, n_pages)
    achieved = nbytes / (ms * 1e-3) / 1e9
    flops = 2 * n_rows * w.n_kv_heads * 2 * w.d * w.d  # the rotation y = x R, K and V
    log(f"quantize_append {ms * 1e3:.1f} us, {achieved:.0f} GB/s, {flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s (x2 split)")
    result = {
        "metric": PREFILL_METRIC, "value": round(n_rows / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 in, f16 hi/lo MFMA, f32 accumulate, int2 out",
        "data": "synthetic",
        "config": {"workload": "gqa96-prefill-8x8192", "sequences": n_seq, "rows_per_sequence": chunk,
                   "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": w.d, "page_tokens": 16,
                   "copies": copies},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic("gqa96-prefill-8x8192", "quantize_append_kernel", APPEND_SOURCES),
                     "kernel": "quantize_append_kernel<128,false>", "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": round(ms * 1e3, 2),
                     "mfma_tflops_algorithmic": round(flops / (ms * 1e-3) / 1e12, 2)},
    }
    if cpu:
        result["cpu_baseline"] = _cpu_append_baseline(k, v, row_seq, row_pos, bt, rt, w, n_rows, log)
    del sets, base
    torch.cuda.empty_cache()
    return result


EXTEND_METRIC = "chunked-prefill attention new rows/s + MFMA TFLOP/s (% of dense bf16 peak), Qwen3-8B layer"
MFMA_PEAK_TFLOPS = 2500.0


def extend_flops(cache_lens, n_new, n_q_heads: int, d: int) -> int:
    """Algorithmic flops of one extend call: per new row i of a sequence with
    P cached tokens, per query head, 2 d multiply-adds for each of the
    P + i + 1 keys it attends (q k and p v)."""
    tot = 0
    for P, n in zip(cache_lens, n_new):
        P, n = int(P), int(n)
        tot += n * P + n * (n + 1) // 2
    return 4 * d * n_q_heads * tot


def extend_line(args, log, cpu: bool) -> dict:
    """Chunked prefill ("extend") over the mixed INT2 cache: the 28-sequence
    Qwen3-8B batch (ragged cached contexts, a 1024-token prefix shared by all)
    each extended by a chunk of 512 new rows, causal.  Launches rotate over
    cache copies totalling >= 1 GiB; HIP events on the launch stream."""
    import torch
    from int2_rotated_kv_oscar_amd import lib, synth
    dev = "cuda:0"
    w = synth.WORKLOADS["qwen3-8b-b28-ragged"]
    n_new = 512
    t0 = time.time()
    inp = synth.decode_inputs(w)
    B = len(inp.seq_lens)
    cu = np.arange(B + 1, dtype=np.int32) * n_new
    rng = synth.rng_for(w.cfg_id, 100)
    kn, vn = synth.kv_rows(rng, B * n_new, w)
    qn = synth.q_rows(rng, B * n_new, w, synth.query_mixers(w))
    cal = synth.calibration_set(w, n_rows=1024)
    rt = lib.build_rotation(cal.q, cal.k, cal.v, w.group_q)
    log(f"extend inputs + calibration {time.time() - t0:.1f}s")

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    r_k = torch.from_numpy(rt["r_k"].astype(np.float32)).to(dev)
    r_v = torch.from_numpy(rt["r_v"].astype(np.float32)).to(dev)
    tau_k, tau_v = float(np.float32(rt["tau_k"])), float(np.float32(rt["tau_v"]))
    int2 = torch.zeros(inp.n_int2_pages * lib.int2_page_bytes(w.d, w.n_kv_heads), dtype=torch.uint8, device=dev)
    bf16 = torch.zeros(inp.n_bf16_pages * lib.bf16_page_bytes(w.d, w.n_kv_heads) // 2, dtype=torch.int16, device=dev)
    cache = lib.make_cache(w.d, w.n_kv_heads, w.n_sink, w.n_recent, int2, bf16)
    bt_q, bt_h = i32(inp.bt_q), i32(inp.bt_h)
    ms, mp, mr = synth.middle_rows(inp)
    lib.quantize_append(cache, bf(inp.k_rows[mr]), bf(inp.v_rows[mr]), i32(ms), i32(mp), bt_q, r_k, r_v, tau_k, tau_v)
    hs, hp, hr = synth.bf16_rows(inp)
    lib.write_bf16(cache, bf(inp.k_rows[hr]), bf(inp.v_rows[hr]), i32(hs), i32(hp), bt_h)
    torch.cuda.synchronize()
    footprint = int2.numel() + bf16.numel() * 2
    copies = max(1, int(np.ceil((1 << 30) / footprint)))
    pools = [(int2, bf16)] + [(int2.clone(), bf16.clone()) for _ in range(copies - 1)]
    caches = [lib.make_cache(w.d, w.n_kv_heads, w.n_sink, w.n_recent, a, b) for a, b in pools]
    q, k_new, v_new = bf(qn), bf(kn), bf(vn)
    cu_d, lens_d = i32(cu), i32(inp.seq_lens)
    max_cache = int(inp.seq_lens.max())
    wsb = lib.extend_workspace_bytes(B, w.n_kv_heads, w.n_q_heads, w.d, w.n_sink, w.n_recent, max_cache, n_new)
    ws = torch.empty(max(1, (wsb + 3) // 4), dtype=torch.int32, device=dev)
    out = torch.empty(B * n_new, w.n_q_heads, w.d, dtype=torch.bfloat16, device=dev)

    def launch(i):
        lib.paged_extend_attn(caches[i % copies], 2, q, k_new, v_new, cu_d, lens_d, max_cache, n_new, bt_q, bt_h,
                              r_k, r_v, out, ws)

    for i in range(max(2, args.warmup)):
        launch(i)
    torch.cuda.synchronize()
    K = max(5, args.steps // 4)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        launch(i)
    e1.record()
    torch.cuda.synchronize()
    ms_call = e0.elapsed_time(e1) / K
    flops = extend_flops(inp.seq_lens, np.full(B, n_new), w.n_q_heads, w.d)
    tflops = flops / (ms_call * 1e-3) / 1e12
    rows = B * n_new
    log(f"extend {ms_call * 1e3:.1f} us per call, {tflops:.1f} TFLOP/s, {rows / (ms_call * 1e-3):.3g} rows/s "
        f"(workspace {wsb / 1e6:.1f} MB, {copies} cache copies)")
    res = {
        "metric": EXTEND_METRIC, "value": round(rows / (ms_call * 1e-3), 1), "unit": "new rows/s",
        "ms_per_call": round(ms_call, 5), "dtype": "int2 codes -> f16 tiles, bf16 raw rows, f32 accumulate",
        "config": {"workload": "qwen3-8b-b28-extend512", "batch": B, "cached_context": "U[4096, 32768], 1024 shared",
                   "new_rows_per_sequence": n_new, "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads,
                   "head_dim": w.d, "cache_copies": copies},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "attend_kernel<128,2,8,2,0>", "algorithmic_flops_per_launch": flops,
                     "avg_launch_us": round(ms_call * 1e3, 2)},
    }
    if cpu:
        from oracle import attention as oatt
        from oracle import layout as olayout
        lim, threads = blas_threads(len(os.sched_getaffinity(0)))
        pool = olayout.Int2Pool(inp.n_int2_pages, w.n_kv_heads, w.d, int2.cpu().numpy())
        bfp = olayout.Bf16Pool(inp.n_bf16_pages, w.n_kv_heads, w.d, bf16.cpu().numpy().view(np.uint16))
        f = lambda x: synth.bf16_bits_to_f32(x).astype(np.float64)  # noqa: E731
        n, dt = 4, 0.0
        while dt < 8.0 and n <= n_new:  # rows 0 .. n-1 of sequence 0, growing until ~10 s
            t0 = time.time()
            oatt.extend_attention(f(qn[:n]), f(kn[:n]), f(vn[:n]), pool, bfp, [0, n], inp.seq_lens[:1], inp.bt_q[:1],
                                  inp.bt_h[:1], rt["r_k"].astype(np.float32), rt["r_v"].astype(np.float32),
                                  w.n_sink, w.n_recent)
            dt = time.time() - t0
            n *= 2
        lim.restore_original_limits()
        res["cpu_baseline"] = {"value": round((n // 2) / dt, 1), "unit": "new rows/s", "cores": threads, "kind": "oracle",
                               "sample": f"oracle float64 extend of the first {n // 2} new rows of sequence 0 "
                                         f"({int(inp.seq_lens[0])} cached tokens); BLAS threads {threads}"}
    del pools, caches
    torch.cuda.empty_cache()
    return res


INT4_METRIC = "INT4 paged decode-attn KV-tokens/s + achieved HBM GB/s (% of peak)"


def int4_decode_line(args, log, w, cpu: bool) -> dict:
    """The INT4-cache decode on the decode workload's shape: the middle history
    quantized to 16 levels in INT4 pages, the same BF16 sink/recent pages.
    Launches rotate over >= 1 GiB of cache copies; HIP events on the stream."""
    import torch
    from int2_rotated_kv_oscar_amd import lib, synth
    dev = "cuda:0"
    inp = synth.decode_inputs(w)
    cal = synth.calibration_set(w, n_rows=1024)
    rt = lib.build_rotation(cal.q, cal.k, cal.v, w.group_q)

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)

    r_k = torch.from_numpy(rt["r_k"].astype(np.float32)).to(dev)
    r_v = torch.from_numpy(rt["r_v"].astype(np.float32)).to(dev)
    tau_k, tau_v = float(np.float32(rt["tau_k"])), float(np.float32(rt["tau_v"]))
    q4 = torch.zeros(inp.n_int2_pages * lib.int4_page_bytes(w.d, w.n_kv_heads), dtype=torch.uint8, device=dev)
    bf16 = torch.zeros(inp.n_bf16_pages * lib.bf16_page_bytes(w.d, w.n_kv_heads) // 2, dtype=torch.int16, device=dev)
    cache = lib.make_cache(w.d, w.n_kv_heads, w.n_sink, w.n_recent, q4, bf16, code_bits=4)
    bt_q, bt_h = i32(inp.bt_q), i32(inp.bt_h)
    ms, mp, mr = synth.middle_rows(inp)
    lib.quantize_append_int4(cache, bf(inp.k_rows[mr]), bf(inp.v_rows[mr]), i32(ms), i32(mp), bt_q, r_k, r_v, tau_k,
                             tau_v)
    hs, hp, hr = synth.bf16_rows(inp)
    lib.write_bf16(cache, bf(inp.k_rows[hr]), bf(inp.v_rows[hr]), i32(hs), i32(hp), bt_h)
    torch.cuda.synchronize()
    footprint = q4.numel() + bf16.numel() * 2 + r_k.numel() * 8
    copies = max(1, int(np.ceil((1 << 30) / footprint)))
    pools = [(q4, bf16, r_k, r_v)] + [(q4.clone(), bf16.clone(), r_k.clone(), r_v.clone()) for _ in range(copies - 1)]
    caches = [lib.make_cache(w.d, w.n_kv_heads, w.n_sink, w.n_recent, a, b, code_bits=4) for a, b, _, _ in pools]
    q = bf(inp.q)
    B = len(inp.seq_lens)
    seq_lens = i32(inp.seq_lens)
    wsb = lib.decode_int4_workspace_bytes(B, w.n_kv_heads, w.n_q_heads, w.d, w.n_sink, w.n_recent, inp.max_seq_len)
    ws = torch.empty(max(1, (wsb + 3) // 4), dtype=torch.int32, device=dev)
    out = torch.empty(B, w.n_q_heads, w.d, dtype=torch.bfloat16, device=dev)

    def launch(i):
        _, _, rk, rv = pools[i % copies]
        lib.paged_decode_attn_int4(caches[i % copies], q, seq_lens, inp.max_seq_len, bt_q, bt_h, rk, rv, out, ws)

    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        launch(i)
    e1.record()
    torch.cuda.synchronize()
    ms_call = e0.elapsed_time(e1) / K
    d, hkv = w.d, w.n_kv_heads
    per_mid = 2 * (d // 2) + 2 * 2 * (d // 32) * 2  # INT4: 2 x d/2 B codes + 2 x 2 n_g x 2 B scale/zero
    mid = raw = pages = 0
    for b, L in enumerate(inp.seq_lens):
        sink, m, rec = synth.regions(int(L), w.n_sink, w.n_recent)
        lo = m[0] if (b == 0 or not w.shared_prefix) else max(m[0], w.shared_prefix)
        mid += max(0, m[1] - lo)
        raw += (sink[1] - sink[0]) + (rec[1] - rec[0]) if (b == 0 or not w.shared_prefix) else (rec[1] - rec[0])
        pages += (int(L) + 15) // 16
    nbytes = (mid * per_mid * hkv + raw * 4 * d * hkv + 2 * d * d * 4 * hkv + 2 * B * w.n_q_heads * d * 2 + pages * 4)
    gbs = nbytes / (ms_call * 1e-3) / 1e9
    tokens = int(inp.seq_lens.sum())
    log(f"int4 decode {ms_call * 1e3:.1f} us per call, {gbs:.0f} GB/s algorithmic")
    res = {
        "metric": INT4_METRIC, "value": round(tokens / (ms_call * 1e-3), 1), "unit": "KV-tokens/s",
        "ms_per_call": round(ms_call, 5), "dtype": "int4 codes -> f16 tiles, f32 accumulate",
        "config": {"workload": w.name + "-int4", "batch": B, "context": inp.max_seq_len, "q_heads": w.n_q_heads,
                   "kv_heads": hkv, "head_dim": d, "cache_copies": copies},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": f"attend_kernel<{d},4,4,1,1> + attend_merge_kernel<{d},16,1>",
                     "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": round(ms_call * 1e3, 2), "note": "avg_launch_us: one call (both launches)"},
    }
    if cpu:
        from oracle import attention as oatt
        from oracle import layout as olayout
        lim, threads = blas_threads(len(os.sched_getaffinity(0)))
        pool = olayout.Int4Pool(inp.n_int2_pages, hkv, d, q4.cpu().numpy())
        bfp = olayout.Bf16Pool(inp.n_bf16_pages, hkv, d, bf16.cpu().numpy().view(np.uint16))
        t0 = time.time()
        oatt.decode_attention(synth.bf16_bits_to_f32(inp.q).astype(np.float64), pool, bfp, inp.seq_lens, inp.bt_q,
                              inp.bt_h, rt["r_k"].astype(np.float32), rt["r_v"].astype(np.float32), w.n_sink,
                              w.n_recent)
        dt = time.time() - t0
        lim.restore_original_limits()
        res["cpu_baseline"] = {"value": round(tokens / dt, 1), "unit": "KV-tokens/s", "cores": threads, "kind": "oracle",
                               "sample": f"oracle float64 decode of the whole INT4 cache ({tokens} tokens); "
                                         f"BLAS threads {threads}"}
    del pools, caches
    torch.cuda.empty_cache()
    return res


GRAM_METRIC = "calibration Gram pooled rows/s + achieved HBM GB/s (% of peak), Qwen3-8B calibration"


def run_calib_gram(args, log) -> int:
    """oscar_calib_gram on the Qwen3-8B calibration set (8192 rows x 32 query
    heads, d = 128, pooled over 8 KV groups of 4): bytes = the bf16 rows read
    + the float64 targets written; inputs rotate over copies totalling >= 1 GiB."""
    import torch
    from int2_rotated_kv_oscar_amd import lib, synth
    dev = "cuda:0"
    w = synth.WORKLOADS["qwen3-8b-b1-32k"]
    cal = synth.calibration_set(w)
    q_bits = synth.to_bf16_bits(cal.q)
    n, hx, d = q_bits.shape
    x0 = torch.from_numpy(np.ascontiguousarray(q_bits).view(np.int16)).to(dev).view(torch.bfloat16)
    copies = args.copies or max(1, int(np.ceil((1 << 30) / q_bits.nbytes)))
    xs = [x0] + [x0.clone() for _ in range(copies - 1)]
    outs = [torch.empty((w.n_kv_heads, d, d), dtype=torch.float64, device=dev) for _ in range(copies)]
    for i in range(args.warmup):
        lib.calib_gram(xs[i % copies], w.n_kv_heads, outs[i % copies])
    torch.cuda.synchronize()
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(K):
        lib.calib_gram(xs[i % copies], w.n_kv_heads, outs[i % copies])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K
    nbytes = q_bits.nbytes + w.n_kv_heads * d * d * 8
    flops = 2 * n * hx * d * d
    achieved = nbytes / (ms * 1e-3) / 1e9
    log(f"calib_gram {ms * 1e3:.1f} us, {achieved:.0f} GB/s, {flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
    result = {
        "metric": GRAM_METRIC, "value": round(n * hx / (ms * 1e-3), 1), "unit": "pooled rows/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 in, bf16 MFMA, f32 blocks, f64 sums", "data": "synthetic",
        "config": {"workload": "qwen3-8b-calibration", "rows": n, "q_heads": hx, "kv_heads": w.n_kv_heads,
                   "head_dim": d, "copies": copies},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "calib_gram_kernel<128>", "algorithmic_bytes_per_launch": nbytes,
                     "avg_launch_us": round(ms * 1e3, 2),
                     "mfma_tflops_algorithmic": round(flops / (ms * 1e-3) / 1e12, 2)},
    }
    if not args.no_cpu_baseline:
        from oracle import rotation as orot
        lim, threads = blas_threads(len(os.sched_getaffinity(0)))
        q64 = cal.q.astype(np.float64)
        t0 = time.time()
        heads = 0
        for h in range(w.n_kv_heads):  # the oracle's Q target, head by head, for about 10 s at most
            orot.calibration_targets(q64[:, 4 * h:4 * h + 4], cal.k[:, h:h + 1].astype(np.float64),
                                     cal.v[:, h:h + 1].astype(np.float64), 4, oc=q64[:, 4 * h:4 * h + 4])
            heads += 1
            if time.time() - t0 > 10.0:
                break
        dt = (time.time() - t0) / 2  # each call forms the Q and the O target
        lim.restore_original_limits()
        result["cpu_baseline"] = {"value": round(n * 4 * heads / dt, 1), "unit": "pooled rows/s", "cores": threads,
                                  "kind": "oracle",
                                  "sample": f"oracle float64 targets of {heads}/{w.n_kv_heads} KV heads "
                                            f"(BLAS pool measured at {threads} threads)"}
    print(json.dumps(result), flush=True)
    return 0


def _cpu_append_baseline(k, v, row_seq, row_pos, bt, rt, w, n_rows, log) -> dict:
    """The oracle (float64 NumPy) quantizing a bounded sample of the same rows."""
    from oracle import cache as ocache
    from oracle import layout as olayout
    cores = len(os.sched_getaffinity(0))
    lim, threads = blas_threads(cores)
    rk = rt["r_k"].astype(np.float32).astype(np.float64)
    rv = rt["r_v"].astype(np.float32).astype(np.float64)
    n_pages = bt.size
    done, dt, n = 0, 0.0, 256
    while dt < 10.0 and done < n_rows:
        sel = slice(done, min(n_rows, done + n))
        pool = olayout.Int2Pool(n_pages, w.n_kv_heads, w.d)
        t0 = time.time()
        ocache.quantize_append(pool, k[sel], v[sel], row_seq[sel], row_pos[sel], bt, rk, rv,
                               float(np.float32(rt["tau_k"])), float(np.float32(rt["tau_v"])), olayout.bf16_to_f64)
        dt += time.time() - t0
        done = sel.stop
        n *= 2
    lim.restore_original_limits()
    log(f"cpu oracle: {done} rows in {dt:.1f}s, BLAS threads {threads}")
    return {"value": round(done / dt, 1), "unit": "rows/s", "cores": threads, "kind": "oracle",
            "sample": f"oracle float64 quantize-append of the first {done} of the {n_rows} rows "
                      f"(all {w.n_kv_heads} KV heads, K and V); BLAS pool limited to {cores} and measured at "
                      f"{threads} threads"}


def _all_bf16_tables(inp):
    B, mp = inp.bt_h.shape
    bt = np.full((B, mp), -1, np.int32)
    n = 0
    for b, L in enumerate(inp.seq_lens):
        k = (int(L) + 15) // 16
        bt[b, :k] = np.arange(n, n + k)
        n += k
    return bt, inp.n_int2_pages, max(n, 1), mp


def _cpu_baseline(inp, w, cache, int2, bf16, rt, tokens, log, cores: int, budget_s: float) -> dict:
    """The oracle (float64 NumPy) decoding the same cache on `cores` host
    threads (the BLAS pool limited to them), for about budget_s seconds."""
    from oracle import attention as oatt
    from oracle import layout as olayout
    from int2_rotated_kv_oscar_amd import lib, synth
    lim, threads = blas_threads(cores)
    pool_q = olayout.Int2Pool(inp.n_int2_pages, w.n_kv_heads, w.d, int2.cpu().numpy())
    pool_h = olayout.Bf16Pool(bf16.numel() * 2 // lib.bf16_page_bytes(w.d, w.n_kv_heads), w.n_kv_heads, w.d,
                              bf16.cpu().numpy().view(np.uint16))
    q = synth.bf16_bits_to_f32(inp.q).astype(np.float64)
    rk = rt["r_k"].astype(np.float32).astype(np.float64)
    rv = rt["r_v"].astype(np.float32).astype(np.float64)
    # bounded sample: as many KV heads of the full-length batch as fit ~10 s
    heads = []
    t0 = time.time()
    for h in range(w.n_kv_heads):
        one_q = olayout.Int2Pool(inp.n_int2_pages, 1, w.d, pool_q.data[:, h:h + 1])
        one_h = olayout.Bf16Pool(pool_h.n_pages, 1, w.d, pool_h.data[:, h:h + 1])
        G = w.group_q
        oatt.decode_attention(q[:, h * G:(h + 1) * G], one_q, one_h, inp.seq_lens, inp.bt_q, inp.bt_h,
                              rk[h:h + 1], rv[h:h + 1], w.n_sink, w.n_recent)
        heads.append(h)
        if time.time() - t0 > budget_s:
            break
    dt = time.time() - t0
    lim.restore_original_limits()
    per_layer = dt * w.n_kv_heads / len(heads)
    log(f"cpu oracle: {len(heads)} KV heads in {dt:.1f}s, BLAS threads {threads}")
    return {"value": round(tokens / per_layer, 1), "unit": "KV-tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"oracle float64 decode of {len(heads)}/{w.n_kv_heads} KV heads of the same cache "
                      f"({tokens} tokens), time scaled to all heads; BLAS pool limited to {cores} and measured at "
                      f"{threads} threads"}


if __name__ == "__main__":
    sys.exit(main())
