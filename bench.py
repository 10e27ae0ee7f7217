#!/usr/bin/env python
"""MLA decode benchmark on one MI355X.

One step = one mla_decode call (query projections, absorption, paged-cache
attention with split-KV merge, W_UV and W_O) for a batch of 64 sequences of
the DeepSeek-V2 layer (d=5120, n_h=128, d_h=128, d_c=512, d_c'=1536, d_R=64),
context lengths uniform on [1024, 8192], 64-token pages in shuffled order,
bf16 weights/cache with fp32 accumulation, query positions equal to each
sequence's length (kv_len = L + 1).  The weights are packed once, before
timing, into the tiled layout the decode GEMMs stream (--weights rows keeps
them row-major; --weights merged runs mla_decode_merged on the products
W_UK,i^T W_UQ,i and W_O,i W_UV,i computed once before timing, tiled).  Inputs are seeded synthetic data resident in HBM; two
full buffer sets (weights + cache) alternate between steps so that the 256 MB
last-level cache cannot serve a step from the previous one.

Prints one JSON line (see the keys below).  --gpus N with N > 1 exits: this
build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MLA decode tokens/s + latent-cache HBM GB/s & MFMA% (n_h=128, d_c=512)"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
BYTES_PER_TOKEN = 1152          # one cached row: (512 + 64) bf16
FLOP_PER_TOKEN = 2 * 128 * 576 + 2 * 128 * 512   # scores + latent accumulation per head


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


WORKLOADS = {
    # name: (batch, lo, hi, config id)
    "batch64": (64, 1024, 8192, 3),
    "batch1": (1, 4096, 4096, 2),
    "long4": (4, 131072, 131072, 4),
}


def build_set(s, B, lo, hi, cid, sub, device, inputs, lib, cfg, weights):
    import numpy as np
    import torch
    L = inputs.make_lengths(B, lo, hi, cid)
    kv = (L + 1).astype(np.int32)
    paged = inputs.make_paged(kv, 64, cid + 100 * sub, shuffle=True)
    offs = np.concatenate([[0], np.cumsum(kv)[:-1]]).astype(np.int64)
    rows = inputs.make_cache_rows(int(kv.sum()), s, cid, "bf16", sub=sub)
    cache = device.bits_tensor(inputs.scatter_rows(rows.bits, paged, offs, fill=0))
    del rows
    W = inputs.make_weights(s, cid + 100 * sub, "bf16")
    Wd = device.weights(W)
    del W
    wbytes = sum(t.numel() * t.element_size() for t in Wd.values())
    wts, packed, merged = lib.make_weights(Wd), None, None
    if weights != "rows":
        # one-time layout change at load; the row-major copies are dropped
        packed = device.workspace(lib.packed_weights_size(cfg))
        rows = wts
        wts = lib.pack_weights(cfg, rows, packed)
        if weights == "merged":
            Mq = torch.empty(s.n_h * s.d_c, s.d_cq, dtype=torch.bfloat16, device="cuda")
            Mo = torch.empty(s.d, s.n_h * s.d_c, dtype=torch.bfloat16, device="cuda")
            lib.merge_weights(cfg, rows, lib.LAYOUT_TILES, Mq, Mo)
            merged = dict(Mq=Mq, Mo=Mo, mw=lib.MergedWeights(wts.W_DQ, wts.W_QR, Mq.data_ptr(),
                                                             Mo.data_ptr(), lib.LAYOUT_TILES))
            wbytes = (Wd["W_DQ"].numel() + Wd["W_QR"].numel() + Mq.numel() + Mo.numel()) * 2
        torch.cuda.synchronize()
        Wd = None
    Hq = inputs.make_hidden(B, s, cid, "bf16", sub=sub)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()  # noqa: E731
    return dict(L=L, kv=kv, paged=paged, cache=cache, Wd=Wd, wts=wts, packed=packed, wbytes=wbytes,
                merged=merged,
                h=device.tensor(Hq), pos=i32(L), kv_d=i32(kv), pt=i32(paged.page_table),
                Hq=Hq, offs=offs)


def host_info():
    """CPU model, the BLAS library numpy calls and its thread count."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas, threads = "unknown", 1
    try:
        import threadpoolctl
        info = [i for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if info:
            blas = f"{info[0].get('internal_api')} {info[0].get('version')}"
            threads = max(int(i.get("num_threads", 1)) for i in info)
    except Exception:  # noqa: BLE001
        pass
    return model, blas, threads


def cpu_baseline(s, st, budget_s, cid):
    """The fp64 oracle on a bounded sample of the same workload: whole
    sequences until the time budget is spent, first in order A (the
    reference: keys and values decompressed per head), then in order B (the
    same algorithm as the GPU path: absorbed query, latent attention, one
    decompression) on the same sequences."""
    import numpy as np

    import oracle
    from mla_latent_kv_15_amd import inputs
    model, blas, threads = host_info()
    W64 = {k: v.f64() for k, v in inputs.make_weights(s, cid, "bf16").items()}
    sc = oracle.default_scale(s.d_h, s.d_r)
    H64 = st["Hq"].f64()

    def one(b, order):
        n = int(st["kv"][b])
        rows = inputs.make_cache_rows(n, s, 9000 + b, "bf16").f64()
        q_c, q_r = oracle.query(H64[b], W64["W_DQ"], W64["W_UQ"], W64["W_QR"], int(st["L"][b]),
                                s.n_h, 10000.0)
        fn = oracle.attend_order_a if order == "A" else oracle.attend_order_b
        t0 = time.perf_counter()
        o = fn(q_c, q_r, rows[:, :s.d_c], rows[:, s.d_c:], W64["W_UK"], W64["W_UV"], sc)
        oracle.integrate(o, W64["W_O"])
        return time.perf_counter() - t0, n

    spent, done, toks = 0.0, 0, 0
    for b in range(len(st["L"])):
        dt, n = one(b, "A")
        spent += dt
        done += 1
        toks += n
        if spent > budget_s:
            break
    spent_b = sum(one(b, "B")[0] for b in range(done))
    return {"value": done / spent, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "blas": blas,
            "sample": f"order-A fp64 decode (query projections, per-head decompressed "
                      f"attention, W_O) of the first {done} of the batch's sequences "
                      f"({toks} cached rows) in {spent:.1f} s; each sequence yields one token; "
                      f"the time to generate the synthetic rows is not counted",
            "order_b": {"value": done / spent_b, "unit": "tokens/s",
                        "sample": f"order-B fp64 decode of the same {done} sequences in "
                                  f"{spent_b:.2f} s"}}


TRAFFIC_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                            "attn_v2_traffic_batch64.txt")


def sclk_files():
    """The GPU's shader-clock level files (the kernel driver lists the
    levels, the current one marked with '*')."""
    import glob
    return sorted(f for f in glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk")
                  if os.access(f, os.R_OK))


def read_sclk(path):
    """The marked (current) level of a pp_dpm_sclk file, in MHz, or None."""
    try:
        with open(path) as f:
            for line in f:
                if "*" in line:
                    return float(line.split(":")[1].strip().lower().split("mhz")[0])
    except (OSError, ValueError, IndexError):
        return None
    return None


def read_power_w(card_dir):
    """The board power the driver reports (hwmon power1_average, else
    power1_input, microwatts) in watts, or None."""
    import glob
    for name in ("power1_average", "power1_input"):
        for f in sorted(glob.glob(os.path.join(card_dir, "hwmon", "hwmon*", name))):
            try:
                with open(f) as fh:
                    return float(fh.read().strip()) * 1e-6
            except (OSError, ValueError):
                continue
    return None


def sample_clock(run_steps, n_steps, what="decode steps", period_s=0.002):
    """Median, min and max shader clock (and board power where readable)
    sampled from sysfs while n_steps calls run back to back; None where the
    driver's files are absent."""
    import threading

    import numpy as np
    import torch
    files = sclk_files()
    if not files:
        return None
    samples = {f: [] for f in files}
    power = {f: [] for f in files}
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            for f in files:
                v = read_sclk(f)
                if v is not None:
                    samples[f].append(v)
                w = read_power_w(os.path.dirname(f))
                if w is not None:
                    power[f].append(w)
            time.sleep(period_s)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    run_steps(n_steps)
    torch.cuda.synchronize()
    stop.set()
    th.join()
    # the busy card is the one whose clock moved most above its lowest level
    best = max(files, key=lambda f: (np.median(samples[f]) if samples[f] else -1.0))
    v = np.array(samples[best])
    if v.size == 0:
        return None
    pw = np.array(power[best])
    return {"sclk_mhz_median": float(np.median(v)), "sclk_mhz_min": float(v.min()),
            "sclk_mhz_max": float(v.max()), "samples": int(v.size),
            "board_power_w_median": float(np.median(pw)) if pw.size else None,
            "board_power_w_max": float(pw.max()) if pw.size else None,
            "source": f"{best} (current level) and its hwmon power, sampled every "
                      f"{period_s * 1e3:.0f} ms over {n_steps} {what} run back to back",
            "bf16_mfma_peak_at_median_tflops": BF16_PEAK_TFLOPS * float(np.median(v)) / 2400.0}


def measured_traffic(workload):
    """HBM bytes per attention launch from the committed counter summary, if
    it was taken on the current attention and planner sources and on this
    workload; otherwise None."""
    if workload != "batch64" or not os.path.exists(TRAFFIC_FILE):
        return None
    from mla_latent_kv_15_amd import profsum
    vals = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("sources_sha256") != profsum.sources_digest():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def mha_baseline(args, B, lo, hi, cid):
    """Attention only, same batch: decode over an MHA-equivalent cache (a key
    and a value per head and token, 64 KB per token) against MLA's latent
    cache (1152 B per token).  Prints one JSON line."""
    import numpy as np
    import torch

    from mla_latent_kv_15_amd import device, inputs, lib
    s = inputs.V2
    cfg = lib.make_config(s, 64, "bf16")
    lib.load()
    st = build_set(s, B, lo, hi, cid, 0, device, inputs, lib, cfg, "tiles")
    kv = st["kv"]
    max_kv = int(kv.max())
    rope = torch.empty(max_kv + 1, s.d_r // 2, 2, dtype=torch.float32, device="cuda")
    lib.rope_table_init(cfg, max_kv + 1, rope)
    q_lat = torch.empty(B, s.n_h, s.row, dtype=torch.bfloat16, device="cuda")
    ws = device.workspace(lib.workspace_size(cfg, lib.OP_DECODE_QUERY, B))
    lib.decode_query(cfg, st["wts"], st["h"], st["pos"], rope, ws, q_lat)
    # the multi-head cache: same pages, rows of 2 * n_h * d_h bf16, N(0,1)
    width = 2 * s.n_h * s.d_h
    gen = torch.Generator(device="cuda")
    gen.manual_seed(cid)
    n_pages = st["paged"].num_pages
    mha_cache = torch.randn(n_pages, 64, width, dtype=torch.bfloat16, device="cuda", generator=gen)
    q_mha = torch.randn(B, s.n_h, s.d_h, dtype=torch.bfloat16, device="cuda", generator=gen)
    ws_m = device.workspace(lib.workspace_size(cfg, lib.OP_MHA_DECODE, B, max_kv, 0))
    ws_a = device.workspace(lib.workspace_size(cfg, lib.OP_DECODE_ATTENTION, B, max_kv, 0))
    o_m = torch.empty(B, s.n_h, s.d_h, dtype=torch.bfloat16, device="cuda")
    o_a = torch.empty(B, s.n_h, s.d_c, dtype=torch.bfloat16, device="cuda")

    def run_mha():
        lib.mha_decode_attention(cfg, q_mha, mha_cache, st["pt"], st["kv_d"], max_kv, 0, ws_m, o_m)

    def run_mla():
        lib.decode_attention(cfg, q_lat, st["cache"], st["pt"], st["kv_d"], max_kv, 0, ws_a, o_a)

    res = {}
    for name, fn, n in (("mha", run_mha, max(3, args.steps // 10)), ("mla", run_mla, args.steps)):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / n
    toks = int(kv.sum())
    mha_bytes = toks * width * 2
    mla_bytes = toks * BYTES_PER_TOKEN
    out = {
        "metric": "decode attention time, MHA-equivalent cache vs MLA latent cache",
        "unit": "ms", "higher_is_better": False, "data": "synthetic", "dtype": "bf16",
        "config": {"workload": f"attention only, DeepSeek-V2 heads (128 x 128), batch {B}, "
                               f"context U[{lo},{hi}], 64-token shuffled pages",
                   "cached_tokens": toks},
        "mha": {"ms": res["mha"], "cache_bytes": mha_bytes,
                "GBps": mha_bytes / (res["mha"] * 1e-3) / 1e9,
                "kernels": "mha_decode_kernel + combine_kernel (plan included)"},
        "mla": {"ms": res["mla"], "cache_bytes": mla_bytes,
                "GBps": mla_bytes / (res["mla"] * 1e-3) / 1e9,
                "kernels": "attn_v2_kernel + combine_v2_kernel (plan included)"},
        "cache_ratio": mha_bytes / mla_bytes,
        "time_ratio": res["mha"] / res["mla"],
    }
    print(json.dumps(out), flush=True)


def backward_measure(args, T):
    """Order-A attention backward (mla_attention_backward) at the V2 head
    shape: T causal queries over T cached rows of one sequence.  Prints one
    JSON line with the algorithmic flop rate (each product counted once,
    causal pairs only; the kernels recompute the scores) against the bf16
    MFMA peak (every product runs on bf16 MFMA with fp32 sums)."""
    import numpy as np
    import torch

    from mla_latent_kv_15_amd import device, inputs, lib
    s = inputs.V2
    cfg = lib.make_config(s, 64, "bf16")
    lib.load()
    N = T
    W = device.weights(inputs.make_weights(s, 60, "bf16"))
    wts = lib.make_weights(W)
    paged = inputs.make_paged([N], 64, 60, shuffle=True)
    rows = inputs.make_cache_rows(N, s, 60, "bf16")
    cache = device.bits_tensor(inputs.scatter_rows(rows.bits, paged, np.array([0]), fill=0))
    q = torch.from_numpy(inputs.normal((T, s.n_h, s.d_h + s.d_r), 1.0, 60,
                                       inputs.STREAM_QUERY)).cuda()
    dO = torch.from_numpy(inputs.normal((T, s.n_h, s.d_h), 1.0, 60, inputs.STREAM_QUERY, 1)).cuda()
    pos = torch.arange(T, dtype=torch.int32, device="cuda")
    pt = torch.from_numpy(paged.page_table[0].astype(np.int32)).cuda()
    ws = device.workspace(lib.workspace_size(cfg, lib.OP_ATTENTION_BACKWARD, T, N, 0))
    f = lambda *shape: torch.empty(*shape, dtype=torch.float32, device="cuda")  # noqa: E731
    outs = (f(s.n_h * s.d_h, s.d_c), f(s.n_h * s.d_h, s.d_c), f(T, s.n_h, s.d_h + s.d_r),
            f(N, s.row))

    def run():
        lib.attention_backward(cfg, wts, q, pos, cache, pt, N, dO, ws, *outs)

    for _ in range(2):
        run()
    torch.cuda.synchronize()
    n = max(2, args.steps // 10)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    h, dh, dr, dc = s.n_h, s.d_h, s.d_r, s.d_c
    pairs = T * (T + 1) // 2                     # causal (query, key) pairs
    flop = 2.0 * (2 * N * h * dh * dc            # K^C, V recomputed
                  + pairs * h * (dh + dr)        # scores
                  + pairs * h * dh               # dp
                  + 2 * pairs * h * dh           # dV, dK^C
                  + pairs * h * (dh + dr)        # dq
                  + pairs * h * dr               # dk^R
                  + 2 * h * dh * dc * N          # dW_UK, dW_UV
                  + 2 * N * h * dh * dc)         # dc
    tflops = flop / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "order-A attention backward (dW_UK, dW_UV, dq, dC)",
        "unit": "ms", "value": ms, "higher_is_better": False, "data": "synthetic",
        "dtype": "bf16 (fp32 sums and outputs)",
        "config": {"workload": f"V2 heads (128 x 128, d_c 512, d_r 64), {T} causal queries over "
                               f"{N} cached rows"},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": tflops / 2500.0, "flop": flop},
    }), flush=True)


def prefill_measure(args, T):
    """Append and causal prefill (mla_append_kv, mla_prefill) of one sequence
    of T tokens at the V2 shape, positions 0..T-1, 64-token shuffled pages,
    tiled weights.  Prints one JSON line: the prefill time and its algorithmic
    flop rate against the bf16 MFMA peak (every product and the attention run
    on bf16 MFMA)."""
    import numpy as np
    import torch

    from mla_latent_kv_15_amd import device, inputs, lib
    s = inputs.V2
    cfg = lib.make_config(s, 64, "bf16")
    lib.load()
    W = device.weights(inputs.make_weights(s, 5, "bf16"))
    rows = lib.make_weights(W)
    packed = device.workspace(lib.packed_weights_size(cfg))
    wts = lib.pack_weights(cfg, rows, packed)
    torch.cuda.synchronize()
    del W, rows
    h = device.tensor(inputs.make_hidden(T, s, 5, "bf16"))
    paged = inputs.make_paged([T], 64, 5, shuffle=True)
    cache = torch.zeros(paged.num_pages, 64, s.row, dtype=torch.bfloat16, device="cuda")
    rope = torch.empty(T + 1, s.d_r // 2, 2, dtype=torch.float32, device="cuda")
    lib.rope_table_init(cfg, T + 1, rope)
    pos = torch.arange(T, dtype=torch.int32, device="cuda")
    slots = torch.from_numpy(paged.slots(0).astype(np.int32)).cuda()
    pt = torch.from_numpy(paged.page_table[0].astype(np.int32)).cuda()
    wsa = device.workspace(lib.workspace_size(cfg, lib.OP_APPEND, T))
    ws = device.workspace(lib.workspace_size(cfg, lib.OP_PREFILL, T, T))
    out = torch.empty(T, s.d, dtype=torch.bfloat16, device="cuda")

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    n = max(2, args.steps // 10)
    append_ms = timed(lambda: lib.append_kv(cfg, wts, h, pos, slots, rope, cache, wsa), n)
    ms = timed(lambda: lib.prefill(cfg, wts, h, pos, cache, pt, T, rope, ws, out), n)
    d, hh, dh, dr, dc, dq = s.d, s.n_h, s.d_h, s.d_r, s.d_c, s.d_cq
    pairs = T * (T + 1) // 2                      # causal (query, key) pairs
    flop = 2.0 * (T * d * dq + T * dq * hh * (dh + dr)      # c^Q, q^C and q^R
                  + 2 * T * dc * hh * dh                     # K^C and V of the T rows
                  + pairs * hh * (dh + dr) + pairs * hh * dh  # scores, P V
                  + T * hh * dh * d)                         # W_O
    tflops = flop / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "causal prefill (mla_prefill, order A)", "unit": "ms", "value": ms,
        "higher_is_better": False, "data": "synthetic", "dtype": "bf16",
        "append_ms": append_ms,
        "config": {"workload": f"DeepSeek-V2 layer, one sequence of {T} tokens, positions "
                               f"0..{T - 1}, 64-token shuffled pages, weights tiled"},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": tflops / 2500.0, "flop": flop},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="batch64", choices=sorted(WORKLOADS))
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--sets", type=int, default=2)
    ap.add_argument("--weights", default="tiles", choices=("tiles", "rows", "merged"),
                    help="weight layout (default: packed into tiles before timing); merged: "
                         "decode from the offline products W_UK^T W_UQ and W_O W_UV")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--baseline", choices=("mha",), default=None,
                    help="instead of the step: time decode attention over an MHA-equivalent "
                         "cache against MLA's on the same batch and exit")
    ap.add_argument("--prefill", type=int, default=0, metavar="T",
                    help="time append + causal prefill of one T-token sequence instead")
    ap.add_argument("--backward", type=int, default=0, metavar="T",
                    help="instead of the step: time the order-A attention backward for T "
                         "queries over T cached rows and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 5 device-to-device copies of MIB MiB (a known-size "
                         "reference for the HBM byte counters) and exit")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; multi-GPU sharding is described "
              "in DESIGN.md but not built (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from mla_latent_kv_15_amd import device, inputs, lib

    torch.cuda.set_device(0)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n}), flush=True)
        return
    lib.load()
    s = inputs.V2
    B, lo, hi, cid = WORKLOADS[args.workload]
    if args.baseline == "mha":
        mha_baseline(args, B, lo, hi, cid)
        return
    if args.backward:
        backward_measure(args, args.backward)
        return
    if args.prefill:
        prefill_measure(args, args.prefill)
        return
    cfg = lib.make_config(s, 64, "bf16")
    log(f"building {args.sets} buffer set(s) for workload {args.workload}")
    sets = [build_set(s, B, lo, hi, cid, k, device, inputs, lib, cfg, args.weights)
            for k in range(args.sets)]
    st0 = sets[0]
    max_kv = int(max(int(st["kv"].max()) for st in sets))
    rope = torch.empty(max_kv + 1, s.d_r // 2, 2, dtype=torch.float32, device="cuda")
    lib.rope_table_init(cfg, max_kv + 1, rope)
    op = lib.OP_DECODE_MERGED if args.weights == "merged" else lib.OP_DECODE
    ws = device.workspace(lib.workspace_size(cfg, op, B, max_kv, args.splits))
    outs = [torch.empty(B, s.d, dtype=torch.bfloat16, device="cuda") for _ in sets]

    def step(i):
        st = sets[i % len(sets)]
        if args.weights == "merged":
            lib.decode_merged(cfg, st["merged"]["mw"], st["h"], st["pos"], st["cache"], st["pt"],
                              st["kv_d"], max_kv, rope, args.splits, ws, outs[i % len(sets)])
        else:
            lib.decode(cfg, st["wts"], st["h"], st["pos"], st["cache"], st["pt"], st["kv_d"],
                       max_kv, rope, args.splits, ws, outs[i % len(sets)])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log("timing")
    # 1) the timed region: K steps back to back, nothing else on the stream
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(args.steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms_step = total_ms / args.steps
    # 2) the same K steps with an event between consecutive steps: the
    # distribution of per-step times
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(args.steps):
        step(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])
    # 3) the same K steps with the library's events around the attention
    # kernel and its merge, on the stream they are launched on
    lib.profile_enable(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    attn_ms, attn_merge_ms, launches = lib.profile_read()
    lib.profile_enable(False)
    # 4) the shader clock while steps run (the peaks above assume 2.4 GHz)
    def run_steps(n):
        for i in range(n):
            step(i)
    clock = sample_clock(run_steps, max(1000, args.steps))
    # the same while only the cache stream runs (mla_decode_attention: query
    # tiles, plan, attention kernel, merge) on a random absorbed query
    qa = (torch.randn(B, s.n_h, s.row, device="cuda") * 0.05).to(torch.bfloat16)
    ws_a = device.workspace(lib.workspace_size(cfg, lib.OP_DECODE_ATTENTION, B, max_kv,
                                               args.splits))
    lat = torch.empty(B, s.n_h, s.d_c, dtype=torch.bfloat16, device="cuda")

    def run_attention(n):
        for i in range(n):
            st = sets[i % len(sets)]
            lib.decode_attention(cfg, qa, st["cache"], st["pt"], st["kv_d"], max_kv, args.splits,
                                 ws_a, lat)
    clock_attention = sample_clock(run_attention, max(2000, args.steps),
                                   "mla_decode_attention calls")
    attn_avg = attn_ms / max(launches, 1)
    am_avg = attn_merge_ms / max(launches, 1)
    # per-launch algorithmic work: the cached rows of the step's batch (sets alternate)
    toks = [int(st["kv"].sum()) for st in sets]
    toks_avg = sum(toks[i % len(sets)] for i in range(args.steps)) / args.steps
    cache_bytes = toks_avg * BYTES_PER_TOKEN
    achieved = cache_bytes / (am_avg * 1e-3) / 1e9
    achieved_k = cache_bytes / (attn_avg * 1e-3) / 1e9
    mfma_tflops = toks_avg * FLOP_PER_TOKEN / (attn_avg * 1e-3) / 1e12
    weight_bytes = st0["wbytes"]
    step_bytes = cache_bytes + weight_bytes

    res = {
        "metric": METRIC,
        "value": B / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{'mla_decode_merged' if args.weights == 'merged' else 'mla_decode'}, "
                        f"DeepSeek-V2 layer, batch {B}, context U[{lo},{hi}], "
                        f"64-token shuffled pages, kv_len = L + 1",
            "batch": B, "context_lo": lo, "context_hi": hi, "page_size": 64,
            "d": s.d, "n_h": s.n_h, "d_h": s.d_h, "d_c": s.d_c, "d_cq": s.d_cq, "d_r": s.d_r,
            "num_splits": args.splits, "buffer_sets": len(sets), "weights": args.weights,
        },
        "ms_per_step_median": float(np.median(per)),
        "ms_per_step_p10": float(np.percentile(per, 10)),
        "ms_per_step_p90": float(np.percentile(per, 90)),
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": measured_traffic(args.workload),
            "kernel": "attn_v2_kernel + combine_v2_kernel (paged latent-cache attention and "
                      "the merge of its split partials)",
            "launch_ms": am_avg,
            "bytes_per_launch": cache_bytes,
            "kernel_only": {"kernel": "attn_v2_kernel", "launch_ms": attn_avg,
                            "achieved": achieved_k, "frac": achieved_k / HBM_PEAK_GBPS},
        },
        "attention_mfma_tflops": mfma_tflops,
        "attention_mfma_frac": mfma_tflops / BF16_PEAK_TFLOPS,
        "clock": clock,
        "clock_attention": clock_attention,
        "step_hbm_GBps": step_bytes / (ms_step * 1e-3) / 1e9,
        "step_bytes": step_bytes,
    }
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(s, st0, args.cpu_seconds, cid)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
