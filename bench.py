"""Benchmark of the MI355X FlashAttention forward (one GPU).

One step = the prefill workload B=4, H=32, N=4096, d=128, bf16 Q/K/V drawn
i.i.d. N(0,1), scale 1/sqrt(128), run once non-causal and once causal (one
launch each).  `value` is algorithmic TFLOP/s over the step: 4*B*H*N^2*d
FLOPs non-causal plus half of that causal, divided by the measured time,
with inputs resident in device memory before the timed region.

Printed as ONE JSON line, which also carries
  * roofline: the dominant kernel (non-causal prefill), its algorithmic
    FLOPs per launch over its average launch time (HIP events on its stream)
    against the dense bf16 MFMA peak, and the HBM traffic per launch taken
    from committed rocprofv3 counter runs when they match the current kernel
    source (null otherwise);
  * cpu_baseline: the fp64 CPU oracle timed on a bounded sample of the same
    workload on this host's cores;
  * other_workloads: the long causal fp16 sequence, the backward pass at the
    prefill configuration (algorithmic FLOPs of its five matrix products,
    2.5x the forward's), grouped-query prefill and decode (32 query heads on
    8 K/V heads), a packed variable-length causal batch, the split-KV decode
    (GB/s over the K+V bytes) and the four quantised forwards (int8 scores
    with fp8 P.V, the all-INT8 form, FP8 with rotated Q and K, and the same
    with P in MXFP4), each timed the same way (informational).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]
                       [--copy-calibration] [--decode-only | --long-only | --quant-only | --backward-only]
       python bench.py --traffic-from FETCH_DIR WRITE_DIR
       python bench.py --mfma-from DIR
       python bench.py --decode-traffic-from FETCH_DIR WRITE_DIR

HBM traffic: two rocprofv3 counter runs of
    python bench.py --no-cpu-baseline --no-extra --steps 3 --warmup 1 --copy-calibration
one with --pmc FETCH_SIZE and one with --pmc WRITE_SIZE (CSV output).  The
--copy-calibration flag adds, before the timed region, three plain device
copies of COPY_BYTES bytes (torch's copy kernel reads and writes exactly that
many bytes), so each counter is scaled by known bytes / what it reads for
the copy.  --traffic-from turns the two runs into profiles/prefill_4k_traffic.json.

MFMA utilisation: one rocprofv3 run of the same command with --pmc MfmaUtil
SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE; --mfma-from turns it into
profiles/prefill_4k_mfma.json (both launches).  Decode HBM bytes: the two traffic runs of
    python bench.py --decode-only --steps 3 --warmup 1 --copy-calibration
and --decode-traffic-from, giving profiles/decode_8k_traffic.json.  Each
record carries a hash of the kernel source it was taken on and is ignored
once that source changes.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attn fwd TFLOP/s & % MFMA peak (prefill); HBM GB/s & % peak (decode)"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16/fp16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # dense fp8 / int8
PEAK_HBM_GBS = 8000.0         # HBM3E
PEAK_CLOCK_GHZ = 2.4          # the engine clock the MFMA peaks are quoted at
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_4k_traffic.json")
COPY_BYTES = 1 << 30          # bytes read (and written) by one calibration copy
PREFILL_KERNEL = "prefill_kernel<128, true, false, 0>"   # bf16, non-causal, all exp2 on v_exp_f32
PREFILL_KERNEL_CAUSAL = "prefill_kernel<128, true, true, 0>"
MFMA_FILE = os.path.join(ROOT, "profiles", "prefill_4k_mfma.json")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_8k_traffic.json")
DECODE_KERNELS = ("decode_partial_kernel<128, true, 1>", "decode_merge_kernel")
KERNEL_SOURCES = ["flashattention_forward_amd/csrc/prefill.hip", "flashattention_forward_amd/csrc/common.h",
                  "flashattention_forward_amd/csrc/seq_shape.h"]
DECODE_SOURCES = ["flashattention_forward_amd/csrc/decode.hip", "flashattention_forward_amd/csrc/common.h",
                  "flashattention_forward_amd/csrc/seq_shape.h"]


def _median(xs):
    ys = sorted(xs)
    n = len(ys)
    return ys[n // 2] if n % 2 else 0.5 * (ys[n // 2 - 1] + ys[n // 2])


def kernel_source_sha(sources=None) -> str:
    """Hash of a kernel's code (the prefill's by default) with comments and
    blank space removed, so that a counter record goes stale when the code
    changes, not its prose."""
    import re
    h = hashlib.sha256()
    for p in (KERNEL_SOURCES if sources is None else sources):
        with open(os.path.join(ROOT, p)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(" ".join(l.split()) for l in text.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


def _current_record(path, sources=None):
    """A committed counter record, or None if missing or taken on other code."""
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    return rec if rec.get("kernel_source_sha") == kernel_source_sha(sources) else None


def traffic_per_launch():
    """HBM bytes per launch of the non-causal prefill kernel from the committed
    counter runs, or None if they were taken on another kernel source."""
    rec = _current_record(TRAFFIC_FILE)
    return None if rec is None else rec.get("hbm_bytes_per_launch")


def _counter_rows(run_dir: str, counter: str, with_time: bool = False):
    """(kernel name, value[, duration ns]) per dispatch of `counter` from a
    rocprofv3 CSV run."""
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") == counter:
                    row = (r["Kernel_Name"], float(r["Counter_Value"]))
                    if with_time:
                        row += (int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),)
                    rows.append(row)
    if not rows:
        raise SystemExit(f"no {counter} rows under {run_dir}")
    return rows


def _write(path, rec):
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def _scaled_bytes(run_dir, counter, kernels, per_call):
    """Counter bytes per call of the listed kernels (per_call dispatches of each
    make one call), scaled by the copy calibration run in the same process."""
    rows = _counter_rows(run_dir, counter)
    copy = [v for k, v in rows if "copy" in k.lower() or "elementwise" in k.lower()]
    if not copy:
        raise SystemExit(f"{counter}: no copy-calibration dispatches under {run_dir}")
    copy_kib = sorted(copy)[len(copy) // 2]
    factor = COPY_BYTES / (copy_kib * 1024.0)
    kib = 0.0
    for name in kernels:
        vals = [v for k, v in rows if name in k]
        if not vals:
            raise SystemExit(f"{counter}: no {name} dispatches under {run_dir}")
        kib += sum(vals) / len(vals) * per_call.get(name, 1)
    return {"counter": counter, "kib_per_call": round(kib, 1), "copy_kib_per_dispatch": round(copy_kib, 1),
            "bytes_per_counter_byte": round(factor, 4), "bytes_per_call": round(kib * 1024.0 * factor)}


def traffic_from(fetch_dir: str, write_dir: str) -> dict:
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the non-causal prefill
    kernel by the copy calibration and write the traffic record."""
    out = {"kernel": PREFILL_KERNEL, "kernel_source_sha": kernel_source_sha(), "copy_bytes": COPY_BYTES}
    total = 0.0
    for name, run_dir, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        r = _scaled_bytes(run_dir, counter, [PREFILL_KERNEL], {})
        out[name] = {"counter": counter, "prefill_kib_per_dispatch": r["kib_per_call"],
                     "copy_kib_per_dispatch": r["copy_kib_per_dispatch"],
                     "bytes_per_counter_byte": r["bytes_per_counter_byte"], "prefill_bytes_per_launch": r["bytes_per_call"]}
        total += r["bytes_per_call"]
    out["hbm_bytes_per_launch"] = round(total)
    return _write(TRAFFIC_FILE, out)


def mfma_from(run_dir: str) -> dict:
    """MFMA utilisation of the prefill kernel from one rocprofv3 run with --pmc
    MfmaUtil SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE: rocprof's derived
    MfmaUtil (busy cycles summed over all SIMDs / (active cycles x SIMDs)),
    the busy cycles per SIMD, and the clock the active-cycle count implies
    over the dispatch (GRBM_GUI_ACTIVE summed over the 8 XCDs); the
    non-causal launch at the top level, the causal one under "causal"."""
    def one(kernel: str) -> dict:
        util = [v for k, v in _counter_rows(run_dir, "MfmaUtil") if kernel in k]
        busy = [v for k, v in _counter_rows(run_dir, "SQ_VALU_MFMA_BUSY_CYCLES") if kernel in k]
        gui = [(v, t) for k, v, t in _counter_rows(run_dir, "GRBM_GUI_ACTIVE", True) if kernel in k]
        if not util or not busy or not gui:
            raise SystemExit(f"no {kernel} dispatches under {run_dir}")
        n = min(len(util), len(busy), len(gui))
        return {"kernel": kernel, "dispatches": n,
                "mfma_util_pct": [round(u, 2) for u in util[:n]],
                "mfma_busy_cycles_per_simd": [round(b / 1024.0) for b in busy[:n]],
                "clock_ghz": [round(g / 8.0 / t, 3) for g, t in gui[:n]],
                "dispatch_us": [round(t / 1e3, 1) for _, t in gui[:n]]}
    rec = one(PREFILL_KERNEL)
    mfmas = 1099511627776.0 / (32 * 32 * 16 * 2)          # 32x32x16 MFMAs per non-causal launch
    rec = {"kernel": PREFILL_KERNEL, "kernel_source_sha": kernel_source_sha(), **{k: v for k, v in rec.items() if k != "kernel"},
           "busy_cycles_per_mfma": round(rec["mfma_busy_cycles_per_simd"][0] * 1024.0 / mfmas, 2),
           "causal": one(PREFILL_KERNEL_CAUSAL)}
    return _write(MFMA_FILE, rec)


def decode_traffic_from(fetch_dir: str, write_dir: str) -> dict:
    """HBM bytes of one split-KV decode call (partial + merge kernels) of the
    decode_8k workload from two counter runs of bench.py --decode-only."""
    out = {"kernels": list(DECODE_KERNELS), "kernel_source_sha": kernel_source_sha(DECODE_SOURCES),
           "copy_bytes": COPY_BYTES, "algorithmic_bytes": 2 * 64 * 32 * 8192 * 128 * 2}
    total = 0
    for name, run_dir, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        out[name] = _scaled_bytes(run_dir, counter, DECODE_KERNELS, {})
        total += out[name]["bytes_per_call"]
    out["hbm_bytes_per_call"] = total
    return _write(DECODE_TRAFFIC_FILE, out)


def copy_calibration():
    """Three plain device copies of COPY_BYTES bytes (untimed)."""
    import torch
    src = torch.ones(COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def timed_launches(fns, steps, warmup):
    """Run the list of launch closures `steps` times after `warmup` rounds;
    returns (total seconds, [average seconds per launch of each closure])."""
    import torch
    for _ in range(warmup):
        for f in fns:
            f()
    torch.cuda.synchronize()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in fns]
          for _ in range(steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for s in range(steps):
        for i, f in enumerate(fns):
            ev[s][i][0].record()
            f()
            ev[s][i][1].record()
    t1.record()
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1) / 1e3
    per = [sum(ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)) / steps / 1e3 for i in range(len(fns))]
    return total, per


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), for the baseline's record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(seconds_target: float = 15.0, max_heads: int = 1024):
    """The fp64 oracle on a bounded sample of the prefill workload: whole
    heads, alternating non-causal and causal, until ~seconds_target."""
    import numpy as np
    import fa_inputs as G
    from oracle import attention as A
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    w = G.WORKLOADS["prefill_4k"]
    flops = 0.0
    heads = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds_target and heads < max_heads:
        b, h = divmod(heads, w.H)
        q, k, v = (G.to_f64(x[0], "bf16") for x in G.draw_qkv(w, heads=[(b, h)]))
        causal = bool(heads % 2)
        A.attention_head(q, k, v, w.scale, causal)
        flops += 4.0 * w.Nq * w.Nk * w.d / (2.0 if causal else 1.0)
        heads += 1
    dt = time.perf_counter() - t0
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "cpu": cpu_model(), "host_cpus": os.cpu_count(),
            "sample": f"{heads} whole heads (alternating non-causal/causal) of B=4 H=32 N=4096 d=128 bf16, "
                      f"fp64 numpy, {dt:.1f} s incl. input generation"}


def cpu_oracle_other(seconds_each: float = 4.0):
    """The fp64 oracle beside the other workloads, each on a bounded sample
    timed on this host: the long causal sequence (query rows of one head
    against all their visible keys), the decode (whole (batch, head) pairs,
    GB/s over their K and V bytes) and the quantised forward (query rows of
    one head, int8 scores and E4M3 P as the oracle emulates them; the head's
    quantisation is outside the timed part)."""
    import numpy as np
    import fa_inputs as G
    from oracle import attention as A
    from oracle import quant as Q
    out = {}
    # long causal sequence: rows spread over the head, each against its visible keys
    w = G.WORKLOADS["long_23400_causal"]
    q, k, v = (G.to_f64(x[0], "fp16") for x in G.draw_qkv(w, heads=[(0, 0)]))
    flops, rows_done, t0 = 0.0, 0, time.perf_counter()
    # blocks of 64 rows at a stride of 2339 across the head, each pass shifted
    # by 64 rows, until the time budget is spent
    for i in range(w.Nq):
        r0 = (i * 2339 + (i // 10) * 64) % (w.Nq - 63)
        rows = np.arange(r0, r0 + 64)
        A.attention_rows(q, k, v, rows, w.scale, True)
        flops += float(np.sum(4.0 * w.d * (rows + 1)))
        rows_done += len(rows)
        if time.perf_counter() - t0 > seconds_each:
            break
    dt = time.perf_counter() - t0
    out["long_23400_causal"] = {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s",
                                "sample": f"{rows_done} query rows of one head (fp16, causal), {dt:.1f} s"}
    # decode: whole (batch, head) pairs
    w = G.WORKLOADS["decode_8k"]
    heads = [divmod(i, w.H) for i in range(32)]
    drawn = [tuple(G.to_f64(x[0], "bf16") for x in G.draw_qkv(w, heads=[bh])) for bh in heads]
    nbytes, pairs, t0 = 0.0, 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds_each:
        q, k, v = drawn[pairs % len(drawn)]
        A.attention_head(q, k, v, w.scale, False)
        nbytes += 2.0 * w.Nk * w.d * 2
        pairs += 1
    dt = time.perf_counter() - t0
    out["decode_8k"] = {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s",
                        "sample": f"{pairs} (batch, head) decodes over 32 drawn pairs, inputs drawn beforehand, "
                                  f"{dt:.1f} s"}
    # quantised forward: query rows of one head
    w = G.WORKLOADS["quant_8k"]
    q, k, v = (G.to_f32(x[0], "bf16") for x in G.draw_qkv(w, heads=[(0, 0)]))
    qi = Q.quantize_inputs(q, k, v)
    ops, rows_done, t0 = 0.0, 0, time.perf_counter()
    for r0 in range(0, w.Nq, 512):
        rows = slice(r0, r0 + 128)
        Q.attention_q8_head(qi["q8"][rows], qi["sq"][rows], qi["k8"], qi["sk"], qi["v8"], qi["sv"], w.scale)
        ops += 4.0 * w.d * w.Nk * 128
        rows_done += 128
        if time.perf_counter() - t0 > seconds_each:
            break
    dt = time.perf_counter() - t0
    out["quant_8k"] = {"value": round(ops / dt / 1e12, 6), "unit": "TOP/s",
                       "sample": f"{rows_done} query rows of one head (int8 scores, E4M3 P), {dt:.1f} s"}
    return out


def rescale_stats(heads: int = 4):
    """How often the running max is raised (O and l rescaled), emulated on the
    CPU over the bench inputs, per (wave of 32 query rows, key tile) pair, for
    three rules: raise on every increase of a row's max (the plain online
    softmax), raise only when a tile's max exceeds the running max by more
    than 8 in log2 units (a threshold on the max), and this library's rule
    (raise when a lane's probabilities against the current max would sum past
    2^14; a lane holds the keys 4h..4h+3 of every 8 of the tile).  A wave
    raises when any of its rows (lanes) does.  The first visible tile of a
    row always sets its max and is counted apart."""
    import numpy as np
    import fa_inputs as G
    log2e = 1.4426950408889634
    out = {}
    cases = [("prefill_4k", G.WORKLOADS["prefill_4k"], "bf16", 64), ("prefill_4k_causal",
             G.WORKLOADS["prefill_4k_causal"], "bf16", 64), ("long_23400_causal", G.WORKLOADS["long_23400_causal"],
                                                              "fp16", 128)]
    for name, w, dt, BN in cases:
        cnt = {"every_increase": 0, "max_plus_8": 0, "tile_sum_2^14": 0, "first_tiles": 0, "wave_tiles": 0}
        for hd in range(heads):
            b, h = divmod(hd * 7 % (w.B * w.H), w.H)
            q, k = (G.to_f64(x[0], dt) for x in G.draw_qkv(w, heads=[(b, h)])[:2])
            Nq, Nk = q.shape[0], k.shape[0]
            for r0 in range(0, Nq, 32):
                rows = np.arange(r0, min(Nq, r0 + 32))
                s = (q[rows] @ k.T) * (w.scale * log2e)
                if w.causal:
                    s = np.where(np.arange(Nk)[None, :] <= rows[:, None] + (Nk - Nq), s, -np.inf)
                    kv_end = min(Nk, (r0 // 256 + 1) * 256 + (Nk - Nq))   # the workgroup's last visible key
                else:
                    kv_end = Nk
                m0 = np.full(len(rows), -np.inf)
                m8 = m0.copy()
                ms = m0.copy()
                half = (np.arange(BN) % 8) >= 4
                for t0 in range(0, kv_end, BN):
                    T = s[:, t0:t0 + BN]
                    tm = T.max(axis=1)
                    cnt["wave_tiles"] += 1
                    if np.all(np.isneginf(ms)) and np.any(np.isfinite(tm)):
                        cnt["first_tiles"] += 1
                    if np.any(tm > m0) and not np.all(np.isneginf(m0)):
                        cnt["every_increase"] += 1
                    m0 = np.maximum(m0, tm)
                    if np.any(tm > m8 + 8) and not np.all(np.isneginf(m8)):
                        cnt["max_plus_8"] += 1
                    m8 = np.where(tm > m8 + 8, np.maximum(m8, tm), m8)
                    if np.any(np.isneginf(ms)):
                        ms = np.maximum(ms, tm)
                    else:
                        with np.errstate(over="ignore"):
                            p = np.exp2(T - ms[:, None])
                        hs = np.stack([p[:, ~half[:T.shape[1]]].sum(axis=1), p[:, half[:T.shape[1]]].sum(axis=1)])
                        if np.any(~(hs <= 2.0 ** 14)):
                            cnt["tile_sum_2^14"] += 1
                            ms = np.maximum(ms, tm)
        n = cnt["wave_tiles"]
        out[name] = {**cnt, "heads": heads, "tile_keys": BN,
                     "rate_every_increase": round(cnt["every_increase"] / n, 5),
                     "rate_max_plus_8": round(cnt["max_plus_8"] / n, 5),
                     "rate_tile_sum": round(cnt["tile_sum_2^14"] / n, 5)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--mfma-from", metavar="DIR")
    ap.add_argument("--decode-traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--decode-only", action="store_true")
    ap.add_argument("--quant-only", action="store_true")
    ap.add_argument("--long-only", action="store_true", help="the long causal sequence alone (counter runs)")
    ap.add_argument("--backward-only", action="store_true",
                    help="the non-causal backward of the prefill workload alone (counter runs)")
    ap.add_argument("--rescale-stats", action="store_true",
                    help="CPU only: how often each max-raising rule rescales, on the bench inputs")
    args = ap.parse_args()
    if args.rescale_stats:
        print(json.dumps(rescale_stats()))
        return
    if args.traffic_from:
        print(json.dumps(traffic_from(*args.traffic_from)))
        return
    if args.mfma_from:
        print(json.dumps(mfma_from(args.mfma_from)))
        return
    if args.decode_traffic_from:
        print(json.dumps(decode_traffic_from(*args.decode_traffic_from)))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path (the forward pass shards by "
              "(batch, head) with no exchange between GPUs, so one GPU's share is the measured unit). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import fa_inputs as G
    import flashattention_forward_amd as F

    F.lib()
    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration()
    if args.decode_only:
        # the split-KV decode of decode_8k alone (for its counter runs)
        wd = G.WORKLOADS["decode_8k"]
        tq, tk, tv = (G.to_torch(x, "bf16") for x in G.draw_qkv(wd, threads=16))
        o = torch.empty_like(tq)
        l = torch.empty((wd.B, wd.H, 1), device="cuda")
        ws = torch.empty(F.workspace_bytes(wd.B, wd.H, 1, wd.Nk, wd.d, 0), device="cuda", dtype=torch.uint8)
        _, per = timed_launches([lambda: F.attn_fwd(tq, tk, tv, scale=wd.scale, out=o, lse=l, workspace=ws)],
                                args.steps, args.warmup)
        print(json.dumps({"workload": "decode_8k", "ms": round(per[0] * 1e3, 4)}))
        return
    if args.long_only:
        # the long causal fp16 sequence alone (for its counter runs)
        wl = G.WORKLOADS["long_23400_causal"]
        tq, tk, tv = (G.to_torch(x, "fp16") for x in G.draw_qkv(wl, threads=16))
        o = torch.empty_like(tq)
        l = torch.empty((wl.B, wl.H, wl.Nq), device="cuda")
        _, per = timed_launches([lambda: F.attn_fwd(tq, tk, tv, causal=True, scale=wl.scale, out=o, lse=l)],
                                args.steps, args.warmup)
        print(json.dumps({"workload": "long_23400_causal", "ms": round(per[0] * 1e3, 4)}))
        return
    if args.backward_only:
        # the non-causal backward of prefill_4k alone (for its counter runs)
        w = G.WORKLOADS["prefill_4k"]
        tq, tk, tv = (G.to_torch(x, "bf16") for x in G.draw_qkv(w, threads=16))
        tdo = G.to_torch(G.draw_tensor(w, "do", threads=16), "bf16")
        o, l = F.attn_fwd(tq, tk, tv, causal=False, scale=w.scale)
        dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
        ws = torch.empty(w.B * w.H * w.Nq * 8, device="cuda", dtype=torch.uint8)
        _, per = timed_launches([lambda: F.attn_bwd(tq, tk, tv, o, tdo, l, causal=False, scale=w.scale, dq=dq, dk=dk,
                                                    dv=dv, workspace=ws)], args.steps, args.warmup)
        print(json.dumps({"workload": "backward_4k", "ms": round(per[0] * 1e3, 4)}))
        return
    if args.quant_only:
        # the quantised forward of quant_8k alone (int8 scores, E4M3 P.V; for its counter runs)
        wq = G.WORKLOADS["quant_8k"]
        tq, tk, tv = (G.to_torch(x, "bf16") for x in G.draw_qkv(wq, threads=16))
        q8, sq = F.quantize_rows_i8(tq)
        k8, sk = F.quantize_rows_i8(tk)
        v8, sv = F.quantize_tensor_e4m3(tv)
        o = torch.empty((wq.B, wq.H, wq.Nq, wq.d), device="cuda", dtype=torch.bfloat16)
        l = torch.empty((wq.B, wq.H, wq.Nq), device="cuda")
        _, per = timed_launches([lambda: F.attn_fwd_q8(q8, k8, v8, sq, sk, sv, scale=wq.scale, out=o, lse=l)],
                                args.steps, args.warmup)
        print(json.dumps({"workload": "quant_8k", "ms": round(per[0] * 1e3, 4)}))
        return
    w = G.WORKLOADS["prefill_4k"]
    q, k, v = (G.to_torch(x, "bf16") for x in G.draw_qkv(w, threads=16))
    out_nc, out_c = torch.empty_like(q), torch.empty_like(q)
    lse_nc = torch.empty((w.B, w.H, w.Nq), device="cuda")
    lse_c = torch.empty_like(lse_nc)
    flops_nc = G.WORKLOADS["prefill_4k"].flops()
    flops_c = G.WORKLOADS["prefill_4k_causal"].flops()
    fns = [lambda: F.attn_fwd(q, k, v, causal=False, scale=w.scale, out=out_nc, lse=lse_nc),
           lambda: F.attn_fwd(q, k, v, causal=True, scale=w.scale, out=out_c, lse=lse_c)]
    total, per = timed_launches(fns, args.steps, args.warmup)
    value = (flops_nc + flops_c) * args.steps / total / 1e12
    achieved = flops_nc / per[0] / 1e12
    traffic = traffic_per_launch()
    mf = _current_record(MFMA_FILE)
    res = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(total / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded i.i.d. N(0,1), rounded to bf16)",
        "config": {"workload": "prefill_4k: B=4 H=32 Nq=Nk=4096 d=128 bf16, scale 1/sqrt(128); one step = one "
                               "non-causal + one causal launch", "global_batch": w.B, "seq_len": w.Nq,
                   "heads": w.H, "head_dim": w.d, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "prefill_kernel<128, bf16, non-causal>",
                     "flops_per_launch": flops_nc,
                     "mfma_util_counted": None if mf is None else {
                         "pct": mf["mfma_util_pct"], "clock_ghz": mf["clock_ghz"],
                         "causal_pct": mf.get("causal", {}).get("mfma_util_pct"),
                         # the nameplate peak scaled to the median clock of the counter run, and this
                         # run's throughput against it (the clock was counted in another run)
                         "peak_at_counted_clock": round(PEAK_BF16_TFLOPS * _median(mf["clock_ghz"]) / PEAK_CLOCK_GHZ, 1),
                         "frac_at_counted_clock": round(achieved / (PEAK_BF16_TFLOPS * _median(mf["clock_ghz"])
                                                                    / PEAK_CLOCK_GHZ), 4),
                         "source": "profiles/prefill_4k_mfma.json (rocprofv3 MfmaUtil)"}},
        "kernels": {
            "prefill_noncausal": {"ms": round(per[0] * 1e3, 4), "tflops": round(flops_nc / per[0] / 1e12, 3),
                                  "frac_peak": round(flops_nc / per[0] / 1e12 / PEAK_BF16_TFLOPS, 4)},
            "prefill_causal": {"ms": round(per[1] * 1e3, 4), "tflops": round(flops_c / per[1] / 1e12, 3),
                               "frac_peak": round(flops_c / per[1] / 1e12 / PEAK_BF16_TFLOPS, 4)},
        },
    }
    del q, k, v, out_nc, out_c, lse_nc, lse_c
    torch.cuda.empty_cache()

    if not args.no_extra:
        other = {}
        # long causal sequence, fp16 d=64
        wl = G.WORKLOADS["long_23400_causal"]
        tq, tk, tv = (G.to_torch(x, "fp16") for x in G.draw_qkv(wl, threads=16))
        o = torch.empty_like(tq)
        l = torch.empty((wl.B, wl.H, wl.Nq), device="cuda")
        _, per = timed_launches([lambda: F.attn_fwd(tq, tk, tv, causal=True, scale=wl.scale, out=o, lse=l)],
                                max(5, args.steps // 2), args.warmup)
        other["long_23400_causal"] = {"ms": round(per[0] * 1e3, 4), "tflops": round(wl.flops() / per[0] / 1e12, 3),
                                      "frac_peak": round(wl.flops() / per[0] / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del tq, tk, tv, o, l
        # backward pass at the prefill configuration: algorithmic FLOPs of its five
        # products (Q K^T, P^T dO, dO V^T, dS K, dS^T Q) = 2.5x the forward's
        tq, tk, tv = (G.to_torch(x, "bf16") for x in G.draw_qkv(w, threads=16))
        tdo = G.to_torch(G.draw_tensor(w, "do", threads=16), "bf16")
        # the software-exp2 split (2 or 4 of every 8 softmax exponentials on the
        # library's polynomial instead of v_exp_f32), non-causal, beside the default
        so, sl = torch.empty_like(tq), torch.empty((w.B, w.H, w.Nq), device="cuda")
        _, pers = timed_launches([lambda sh=sh: F.attn_fwd_exp2_split(tq, tk, tv, sh, causal=False, scale=w.scale,
                                                                      out=so, lse=sl) for sh in (0, 2, 4)],
                                 max(5, args.steps // 2), args.warmup)
        other["prefill_4k_exp2_split"] = {
            "ms_by_poly_share": {f"{sh}/8": round(t * 1e3, 4) for sh, t in zip((0, 2, 4), pers)},
            "tflops_by_poly_share": {f"{sh}/8": round(flops_nc / t / 1e12, 3) for sh, t in zip((0, 2, 4), pers)}}
        del so, sl
        dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
        ws = torch.empty(w.B * w.H * w.Nq * 8, device="cuda", dtype=torch.uint8)
        for causal in (False, True):
            o, l = F.attn_fwd(tq, tk, tv, causal=causal, scale=w.scale)
            _, per = timed_launches([lambda: F.attn_bwd(tq, tk, tv, o, tdo, l, causal=causal, scale=w.scale, dq=dq,
                                                        dk=dk, dv=dv, workspace=ws)],
                                    max(5, args.steps // 2), args.warmup)
            fl = 2.5 * (flops_c if causal else flops_nc)
            other["backward_4k_causal" if causal else "backward_4k"] = {
                "ms": round(per[0] * 1e3, 4), "tflops": round(fl / per[0] / 1e12, 3),
                "frac_peak": round(fl / per[0] / 1e12 / PEAK_BF16_TFLOPS, 4), "flops": fl}
            del o, l
        del tq, tk, tv, tdo, dq, dk, dv, ws
        torch.cuda.empty_cache()
        # grouped-query prefill: 32 query heads on 8 K/V heads, causal
        wg = G.WORKLOADS["gqa_4k_causal"]
        tq = G.to_torch(G.draw_tensor(wg, "q", threads=16), "bf16")
        wgk = G.shrink(wg, H=8)
        tk, tv = (G.to_torch(G.draw_tensor(wgk, t, threads=16), "bf16") for t in ("k", "v"))
        o = torch.empty_like(tq)
        l = torch.empty((wg.B, wg.H, wg.Nq), device="cuda")
        _, per = timed_launches([lambda: F.attn_fwd(tq, tk, tv, causal=True, scale=wg.scale, out=o, lse=l)],
                                args.steps, args.warmup)
        other["gqa_4k_causal"] = {"ms": round(per[0] * 1e3, 4), "tflops": round(wg.flops() / per[0] / 1e12, 3),
                                  "frac_peak": round(wg.flops() / per[0] / 1e12 / PEAK_BF16_TFLOPS, 4),
                                  "heads": "32 query / 8 K/V"}
        # its backward (dK, dV of a K/V head summed over its 4 query heads)
        tdo = G.to_torch(G.draw_tensor(wg, "do", threads=16), "bf16")
        dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
        ws = torch.empty(wg.B * wg.H * wg.Nq * 8, device="cuda", dtype=torch.uint8)
        _, per = timed_launches([lambda: F.attn_bwd(tq, tk, tv, o, tdo, l, causal=True, scale=wg.scale, dq=dq, dk=dk,
                                                    dv=dv, workspace=ws)], max(5, args.steps // 2), args.warmup)
        fl = 2.5 * wg.flops()
        other["backward_gqa_4k_causal"] = {"ms": round(per[0] * 1e3, 4), "tflops": round(fl / per[0] / 1e12, 3),
                                           "frac_peak": round(fl / per[0] / 1e12 / PEAK_BF16_TFLOPS, 4),
                                           "heads": "32 query / 8 K/V"}
        del tq, tk, tv, o, l, tdo, dq, dk, dv, ws
        # packed variable-length batch: 16 sequences of seeded lengths in [128, 4096],
        # 32 query heads on 8 K/V heads, causal; FLOPs over the visible pairs
        lens = np.random.default_rng([0, 7]).integers(128, 4097, 16)
        cu = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).cuda()
        tot = int(lens.sum())
        wv = G.Workload("varlen_mix", 7, 1, 32, tot, tot, 128, "bf16", 1.0, True, 128 ** -0.5)
        tq = G.to_torch(G.draw_tensor(wv, "q", threads=16)[0], "bf16")
        wvk = G.shrink(wv, H=8)
        tk, tv = (G.to_torch(G.draw_tensor(wvk, t, threads=16)[0], "bf16") for t in ("k", "v"))
        o = torch.empty_like(tq)
        l = torch.empty((32, tot), device="cuda")
        mx = int(lens.max())
        _, per = timed_launches([lambda: F.attn_fwd_varlen(tq, tk, tv, cu, cu, mx, mx, causal=True, scale=wv.scale,
                                                           out=o, lse=l)], args.steps, args.warmup)
        fl = float(sum(2.0 * 32 * n * n * 128 for n in lens))
        other["varlen_mix_causal"] = {"ms": round(per[0] * 1e3, 4), "tflops": round(fl / per[0] / 1e12, 3),
                                      "frac_peak": round(fl / per[0] / 1e12 / PEAK_BF16_TFLOPS, 4),
                                      "tokens": tot, "sequences": 16, "flops": fl}
        # its backward
        tdo = G.to_torch(G.draw_tensor(wv, "do", threads=16)[0], "bf16")
        dq, dk, dv = torch.empty_like(tq), torch.empty_like(tk), torch.empty_like(tv)
        ws = torch.empty(32 * tot * 8, device="cuda", dtype=torch.uint8)
        _, per = timed_launches([lambda: F.attn_bwd_varlen(tq, tk, tv, o, tdo, l, cu, cu, mx, mx, causal=True,
                                                           scale=wv.scale, dq=dq, dk=dk, dv=dv, workspace=ws)],
                                max(5, args.steps // 2), args.warmup)
        other["backward_varlen_mix_causal"] = {"ms": round(per[0] * 1e3, 4),
                                               "tflops": round(2.5 * fl / per[0] / 1e12, 3),
                                               "frac_peak": round(2.5 * fl / per[0] / 1e12 / PEAK_BF16_TFLOPS, 4)}
        del tq, tk, tv, o, l, cu, tdo, dq, dk, dv, ws
        torch.cuda.empty_cache()
        # grouped-query decode: 32 query heads on 8 K/V heads; GB/s over the K/V bytes
        # that must be read once (the 8 K/V heads)
        wgd = G.WORKLOADS["gqa_decode_8k"]
        tq = G.to_torch(G.draw_tensor(wgd, "q", threads=16), "bf16")
        wgdk = G.shrink(wgd, H=8)
        tk, tv = (G.to_torch(G.draw_tensor(wgdk, t, threads=16), "bf16") for t in ("k", "v"))
        o = torch.empty_like(tq)
        l = torch.empty((wgd.B, wgd.H, 1), device="cuda")
        ws = torch.empty(F.workspace_bytes(wgd.B, wgd.H, 1, wgd.Nk, wgd.d, 0, Hkv=8), device="cuda",
                         dtype=torch.uint8)
        _, per = timed_launches([lambda: F.attn_fwd(tq, tk, tv, scale=wgd.scale, out=o, lse=l, workspace=ws)],
                                args.steps, args.warmup)
        kvb = 2 * wgd.B * 8 * wgd.Nk * wgd.d * 2
        other["gqa_decode_8k"] = {"ms": round(per[0] * 1e3, 4), "gbs_kv": round(kvb / per[0] / 1e9, 1),
                                  "frac_hbm_peak": round(kvb / per[0] / 1e9 / PEAK_HBM_GBS, 4), "kv_bytes": kvb,
                                  "heads": "32 query / 8 K/V"}
        del tq, tk, tv, o, l, ws
        torch.cuda.empty_cache()
        # split-KV decode
        wd = G.WORKLOADS["decode_8k"]
        tq, tk, tv = (G.to_torch(x, "bf16") for x in G.draw_qkv(wd, threads=16))
        o = torch.empty_like(tq)
        l = torch.empty((wd.B, wd.H, 1), device="cuda")
        splits = F.decode_splits(wd.B, wd.H, wd.Nk, wd.d)
        ws = torch.empty(F.workspace_bytes(wd.B, wd.H, 1, wd.Nk, wd.d, 0), device="cuda", dtype=torch.uint8)
        _, per = timed_launches([lambda: F.attn_fwd(tq, tk, tv, scale=wd.scale, out=o, lse=l, workspace=ws)],
                                args.steps, args.warmup)
        kv_bytes = 2 * wd.B * wd.H * wd.Nk * wd.d * 2
        other["decode_8k"] = {"ms": round(per[0] * 1e3, 4), "splits": splits,
                              "gbs_kv": round(kv_bytes / per[0] / 1e9, 1),
                              "frac_hbm_peak": round(kv_bytes / per[0] / 1e9 / PEAK_HBM_GBS, 4),
                              "kv_bytes": kv_bytes}
        drec = _current_record(DECODE_TRAFFIC_FILE, DECODE_SOURCES)
        if drec is not None:
            # all HBM bytes of the call as the counters saw them (K, V, Q, partials)
            hb = drec["hbm_bytes_per_call"]
            other["decode_8k"].update({"hbm_bytes_counted": hb, "gbs_counted": round(hb / per[0] / 1e9, 1),
                                       "frac_hbm_peak_counted": round(hb / per[0] / 1e9 / PEAK_HBM_GBS, 4)})
        del tq, tk, tv, o, l, ws
        torch.cuda.empty_cache()
        # quantised forward (timing covers attn_fwd_q8 only; quantisation reported apart)
        wq = G.WORKLOADS["quant_8k"]
        tq, tk, tv = (G.to_torch(x, "bf16") for x in G.draw_qkv(wq, threads=16))
        q8, sq = F.quantize_rows_i8(tq)
        k8, sk = F.quantize_rows_i8(tk)
        v8, sv = F.quantize_tensor_e4m3(tv)
        o = torch.empty((wq.B, wq.H, wq.Nq, wq.d), device="cuda", dtype=torch.bfloat16)
        l = torch.empty((wq.B, wq.H, wq.Nq), device="cuda")
        _, per = timed_launches([lambda: F.attn_fwd_q8(q8, k8, v8, sq, sk, sv, scale=wq.scale, out=o, lse=l)],
                                args.steps, args.warmup)
        _, perq = timed_launches([lambda: (F.quantize_rows_i8(tq), F.quantize_rows_i8(tk),
                                           F.quantize_tensor_e4m3(tv))], 5, 1)
        ops = wq.flops()
        other["quant_8k"] = {"ms": round(per[0] * 1e3, 4), "tops": round(ops / per[0] / 1e12, 3),
                             "frac_fp8_peak": round(ops / per[0] / 1e12 / PEAK_FP8_TFLOPS, 4),
                             "quantize_ms": round(perq[0] * 1e3, 4)}
        # the all-INT8 variant on the same inputs (int8 per-tensor V, int8 P)
        v8i, svi = F.quantize_tensor_i8(tv)
        _, per = timed_launches([lambda: F.attn_fwd_i8(q8, k8, v8i, sq, sk, svi, scale=wq.scale, out=o, lse=l)],
                                args.steps, args.warmup)
        other["quant_i8_8k"] = {"ms": round(per[0] * 1e3, 4), "tops": round(ops / per[0] / 1e12, 3),
                                "frac_int8_peak": round(ops / per[0] / 1e12 / PEAK_FP8_TFLOPS, 4)}
        # rotated FP8 (random-sign Hadamard + block E4M3 of Q and K; V and P as above)
        sgn = torch.from_numpy(G.draw_signs(90, wq.d)).cuda()
        f8q, fsq = F.rotate_quantize_e4m3(tq, sgn, 64)
        f8k, fsk = F.rotate_quantize_e4m3(tk, sgn, 64)
        _, per = timed_launches([lambda: F.attn_fwd_fp8(f8q, f8k, v8, fsq, fsk, sv, scale=wq.scale, out=o, lse=l)],
                                args.steps, args.warmup)
        _, perr = timed_launches([lambda: (F.rotate_quantize_e4m3(tq, sgn, 64), F.rotate_quantize_e4m3(tk, sgn, 64))],
                                 5, 1)
        _, per4 = timed_launches([lambda: F.attn_fwd_fp4p(f8q, f8k, v8, fsq, fsk, sv, scale=wq.scale, out=o, lse=l)],
                                 args.steps, args.warmup)
        other["quant_fp4p_8k"] = {"ms": round(per4[0] * 1e3, 4), "tflops": round(ops / per4[0] / 1e12, 3),
                                  "frac_fp8_peak": round(ops / per4[0] / 1e12 / PEAK_FP8_TFLOPS, 4),
                                  "p_format": "MXFP4 (E2M1, one E8M0 scale per 32 keys)"}
        other["quant_fp8_rotated_8k"] = {"ms": round(per[0] * 1e3, 4), "tflops": round(ops / per[0] / 1e12, 3),
                                         "frac_fp8_peak": round(ops / per[0] / 1e12 / PEAK_FP8_TFLOPS, 4),
                                         "rotate_quantize_qk_ms": round(perr[0] * 1e3, 4), "block_rows": 64}
        del tq, tk, tv, q8, k8, v8, sq, sk, sv, o, l, v8i, svi, f8q, f8k, fsq, fsk, sgn
        torch.cuda.empty_cache()
        res["other_workloads"] = other

    res["build_info"] = F.build_info()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline()
        if not args.no_extra:
            res["cpu_oracle_other"] = cpu_oracle_other()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
