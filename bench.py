#!/usr/bin/env python3
"""Benchmark of the MLA position-independent KV path on one MI355X.

One step is the per-batch GPU work of the path on the rotate-gather workload
(64 requests x 32768 assembled tokens from a 4096-chunk registry, chunk
lengths uniform in [32, 512], 80% registry hits): the per-entry trig pass and
the rotate-gather kernel, with the chunk table's device image and the pool
already resident in HBM.  ``value`` is assembled KV tokens per second.

Further legs time MLA decode with rotation on load (batch 64 x 8192 tokens
x 16 heads; batch 32 x 32768 x 128 heads with 16 splits), the chunked
tail-prefill (4096 queries over 65536 rows, 16 heads: rotate-gather of the
cache, then the prefill over it), its non-absorbed form (per-head up-projection
of the assembled cache, then attention with 192-wide keys) and the GQA/MHA comparison (the same chunk
table over an 8 x 128 grouped-query pool with the whole key rotated) with the
same methodology, each with its own roofline, and the host chunk-table producer
(content-defined chunking, fingerprints and registry lookups for 64 requests
x 32768 tokens against a warm registry; host work, no GPU).  The CPU oracle
is timed on a bounded sample of the rotate-gather batch as ``cpu_baseline``
(and of the producer batch inside the producer leg).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--legs ...]
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

METRIC = "assembled KV tokens/s and MLA decode GB/s (% of HBM peak) vs CPU oracle"
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
ROW_BYTES = 1152
CSRC = os.path.join(ROOT, "mla_position_independent_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# sources that define each timed kernel (a counter record is valid only for these bytes)
KERNEL_SOURCES = {
    # the gather's reads follow the host's grouping of the entries (irm_table.cpp)
    "rotate_gather_kernel": ["irm_gather.hip", "irm_device.h", "irm_table.cpp", "irm_internal.h"],
    "decode_private_kernel": ["irm_decode.hip", "irm_attn.h", "irm_device.h"],
    "decode_shared_kernel": ["irm_decode.hip", "irm_attn.h", "irm_device.h"],
    "prefill_kernel": ["irm_prefill.hip", "irm_attn.h", "irm_device.h"],
    "gqa_rotate_gather_kernel": ["irm_gqa.hip", "irm_device.h"],
    "mha_prefill_kernel": ["irm_nonabsorbed.hip", "irm_attn.h", "irm_device.h"],
}


def log(msg: str):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(key: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current source of that kernel; else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(key)
    kernel = key.split(":")[0]
    if not ent or ent.get("source_sha256_16") != kernel_source_hash(kernel):
        return None
    return ent.get("hbm_bytes_per_launch")


def _counter_rows(path: str):
    """(kernel name, counter name, value) of every dispatch in the rocprofv3
    counter CSVs under path."""
    import csv
    import glob
    files = [path] if os.path.isfile(path) else glob.glob(os.path.join(path, "**", "*counter_collection.csv"),
                                                        recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {path}")
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                yield row["Kernel_Name"], row["Counter_Name"], float(row["Counter_Value"])


def _mean_counter(path: str, counter: str, match) -> tuple:
    vals = [v for k, c, v in _counter_rows(path) if c == counter and match(k)]
    if not vals:
        raise SystemExit(f"no {counter} values for the selected kernel under {path}")
    return sum(vals) / len(vals), len(vals)


def ingest_counters(key: str, fetch_dir: str, write_dir: str, cal_fetch_dir: str, cal_write_dir: str):
    """Turn two counter runs of a kernel (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) into HBM bytes per launch, each scaled by what the same counter
    reads for a plain 1 GiB device copy, and record them in profiles/traffic.json."""
    kernel = key.split(":")[0]
    mk = lambda k: kernel in k
    is_copy = lambda k: "copy" in k.lower() and "fill" not in k.lower()
    copy_bytes = float(1 << 30)
    f_kib, nf = _mean_counter(fetch_dir, "FETCH_SIZE", mk)
    w_kib, nw = _mean_counter(write_dir, "WRITE_SIZE", mk)
    cf_kib, _ = _mean_counter(cal_fetch_dir, "FETCH_SIZE", is_copy)
    cw_kib, _ = _mean_counter(cal_write_dir, "WRITE_SIZE", is_copy)
    f_scale = copy_bytes / (cf_kib * 1024.0)
    w_scale = copy_bytes / (cw_kib * 1024.0)
    fetch = f_kib * 1024.0 * f_scale
    write = w_kib * 1024.0 * w_scale
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        rec = {}
    rec[key] = {"source_sha256_16": kernel_source_hash(kernel), "hbm_bytes_per_launch": round(fetch + write),
                "fetch_bytes_per_launch": round(fetch), "write_bytes_per_launch": round(write),
                "fetch_kib_raw": round(f_kib, 1), "write_kib_raw": round(w_kib, 1), "dispatches": [nf, nw],
                "copy_calibration": {"bytes": copy_bytes, "fetch_kib": round(cf_kib, 1), "write_kib": round(cw_kib, 1),
                                     "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4)}}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    log(f"{key}: fetch {fetch / 1e6:.1f} MB, write {write / 1e6:.1f} MB per launch -> {TRAFFIC_FILE}")


class ClockSampler:
    """Samples the GPU's shader clock from sysfs on a host thread while a leg
    runs (the part lowers its clock under sustained load, so MFMA-bound
    rates depend on it).  Reads the current level of pp_dpm_sclk or the
    hwmon sclk input of the first amdgpu card that has one; reports nothing
    where neither exists.  The card's power reading (hwmon power1_average or
    power1_input) and its power cap are sampled beside it where they exist;
    that reading is the firmware's running average, which trails a leg of a
    few tens of milliseconds, so it is context for the clock, not a measure
    of the leg's own draw."""

    def __init__(self, period_s: float = 0.002):
        import glob
        import threading
        self.period = period_s
        self.samples = []
        self.source = None
        for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
            for cand in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*", "freq1_input"))):
                label = os.path.join(os.path.dirname(cand), "freq1_label")
                try:
                    if open(label).read().strip().lower() == "sclk":
                        self.source = ("hwmon", cand)
                        break
                except OSError:
                    pass
            if self.source is None and os.path.exists(os.path.join(dev, "pp_dpm_sclk")):
                self.source = ("dpm", os.path.join(dev, "pp_dpm_sclk"))
            if self.source is not None:
                break
        self.power_path = self.cap_w = None
        self.power = []
        for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
            for h in sorted(glob.glob(os.path.join(dev, "hwmon", "hwmon*"))):
                for name in ("power1_average", "power1_input"):
                    if self.power_path is None and os.path.exists(os.path.join(h, name)):
                        self.power_path = os.path.join(h, name)
                        try:
                            self.cap_w = int(open(os.path.join(h, "power1_cap")).read().strip()) / 1e6
                        except (OSError, ValueError):
                            pass
            if self.power_path is not None:
                break
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        kind, path = self.source
        with open(path) as f:
            txt = f.read()
        if kind == "hwmon":
            return int(txt.strip()) / 1e6
        for line in txt.splitlines():
            if line.strip().endswith("*"):
                tok = line.split(":", 1)[1].strip().split()[0].lower()
                return float(tok.replace("mhz", ""))
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read() if self.source is not None else None
                if v:
                    self.samples.append(v)
                if self.power_path is not None:
                    with open(self.power_path) as f:
                        self.power.append(int(f.read().strip()) / 1e6)
            except (OSError, ValueError, IndexError):
                pass
            self._stop.wait(self.period)

    def __enter__(self):
        if self.source is not None or self.power_path is not None:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self.source is not None or self.power_path is not None:
            self._stop.set()
            self._thread.join()

    def summary(self):
        if not self.samples and not self.power:
            return None
        res = {}
        if self.samples:
            v = sorted(self.samples)
            res.update({"median_mhz": v[len(v) // 2], "min_mhz": v[0], "max_mhz": v[-1], "samples": len(v),
                        "source": self.source[0]})
        if self.power:
            pw = sorted(self.power)
            res.update({"power_median_w": round(pw[len(pw) // 2], 1), "power_max_w": round(pw[-1], 1),
                        "power_cap_w": self.cap_w})
        return res


def frac_at_clock(frac: float, clk):
    """A fraction of the 2.4 GHz peak restated against the peak at the shader
    clock sampled during the timed loop (the part runs sustained MFMA-heavy
    kernels below 2.4 GHz); None without a clock sample."""
    if not clk or not clk.get("median_mhz"):
        return None
    return round(frac * 2400.0 / clk["median_mhz"], 4)


# After the GPU has idled (while a leg draws its inputs on the host) its
# shader clock ramps up over the first tens of milliseconds of sustained
# work: the long decode's first 20 calls after 3 warm-up calls take 0.45 ms
# each against 0.40 ms after 200.  The decode and prefill legs therefore warm
# up for at least this long, so that their timed loops see the rate that a
# running decode or prefill loop sees; the headline step keeps exactly the
# warm-up steps it is given.
LEG_WARM_MS = 150.0


def time_leg(fn, steps: int, warmup: int, inner_events: bool = True, min_warm_ms: float = 0.0):
    """Run fn(ev_mid_or_None) warmup times, then more untimed calls until at
    least min_warm_ms have passed since the first, then steps timed calls.
    Returns wall ms per timed step (synchronised on both sides of the timed
    region), the median event time of the part fn brackets (ms), the mean of
    those event times, the shader clock sampled during the timed region, and
    the number of untimed calls made."""
    import torch
    t_w = time.perf_counter()
    n_warm = 0
    for _ in range(warmup):
        fn(None)
        n_warm += 1
    torch.cuda.synchronize()
    while (time.perf_counter() - t_w) * 1e3 < min_warm_ms:
        # enqueue about the calls the remaining time holds, at the rate so far
        per_ms = (time.perf_counter() - t_w) * 1e3 / max(n_warm, 1)
        more = max(1, min(1000, int((min_warm_ms - (time.perf_counter() - t_w) * 1e3) / max(per_ms, 1e-3)) + 1))
        for _ in range(more):
            fn(None)
            n_warm += 1
        torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    with ClockSampler() as clk:
        t0 = time.perf_counter()
        for k in range(steps):
            fn(evs[k] if inner_events else None)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
    kern = sorted(a.elapsed_time(b) for a, b in evs) if inner_events else []
    med = kern[len(kern) // 2] if kern else None
    mean = sum(kern) / len(kern) if kern else None
    return (t1 - t0) * 1e3 / steps, med, mean, clk.summary(), n_warm


_SCRUB = []


def time_cold(fn, n: int = 5):
    """Median event time (ms) of fn over n launches, each right behind a 512 MB
    write and a read of the same 512 MB on the same stream, which evict the
    256 MB Infinity Cache.  The read after the write drains the write's dirty
    lines before fn starts (a write alone leaves up to 256 MB of dirty lines
    whose write-back is charged to fn: +15% on the batched decode), and the
    scrub is enqueued together with fn, so fn is already queued when the
    scrub ends and the events hold fn's GPU time alone (no launch gap), to be
    set beside the timed loop's back-to-back median.  Returns (cold ms, ms
    of the same calls behind a 32 MB read instead of the scrub)."""
    import torch
    if not _SCRUB:
        _SCRUB.append(torch.ones(512 << 18, dtype=torch.int32, device="cuda"))
    scrub = _SCRUB[0]

    def one(cold: bool):
        if cold:
            scrub.fill_(2)
            scrub.sum()
        else:
            scrub[: 8 << 20].sum()  # a 32 MB read ahead, long enough that fn is queued when it ends
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    one(False)
    cold = sorted(one(True) for _ in range(n))
    warm = sorted(one(False) for _ in range(n))
    return cold[n // 2], warm[n // 2]


def time_events(fn, n: int = 10):
    """Median event time (ms) of fn over n back-to-back calls (events around
    each call, one synchronisation at the end, as in the timed loops), after
    one untimed call."""
    import torch
    fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    return ts[len(ts) // 2]


def leg_gather(args, irm, torch, synth, make=None, label="rotate-gather"):
    """One step = the per-batch device work of a new chunk table on the
    rotate-gather batch: the row-map and trig passes (irm_table_prepare) and
    the rotate-gather kernel, with the table's image and the pool in HBM."""
    log(f"{label}: generating 64 x 32768-token batch")
    w = (make or synth.rotate_gather_batch)()
    pool = irm.to_device_bf16(w.pool)
    inv = irm.rope_inv_freq(w.theta)
    t = irm.Table(w.chunks, w.seq_first, w.pool.shape[0]).upload(inv)
    out = torch.empty((t.total_rows, 576), dtype=torch.bfloat16, device="cuda")

    def step(ev):
        t.prepare(inv)                      # row map + per-entry trig (double sincos)
        if ev is not None:
            ev[0].record()
        irm.rotate_gather(t, pool, out=out)
        if ev is not None:
            ev[1].record()

    ms, kern_ms, kern_mean, clk, _ = time_leg(step, args.steps, args.warmup)
    tokens = t.total_rows
    alg_bytes = 2 * ROW_BYTES * tokens
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    # the kernel reads each pool run that several entries place once: its
    # least traffic is those rows read once plus every assembled row written
    gs = t.gather_stats()
    min_bytes = ROW_BYTES * (gs["read_rows"] + tokens)
    traffic = measured_traffic("rotate_gather_kernel" + ("" if make is None else ":" + w.name))
    cold_ms, warm1_ms = time_cold(lambda: irm.rotate_gather(t, pool, out=out))
    prep_ms = time_events(lambda: t.prepare(inv))
    upload_ms = time_events(lambda: t.upload(inv, dev_buf=t._dev))
    log(f"{label}: pool rows read {gs['read_rows']} of {tokens} assembled ({gs['n_items']} work items); "
        f"{min_bytes / (kern_ms * 1e-3) / 1e9:.0f} GB/s of least traffic")
    log(f"{label}: {ms:.3f} ms/step, kernel {kern_ms:.3f} ms (median), {achieved:.0f} GB/s; behind a cache scrub "
        f"{cold_ms:.3f} ms, behind a small kernel {warm1_ms:.3f} ms; prepare {prep_ms:.3f} ms, upload with its "
        f"copy {upload_ms:.3f} ms")
    res = {
        "tokens": tokens, "ms_per_step": ms, "kernel_ms": kern_ms, "entries": int(t.n_chunks),
        "mean_entry_len": round(tokens / max(1, t.n_chunks), 1),
        "table_prepare_ms": round(prep_ms, 4),
        "table_upload_ms": round(upload_ms, 4),
        # the host image copied by the upload (the trig, row-map and work-item
        # regions are written by the device passes)
        "table_h2d_bytes": int(gs["host_bytes"]),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "rotate_gather_kernel",
                     "kernel_ms_median": round(kern_ms, 4), "kernel_ms_mean": round(kern_mean, 4),
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "pool_rows_read": int(gs["read_rows"]),
                     "min_traffic_bytes_per_launch": int(min_bytes),
                     "min_traffic_frac": round(min_bytes / (kern_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "cold_cache_kernel_ms": round(cold_ms, 4),
                     "cold_cache_frac": round(alg_bytes / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "warm_behind_small_kernel_ms": round(warm1_ms, 4)},
        "sclk": clk,
        "workload": w, "table": t,
    }
    return res


def leg_gather_cdc(args, irm, torch, synth):
    """The rotate-gather batch with CDC-like chunk lengths (mean ~127 instead
    of 272): about twice the entries, the harder per-entry case."""
    r = leg_gather(args, irm, torch, synth, make=synth.rotate_gather_cdc_batch, label="rotate-gather (CDC lengths)")
    w = r.pop("workload")
    r.pop("table")
    r["workload"] = w.name
    r["value"] = round(r["tokens"] / (r["ms_per_step"] * 1e-3), 1)
    r["unit"] = "assembled KV tokens/s"
    return r


def _delta0_chunks(chunks):
    """The same entries with every delta 0 (p_src = p_tgt): the same pool
    rows, read through the same row map, with nothing to rotate."""
    c = chunks.copy()
    c["p_src"] = c["p_tgt"]
    return c


def leg_decode(args, irm, torch, synth, name, make):
    """One call = the split pass and the combine pass over the batch, the
    table prepared once (a decode loop reuses a sequence's table every step).
    Besides the call itself (rows gathered through the chunk table, k_r
    rotated on load), the same batch is decoded twice more to price the
    rotation: over the same rows with every delta set to 0 (same row map and
    scattered rows, nothing rotated), and over the cache assembled by
    rotate-gather beforehand, as one fresh entry per sequence (contiguous
    rows, nothing rotated)."""
    import numpy as np
    log(f"{name}: generating")
    w = make()
    pool = irm.to_device_bf16(w.pool)
    t = irm.Table(w.chunks, w.seq_first, w.pool.shape[0]).upload(irm.rope_inv_freq(w.theta))
    ql, qr = irm.to_device_bf16(w.q_lat), irm.to_device_bf16(w.q_rope)
    H = w.n_heads
    out = torch.empty((w.n_seq, H, 512), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(irm.decode_workspace_bytes(t, H, w.n_splits), dtype=torch.uint8, device="cuda")

    def call(table, kv):
        irm.mla_decode(ql, qr, table, kv, n_splits=w.n_splits, scale=w.scale, out=out, workspace=ws)

    def step(ev):
        if ev is not None:
            ev[0].record()
        call(t, pool)
        if ev is not None:
            ev[1].record()

    ms, kern_ms, kern_mean, clk, n_warm = time_leg(step, args.steps, args.warmup, min_warm_ms=args.leg_warm_ms)
    cold_ms, warm1_ms = time_cold(lambda: step(None))

    # the price of the rotation on load
    t0 = irm.Table(_delta0_chunks(w.chunks), w.seq_first, w.pool.shape[0]).upload(irm.rope_inv_freq(w.theta))
    assembled = irm.rotate_gather(t, pool)
    base = t.seq_base()
    rows = [(int(base[s]), int(base[s + 1] - base[s]), 0, 0, 1) for s in range(t.n_seq)]
    tf = irm.Table(np.array(rows, irm.CHUNK_DTYPE), np.arange(t.n_seq + 1, dtype=np.uint32), t.total_rows).upload()
    torch.cuda.synchronize()
    variants = {}
    for rnd in range(3):     # interleaved rounds: the clock drifts with the chip's temperature
        for key, tab, kv in (("rotate_on_load", t, pool), ("same_rows_delta0", t0, pool),
                             ("assembled_contiguous", tf, assembled)):
            variants.setdefault(key, []).append(time_events(lambda: call(tab, kv), 10))
    rot = {k: round(sorted(v)[1], 4) for k, v in variants.items()}
    rot["rotation_cost_frac"] = round(rot["rotate_on_load"] / rot["same_rows_delta0"] - 1.0, 4)
    rot["table_and_gather_cost_frac"] = round(rot["rotate_on_load"] / rot["assembled_contiguous"] - 1.0, 4)
    rot["method"] = ("median of 10 back-to-back calls per variant, middle of 3 interleaved rounds; "
                     "same_rows_delta0 = the same entries with p_src = p_tgt")
    del assembled, tf, t0

    # the split pass runs one 16-head group per workgroup unless the head
    # count is a multiple of 64 (four groups share every KV tile)
    kernel = "decode_shared_kernel" if H % 64 == 0 else "decode_private_kernel"
    kv = ROW_BYTES * t.total_rows
    qo = w.n_seq * H * (576 + 512) * 2
    alg_bytes = kv + qo
    flops = 2 * (576 + 512) * H * t.total_rows
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    log(f"{name}: {kern_ms:.3f} ms/call (median), {achieved:.0f} GB/s, {flops / kern_ms / 1e9:.0f} TFLOP/s; "
        f"behind a cache scrub {cold_ms:.3f} ms, behind a small kernel {warm1_ms:.3f} ms; rotation {rot}")
    cpu = None
    if not args.no_cpu_baseline:
        log(f"{name}: oracle on a sample of the batch")
        cpu = cpu_baseline_decode(w, args.cpu_seconds_legs)
    return {
        "workload": w.name, "ms_per_call": round(kern_ms, 4), "tokens": t.total_rows, "n_splits": w.n_splits,
        "cpu_baseline": cpu,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(kernel + ":" + w.name),
                     "kernel": kernel + " + decode_combine_kernel",
                     "kernel_ms_median": round(kern_ms, 4), "kernel_ms_mean": round(kern_mean, 4),
                     "algorithmic_bytes_per_launch": alg_bytes,
                     "cold_cache_kernel_ms": round(cold_ms, 4),
                     "cold_cache_frac": round(alg_bytes / (cold_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "warm_behind_small_kernel_ms": round(warm1_ms, 4)},
        "mfma_tflops": round(flops / (kern_ms * 1e-3) / 1e12, 2),
        "mfma_frac": round(flops / (kern_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, 4),
        "mfma_frac_at_sampled_clock": frac_at_clock(flops / (kern_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFS, clk),
        "rotation_on_load": rot,
        "sclk": clk,
        "warmup_calls": n_warm,
    }


def leg_tiny(args, irm, torch, synth):
    """The 1-sequence, 1024-row, 16-head decode: a latency case, reported in
    microseconds per call (split pass + combine), with the oracle beside it."""
    w = synth.tiny_decode()
    pool = irm.to_device_bf16(w.pool)
    t = irm.Table(w.chunks, w.seq_first, w.pool.shape[0]).upload(irm.rope_inv_freq(w.theta))
    ql, qr = irm.to_device_bf16(w.q_lat), irm.to_device_bf16(w.q_rope)
    out = torch.empty((1, w.n_heads, 512), dtype=torch.bfloat16, device="cuda")
    ws_bytes = irm.decode_workspace_bytes(t, w.n_heads, 0)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    # the split count the library picks (its workspace matches that count's)
    n_splits = next((s for s in range(1, 65) if irm.decode_workspace_bytes(t, w.n_heads, s) == ws_bytes), 0)

    def step(ev):
        if ev is not None:
            ev[0].record()
        irm.mla_decode(ql, qr, t, pool, scale=w.scale, out=out, workspace=ws)  # the library's split count
        if ev is not None:
            ev[1].record()

    ms, kern_ms, _, _, _ = time_leg(step, args.steps, args.warmup)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            reps = 0
            while reps == 0 or time.perf_counter() - t0 < 1.0:
                c, k = _oracle_rows(w, 0, oracle.rope_inv_freq(w.theta))
                oracle.mla_decode(oracle.bf16_to_f64(w.q_lat[0]), oracle.bf16_to_f64(w.q_rope[0]), c, k, w.scale)
                reps += 1
            cpu = {"value": round((time.perf_counter() - t0) / reps * 1e6, 1), "unit": "us per call", "cores": 1,
                   "kind": "oracle", "host": host_cpu(), "sample": f"the whole case, {reps} calls"}
    log(f"tiny decode: {kern_ms * 1e3:.1f} us per call")
    return {"workload": w.name, "us_per_call": round(kern_ms * 1e3, 2), "n_splits": n_splits,
            "kernel": "decode_private_kernel + decode_combine_kernel", "cpu_baseline": cpu}


def leg_prefill(args, irm, torch, synth, assembled: bool = True, fused: bool = True):
    """One call = assemble the 65536-row cache with rotate-gather, then the
    causal prefill of the 4096 queries over it (irm_mla_prefill_assembled).
    The roofline is the prefill kernel's own time (events around it); the
    single-kernel path with rotation on load (irm_mla_prefill_tail) is timed
    too, for comparison."""
    log("tail-prefill: generating")
    w = synth.tail_prefill()
    pool = irm.to_device_bf16(w.pool)
    t = irm.Table(w.chunks, w.seq_first, w.pool.shape[0]).upload(irm.rope_inv_freq(w.theta))
    ql, qr = irm.to_device_bf16(w.q_lat), irm.to_device_bf16(w.q_rope)
    nq, H = w.q_lat.shape[0], w.n_heads
    out = torch.empty((nq, H, 512), dtype=torch.bfloat16, device="cuda")
    kv = torch.empty((t.total_rows, 576), dtype=torch.bfloat16, device="cuda")

    def step(ev):
        irm.rotate_gather(t, pool, out=kv)
        if ev is not None:
            ev[0].record()
        irm.mla_prefill_assembled(ql, qr, w.q_pos0, kv, scale=w.scale, out=out)
        if ev is not None:
            ev[1].record()

    def fused_call(ev):
        if ev is not None:
            ev[0].record()
        irm.mla_prefill_tail(ql, qr, w.q_pos0, t, pool, scale=w.scale, out=out)
        if ev is not None:
            ev[1].record()

    n_steps, n_warm = max(3, args.steps // 4), min(args.warmup, 2)
    if not assembled:   # profiling the fused kernel alone
        fused_ms = time_leg(fused_call, n_steps, n_warm, min_warm_ms=args.leg_warm_ms)[1]
        log(f"tail-prefill, rotation on load in one kernel: {fused_ms:.3f} ms")
        return None
    ms, kern_ms, kern_mean, clk, warm_calls = time_leg(step, n_steps, n_warm, min_warm_ms=args.leg_warm_ms)
    fused_ms = time_leg(fused_call, n_steps, 1, min_warm_ms=args.leg_warm_ms)[1] if fused else None
    pairs = nq * w.q_pos0 + nq * (nq + 1) // 2      # visible (query, key) pairs
    flops = pairs * H * 2 * (576 + 512)
    achieved = flops / (kern_ms * 1e-3) / 1e12
    log(f"tail-prefill: {ms:.3f} ms/call (rotate-gather + prefill over the assembled cache; prefill kernel "
        f"{kern_ms:.3f} ms, {achieved:.0f} TFLOP/s); rotation on load in one kernel: "
        + ("not timed" if fused_ms is None else f"{fused_ms:.3f} ms"))
    cpu = None
    if not args.no_cpu_baseline:
        log("tail-prefill: oracle on the first queries")
        cpu = cpu_baseline_prefill(w, args.cpu_seconds_legs)
    return {
        "workload": w.name, "ms_per_call": round(ms, 4), "queries": nq, "kv_rows": t.total_rows,
        "cpu_baseline": cpu,
        "call": "irm_rotate_gather + irm_mla_prefill_assembled",
        "prefill_kernel_ms": round(kern_ms, 4),
        "fused_rotate_on_load_ms": None if fused_ms is None else round(fused_ms, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4),
                     "traffic": measured_traffic("prefill_kernel"), "kernel": "prefill_kernel (assembled cache)",
                     "kernel_ms_median": round(kern_ms, 4), "kernel_ms_mean": round(kern_mean, 4),
                     "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": ROW_BYTES * t.total_rows + nq * H * (576 + 512) * 2,
                     "frac_at_sampled_clock": frac_at_clock(achieved / MFMA_BF16_PEAK_TFS, clk)},
        "sclk": clk,
        "warmup_calls": warm_calls,
    }


def leg_nonabsorbed(args, irm, torch, synth):
    """Non-absorbed MLA prefill on the tail-prefill workload: the assembled
    65536-row cache is up-projected per head (irm_mla_kv_upproj, random
    W_UK / W_UV), then the 4096 queries attend with 192-wide keys and 128-wide
    values per head (irm_mla_prefill_nonabsorbed).  Roofline on the attention
    kernel; the up-projection is timed on its own."""
    log("non-absorbed prefill: generating")
    w = synth.tail_prefill()
    pool = irm.to_device_bf16(w.pool)
    t = irm.Table(w.chunks, w.seq_first, w.pool.shape[0]).upload(irm.rope_inv_freq(w.theta))
    q_nope, wk, wv = synth.nonabsorbed_inputs(1005, w.q_lat.shape[0], w.n_heads)
    qn, qr = irm.to_device_bf16(q_nope), irm.to_device_bf16(w.q_rope)
    wk, wv = irm.to_device_bf16(wk), irm.to_device_bf16(wv)
    nq, H = qn.shape[0], qn.shape[1]
    kv = irm.rotate_gather(t, pool)
    kvh = torch.empty((H, kv.shape[0], 256), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((nq, H, 128), dtype=torch.bfloat16, device="cuda")

    def up(ev):
        if ev is not None:
            ev[0].record()
        irm.mla_kv_upproj(kv, wk, wv, out=kvh)
        if ev is not None:
            ev[1].record()

    def attend(ev):
        if ev is not None:
            ev[0].record()
        irm.mla_prefill_nonabsorbed(qn, qr, w.q_pos0, kv, kvh, scale=w.scale, out=out)
        if ev is not None:
            ev[1].record()

    n_steps = max(3, args.steps // 2)
    up_ms = time_leg(up, n_steps, min(args.warmup, 2), min_warm_ms=args.leg_warm_ms)[1]
    _, kern_ms, _, clk, warm_calls = time_leg(attend, n_steps, min(args.warmup, 2), min_warm_ms=args.leg_warm_ms)
    pairs = nq * w.q_pos0 + nq * (nq + 1) // 2
    flops = pairs * H * 2 * (192 + 128)
    up_flops = 2 * kv.shape[0] * 512 * 256 * H
    achieved = flops / (kern_ms * 1e-3) / 1e12
    up_tfs = up_flops / (up_ms * 1e-3) / 1e12
    log(f"non-absorbed prefill: up-projection {up_ms:.3f} ms ({up_tfs:.0f} TFLOP/s), attention {kern_ms:.3f} ms "
        f"({achieved:.0f} TFLOP/s)")
    return {
        "workload": w.name + "_nonabsorbed", "ms_per_call": round(up_ms + kern_ms, 4), "queries": nq,
        "kv_rows": int(kv.shape[0]), "call": "irm_mla_kv_upproj + irm_mla_prefill_nonabsorbed (over the assembled cache)",
        "upproj_ms": round(up_ms, 4), "upproj_tflops": round(up_tfs, 1), "attention_ms": round(kern_ms, 4),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFS,
                     "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFS, 4),
                     "traffic": measured_traffic("mha_prefill_kernel"), "kernel": "mha_prefill_kernel",
                     "algorithmic_flops_per_launch": flops,
                     "frac_at_sampled_clock": frac_at_clock(achieved / MFMA_BF16_PEAK_TFS, clk)},
        "sclk": clk,
        "warmup_calls": warm_calls,
    }


def leg_gqa(args, irm, torch, gather):
    """GQA/MHA comparison: the rotate-gather batch's chunk table over a
    grouped-query pool (8 KV heads x head_dim 128, rows [K | V] = 4096 B),
    where every reused row has its whole key rotated.  Same methodology as the
    MLA rotate-gather leg; the pool is drawn on the device (seeded)."""
    n_kv, d = 8, 128
    t, w = gather["table"], gather["workload"]
    width = 2 * n_kv * d
    log(f"gqa rotate-gather: drawing a {w.pool.shape[0]} x {width} bf16 pool on the device")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(3003)
    pool = torch.randn((w.pool.shape[0], width), dtype=torch.bfloat16, device="cuda", generator=gen)
    out = torch.empty((t.total_rows, width), dtype=torch.bfloat16, device="cuda")
    inv = irm.gqa_inv_freq(w.theta, d)

    def step(ev):
        if ev is not None:
            ev[0].record()
        irm.gqa_rotate_gather(t, pool, n_kv, d, inv, out=out)
        if ev is not None:
            ev[1].record()

    ms, kern_ms, _, _, _ = time_leg(step, args.steps, args.warmup)
    tokens = t.total_rows
    alg_bytes = 2 * 2 * width * tokens
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    ratio = kern_ms / gather["kernel_ms"]
    # the MLA kernel reads each shared pool run once, this one every placement:
    # its bytes per assembled row against the row-by-row MLA figure (2304 B)
    bytes_ratio = (2 * 2 * width) / (2 * ROW_BYTES)
    log(f"gqa rotate-gather: {kern_ms:.3f} ms/call, {achieved:.0f} GB/s; {ratio:.2f}x the MLA rotate-gather time "
        f"(which reads each shared pool run once); {bytes_ratio:.2f}x the bytes per row of a row-by-row MLA gather")
    return {
        "workload": f"gqa_{n_kv}x{d}_" + w.name, "ms_per_call": round(kern_ms, 4), "tokens": tokens,
        "row_bytes": 2 * width, "rotated_bytes_per_token": n_kv * d * 2, "mla_rotated_bytes_per_token": 128,
        "time_vs_mla_rotate_gather": round(ratio, 3),
        "bytes_per_row_vs_mla_row_by_row": round(bytes_ratio, 3),
        "note": "this kernel reads every placement of a reused row; the MLA rotate-gather reads each shared pool "
                "run once, so the time ratio holds that saving as well as the per-row bytes",
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic("gqa_rotate_gather_kernel"),
                     "kernel": "gqa_trig_kernel + gqa_rotate_gather_kernel",
                     "algorithmic_bytes_per_launch": alg_bytes},
    }


def leg_producer(args, irm, synth, oracle_seconds: float):
    """Host chunk-table producer: irm_registry_assemble on 64 requests x 32768
    tokens (shared documents at shifted offsets, 80% of segments), the
    registry warmed by one earlier batch of the same mix."""
    import numpy as np
    warm = synth.token_requests(seed=1106)
    reqs = synth.token_requests(seed=1006)
    n_tok = int(sum(r.size for r in reqs))
    threads = min(16, os.cpu_count() or 1)  # the host share of one GPU
    times = []
    for k in range(args.warmup + args.steps):
        reg = irm.Registry(0)
        reg.assemble(warm, n_threads=threads)
        t0 = time.perf_counter()
        chunks, seq_first, _ = reg.assemble(reqs, n_threads=threads)
        dt = time.perf_counter() - t0
        if k >= args.warmup:
            times.append(dt)
    ms = 1e3 * float(np.median(times))
    hit_tok = float(chunks["len"][chunks["flags"] == 0].sum()) / n_tok
    log(f"producer: {ms:.3f} ms per batch, {n_tok / (ms * 1e-3):.4g} tokens/s on {threads} threads, "
        f"{hit_tok:.1%} of tokens from the registry")
    # the same batch with the S1 fallback (missed chunks looked up again as 128-token windows)
    p_s1 = irm.cdc_params(fallback_window=128)
    times_s1 = []
    for k in range(args.warmup + args.steps):
        reg = irm.Registry(0)
        reg.assemble(warm, params=p_s1, n_threads=threads)
        t0 = time.perf_counter()
        c_s1, _, _ = reg.assemble(reqs, params=p_s1, n_threads=threads)
        if k >= args.warmup:
            times_s1.append(time.perf_counter() - t0)
    ms_s1 = 1e3 * float(np.median(times_s1))
    hit_s1 = float(c_s1["len"][c_s1["flags"] == 0].sum()) / n_tok
    log(f"producer with the S1 fallback: {ms_s1:.3f} ms per batch, {hit_s1:.1%} of tokens from the registry")
    res = {"workload": "token_requests_64x32768", "ms_per_call": round(ms, 4), "tokens": n_tok,
           "value": round(n_tok / (ms * 1e-3), 1), "unit": "tokens/s (host)", "threads": threads,
           "entries": int(chunks.shape[0]), "registry_token_fraction": round(hit_tok, 4),
           "s1_fallback_128": {"ms_per_call": round(ms_s1, 4), "entries": int(c_s1.shape[0]),
                               "registry_token_fraction": round(hit_s1, 4)}}
    if oracle_seconds > 0:
        from oracle import irm_producer
        oreg = irm_producer.Registry(0)
        for r in warm[:4]:
            oreg.assemble(list(r))
        done, spent = 0, 0.0
        for r in reqs:
            t0 = time.perf_counter()
            oreg.assemble(list(r))
            spent += time.perf_counter() - t0
            done += r.size
            if spent >= oracle_seconds:
                break
        res["cpu_baseline"] = {"value": round(done / spent, 1), "unit": "tokens/s", "cores": 1, "kind": "oracle",
                               "sample": f"{done} tokens of the batch, {spent:.1f} s single-threaded Python"}
    return res


def cpu_baseline(w, seconds: float):
    """The oracle, single-threaded, on the first requests of the rotate-gather
    batch until ``seconds`` of CPU work have been spent (at least one)."""
    import numpy as np
    from threadpoolctl import threadpool_limits
    import oracle

    inv = oracle.rope_inv_freq(w.theta)
    done_tokens, done_req, spent = 0, 0, 0.0
    with threadpool_limits(limits=1):
        while done_req < w.n_seq and (spent < seconds or done_req == 0):
            s = done_req
            lo, hi = int(w.seq_first[s]), int(w.seq_first[s + 1])
            sub = w.chunks[lo:hi]
            t0 = time.perf_counter()
            (g, d, _), = oracle.expand_table(sub, np.array([0, hi - lo]), w.pool.shape[0])
            c, k = oracle.assemble_rows(w.pool, g, d, inv)
            spent += time.perf_counter() - t0
            done_tokens += g.shape[0]
            done_req += 1
    return {"value": round(done_tokens / spent, 1), "unit": "assembled KV tokens/s", "cores": 1,
            "kind": "oracle", "host": host_cpu(),
            "sample": f"first {done_req} of {w.n_seq} requests ({done_tokens} tokens), "
                      f"{spent:.1f} s single-threaded float64 numpy"}


def host_cpu() -> str:
    """Host cores and CPU model, for the oracle baselines."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"1 of {os.cpu_count()} host cores ({model})"


def _oracle_rows(w, b, inv):
    """Assembled rows of sequence b by the oracle (table expansion, float64
    rotation)."""
    import numpy as np
    import oracle
    lo, hi = int(w.seq_first[b]), int(w.seq_first[b + 1])
    (g, d, _), = oracle.expand_table(w.chunks[lo:hi], np.array([0, hi - lo]), w.pool.shape[0])
    return oracle.assemble_rows(w.pool, g, d, inv)


def cpu_baseline_decode(w, seconds: float):
    """The oracle, single-threaded, on whole sequences of a decode batch (row
    assembly and attention) until ``seconds`` have been spent (at least one);
    algorithmic bytes per second as for the GPU leg."""
    from threadpoolctl import threadpool_limits
    import oracle

    inv = oracle.rope_inv_freq(w.theta)
    done, tokens, spent = 0, 0, 0.0
    with threadpool_limits(limits=1):
        while done < w.n_seq and (spent < seconds or done == 0):
            t0 = time.perf_counter()
            c, k = _oracle_rows(w, done, inv)
            oracle.mla_decode(oracle.bf16_to_f64(w.q_lat[done]), oracle.bf16_to_f64(w.q_rope[done]), c, k, w.scale)
            spent += time.perf_counter() - t0
            tokens += c.shape[0]
            done += 1
    nbytes = ROW_BYTES * tokens + done * w.n_heads * (576 + 512) * 2
    return {"value": round(nbytes / spent / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle", "host": host_cpu(),
            "sample": f"first {done} of {w.n_seq} sequences ({tokens} cached tokens, {w.n_heads} heads), "
                      f"{spent:.1f} s single-threaded float64 numpy"}


def cpu_baseline_prefill(w, seconds: float):
    """The oracle, single-threaded: the 65536-row cache assembled once (timed
    apart), then the first queries of the tail in blocks of 4 until
    ``seconds`` of attention have been spent; algorithmic flops per second of
    the attention as for the GPU leg."""
    from threadpoolctl import threadpool_limits
    import oracle

    inv = oracle.rope_inv_freq(w.theta)
    nq, H = w.q_lat.shape[0], w.n_heads
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        c, k = _oracle_rows(w, 0, inv)
        assemble_s = time.perf_counter() - t0
        done, spent, flops = 0, 0.0, 0.0
        while done < nq and (spent < seconds or done == 0):
            hi = min(nq, done + 4)
            t0 = time.perf_counter()
            oracle.mla_prefill_tail(oracle.bf16_to_f64(w.q_lat[done:hi]), oracle.bf16_to_f64(w.q_rope[done:hi]),
                                    c, k, w.q_pos0 + done, w.scale)
            spent += time.perf_counter() - t0
            flops += sum(w.q_pos0 + i + 1 for i in range(done, hi)) * H * 2 * (576 + 512)
            done = hi
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": 1, "kind": "oracle", "host": host_cpu(),
            "sample": f"first {done} of {nq} queries over {c.shape[0]} rows ({spent:.1f} s of attention; the "
                      f"cache assembly took {assemble_s:.1f} s apart), single-threaded float64 numpy"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--legs", default="gather,gather_cdc,tiny,decode,long_decode,prefill,nonabsorbed,gqa,producer",
                    help="comma list; without gather only the named legs run (profiling, no JSON line)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cpu-seconds-legs", type=float, default=5.0,
                    help="oracle seconds per decode / prefill leg (its own cpu_baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--leg-warm-ms", type=float, default=LEG_WARM_MS,
                    help="least warm-up time of the decode and prefill legs (0 in profiling mode)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="run a plain 1 GiB device copy (for scaling HBM counters) and exit")
    ap.add_argument("--profile", action="store_true",
                    help="run the named legs only, without the JSON line or the CPU baseline")
    ap.add_argument("--ingest-counters", nargs=5, metavar=("KEY", "FETCH", "WRITE", "CAL_FETCH", "CAL_WRITE"),
                    help="record rocprofv3 FETCH_SIZE/WRITE_SIZE runs of a kernel (scaled by the copy runs) "
                         "in profiles/traffic.json and exit; KEY is e.g. rotate_gather_kernel or "
                         "decode_private_kernel:<workload name>")
    args = ap.parse_args()
    if args.ingest_counters:
        ingest_counters(*args.ingest_counters)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path shards by request "
              "or sequence with no exchange, and the benchmark measures one GPU's share.", file=sys.stderr)
        sys.exit(2)

    import torch
    import mla_position_independent_amd as irm
    import synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    irm.lib()

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied 1 GiB x 5")
        return

    legs = [x.strip() for x in args.legs.split(",") if x.strip()]
    if args.profile or "gather" not in legs:
        # profiling mode: run the requested legs only, no JSON line, no oracle
        args.no_cpu_baseline = True
        args.leg_warm_ms = 0.0  # counters and traces need no settled clock
        g = None
        for name in legs:
            if name == "gather":
                g = leg_gather(args, irm, torch, synth)
            elif name == "gather_cdc":
                leg_gather_cdc(args, irm, torch, synth)
            elif name == "tiny":
                leg_tiny(args, irm, torch, synth)
            elif name == "decode":
                leg_decode(args, irm, torch, synth, "batched decode", synth.batched_decode)
            elif name == "long_decode":
                leg_decode(args, irm, torch, synth, "long decode", synth.long_decode)
            elif name == "prefill":        # the assembled-cache pair only (one prefill instantiation)
                leg_prefill(args, irm, torch, synth, fused=False)
            elif name == "prefill_fused":  # the single kernel with rotation on load only
                leg_prefill(args, irm, torch, synth, assembled=False)
            elif name == "producer":
                leg_producer(args, irm, synth, 0.0)
            elif name == "nonabsorbed":
                leg_nonabsorbed(args, irm, torch, synth)
            elif name == "gqa":
                leg_gqa(args, irm, torch, leg_gather(args, irm, torch, synth) if g is None else g)
        return
    g = leg_gather(args, irm, torch, synth)
    extra = {}
    if "gather_cdc" in legs:
        extra["gather_cdc"] = leg_gather_cdc(args, irm, torch, synth)
    if "tiny" in legs:
        extra["tiny_decode"] = leg_tiny(args, irm, torch, synth)
    if "decode" in legs:
        extra["decode"] = leg_decode(args, irm, torch, synth, "batched decode", synth.batched_decode)
    if "long_decode" in legs:
        extra["long_decode"] = leg_decode(args, irm, torch, synth, "long decode", synth.long_decode)
    if "prefill" in legs:
        extra["prefill"] = leg_prefill(args, irm, torch, synth)
    if "nonabsorbed" in legs:
        extra["prefill_nonabsorbed"] = leg_nonabsorbed(args, irm, torch, synth)
    if "gqa" in legs:
        extra["gqa_comparison"] = leg_gqa(args, irm, torch, g)
    if "producer" in legs:
        extra["producer"] = leg_producer(args, irm, synth, 0.0 if args.no_cpu_baseline else 3.0)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on a sample of the rotate-gather batch")
        cpu = cpu_baseline(g["workload"], args.cpu_seconds)

    w = g["workload"]
    line = {
        "metric": METRIC,
        "value": round(g["tokens"] / (g["ms_per_step"] * 1e-3), 1),
        "unit": "assembled KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(g["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16 rows; chunk tables from the pages' CDC bounds)",
        "config": {"workload": w.name, "requests": w.n_seq, "tokens_per_request": 32768,
                   "registry_chunks": w.meta["n_registry"], "chunk_len": "uniform[32,512]",
                   "hit_fraction_by_entry": 0.8, "p_src_range": [0, 131072], "row": "576 x bf16",
                   "step": "per-batch device passes of the chunk table (row map + per-entry trig) + rotate-gather, "
                           "the table's image and the pool resident in HBM"},
        "table_prepare_ms": g["table_prepare_ms"],
        "table_upload_ms": g["table_upload_ms"],
        "table_h2d_bytes": g["table_h2d_bytes"],
        "sclk": g["sclk"],
        "roofline": g["roofline"],
        "cpu_baseline": cpu,
        "legs": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
