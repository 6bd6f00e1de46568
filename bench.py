"""Benchmark of the AXELRAM-style write + score path on one MI355X.

A step is one pass of the whole hot path over the LLaMA-3.1-8B-shaped GQA
decode cache (batch 8, 8 KV heads, 32 query heads, d = 128, b = 3, 32768
tokens, fp16 keys): quantize every key (normalise, sign pattern, WHT,
Lloyd-Max bucketize, pack) and score every query head against the packed
cache (query transform, LUT in LDS, lookup-accumulate).  Inputs are resident
in HBM before timing starts.

Prints one JSON line:
  * value: keys per second through the timed steps (whole-job throughput);
  * roofline: the score kernel (the kernel the bandwidth target names) with
    every launch reading its records from HBM (back to back over eight copies
    of the cache, four times the Infinity Cache), duration from HIP events on
    the stream it runs on; roofline_write: the write kernel alike;
  * configs: write and score kernel times on every workload shape (tiny;
    LLaMA decode; all 36 Qwen2.5-3B layers; long context at b = 2, 3, 4; the
    nine write-sweep cells), each kernel cycling over enough buffer copies
    that its inputs come from HBM.  Per-kernel loops run from a captured
    graph (one pass over the copies, replayed): a launch through the Python
    binding costs the host ~20-30 us, more than the shorter kernels take;
  * cpu_baseline: the fp64 oracle on bounded samples of every workload, its
    quantize and score rates reported separately.

--profile KERNEL runs only that kernel's timed loop (for a rocprofv3 kernel
trace or counter pass whose averages then cover exactly those launches) and
prints its HIP-event figure.
"""

import argparse
import gc
import glob
import hashlib
import json
import math
import os
import re
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
CUS, CLOCK_HZ = 256, 2.4e9        # MI355X compute units and peak engine clock
METRIC = "quantized keys scored/sec + achieved HBM GB/s (d=128, b=3, GQA decode)"
CSRC = os.path.join(ROOT, "lut_attention_scoring_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")

# Sources whose compiled code a kernel's counter figures depend on.
KERNEL_SOURCES = {
    "write": ["axr_write.hip", "axr_keyquant.h", "axr_device.h", "axr_internal.h"],
    "score": ["axr_score.hip", "axr_keyquant.h", "axr_device.h", "axr_internal.h"],
    "fused": ["axr_score.hip", "axr_keyquant.h", "axr_device.h", "axr_internal.h"],
}

WARM_MS = 30.0   # time each kernel runs untimed before its timed launches
SETTLE_MS = 100.0  # step loop run untimed before the warmup steps


def sources_sha1(kernel):
    h = hashlib.sha1()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def counter_traffic(kernel):
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE / WRITE_SIZE passes
    summarised in profiles/: each summary carries a line
      counter-traffic: kernel=K sources_sha1=S fetch_kib=F write_kib=W
                       fetch_factor=a write_factor=b
    written from the run that took the counters (S is the SHA-1 of the
    kernel's sources in that run).  Bytes = (F a + W b) * 1024 if S equals the
    current sources' SHA-1, else None (the kernel changed since)."""
    want = sources_sha1(kernel)
    pat = re.compile(r"counter-traffic:\s*kernel=(\w+)\s+sources_sha1=([0-9a-f]+)\s+"
                     r"fetch_kib=([0-9.]+)\s+write_kib=([0-9.]+)\s+fetch_factor=([0-9.]+)\s+"
                     r"write_factor=([0-9.]+)")
    for path in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        with open(path) as f:
            for m in pat.finditer(f.read()):
                if m.group(1) == kernel and m.group(2) == want:
                    fk, wk, ff, wf = (float(m.group(i)) for i in range(3, 7))
                    return (fk * ff + wk * wf) * 1024.0
    return None


def counter_valu(kernel):
    """VALU wave instructions per launch from the rocprofv3 SQ_INSTS_VALU pass
    summarised in profiles/ (a line "counter-valu: kernel=K sources_sha1=S
    valu_per_launch=V"), gated on the sources' SHA-1 like counter_traffic."""
    want = sources_sha1(kernel)
    pat = re.compile(r"counter-valu:\s*kernel=(\w+)\s+sources_sha1=([0-9a-f]+)\s+"
                     r"valu_per_launch=([0-9.]+)")
    for path in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        with open(path) as f:
            for m in pat.finditer(f.read()):
                if m.group(1) == kernel and m.group(2) == want:
                    return float(m.group(3))
    return None


def valu_issue(kernel, us):
    """Wave64 VALU instructions per CU-cycle over a launch of `us` (256 CUs at
    2.4 GHz), from the counted instructions; None without a current count."""
    v = counter_valu(kernel)
    return None if v is None else round(v / (CUS * CLOCK_HZ * us * 1e-6), 3)


def launches_ms(torch, stream, fn, reps, warm_ms=WARM_MS):
    """Average duration of `reps` back-to-back launches of fn, from HIP events
    recorded on the stream the kernels run on.  Before the start event the
    kernel runs untimed for `warm_ms` of wall time, and a few more launches
    are queued right before the event: the chip needs several milliseconds of
    a given load before its clock settles, and that transient belongs to no
    kernel.  Python's cyclic garbage collector is held off (a full collection
    of this process stalls the launching thread for tens of milliseconds)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gc.collect()
    gc.disable()
    try:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < warm_ms * 1e-3:
            for _ in range(8):
                fn()
            torch.cuda.synchronize()
        for _ in range(8):
            fn()
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
    finally:
        gc.enable()
    return e0.elapsed_time(e1) / reps


def graph_ms(torch, stream, fn, calls, reps, warm_ms=WARM_MS):
    """Average duration of one of `calls` launches of fn captured in a HIP
    graph, replayed back to back between HIP events: the host takes ~20-30 us
    per launch through the binding, longer than the shorter kernels run, so
    host-launched loops would time the host for them.  The graph holds one
    pass of fn over the rotating copies (`calls` launches); it is replayed
    untimed for `warm_ms` first (clock settling), then `reps` launches' worth
    of replays are timed."""
    dev = torch.device("cuda:0")
    for _ in range(calls):                      # eager pass: lazy initialisation
        fn()
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for _ in range(calls):
            fn()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls):
            fn()
    torch.cuda.synchronize()
    n = max(1, reps // calls)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    gc.collect()
    gc.disable()
    try:
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < warm_ms * 1e-3:
            graph.replay()
            torch.cuda.synchronize()
        graph.replay()
        e0.record(stream)
        for _ in range(n):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    finally:
        gc.enable()
    del graph
    return e0.elapsed_time(e1) / (n * calls)


class Rotor:
    """Calls fn(copy) cycling over buffer copies."""

    def __init__(self, copies, fn):
        self.copies, self.fn, self.i = copies, fn, 0

    def __call__(self):
        c = self.copies[self.i % len(self.copies)]
        self.i += 1
        self.fn(c)


def graph_calls(k):
    """Launches per captured graph: whole passes over the k copies, >= 16."""
    return k * max(1, math.ceil(16 / k))


def n_copies(bytes_per_copy, min_copies=4, cycle_bytes=1 << 30):
    """Copies to cycle over so that one cycle moves >= 1 GiB (four times the
    256 MB Infinity Cache) and at least `min_copies`."""
    return max(min_copies, math.ceil(cycle_bytes / max(bytes_per_copy, 1)))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed step loop before the warmup steps (clock settling)")
    ap.add_argument("--cold-reps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the every-workload section")
    ap.add_argument("--profile", choices=["score_rotating", "score_resident", "write",
                                          "qwen_score", "long_score_b2", "long_score_b3",
                                          "long_score_b4", "write_sweep", "fused",
                                          "calibrate"],
                    help="run only this kernel's timed loop and print its figure "
                         "(calibrate: a 1 GiB read stream and a 1 GiB write stream, "
                         "the known sizes that scale rocprofv3's FETCH_SIZE and WRITE_SIZE)")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# Inputs
# ---------------------------------------------------------------------------

def gen_parallel(fns, workers=16):
    """Runs the generators in threads (numpy's generators release the GIL)."""
    with ThreadPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(lambda f: f(), fns))


def score_bytes_per_key(d, b, G):
    return d * b // 8 + 4 + 4 * G


def write_bytes_per_key(d, b, elt):
    return d * elt + d * b // 8 + 4


# ---------------------------------------------------------------------------
# Every workload shape
# ---------------------------------------------------------------------------

def time_write(torch, axr, stream, keys, bits, b, reps):
    """Write kernel over rotating copies of the keys (records and norms of
    each copy written to their own buffers)."""
    dev = keys.device
    n = keys.numel() // keys.shape[-1]
    d = keys.shape[-1]
    per = write_bytes_per_key(d, b, keys.element_size()) * n
    k = n_copies(per, min_copies=2)
    copies = [keys] + [keys.clone() for _ in range(k - 1)]
    outs = [(torch.empty(n, d * b // 32, dtype=torch.int32, device=dev),
             torch.empty(n, dtype=torch.float32, device=dev)) for _ in range(k)]
    pairs = list(zip(copies, outs))
    rot = Rotor(pairs, lambda c: axr.quantize_keys(c[0], bits, b, packed=c[1][0],
                                                   norms=c[1][1]))
    ms = graph_ms(torch, stream, rot, graph_calls(k), reps)
    del copies, outs, pairs
    return {"us": ms * 1e3, "keys_per_s": n / (ms * 1e-3), "bytes": per,
            "GB_per_s": per / (ms * 1e6), "frac_hbm": per / (ms * 1e6) / HBM_PEAK_GBS,
            "copies": k}


def table_read_bytes_per_key(d, b, G):
    """LDS bytes of table entries the score kernel reads per key: d/P lookups
    of 16 bytes (four heads) per group of four query heads, with P the
    coordinates per table entry that the library picks for (d, b)."""
    if d == 128:
        p = 4 if b == 2 else 2
    elif b == 4 or (d == 512 and b == 3):
        p = 1
    else:
        p = 2
    return (d // p) * ((G + 3) // 4) * 16


def time_fused(torch, axr, stream, keys, q, bits, b, reps):
    """Quantize-and-score over rotating copies of the keys, each with its own
    records, norms and score rows."""
    dev = keys.device
    B, Hkv, T, d = keys.shape
    Hq = q.shape[1]
    n = B * Hkv * T
    per = (write_bytes_per_key(d, b, keys.element_size()) + 4 * (Hq // Hkv)) * n
    k = n_copies(per, min_copies=2)
    copies = [(keys if i == 0 else keys.clone(),
               torch.empty(B, Hkv, T, d * b // 32, dtype=torch.int32, device=dev),
               torch.empty(B, Hkv, T, dtype=torch.float32, device=dev),
               torch.empty(B, Hq, T, dtype=torch.float32, device=dev)) for i in range(k)]
    rot = Rotor(copies, lambda c: axr.quantize_score(c[0], q, bits, b, packed=c[1], norms=c[2],
                                                     out=c[3]))
    ms = graph_ms(torch, stream, rot, graph_calls(k), reps)
    del copies
    return {"us": ms * 1e3, "keys_per_s": n / (ms * 1e-3), "bytes": per,
            "GB_per_s": per / (ms * 1e6), "frac_hbm": per / (ms * 1e6) / HBM_PEAK_GBS,
            "copies": k}


def time_score(torch, axr, stream, q, packed, norms, bits, b, reps, min_copies=4):
    """Score kernel over rotating copies of records, norms and score rows."""
    B, Hq, _ = q.shape
    _, Hkv, T, W = packed.shape
    n = B * Hkv * T
    d = q.shape[-1]
    per = score_bytes_per_key(d, b, Hq // Hkv) * n
    k = n_copies(per, min_copies=min_copies)
    copies = [(packed, norms, torch.empty(B, Hq, T, device=q.device))] + [
        (packed.clone(), norms.clone(), torch.empty(B, Hq, T, device=q.device))
        for _ in range(k - 1)]
    rot = Rotor(copies, lambda c: axr.score(q, c[0], c[1], bits, b, out=c[2]))
    ms = graph_ms(torch, stream, rot, graph_calls(k), reps)
    del copies
    lds = n * table_read_bytes_per_key(d, b, Hq // Hkv)
    return {"us": ms * 1e3, "keys_per_s": n / (ms * 1e-3),
            "head_scores_per_s": n * (Hq // Hkv) / (ms * 1e-3), "bytes": per,
            "lds_table_bytes": lds,
            "lds_B_per_cu_cycle": round(lds / (CUS * CLOCK_HZ * ms * 1e-3), 1),
            "GB_per_s": per / (ms * 1e6), "frac_hbm": per / (ms * 1e6) / HBM_PEAK_GBS,
            "copies": k}


def configs_section(torch, axr, W, stream, reps):
    dev = torch.device("cuda:0")
    out = {}

    # tiny: 4096 keys, one query (latency-bound; fits every cache)
    w = W.tiny()
    keys, q = w["keys"].to(dev), w["q"].to(dev)
    packed, norms = axr.quantize_keys(keys, w["sign_bits"], 3)
    wr = graph_ms(torch, stream, lambda: axr.quantize_keys(keys, w["sign_bits"], 3,
                                                           packed=packed, norms=norms), 16, reps)
    sc = torch.empty(1, 1, 4096, device=dev)
    sr = graph_ms(torch, stream, lambda: axr.score(q, packed.view(1, 1, 4096, 12),
                                                   norms.view(1, 1, 4096), w["sign_bits"], 3,
                                                   out=sc), 16, reps)
    pk1, nm1 = packed.view(1, 1, 4096, 12), norms.view(1, 1, 4096)
    fr = graph_ms(torch, stream, lambda: axr.quantize_score(keys, q, w["sign_bits"], 3,
                                                            packed=pk1, norms=nm1, out=sc),
                  16, reps)
    out["tiny_d128_b3_n4096"] = {"keys": 4096, "write_us": wr * 1e3, "score_us": sr * 1e3,
                                 "quantize_score_us": fr * 1e3,
                                 "note": "back to back from a graph; 0.2 MiB per launch, "
                                         "latency-bound; quantize_score = both in one launch"}
    log("configs: tiny done")

    # LLaMA-3.1-8B decode cache (the headline workload)
    w = W.llama_decode()
    keys, q, bits = w["keys"].to(dev), w["q"].to(dev), w["sign_bits"]
    del w
    packed, norms = axr.quantize_keys(keys, bits, 3)
    out["llama31_8b_gqa_decode_d128_b3"] = {
        "keys": keys.numel() // 128,
        "write": time_write(torch, axr, stream, keys, bits, 3, reps),
        "score": time_score(torch, axr, stream, q, packed, norms, bits, 3, reps)}
    del keys, q, packed, norms
    torch.cuda.empty_cache()
    log("configs: LLaMA done")

    # Qwen2.5-3B: all 36 layers, each with its own cache; one pass quantizes
    # (then scores) every layer back to back, 36 x 186 MB from HBM
    layers = gen_parallel([lambda l=l: W.qwen_layer(l) for l in range(W.QWEN_LAYERS)])
    L = len(layers)
    bits = layers[0]["sign_bits"]
    lk = [x["keys"].to(dev) for x in layers]
    lq = [x["q"].to(dev) for x in layers]
    del layers
    lp = [axr.quantize_keys(k, bits, 4) for k in lk]
    B, Hkv, T, d = lk[0].shape
    Hq = lq[0].shape[1]
    ls = [torch.empty(B, Hq, T, device=dev) for _ in range(L)]
    n = B * Hkv * T

    # one graph holds a pass over the 36 layers
    write_one = Rotor(list(zip(lk, lp)), lambda c: axr.quantize_keys(
        c[0], bits, 4, packed=c[1][0], norms=c[1][1]))
    score_one = Rotor(list(zip(lq, lp, ls)), lambda c: axr.score(
        c[0], c[1][0], c[1][1], bits, 4, out=c[2]))
    passes = max(2, reps // 4)
    wms = graph_ms(torch, stream, write_one, L, passes * L) * L
    sms = graph_ms(torch, stream, score_one, L, passes * L) * L
    wb = write_bytes_per_key(d, 4, 2) * n
    sb = score_bytes_per_key(d, 4, Hq // Hkv) * n
    out["qwen25_3b_layer_sweep_d128_b4"] = {
        "layers": L, "keys_per_layer": n,
        "write_all_layers_us": wms * 1e3, "score_all_layers_us": sms * 1e3,
        "write_per_layer_us": wms * 1e3 / L, "score_per_layer_us": sms * 1e3 / L,
        "write_GB_per_s": wb * L / (wms * 1e6), "score_GB_per_s": sb * L / (sms * 1e6),
        "write_frac_hbm": wb * L / (wms * 1e6) / HBM_PEAK_GBS,
        "score_frac_hbm": sb * L / (sms * 1e6) / HBM_PEAK_GBS,
        "score_keys_per_s": n * L / (sms * 1e-3), "write_keys_per_s": n * L / (wms * 1e-3),
        "score_lds_B_per_cu_cycle": round(n * L * table_read_bytes_per_key(d, 4, Hq // Hkv) /
                                          (CUS * CLOCK_HZ * sms * 1e-3), 1),
        "note": "one pass = every layer back to back on its own cache (layer sum); "
                f"{passes} passes timed"}
    del lk, lq, lp, ls
    torch.cuda.empty_cache()
    log("configs: Qwen done")

    # long context, b = 2, 3, 4 (the keys do not depend on b)
    w = W.long_context(b=3)
    keys, q, bits = w["keys"].to(dev), w["q"].to(dev), w["sign_bits"]
    del w
    lc = {}
    for b in (2, 3, 4):
        packed, norms = axr.quantize_keys(keys, bits, b)
        lc[f"b{b}"] = {"write": time_write(torch, axr, stream, keys, bits, b, reps),
                       "score": time_score(torch, axr, stream, q, packed, norms, bits, b, reps)}
        if b == 3:   # G = 8 in one launch (two tables per block)
            lc["b3"]["quantize_score"] = time_fused(torch, axr, stream, keys, q, bits, b, reps)
        del packed, norms
    out["long_context_t131072_d128"] = dict(keys=keys.numel() // 128, **lc)
    del keys, q
    torch.cuda.empty_cache()
    log("configs: long context done")

    out["write_sweep_t32768x8"] = write_sweep_section(torch, axr, W, stream, reps)
    log("configs: write sweep done")
    return out


def time_shaped_stream(torch, axr, stream, in_bytes, out_bytes, reps):
    """The bare read-then-write stream probe with the given traffic, cycling
    over enough disjoint regions that every launch reads from HBM."""
    dev = torch.device("cuda:0")
    k = n_copies(in_bytes + out_bytes, min_copies=2)
    ins = [torch.empty(in_bytes, dtype=torch.uint8, device=dev) for _ in range(k)]
    outs = [torch.empty(out_bytes, dtype=torch.uint8, device=dev) for _ in range(k)]
    rot = Rotor(list(zip(ins, outs)), lambda c: axr.probe_read_write(c[0], in_bytes, c[1],
                                                                    out_bytes))
    ms = graph_ms(torch, stream, rot, graph_calls(k), reps)
    del ins, outs
    return ms


def write_sweep_section(torch, axr, W, stream, reps):
    """Write kernel on the nine sweep cells (32768 tokens x 8 KV heads of bf16
    keys, d x b; the keys do not depend on b), each beside the bare stream with
    the same traffic (keys in, records and norms out), both from HBM."""
    dev = torch.device("cuda:0")
    ws = {}
    for d in (128, 256, 512):
        w = W.write_sweep(d=d, b=3)
        keys, bits = w["keys"].to(dev), w["sign_bits"]
        del w
        n = keys.numel() // d
        for b in (2, 3, 4):
            r = time_write(torch, axr, stream, keys, bits, b, reps)
            st = time_shaped_stream(torch, axr, stream, n * d * 2, n * (d * b // 8 + 4), reps)
            r["shaped_stream_us"] = st * 1e3
            r["frac_of_shaped_stream"] = st * 1e3 / r["us"]
            ws[f"d{d}_b{b}"] = r
        del keys
        torch.cuda.empty_cache()
    return ws


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on bounded samples of every workload
# ---------------------------------------------------------------------------

def cpu_baseline():
    """The fp64 oracle as it stands, on a bounded, stated sample of every
    workload (quantize = write path, score = read path, timed separately).
    BLAS threads are pinned to the process's CPU affinity count; only the
    dense Hadamard product uses them, the rest of the oracle runs on one."""
    import numpy as np
    import threadpoolctl
    import torch
    import workloads as W
    from oracle import axelram as A

    cores = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    per = {}

    def run(name, keys, q, bits, b, note):
        k = keys.to(torch.float64).numpy()
        s = A.signs_from_bits(bits)
        t0 = time.perf_counter()
        wr = A.write_path(k, s, b)
        tq = time.perf_counter() - t0
        n = int(np.prod(k.shape[:-1]))
        entry = {"keys": n, "quantize_s": tq, "quantize_keys_per_s": n / tq, "sample": note}
        if q is not None:
            qq = q.to(torch.float64).numpy()
            t0 = time.perf_counter()
            A.read_path(qq, wr["packed"], wr["norms"], s, b)
            ts = time.perf_counter() - t0
            entry.update({"score_s": ts, "score_keys_per_s": n / ts,
                          "quantize_and_score_keys_per_s": n / (tq + ts)})
        per[name] = entry
        return entry

    with threadpoolctl.threadpool_limits(limits=cores, user_api="blas"):
        w = W.tiny()
        run("tiny_d128_b3_n4096", w["keys"], w["q"], w["sign_bits"], 3, "all 4096 keys, 1 query")
        w = W.llama_decode(B=1, T=16384)
        head = run("llama31_8b_gqa_decode_d128_b3", w["keys"], w["q"], w["sign_bits"], 3,
                   "the workload's recipe at batch 1 and 16384 tokens: 8 KV heads x 16384 = "
                   "131072 keys, 32 query heads")
        del w
        tq = ts = nk = 0.0
        for layer in range(W.QWEN_LAYERS):
            w = W.qwen_layer(layer, B=1, T=1024)
            e = run(f"qwen_layer{layer}", w["keys"], w["q"], w["sign_bits"], 4, "")
            tq, ts, nk = tq + e["quantize_s"], ts + e["score_s"], nk + e["keys"]
            del per[f"qwen_layer{layer}"]
        per["qwen25_3b_layer_sweep_d128_b4"] = {
            "keys": int(nk), "quantize_keys_per_s": nk / tq, "score_keys_per_s": nk / ts,
            "quantize_and_score_keys_per_s": nk / (tq + ts),
            "quantize_s": tq, "score_s": ts,
            "sample": "every one of the 36 layers, generated with batch 1 and 1024 tokens "
                      "(2 KV heads, 16 query heads): 2048 keys per layer"}
        w = W.long_context(b=3, T=8192)
        for b in (2, 3, 4):
            run(f"long_context_b{b}", w["keys"], w["q"], w["sign_bits"], b,
                "the workload's recipe at 8192 tokens: 8 KV heads x 8192 = 65536 keys, "
                "64 query heads")
        del w
        for d in (128, 256, 512):
            w = W.write_sweep(d=d, b=3, T=4096)
            for b in (2, 3, 4):
                run(f"write_sweep_d{d}_b{b}", w["keys"], None, w["sign_bits"], b,
                    "the workload's recipe at 4096 tokens: 8 KV heads x 4096 = 32768 keys "
                    "(write path only)")
            del w
    total = sum(e.get("quantize_s", 0.0) + e.get("score_s", 0.0) for e in per.values())
    return {"value": head["quantize_and_score_keys_per_s"], "unit": "keys/s", "cores": int(cores),
            "kind": "oracle",
            "sample": "LLaMA-3.1-8B decode cache recipe at batch 1, 8 KV heads x 16384 tokens "
                      "(131072 keys) quantized and scored by 32 query heads, fp64 numpy; every "
                      f"other workload sampled in per_config; host reports {os.cpu_count()} CPUs, "
                      f"{cores} in this process's affinity (BLAS threads)",
            "per_config": per, "oracle_seconds_sampled": total}


# ---------------------------------------------------------------------------
# Main
# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: there is no multi-GPU path "
              "(the score and write paths shard with no exchange)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import lut_attention_scoring_amd as axr
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    log("generating LLaMA-3.1-8B-shaped decode cache")
    w = W.llama_decode()
    B, Hkv, T, d = w["keys"].shape
    Hq = w["q"].shape[1]
    G = Hq // Hkv
    b, bits = w["b"], w["sign_bits"]
    n = B * Hkv * T
    keys = w["keys"].to(dev)
    q = w["q"].to(dev)
    del w
    packed = torch.empty(B, Hkv, T, d * b // 32, dtype=torch.int32, device=dev)
    norms = torch.empty(B, Hkv, T, dtype=torch.float32, device=dev)
    scores = torch.empty(B, Hq, T, dtype=torch.float32, device=dev)
    axr.quantize_keys(keys, bits, b, packed=packed, norms=norms)
    wbytes = n * write_bytes_per_key(d, b, keys.element_size())
    sbytes = n * score_bytes_per_key(d, b, G)

    if args.profile:
        k = args.profile
        if k == "calibrate":
            del keys, q, packed, norms, scores
            torch.cuda.empty_cache()
            gib = 1 << 30
            buf = torch.empty(gib, dtype=torch.uint8, device=dev)
            sink = torch.zeros(16, dtype=torch.int32, device=dev)
            buf.fill_(1)
            torch.cuda.synchronize()
            rd = launches_ms(torch, stream, lambda: axr.probe_read_stream(buf, sink, gib),
                             max(args.steps, 3), warm_ms=0.0)
            wr = launches_ms(torch, stream, lambda: axr.probe_read_write(sink, 0, buf, gib),
                             max(args.steps, 3), warm_ms=0.0)
            print(json.dumps({"profile": k, "read_stream_bytes": gib, "read_stream_us": rd * 1e3,
                              "read_write_stream_write_bytes": gib,
                              "read_write_stream_us": wr * 1e3}), flush=True)
            return
        if k == "write_sweep":
            del keys, q, packed, norms, scores
            torch.cuda.empty_cache()
            print(json.dumps({"profile": k, **write_sweep_section(torch, axr, W, stream,
                                                                  args.steps)}), flush=True)
            return
        if k in ("score_rotating", "score_resident"):
            r = time_score(torch, axr, stream, q, packed, norms, bits, b, args.steps,
                           min_copies=4 if k == "score_rotating" else 1) \
                if k == "score_rotating" else None
            if r is None:
                ms = graph_ms(torch, stream,
                              lambda: axr.score(q, packed, norms, bits, b, out=scores),
                              16, args.steps)
                r = {"us": ms * 1e3, "GB_per_s": sbytes / (ms * 1e6)}
        elif k == "write":
            r = time_write(torch, axr, stream, keys, bits, b, args.steps)
        elif k == "fused":
            r = time_fused(torch, axr, stream, keys, q, bits, b, args.steps)
        else:
            del keys
            if k == "qwen_score":
                w = W.qwen_layer(0)
                bb = 4
            else:
                bb = int(k[-1])                   # long_score_b2 / b3 / b4
                w = W.long_context(b=bb)
            kk, qq = w["keys"].to(dev), w["q"].to(dev)
            pk, nm = axr.quantize_keys(kk, w["sign_bits"], bb)
            r = time_score(torch, axr, stream, qq, pk, nm, w["sign_bits"], bb, args.steps)
        print(json.dumps({"profile": k, **r}), flush=True)
        return

    # A step quantizes every key (records and norms stored) and scores every
    # query head against them: one launch of the quantize-and-score kernel.
    # The same work as two launches (write kernel, then score kernel) is
    # timed the same way beside it.
    def step():
        axr.quantize_score(keys, q, bits, b, packed=packed, norms=norms, out=scores)

    def step_two_launches():
        axr.quantize_keys(keys, bits, b, packed=packed, norms=norms)
        axr.score(q, packed, norms, bits, b, out=scores)

    # Steps run untimed for settle_ms first: a write + score loop starting
    # from an idle chip runs its first ~10 ms up to half slower while the
    # clock ramps; then the warmup steps, then the timed steps (wall clock
    # between two synchronisations), then as many two-launch steps with HIP
    # events around each kernel (on the stream the kernels run on) for the
    # split.
    log(f"settle {args.settle_ms:.0f} ms, warmup {args.warmup}, timing {args.steps} steps")
    gc.collect()
    gc.disable()

    def timed_steps(fn):
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < args.settle_ms * 1e-3:
            for _ in range(16):
                fn()
            torch.cuda.synchronize()
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            fn()
        torch.cuda.synchronize()
        return time.perf_counter() - t0

    elapsed = timed_steps(step)
    elapsed_two = timed_steps(step_two_launches)
    # The same number of steps again with HIP events around each kernel, for
    # the split between the two: an event recorded between the kernels costs
    # the GPU ~2 us, so these are not the timed steps.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for e in ev:
        e[0].record(stream)
        axr.quantize_keys(keys, bits, b, packed=packed, norms=norms)
        e[1].record(stream)
        axr.score(q, packed, norms, bits, b, out=scores)
        e[2].record(stream)
    torch.cuda.synchronize()
    gc.enable()
    ms_per_step = elapsed * 1e3 / args.steps
    ms_per_step_two = elapsed_two * 1e3 / args.steps
    step_write_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    step_score_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps

    def per_launch_ms(fn, reps):
        return launches_ms(torch, stream, fn, reps)

    def per_graph_ms(fn, reps, calls=16):
        return graph_ms(torch, stream, fn, calls, reps)

    log("per-kernel timing")
    fused_hbm = time_fused(torch, axr, stream, keys, q, bits, b, args.steps)
    write_hbm = time_write(torch, axr, stream, keys, bits, b, args.steps)
    score_hbm = time_score(torch, axr, stream, q, packed, norms, bits, b, args.steps)
    score_res_ms = per_graph_ms(lambda: axr.score(q, packed, norms, bits, b, out=scores),
                                args.steps)

    # Decode step on the same cache: one new key per (sequence, KV head)
    # appended at the last slot, then every sequence scored up to it.
    log("decode-step timing")
    rng = np.random.default_rng(105)
    new_k = torch.from_numpy(rng.standard_normal((B, Hkv, d)).astype(np.float32)).to(
        keys.dtype).to(dev)
    pos = torch.full((B,), T - 1, dtype=torch.int32, device=dev)
    lens = pos + 1

    def append():
        axr.append_keys(new_k, bits, b, packed, norms, pos)

    def decode_step():
        append()
        axr.score(q, packed, norms, bits, b, out=scores, lens=lens)

    append_ms = per_graph_ms(append, args.steps)
    decode_ms = per_launch_ms(decode_step, args.steps)
    fused_ms = per_graph_ms(
        lambda: axr.decode_step(q, new_k, bits, b, packed, norms, pos, out=scores), args.steps)
    side = torch.cuda.Stream(dev)
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        decode_step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        decode_step()
    torch.cuda.synchronize()
    decode_graph_ms = per_launch_ms(graph.replay, args.steps)
    del graph

    log("softmax timing")
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    ws = torch.empty(max(8, axr.score_softmax_workspace_bytes(B, Hq, Hkv, T, d, b)),
                     dtype=torch.uint8, device=dev)
    softmax_ms = per_launch_ms(
        lambda: axr.score_softmax(q, packed, norms, bits, b, out=scores, lse=lse, workspace=ws),
        args.steps)

    # Score kernel alone after 2 GiB of reads (cold cache, single launches).
    log("cold-cache score timing")
    flush = torch.ones(1 << 29, dtype=torch.float32, device=dev)
    flush_bytes = flush.numel() * flush.element_size()
    sink = torch.empty((), dtype=torch.float32, device=dev)
    cold = []
    for _ in range(args.cold_reps):
        torch.sum(flush, dim=0, out=sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        axr.score(q, packed, norms, bits, b, out=scores)
        e1.record(stream)
        torch.cuda.synchronize()
        cold.append(e0.elapsed_time(e1))
    cold.sort()
    cold_ms = cold[len(cold) // 2]

    # Bare streams with the kernels' traffic (include/axr_probe.h): a 2 GiB
    # read, the score kernel's (records + norms in, scores out) back to back
    # on one region and cycling over four, and the write kernel's.
    log("bandwidth probes")
    psink = torch.zeros(4, dtype=torch.int32, device=dev)
    read_ms = per_launch_ms(lambda: axr.probe_read_stream(flush, psink), 10)
    score_in = n * (d * b // 8 + 4)
    score_out = n * 4 * G
    shaped_ms = per_graph_ms(lambda: axr.probe_read_write(keys, score_in, scores, score_out),
                             args.steps)
    kb = keys.view(torch.uint8).reshape(-1)
    nreg = 4
    regions = [(kb[r * score_in:(r + 1) * score_in], torch.empty_like(scores))
               for r in range(min(nreg, kb.numel() // score_in))]
    rot_stream_ms = per_graph_ms(
        Rotor(regions, lambda c: axr.probe_read_write(c[0], score_in, c[1], score_out)),
        args.steps, graph_calls(len(regions)))
    del regions, kb
    # LDS: the score kernel's table-read pattern in a bare loop, one
    # 1024-thread block per CU (include/axr_probe.h)
    lds_out = torch.empty(262144, dtype=torch.int32, device=dev)
    lds_iters = 256
    lds_bytes_cu = axr.probe_lds_read(lds_iters, lds_out)
    lds_ms = per_launch_ms(lambda: axr.probe_lds_read(lds_iters, lds_out), 20)
    lds_peak = lds_bytes_cu / (lds_ms * 1e-3 * CLOCK_HZ)
    del lds_out
    write_in = n * d * keys.element_size()
    write_out = n * (d * b // 8 + 4)
    wscratch = torch.empty(write_out, dtype=torch.uint8, device=dev)
    wshaped_ms = per_graph_ms(lambda: axr.probe_read_write(keys, write_in, wscratch, write_out),
                              args.steps)
    del flush, sink, wscratch

    # Write path with the comparison transforms (block-quaternion rotations)
    # on the prefill write-sweep keys, b = 3.
    log("write-transform comparison")
    wt = {}
    for dd in (128, 256, 512):
        ws_keys = W.write_sweep(d=dd, b=3)["keys"].to(dev)
        nk = ws_keys.numel() // dd
        pk = torch.empty(nk, dd * 3 // 32, dtype=torch.int32, device=dev)
        nm = torch.empty(nk, dtype=torch.float32, device=dev)
        qs = torch.from_numpy(W.isoquant_quaternions(dd)).to(dev)
        sb = W.sign_bits(dd)
        kbytes = nk * (dd * 2 + dd * 3 // 8 + 4)
        for name, fn in (
                ("wht", lambda: axr.quantize_keys(ws_keys, sb, 3, packed=pk, norms=nm)),
                ("isoquant_full", lambda: axr.quantize_keys_isoquant(ws_keys, qs, 3, True, pk, nm)),
                ("isoquant_fast", lambda: axr.quantize_keys_isoquant(ws_keys, qs, 3, False, pk, nm))):
            t_ms = per_graph_ms(fn, args.steps)
            wt[f"d{dd}_{name}"] = {"us": t_ms * 1e3, "GB_per_s": kbytes / (t_ms * 1e6)}
        del ws_keys, pk, nm

    # One-time sign-pattern selection: 200 candidates on 8 calibration layers.
    log("sign-pattern selection timing")
    cal = W.calibration_samples()
    cal_k, cal_q = cal["keys"].to(dev), cal["q"].to(dev)
    cands = W.sign_candidates(d)
    axr.sign_selection_errors(cal_k, cal_q, cands[:2], 4)
    torch.cuda.synchronize()
    gc.collect()
    gc.disable()
    t_sel = time.perf_counter()
    sel_idx, sel_obj = axr.select_sign_pattern(cal_k, cal_q, cands, 4)
    sel_ms = (time.perf_counter() - t_sel) * 1e3
    gc.enable()
    del cal_k, cal_q

    del keys, packed, norms, scores, q
    torch.cuda.empty_cache()
    configs = None
    if not args.no_configs:
        log("every workload")
        configs = configs_section(torch, axr, W, stream, args.steps)

    out = {
        "metric": METRIC,
        "value": n / (ms_per_step * 1e-3),
        "unit": "keys/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "llama31_8b_gqa_decode_d128_b3", "batch": B, "kv_heads": Hkv,
                   "q_heads": Hq, "context": T, "d": d, "b": b, "key_dtype": "f16",
                   "query_dtype": "f16", "keys_per_step": n,
                   "arithmetic": "fp32 transform and norms, int32 fixed-point table sums",
                   "step": "one axr_quantize_score launch: every key quantized (records "
                           "and norms stored) and scored against every query head",
                   "settle_ms": args.settle_ms},
        "roofline": {"kernel": "score", "source": f"HBM ({score_hbm['copies']} rotating "
                                                  "copies of the cache)",
                     "bound": "hbm", "achieved": round(score_hbm["GB_per_s"], 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(score_hbm["GB_per_s"] / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic("score"), "bytes_per_launch": sbytes,
                     "us": score_hbm["us"],
                     "valu_per_cu_cycle": valu_issue("score", score_hbm["us"]),
                     "lds": {"table_bytes_per_launch": score_hbm["lds_table_bytes"],
                             "achieved_B_per_cu_cycle": score_hbm["lds_B_per_cu_cycle"],
                             "probe_B_per_cu_cycle": round(lds_peak, 1),
                             "frac": round(score_hbm["lds_B_per_cu_cycle"] / lds_peak, 3),
                             "note": "16-byte table reads per launch (d/P lookups per key "
                                     "per group of four heads) against a bare loop of the "
                                     "same reads (include/axr_probe.h), per CU-cycle at "
                                     "2.4 GHz"}},
        "roofline_fused": {"kernel": "quantize_score (the step)",
                           "source": f"HBM ({fused_hbm['copies']} rotating copies of keys "
                                     "and outputs)",
                           "bound": "hbm", "achieved": round(fused_hbm["GB_per_s"], 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(fused_hbm["GB_per_s"] / HBM_PEAK_GBS, 4),
                           "traffic": counter_traffic("fused"),
                           "bytes_per_launch": fused_hbm["bytes"], "us": fused_hbm["us"],
                           "valu_per_cu_cycle": valu_issue("fused", fused_hbm["us"])},
        "step_two_launches": {"ms_per_step": ms_per_step_two,
                              "value": n / (ms_per_step_two * 1e-3),
                              "note": "the same step as the write kernel then the score "
                                      "kernel, timed the same way right after the fused "
                                      "steps"},
        "roofline_write": {"kernel": "write", "source": f"HBM ({write_hbm['copies']} rotating "
                                                        "copies of the keys)",
                           "bound": "hbm", "achieved": round(write_hbm["GB_per_s"], 1),
                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(write_hbm["GB_per_s"] / HBM_PEAK_GBS, 4),
                           "traffic": counter_traffic("write"), "bytes_per_launch": wbytes,
                           "us": write_hbm["us"],
                           "valu_per_cu_cycle": valu_issue("write", write_hbm["us"])},
        "step_kernels": {"write_us": step_write_ms * 1e3, "score_us": step_score_ms * 1e3,
                         "note": "HIP events around each kernel in a second pass of as many "
                                 "steps right after the timed ones (events between the "
                                 "kernels cost GPU time, so they stay out of the timed steps); "
                                 "the score kernel there reads records the write kernel has "
                                 "just written"},
        "ceiling": {
            "read_stream_GB_per_s": flush_bytes / (read_ms * 1e-3) / 1e9,
            "read_stream_bytes": flush_bytes,
            "score_shaped_stream_cache_resident_us": shaped_ms * 1e3,
            "score_shaped_stream_rotating_us": rot_stream_ms * 1e3,
            "score_shaped_stream_rotating_GB_per_s": sbytes / (rot_stream_ms * 1e6),
            "score_hbm_frac_of_rotating_stream": rot_stream_ms / (score_hbm["us"] * 1e-3),
            "write_shaped_stream_us": wshaped_ms * 1e3,
            "write_shaped_stream_GB_per_s": wbytes / (wshaped_ms * 1e6),
            "write_frac_of_shaped_stream": wshaped_ms / (write_hbm["us"] * 1e-3),
            "lds_read_B_per_cu_cycle": lds_peak,
            "lds_read_probe_us": lds_ms * 1e3,
        },
        "kernels": {
            "write_hbm": write_hbm,
            "score_hbm": score_hbm,
            "score_cache_resident": {
                "us": score_res_ms * 1e3, "keys_per_s": n / (score_res_ms * 1e-3),
                "GB_per_s": sbytes / (score_res_ms * 1e6),
                "frac_of_peak_cache_resident": sbytes / (score_res_ms * 1e6) / HBM_PEAK_GBS,
                "note": "back to back on one copy, replayed from a graph: the 136 MiB working "
                        "set is served from the 256 MB Infinity Cache, not HBM"},
            "score_cold_cache": {"us_median": cold_ms * 1e3, "keys_per_s": n / (cold_ms * 1e-3),
                                 "GB_per_s": sbytes / (cold_ms * 1e6),
                                 "frac_hbm": sbytes / (cold_ms * 1e6) / HBM_PEAK_GBS,
                                 "note": "single launches after 2 GiB of reads"},
            "score_softmax": {"us": softmax_ms * 1e3, "keys_per_s": n / (softmax_ms * 1e-3),
                              "note": "score kernel with split-T partials + row normalisation, "
                                      "back to back"},
            "write_transforms_b3": wt,
            "sign_selection": {"ms": sel_ms, "candidates": len(cands),
                               "calibration_samples": int(cal["keys"].shape[0]),
                               "keys_per_sample": int(cal["keys"][0].numel() // d),
                               "chosen": sel_idx,
                               "objective_default": float(sel_obj[0]),
                               "objective_chosen": float(sel_obj[sel_idx]),
                               "objective_worst": float(sel_obj.max())},
            "decode_step": {"us": decode_ms * 1e3, "graph_replay_us": decode_graph_ms * 1e3,
                            "fused_us": fused_ms * 1e3, "append_us": append_ms * 1e3,
                            "appended_keys": B * Hkv, "scored_keys": n,
                            "note": "append one key per (sequence, KV head) + ragged score, "
                                    "host-launched back to back (us) and replayed from a "
                                    "graph; fused = one launch (axr_decode_step) and append "
                                    "alone, both replayed from a graph"},
        },
        "configs": configs,
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on bounded samples")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
