"""Benchmark of the AXELRAM-style write + score path on one MI355X.

A step is one pass of the whole hot path over the LLaMA-3.1-8B-shaped GQA
decode cache (batch 8, 8 KV heads, 32 query heads, d = 128, b = 3, 32768
tokens, fp16 keys): quantize every key (normalise, sign pattern, WHT,
Lloyd-Max bucketize, pack) and score every query head against the packed
cache (query transform, LUT in LDS, lookup-accumulate).  Inputs are resident
in HBM before timing starts.

Prints one JSON line.  Per-kernel durations come from HIP events recorded on
the stream the kernels run on; the score kernel is also timed alone on a cold
cache (2 GiB of reads between launches) for its HBM roofline.

With --workloads it instead prints one JSON line per workload shape with the
write and score kernel times (--steps launches each after --warmup).
"""

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "quantized keys scored/sec + achieved HBM GB/s (d=128, b=3, GQA decode)"
CSRC = os.path.join(ROOT, "lut_attention_scoring_amd", "csrc")

# HBM bytes per launch on this workload from rocprofv3 FETCH_SIZE and
# WRITE_SIZE passes (profiles/*_llama31_8b_decode_d128_b3.md): FETCH_SIZE x 2.0
# + WRITE_SIZE x 1.0, factors from a 2 GiB read and a 2 GiB fill in the same
# runs.  Valid only for the kernel sources they were taken on (SHA-1 of the
# files below); otherwise traffic is reported as null.
COUNTER_TRAFFIC = {
    "write": {"sources": ["axr_write.hip", "axr_keyquant.h", "axr_device.h", "axr_internal.h"],
              "sha1": "fb9d2b6f897ea1fac17492de7689ee757b947702",
              "bytes": (262196.1 * 2.0 + 106531.1) * 1024},
    "score": {"sources": ["axr_score.hip", "axr_device.h", "axr_internal.h"],
              "sha1": "fee22021ac8518faff9cdd4adecb29aa7743c683",
              "bytes": (53432.2 * 2.0 + 34485.5) * 1024},
}


def counter_traffic(kernel):
    import hashlib
    entry = COUNTER_TRAFFIC[kernel]
    h = hashlib.sha1()
    for name in entry["sources"]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return entry["bytes"] if h.hexdigest() == entry["sha1"] else None


WARM_MS = 30.0   # time each kernel runs untimed before its timed launches


def launches_ms(torch, stream, fn, reps, warm_ms=WARM_MS):
    """Average duration of `reps` back-to-back launches of fn, from HIP events
    recorded on the stream the kernels run on.  Before the start event the
    kernel runs untimed for `warm_ms` of wall time, and a few more launches
    are queued right before the event: the chip needs several milliseconds of
    a given load before its clock settles (the first couple of hundred score
    launches after other work run up to a third slower), and that transient
    belongs to neither kernel.  Python's cyclic garbage collector is held
    off (a full collection of this process stalls the launching thread for
    tens of milliseconds)."""
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


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    # ~17 ms of steps: the clock takes ~10 ms of this load to settle
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--cold-reps", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workloads", action="store_true",
                    help="instead of the benchmark line: time the write and score kernels "
                         "on every workload shape, one JSON line per workload")
    return ap.parse_args()


def workload_table(args):
    """Write and score kernel times on every workload shape: each kernel is
    launched `steps` times back to back between HIP events on its stream,
    right behind untimed launches of the same kernel (inputs resident in
    HBM, Python's collector off)."""
    import torch
    import lut_attention_scoring_amd as axr
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    def per_launch_ms(fn):
        return launches_ms(torch, stream, fn, args.steps)

    cases = [("tiny_d128_b3", lambda: W.tiny()),
             ("llama31_8b_decode_d128_b3", lambda: W.llama_decode()),
             ("qwen25_3b_layer0_d128_b4", lambda: W.qwen_layer(0)),
             ("qwen25_3b_layer35_d128_b4", lambda: W.qwen_layer(W.QWEN_LAYERS - 1))]
    cases += [(f"long_context_d128_b{b}", lambda b=b: W.long_context(b=b)) for b in (2, 3, 4)]
    cases += [(f"write_sweep_d{d}_b{b}", lambda d=d, b=b: W.write_sweep(d=d, b=b))
              for d in (128, 256, 512) for b in (2, 3, 4)]
    for name, make in cases:
        w = make()
        keys = w["keys"].to(dev)
        B, Hkv, T, d = keys.shape
        b, bits = w["b"], w["sign_bits"]
        n = B * Hkv * T
        packed, norms = axr.quantize_keys(keys, bits, b)
        write_ms = per_launch_ms(lambda: axr.quantize_keys(keys, bits, b, packed=packed,
                                                           norms=norms))
        write_bytes = n * (d * keys.element_size() + d * b // 8 + 4)
        line = {"workload": name, "keys": n, "d": d, "b": b, "key_dtype": str(keys.dtype),
                "write_us": write_ms * 1e3, "write_GB_per_s": write_bytes / (write_ms * 1e6),
                "write_frac_hbm": write_bytes / (write_ms * 1e6) / HBM_PEAK_GBS}
        if w["q"] is not None:
            q = w["q"].to(dev)
            Hq = q.shape[1]
            scores = torch.empty(B, Hq, T, dtype=torch.float32, device=dev)
            score_ms = per_launch_ms(lambda: axr.score(q, packed, norms, bits, b, out=scores))
            score_bytes = n * (d * b // 8 + 4 + 4 * (Hq // Hkv))
            line.update({"G": Hq // Hkv, "score_us": score_ms * 1e3,
                         "score_GB_per_s": score_bytes / (score_ms * 1e6),
                         "score_frac_hbm": score_bytes / (score_ms * 1e6) / HBM_PEAK_GBS})
            del q, scores
        print(json.dumps(line), flush=True)
        del keys, packed, norms, w
        torch.cuda.empty_cache()


def cpu_baseline(w):
    """The fp64 oracle, as it stands, on batch elements [0, 6) of the same
    workload (6 x 8 KV heads x 32768 tokens = 1572864 keys, 32 query heads)."""
    import numpy as np
    import threadpoolctl
    from oracle import axelram as A

    import torch
    nb = 6
    keys = w["keys"][0:nb].to(dtype=torch.float64).numpy()
    q = w["q"][0:nb].to(dtype=torch.float64).numpy()
    s = A.signs_from_bits(w["sign_bits"])
    t0 = time.perf_counter()
    wr = A.write_path(keys, s, w["b"])
    A.read_path(q, wr["packed"], wr["norms"], s, w["b"])
    dt = time.perf_counter() - t0
    n = keys.shape[0] * keys.shape[1] * keys.shape[2]
    threads = max([p.get("num_threads", 1) for p in threadpoolctl.threadpool_info()
                   if p.get("user_api") == "blas"] or [1])
    return {"value": n / dt, "unit": "keys/s", "cores": int(threads), "kind": "oracle",
            "sample": f"batch elements 0-{nb - 1} of 8: {n} keys ({nb} x 8 KV heads x 32768 tokens) "
                      f"quantized and scored by 32 query heads each, fp64 numpy, {dt:.1f} s; "
                      f"host reports {os.cpu_count()} CPUs"}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: there is no multi-GPU path "
              "(the score and write paths shard with no exchange)",
              file=sys.stderr)
        sys.exit(2)
    if args.workloads:
        workload_table(args)
        return

    import torch
    import lut_attention_scoring_amd as axr
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating LLaMA-3.1-8B-shaped decode cache")
    w = W.llama_decode()
    B, Hkv, T, d = w["keys"].shape
    Hq = w["q"].shape[1]
    b, bits = w["b"], w["sign_bits"]
    n = B * Hkv * T
    keys = w["keys"].to(dev)
    q = w["q"].to(dev)
    packed = torch.empty(B, Hkv, T, d * b // 32, dtype=torch.int32, device=dev)
    norms = torch.empty(B, Hkv, T, dtype=torch.float32, device=dev)
    scores = torch.empty(B, Hq, T, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        axr.quantize_keys(keys, bits, b, packed=packed, norms=norms)
        axr.score(q, packed, norms, bits, b, out=scores)

    # The collector runs before the warmup, so that the GPU idles only for
    # the synchronisation between the warmup and the timed steps.
    log(f"warmup {args.warmup}, timing {args.steps} steps")
    gc.collect()
    gc.disable()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gc.enable()
    ms_per_step = elapsed * 1e3 / args.steps

    def per_launch_ms(fn, reps):
        return launches_ms(torch, stream, fn, reps)

    log("per-kernel timing")
    write_ms = per_launch_ms(lambda: axr.quantize_keys(keys, bits, b, packed=packed, norms=norms),
                             args.steps)
    score_ms = per_launch_ms(lambda: axr.score(q, packed, norms, bits, b, out=scores), args.steps)

    # Decode step on the same cache: one new key per (sequence, KV head)
    # appended at the last slot, then every sequence scored up to it.
    log("decode-step timing")
    import numpy as np
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

    append_ms = per_launch_ms(append, args.steps)
    decode_ms = per_launch_ms(decode_step, args.steps)
    fused_ms = per_launch_ms(
        lambda: axr.decode_step(q, new_k, bits, b, packed, norms, pos, out=scores), args.steps)

    # The same step captured once in a HIP graph and replayed (one launch
    # per step from the host).
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

    # Attention probabilities: scores with split-T softmax partials, then the
    # row normalisation (scale 1/sqrt(d)); written over `scores`.
    log("softmax timing")
    lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    ws = torch.empty(max(8, axr.score_softmax_workspace_bytes(B, Hq, Hkv, T, d, b)),
                     dtype=torch.uint8, device=dev)
    softmax_ms = per_launch_ms(
        lambda: axr.score_softmax(q, packed, norms, bits, b, out=scores, lse=lse, workspace=ws),
        args.steps)

    # Score kernel alone on a cold cache: read 2 GiB between launches, which
    # evicts the 136 MiB working set from the 256 MB Infinity Cache and L2
    # without leaving dirty lines behind.
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

    # ... and back to back over three copies of the cache (3 x 136 MiB, more
    # than the Infinity Cache holds): each launch's records, norms and scores
    # were last touched two launches (~280 MB of traffic) earlier, so they
    # come from HBM, without a single launch's start-up in the figure.
    log("rotating-cache score timing")
    copies = [(packed, norms, scores)] + [
        (packed.clone(), norms.clone(), torch.empty_like(scores)) for _ in range(2)]
    rot = [0]

    def score_rotating():
        pk, nm, sc = copies[rot[0] % 3]
        rot[0] += 1
        axr.score(q, pk, nm, bits, b, out=sc)

    rotating_ms = per_launch_ms(score_rotating, 3 * (args.steps // 3) or 3)
    # the bare stream with the score kernel's traffic, rotating the same way:
    # three disjoint 109 MB regions of the key tensor in, the three score
    # buffers out (the HBM-sourced ceiling for this kernel)
    score_in_rot = n * (d * b // 8 + 4)
    score_out_rot = n * 4 * (Hq // Hkv)
    key_bytes = keys.view(torch.uint8).reshape(-1)

    def stream_rotating():
        r = rot[0] % 3
        rot[0] += 1
        axr.probe_read_write(key_bytes[r * score_in_rot:(r + 1) * score_in_rot], score_in_rot,
                             copies[r][2], score_out_rot)

    rotating_stream_ms = per_launch_ms(stream_rotating, 3 * (args.steps // 3) or 3)
    del copies, key_bytes

    # Achievable-bandwidth ceilings on this machine (include/axr_probe.h): a
    # bare 2 GiB read stream, and streams with the score kernel's and the
    # write kernel's traffic (read bytes, then write bytes, per block).
    log("bandwidth probes")
    psink = torch.zeros(4, dtype=torch.int32, device=dev)
    read_ms = per_launch_ms(lambda: axr.probe_read_stream(flush, psink), 10)
    score_in = n * (d * b // 8 + 4)
    score_out = n * 4 * (Hq // Hkv)
    shaped_ms = per_launch_ms(lambda: axr.probe_read_write(keys, score_in, scores, score_out),
                              args.steps)
    # and one with the write kernel's traffic (the keys in, records and norms out)
    write_in = n * d * keys.element_size()
    write_out = n * (d * b // 8 + 4)
    wscratch = torch.empty(write_out, dtype=torch.uint8, device=dev)
    wshaped_ms = per_launch_ms(lambda: axr.probe_read_write(keys, write_in, wscratch, write_out),
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
        kb = nk * (dd * 2 + dd * 3 // 8 + 4)
        for name, fn in (
                ("wht", lambda: axr.quantize_keys(ws_keys, sb, 3, packed=pk, norms=nm)),
                ("isoquant_full", lambda: axr.quantize_keys_isoquant(ws_keys, qs, 3, True, pk, nm)),
                ("isoquant_fast", lambda: axr.quantize_keys_isoquant(ws_keys, qs, 3, False, pk, nm))):
            t_ms = per_launch_ms(fn, args.steps)
            wt[f"d{dd}_{name}"] = {"ms": t_ms, "GB_per_s": kb / (t_ms * 1e-3) / 1e9}
        del ws_keys, pk, nm

    # One-time sign-pattern selection: 200 candidates on 8 calibration layers
    # (B=1, 2 KV heads, 16 query heads, 2048 tokens, b=4).
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

    write_bytes_per_key = d * keys.element_size() + d * b // 8 + 4
    score_bytes_per_key = d * b // 8 + 4 + 4 * (Hq // Hkv)
    write_bytes = n * write_bytes_per_key
    score_bytes = n * score_bytes_per_key
    write_gbs = write_bytes / (write_ms * 1e-3) / 1e9
    score_gbs = score_bytes / (score_ms * 1e-3) / 1e9
    cold_gbs = score_bytes / (cold_ms * 1e-3) / 1e9
    dominant = "write" if write_ms >= score_ms else "score"
    dom_gbs = write_gbs if dominant == "write" else score_gbs
    dom_bytes = write_bytes if dominant == "write" else score_bytes

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
                   "keys_per_step": n},
        "roofline": {"kernel": f"{dominant}_kernel", "bound": "hbm",
                     "achieved": round(dom_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(dom_gbs / HBM_PEAK_GBS, 4),
                     "traffic": counter_traffic(dominant),
                     "bytes_per_launch": dom_bytes},
        "ceiling": {
            "read_stream_GB_per_s": flush_bytes / (read_ms * 1e-3) / 1e9,
            "read_stream_bytes": flush_bytes,
            "score_shaped_stream_GB_per_s": (score_in + score_out) / (shaped_ms * 1e-3) / 1e9,
            "score_shaped_stream_ms": shaped_ms,
            "score_frac_of_shaped_stream": shaped_ms / score_ms,
            "score_shaped_stream_rotating_GB_per_s":
                (score_in_rot + score_out_rot) / (rotating_stream_ms * 1e-3) / 1e9,
            "score_shaped_stream_rotating_ms": rotating_stream_ms,
            "score_rotating_frac_of_rotating_stream": rotating_stream_ms / rotating_ms,
            "write_shaped_stream_GB_per_s": (write_in + write_out) / (wshaped_ms * 1e-3) / 1e9,
            "write_shaped_stream_ms": wshaped_ms,
            "write_frac_of_shaped_stream": wshaped_ms / write_ms,
        },
        "kernels": {
            "write": {"ms": write_ms, "keys_per_s": n / (write_ms * 1e-3),
                      "GB_per_s": write_gbs, "frac_hbm": write_gbs / HBM_PEAK_GBS,
                      "bytes_per_key": write_bytes_per_key,
                      "traffic": counter_traffic("write")},
            "score": {"ms": score_ms, "keys_per_s": n / (score_ms * 1e-3),
                      "head_scores_per_s": n * (Hq // Hkv) / (score_ms * 1e-3),
                      "GB_per_s": score_gbs, "frac_hbm": score_gbs / HBM_PEAK_GBS,
                      "bytes_per_key": score_bytes_per_key,
                      "traffic": counter_traffic("score")},
            "score_cold_cache": {"ms_median": cold_ms, "keys_per_s": n / (cold_ms * 1e-3),
                                 "GB_per_s": cold_gbs, "frac_hbm": cold_gbs / HBM_PEAK_GBS},
            "score_rotating_caches": {
                "ms": rotating_ms, "keys_per_s": n / (rotating_ms * 1e-3),
                "GB_per_s": score_bytes / (rotating_ms * 1e6),
                "frac_hbm": score_bytes / (rotating_ms * 1e6) / HBM_PEAK_GBS,
                "note": "back to back over 3 copies of the cache (408 MiB > 256 MB Infinity Cache)"},
            "score_softmax": {"ms": softmax_ms, "keys_per_s": n / (softmax_ms * 1e-3),
                              "note": "score kernel with split-T partials + row normalisation"},
            "write_transforms_b3": wt,
            "sign_selection": {"ms": sel_ms, "candidates": len(cands),
                               "calibration_samples": int(cal["keys"].shape[0]),
                               "keys_per_sample": int(cal["keys"][0].numel() // d),
                               "chosen": sel_idx,
                               "objective_default": float(sel_obj[0]),
                               "objective_chosen": float(sel_obj[sel_idx]),
                               "objective_worst": float(sel_obj.max())},
            "decode_step": {"ms": decode_ms, "graph_replay_ms": decode_graph_ms,
                            "fused_ms": fused_ms,
                            "append_ms": append_ms,
                            "appended_keys": B * Hkv, "scored_keys": n,
                            "note": "append one key per (sequence, KV head) + ragged score; "
                                    "fused = one launch (axr_decode_step)"},
        },
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
