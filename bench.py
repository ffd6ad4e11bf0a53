#!/usr/bin/env python3
"""Benchmark of the packed-cache hot path on one MI355X.

Workload (default): Qwen2.5-3B-shaped decode -- 36 layers, 16 query heads, 2 KV
heads, head_dim 128, one sequence of 131072 cached tokens, K3V3 Block-GTQ cache,
synthetic seeded inputs (packed_cache_attention_amd.synth).

Phases, all on the GPU through the C ABI (libkvq.so):
  prefill  (untimed setup, measured separately): per layer, exact block energies
           of K and V, greedy K / uniform V allocation, bulk quantize+pack.
  step     (the timed unit): per layer, append the new token's K/V and run the
           split-K decode attention over the packed cache in one launch
           (kvq_decode_step_partials: the append happens inside the attention
           kernel), then the log-sum-exp merge (kvq_merge_partials).  --unfused
           appends with kvq_quantize_pack as a launch of its own instead.  The
           36-layer step is captured once in a HIP graph and replayed.

value = algorithmic bytes of one step (packed cache read by attention + queries
+ outputs + appended token) / measured step time, in GB/s.  The dominant kernel's
average duration is measured with one pair of HIP events around the 36 layers'
split-phase launches issued back to back on the stream they run on (the GPU is
held by a spin while the host enqueues them), which matches the kernel durations
rocprofv3 reports.  A CPU baseline runs the oracle (test infrastructure) on a
bounded sample of the same workload.

After the timed steps, --reps more steps are timed one by one (median, p10, p90).
Labelled lines (--extra) repeat the step measurement on the other workloads -- the
32K Llama-3.1-8B-shaped layer (its 19 MB step fits the 256 MB memory-side cache, so
a 1 GiB read evicts it before every repetition), the 512K context, the 16-sequence
batch -- and on the 128K shape in the K-only value mode (V16) and with the generic
decode kernel; each reports its median step and its kernel's roofline fraction.

`python bench.py --traffic-from FETCH.csv WRITE.csv` instead turns two rocprofv3
--pmc runs (FETCH_SIZE, then WRITE_SIZE, of this script with --copy-probe-mib)
into HBM bytes per decode launch, calibrated against the plain copy kernel.
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

HBM_PEAK_GBPS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0  # dense fp16 matrix-core peak (no sparsity)
METRIC = "packed-cache decode-attn GB/s (% HBM peak) + quantize tokens/s, 128K K3V3"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash(kernel: str) -> str:
    names = (["kvq_decode_mfma.h", "kvq_decode_mfma.hip", "kvq_internal.h"] if kernel == "mfma"
             else ["kvq_decode.hip", "kvq_internal.h"])
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "packed_cache_attention_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from(fetch_csv: str, write_csv: str, copy_mib: int, workload: str):
    """HBM bytes per decode launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs (KiB per
    dispatch), each scaled by the ratio of known bytes to the counter's reading for the
    plain copy kernel of copy_mib MiB in the same run."""
    import csv

    def per_kernel(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r["Counter_Name"] == counter]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        dec_rows = [r for r in rows if "decode_mfma_kernel" in r["Kernel_Name"]]
        # the per-layer step launches only (the layer-batched capability launch has a
        # larger grid): the modal grid size among the decode dispatches
        grids = [r["Grid_Size"] for r in dec_rows]
        grid = max(set(grids), key=grids.count) if grids else None
        dec = [float(r["Counter_Value"]) for r in dec_rows if r["Grid_Size"] == grid]
        # the copy probe: the last three copy dispatches of the run (nothing follows them)
        cp = [r for r in rows if "copy" in r["Kernel_Name"].lower()][-3:]
        big = [float(r["Counter_Value"]) for r in cp]
        return (sum(dec) / len(dec) if dec else None), (sum(big) / len(big) if big else None), len(dec), \
            (cp[0]["Kernel_Name"][:60] if cp else "")

    f_dec, f_copy, n_f, copy_name = per_kernel(fetch_csv, "FETCH_SIZE")
    w_dec, w_copy, n_w, _ = per_kernel(write_csv, "WRITE_SIZE")
    copy_bytes = copy_mib * (1 << 20)
    ff = copy_bytes / (f_copy * 1024.0)
    fw = copy_bytes / (w_copy * 1024.0)
    hbm = f_dec * 1024.0 * ff + w_dec * 1024.0 * fw
    out = {"kernel": "decode_mfma_kernel", "source_sha256_16": kernel_source_hash("mfma"),
           "fetch_kib_per_launch": round(f_dec, 1), "write_kib_per_launch": round(w_dec, 1),
           "launches": [n_f, n_w], "copy_kernel": copy_name, "copy_bytes": copy_bytes,
           "copy_fetch_kib": round(f_copy, 1), "copy_write_kib": round(w_copy, 1),
           "fetch_scale": round(ff, 4), "write_scale": round(fw, 4), "hbm_bytes_per_launch": int(hbm)}
    tf = {}
    if os.path.exists(TRAFFIC_FILE):
        tf = json.load(open(TRAFFIC_FILE))
    tf[workload] = out
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(tf, f, indent=1, sort_keys=True)
    print(json.dumps(out))


MALL_BYTES = 256 << 20  # MI355X Infinity Cache (memory-side, in front of HBM)


def gen_inputs(wl, seed, dev):
    """Seeded K/V rows of every (layer, sequence) [L, rows, H, d], the decode step's new
    token [L, S, H, d] and its queries [L, S, H_q, d], resident on dev (binary16)."""
    import numpy as np
    import torch
    from packed_cache_attention_amd import synth
    L, Hq, H, d = wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    lens = list(wl.seq_lens)
    S = len(lens)
    rows = sum(lens)
    Kall = torch.empty(L, rows, H, d, dtype=torch.float16, device=dev)
    Vall = torch.empty_like(Kall)
    Qall = torch.empty(L, S, Hq, d, dtype=torch.float16, device=dev)
    row0 = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    for l in range(L):
        for s in range(S):
            k, v, _ = synth.gen_layer(wl, s, l, seed=seed, device=dev)
            Kall[l, row0[s]:row0[s] + lens[s]] = k
            Vall[l, row0[s]:row0[s] + lens[s]] = v
    Knew = torch.empty(L, S, H, d, dtype=torch.float16, device=dev)
    Vnew = torch.empty_like(Knew)
    for l in range(L):
        for s in range(S):
            k, v, q = synth.gen_new_token(wl, s, l, lens[s], 0, seed=seed, device=dev)
            Knew[l, s], Vnew[l, s] = k, v
            Qall[l, s] = q
    torch.cuda.synchronize()
    return Kall, Vall, Qall, Knew, Vnew, row0


class MallFlush:
    """Evicts the 256 MB memory-side cache: a plain streaming read of 1 GiB (the
    library's read probe) enqueued before a timed repetition."""

    def __init__(self, dev):
        import torch
        from packed_cache_attention_amd import kvq
        self.kvq = kvq
        self.buf = torch.ones((4 * MALL_BYTES) // 4, dtype=torch.float32, device=dev)
        self.nb = 8 * torch.cuda.get_device_properties(dev).multi_processor_count
        self.sink = torch.empty(self.nb, dtype=torch.int32, device=dev)

    def __call__(self):
        self.kvq.read_probe(self.buf, self.sink, self.nb)


def time_reps(run, reps, flush=None):
    """Milliseconds of each of `reps` calls of run(), one event pair around each (after
    the flush, when given, so it is not timed)."""
    import numpy as np
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        if flush is not None:
            flush()
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) for a, b in evs])


def pct(x):
    import numpy as np
    return {"p10": round(float(np.percentile(x, 10)), 5), "p50": round(float(np.percentile(x, 50)), 5),
            "p90": round(float(np.percentile(x, 90)), 5)}


def workload_line(args, key, kern_name, v_bits=None, label=None, reps=60, flush=None):
    """One labelled decode-step measurement on another workload (or the K-only value
    mode of one): the same fused step as the headline (per layer the append inside the
    attention launch, then the merge), captured in a HIP graph, `reps` repetitions
    timed one by one (each after a memory-side-cache flush when the step's bytes fit in
    it), and the split-phase kernel's average launch time (36 or 28 layers back to
    back; a flushed single launch each when they fit).  Reports medians."""
    import dataclasses
    import numpy as np
    import torch
    from packed_cache_attention_amd import kvq, synth
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[key]
    if v_bits is not None:
        wl = dataclasses.replace(wl, v_bits=v_bits, name=wl.name.rsplit("-", 1)[0] + "-k%dv%d" % (wl.k_budget // 64,
                                                                                                 v_bits))
    kern = {"auto": kvq.DECODE_AUTO, "generic": kvq.DECODE_GENERIC, "mfma": kvq.DECODE_MFMA}[kern_name]
    L, Hq, H, d = wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    lens = list(wl.seq_lens)
    S = len(lens)
    warm = 3
    cap = synth.ceil_to(max(lens) + 2 * warm + reps + 16, 64)
    g = kvq.geom(H, wl.k_budget, wl.v_bits, cap)
    region = kvq.cache_bytes(g)
    tpb = kvq.tile_bytes(g) // 64
    t0 = time.perf_counter()
    Kall, Vall, Qall, Knew, Vnew, row0 = gen_inputs(wl, args.seed, dev)
    cache = torch.zeros(L, S * region, dtype=torch.uint8, device=dev)
    e = torch.zeros(2, H, d // 2, 2, dtype=torch.int64, device=dev)
    kbits = torch.empty(L, H, d // 2, dtype=torch.uint8, device=dev)
    ksig = torch.empty(L, H, d // 2, dtype=torch.float32, device=dev)
    vbits = torch.empty_like(kbits)
    vsig = torch.empty_like(ksig)
    off = torch.arange(S, dtype=torch.int64, device=dev) * region
    v_budget = (16 if wl.v_bits == 16 else wl.v_bits) * (d // 2)
    first0 = torch.zeros(S, dtype=torch.int64, device=dev)
    nnew0 = torch.tensor(lens, dtype=torch.int32, device=dev)
    src0 = torch.tensor(row0, dtype=torch.int64, device=dev)
    for l in range(L):
        e.zero_()
        for s in range(S):
            xs = slice(int(row0[s]), int(row0[s]) + lens[s])
            kvq.block_energy(g, Kall[l, xs], e[0])
            kvq.block_energy(g, Vall[l, xs], e[1])
        kvq.allocate_bits(g, e[0], wl.k_budget, kvq.GREEDY, kbits[l], ksig[l])
        kvq.allocate_bits(g, e[1], v_budget, kvq.UNIFORM, vbits[l], vsig[l])
        kvq.quantize_pack(g, Kall[l], Vall[l], first0, nnew0, src0, max(lens), kbits[l], ksig[l], vsig[l], cache[l],
                          off)
    torch.cuda.synchronize()
    del Kall, Vall
    t_setup = time.perf_counter() - t0
    seq_len = torch.tensor([n + 1 for n in lens], dtype=torch.int32, device=dev)
    plan = kvq.decode_plan(g, Hq, S, cap, kern, 0)
    partials = torch.empty(L, plan["workspace"] // 4, dtype=torch.float32, device=dev)  # partials (+ query table)
    out = torch.empty(L, S, Hq, d, dtype=torch.float32, device=dev)

    def launch(l):
        kvq.decode_step_partials(g, Qall[l], Knew[l], Vnew[l], cache[l], off, seq_len, cap, kbits[l], ksig[l], vsig[l],
                                 partials[l], kernel=kern)

    def step():
        for l in range(L):
            launch(l)
            kvq.merge_partials(S, Hq, plan["n_split"], partials[l], out[l])
        seq_len.add_(1)

    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s_cap):
        with torch.cuda.graph(graph, stream=s_cap):
            step()
    torch.cuda.current_stream().wait_stream(s_cap)
    torch.cuda.synchronize()
    for _ in range(warm):
        graph.replay()
    torch.cuda.synchronize()
    ln0 = seq_len.cpu().numpy().astype(np.int64)
    cache_read = L * int(ln0.sum() + S * (reps - 1) / 2) * H * tpb  # mean over the repetitions
    step_bytes = cache_read + L * (S * Hq * d * (2 + 4) + S * H * (2 * d * 2 + tpb))
    flushed = flush is not None and step_bytes < 2 * MALL_BYTES
    ms = time_reps(graph.replay, reps, flush if flushed else None)
    med = float(np.median(ms))
    # the split-phase kernel: layers back to back (or one flushed launch each)
    kd0 = torch.cuda.Event(enable_timing=True)
    kd1 = torch.cuda.Event(enable_timing=True)
    ln = seq_len.cpu().numpy().astype(np.int64)
    launch_bytes = float(ln.sum()) * H * tpb + S * H * (2 * d * 2 + tpb)
    if flushed:
        us = 1e3 * time_reps(lambda: launch(0), reps, flush)
    else:
        us = []
        for _ in range(5):
            torch.cuda._sleep(20_000_000)
            kd0.record()
            for l in range(L):
                launch(l)
            kd1.record()
            torch.cuda.synchronize()
            us.append(1e3 * kd0.elapsed_time(kd1) / L)
        us = np.array(us)
    kus = float(np.median(us))
    kname = "decode_mfma_kernel" if plan["kernel"] == kvq.DECODE_MFMA else "decode_generic_kernel"
    gbps = step_bytes / (med / 1e3) / 1e9
    kgbps = launch_bytes / (kus / 1e6) / 1e9
    res = {"label": label or wl.name, "workload": wl.name, "layers": L, "q_heads": Hq, "kv_heads": H, "batch": S,
           "context": lens if S > 1 else lens[0], "k_budget": wl.k_budget, "v_bits": wl.v_bits,
           "entry_point": "kvq_decode_step_partials + kvq_merge_partials (graph)", "kernel": kname,
           "n_split": plan["n_split"], "tiles_per_split": plan["tiles_per_split"], "reps": reps,
           "mall_flushed": flushed, "ms_per_step_median": round(med, 5), "ms_per_step_percentiles": pct(ms),
           "value": round(gbps, 2), "unit": "GB/s", "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
           "step_bytes": int(step_bytes),
           "roofline": {"kernel": kname, "bound": "hbm", "achieved": round(kgbps, 2), "peak": HBM_PEAK_GBPS,
                        "unit": "GB/s", "frac": round(kgbps / HBM_PEAK_GBPS, 4), "avg_launch_us": round(kus, 3),
                        "algorithmic_bytes_per_launch": int(launch_bytes), "bytes_per_token_head": tpb},
           "setup_s": round(t_setup, 2)}
    log("%s: %.4f ms/step median of %d%s = %.1f GB/s (%.1f%% of HBM peak); %s %.2f us/launch = %.1f%% of peak"
        % (res["label"], med, reps, " (flushed)" if flushed else "", gbps, 100 * gbps / HBM_PEAK_GBPS, kname, kus,
           100 * kgbps / HBM_PEAK_GBPS))
    del cache, partials, out, graph
    torch.cuda.empty_cache()
    return res


def rot_line(args, reps=60):
    """The rotated TurboQuant-MSE variant at the 128K Qwen2.5-3B shape (K3V3: every
    rotated coordinate at 3 bits, values rotated too).  Prefill: kvq_rot_quantize_pack
    per layer (timed: tokens/s).  Step per layer: the queries rotated, the new token
    rotated and packed and the split decode over the rotated cache in one launch
    (kvq_rot_decode_step_partials: the headline's kernel with the rotation in its
    prologue, uniform widths, scales RN32(1/sqrt(128))), the merge, the outputs rotated
    back (kvq_rot_back); captured in a
    HIP graph, `reps` repetitions timed one by one."""
    import numpy as np
    import torch
    from packed_cache_attention_amd import kvq, synth
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS["c3"]
    L, Hq, H, d = wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    lens = list(wl.seq_lens)
    S = len(lens)
    warm = 3
    cap = synth.ceil_to(max(lens) + 2 * warm + reps + 16, 64)
    g = kvq.geom(H, wl.k_budget, wl.v_bits, cap)
    region = kvq.cache_bytes(g)
    tpb = kvq.tile_bytes(g) // 64
    Kall, Vall, Qall, Knew, Vnew, row0 = gen_inputs(wl, args.seed, dev)
    ksg = torch.stack([synth.rot_signs(H, seed=args.seed, layer=l) for l in range(L)]).to(dev)
    vsg = torch.stack([synth.rot_signs(H, seed=args.seed + 1, layer=l) for l in range(L)]).to(dev)
    sig = float(np.array([kvq.ROT_SIGMA_BITS], np.uint32).view(np.float32)[0])
    kbits = torch.full((H, d // 2), wl.k_budget // (d // 2), dtype=torch.uint8, device=dev)
    rsig = torch.full((H, d // 2), sig, dtype=torch.float32, device=dev)
    cache = torch.zeros(L, S * region, dtype=torch.uint8, device=dev)
    off = torch.arange(S, dtype=torch.int64, device=dev) * region
    first0 = torch.zeros(S, dtype=torch.int64, device=dev)
    nnew0 = torch.tensor(lens, dtype=torch.int32, device=dev)
    src0 = torch.tensor(row0, dtype=torch.int64, device=dev)

    def prefill():
        for l in range(L):
            kvq.rot_quantize_pack(g, Kall[l], Vall[l], first0, nnew0, src0, max(lens), ksg[l], vsg[l], None, cache[l],
                                  off)

    prefill()
    torch.cuda.synchronize()
    pq = time_reps(prefill, 3)
    t_q = float(np.median(pq)) / 1e3
    del Kall, Vall
    seq_len = torch.tensor(lens, dtype=torch.int32, device=dev) + 1
    plan = kvq.decode_plan(g, Hq, S, cap)
    part = torch.empty(L, plan["workspace"] // 4, dtype=torch.float32, device=dev)
    out = torch.empty(L, S, Hq, d, dtype=torch.float32, device=dev)

    def launch(l):
        kvq.rot_decode_step_partials(g, Qall[l], Knew[l], Vnew[l], cache[l], off, seq_len, cap, kbits, rsig, rsig,
                                     ksg[l], vsg[l], part[l])

    def step():
        for l in range(L):
            launch(l)
            kvq.merge_partials(S, Hq, plan["n_split"], part[l], out[l])
            kvq.rot_back(g, out[l], vsg[l])
        seq_len.add_(1)

    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    s_cap = torch.cuda.Stream()
    s_cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s_cap):
        with torch.cuda.graph(graph, stream=s_cap):
            step()
    torch.cuda.current_stream().wait_stream(s_cap)
    torch.cuda.synchronize()
    for _ in range(warm):
        graph.replay()
    torch.cuda.synchronize()
    ln0 = seq_len.cpu().numpy().astype(np.int64)
    step_bytes = L * (int(ln0.sum() + S * (reps - 1) / 2) * H * tpb + S * Hq * d * (2 + 4) + S * H * (2 * d * 2 + tpb))
    ms = time_reps(graph.replay, reps)
    med = float(np.median(ms))
    kd0 = torch.cuda.Event(enable_timing=True)
    kd1 = torch.cuda.Event(enable_timing=True)
    us = []
    for _ in range(5):
        torch.cuda._sleep(20_000_000)
        kd0.record()
        for l in range(L):
            launch(l)
        kd1.record()
        torch.cuda.synchronize()
        us.append(1e3 * kd0.elapsed_time(kd1) / L)
    kus = float(np.median(us))
    ln = seq_len.cpu().numpy().astype(np.int64)
    launch_bytes = float(ln.sum()) * H * tpb
    gbps = step_bytes / (med / 1e3) / 1e9
    kgbps = launch_bytes / (kus / 1e6) / 1e9
    rows = sum(lens)
    res = {"label": "rotated TQ-MSE variant (random-sign Hadamard keys and values) at the 128K shape, K3V3",
           "workload": wl.name + "-rotated", "entry_point": "kvq_rot_decode_step_partials + "
           "kvq_merge_partials + kvq_rot_back (graph)", "reps": reps,
           "ms_per_step_median": round(med, 5), "ms_per_step_percentiles": pct(ms), "value": round(gbps, 2),
           "unit": "GB/s", "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2), "step_bytes": int(step_bytes),
           "roofline": {"kernel": "decode_mfma_kernel" if plan["kernel"] == kvq.DECODE_MFMA else
                        "decode_generic_kernel", "bound": "hbm", "achieved": round(kgbps, 2),
                        "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(kgbps / HBM_PEAK_GBPS, 4),
                        "avg_launch_us": round(kus, 3), "algorithmic_bytes_per_launch": int(launch_bytes)},
           "rot_quantize_ms": round(t_q * 1e3, 4), "rot_quantize_tokens_per_s": round(rows / t_q, 1),
           "rot_quantize_GBps": round(rows * H * L * (2 * d * 2 + tpb) / t_q / 1e9, 1)}
    log("%s: %.4f ms/step median of %d = %.1f GB/s (%.1f%% of HBM peak); decode kernel %.2f us/launch; bulk rotated "
        "quantize %.3f ms for %d layers (%.3g tokens/s)" % (res["label"], med, reps, gbps, 100 * gbps / HBM_PEAK_GBPS,
                                                          kus, t_q * 1e3, L, rows / t_q))
    del cache, part, out, graph
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3", choices=["c2", "c3", "c4", "c5"])
    ap.add_argument("--kernel", default="auto", choices=["auto", "generic", "mfma"])
    ap.add_argument("--tiles-per-split", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true", help="time eager launches instead of a graph replay")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--unfused", action="store_true",
                    help="append with kvq_quantize_pack as a launch of its own instead of inside the attention kernel")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--prefill-chunk", type=int, default=2048,
                    help="also time chunked prefill attention: each sequence's last N tokens as one chunk of "
                         "queries over its whole packed context (0: skip)")
    ap.add_argument("--prefill-split", type=int, default=0, help="key-range splits for the chunk (0: planner)")
    ap.add_argument("--read-probe-gib", type=float, default=4.0,
                    help="size of the plain read-bandwidth probe (0: skip)")
    ap.add_argument("--window", type=int, default=128,
                    help="also time the fp16 recent-window step with this many recent tokens unquantized (0: skip)")
    ap.add_argument("--ramp", type=int, default=100,
                    help="untimed steps before the timed region, after the warm-up (clock ramp)")
    ap.add_argument("--reps", type=int, default=60,
                    help="repetitions timed one by one after the timed steps, for the median and percentiles")
    ap.add_argument("--extra", default="c2,c4,c5,c3-konly,c3-generic,c3-rot",
                    help="labelled lines on other workloads: c2, c4, c5 (fused step), c3-konly (the K-only "
                         "value mode, V16, at the 128K shape), c3-generic (the generic kernel at K3V3), c3-rot (the "
                         "rotated TQ-MSE variant at the 128K shape); '' = none")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(args.traffic_from[0], args.traffic_from[1], args.copy_probe_mib or 256,
                     {"c2": "c2-llama8b-layer-32k-k2v2", "c3": "c3-qwen3b-36layer-128k-k3v3",
                      "c4": "c4-qwen3b-36layer-512k-k3v3", "c5": "c5-r1qwen7b-28layer-16seq-4k32k-k3v2"}[args.workload])
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the hot path is data-parallel per (sequence, layer, KV head) "
              "and this build runs no multi-GPU configuration (see the sharding design notes). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from packed_cache_attention_amd import kvq, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    kern = {"auto": kvq.DECODE_AUTO, "generic": kvq.DECODE_GENERIC, "mfma": kvq.DECODE_MFMA}[args.kernel]

    wl = synth.WORKLOADS[args.workload]
    L, Hq, H, d = wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    lens = list(wl.seq_lens)
    S = len(lens)
    # every step appends one token: eager warm-up, graph warm-up, timed steps, kernel-timing steps
    extra = 2 * max(1, args.warmup) + args.steps + min(args.steps, 10) + 4 + args.reps + args.ramp
    cap = synth.ceil_to(max(lens) + extra, 64)
    g = kvq.geom(H, wl.k_budget, wl.v_bits, cap)
    region = kvq.cache_bytes(g)
    tile = kvq.tile_bytes(g)
    bytes_per_token_head = tile // 64
    log("workload %s: %d layers, %d q / %d kv heads, %d seq(s), lengths %s, K budget %d, V %d bits; "
        "capacity %d, %.1f MB packed per layer" % (wl.name, L, Hq, H, S, lens[:4], wl.k_budget, wl.v_bits, cap,
                                                    S * region / 1e6))

    # ------------------------------------------------------------ inputs (resident in HBM)
    t0 = time.perf_counter()
    rows = sum(lens)
    Kall, Vall, Qall, Knew, Vnew, row0 = gen_inputs(wl, args.seed, dev)
    log("generated inputs in %.1f s (%.2f GB fp16 K/V)" % (time.perf_counter() - t0, 2 * Kall.numel() * 2 / 1e9))

    # ------------------------------------------------------------ prefill: energy, allocation, bulk quantize
    cache = torch.zeros(L, S * region, dtype=torch.uint8, device=dev)
    eK = torch.zeros(L, H, d // 2, 2, dtype=torch.int64, device=dev)
    eV = torch.zeros_like(eK)
    kbits = torch.empty(L, H, d // 2, dtype=torch.uint8, device=dev)
    ksig = torch.empty(L, H, d // 2, dtype=torch.float32, device=dev)
    vbits = torch.empty_like(kbits)
    vsig = torch.empty_like(ksig)
    off = torch.arange(S, dtype=torch.int64, device=dev) * region
    first0 = torch.zeros(S, dtype=torch.int64, device=dev)
    nnew0 = torch.tensor(lens, dtype=torch.int32, device=dev)
    src0 = torch.tensor(row0, dtype=torch.int64, device=dev)
    v_budget = wl.v_bits * (d // 2)

    def prefill(ev=None):
        eK.zero_()
        eV.zero_()
        for l in range(L):
            if ev: ev["e0"][l].record()
            for s in range(S):
                xs = slice(int(row0[s]), int(row0[s]) + lens[s])
                kvq.block_energy(g, Kall[l, xs], eK[l])
                kvq.block_energy(g, Vall[l, xs], eV[l])
            if ev: ev["a0"][l].record()
            kvq.allocate_bits(g, eK[l], wl.k_budget, kvq.GREEDY, kbits[l], ksig[l])
            kvq.allocate_bits(g, eV[l], v_budget, kvq.UNIFORM, vbits[l], vsig[l])
            if ev: ev["q0"][l].record()
            kvq.quantize_pack(g, Kall[l], Vall[l], first0, nnew0, src0, max(lens), kbits[l], ksig[l], vsig[l],
                              cache[l], off)
            if ev: ev["q1"][l].record()

    prefill()
    torch.cuda.synchronize()
    reps = 3
    evs = [{k: [torch.cuda.Event(enable_timing=True) for _ in range(L)] for k in ("e0", "a0", "q0", "q1")}
           for _ in range(reps)]
    tp0 = torch.cuda.Event(enable_timing=True)
    tp1 = torch.cuda.Event(enable_timing=True)
    tp0.record()
    for r in range(reps):
        prefill(evs[r])
    tp1.record()
    torch.cuda.synchronize()
    t_energy = np.mean([sum(e["e0"][l].elapsed_time(e["a0"][l]) for l in range(L)) for e in evs]) / 1e3
    t_alloc = np.mean([sum(e["a0"][l].elapsed_time(e["q0"][l]) for l in range(L)) for e in evs]) / 1e3
    t_quant = np.mean([sum(e["q0"][l].elapsed_time(e["q1"][l]) for l in range(L)) for e in evs]) / 1e3
    t_prefill = tp0.elapsed_time(tp1) / 1e3 / reps
    tok_heads = rows * H * L
    quant_bytes = tok_heads * (2 * d * 2 + bytes_per_token_head)
    energy_bytes = tok_heads * 2 * d * 2
    log("prefill: energy %.3f ms (%.0f GB/s), alloc %.3f ms, quantize %.3f ms (%.0f GB/s, %.3g tokens/s)"
        % (t_energy * 1e3, energy_bytes / t_energy / 1e9, t_alloc * 1e3, t_quant * 1e3,
           quant_bytes / t_quant / 1e9, rows / t_quant))

    # ------------------------------------------------------------ decode step
    cur = torch.tensor(lens, dtype=torch.int64, device=dev)          # slot of the next token
    seq_len = (cur + 1).to(torch.int32)                               # attended tokens incl. the new one
    src_new = torch.arange(S, dtype=torch.int64, device=dev)
    ones32 = torch.ones(S, dtype=torch.int32, device=dev)
    max_len = cap
    plan = kvq.decode_plan(g, Hq, S, max_len, kern, args.tiles_per_split)
    n_split = plan["n_split"]
    partials = torch.empty(L, plan["workspace"] // 4, dtype=torch.float32, device=dev)  # partials (+ query table)
    out = torch.empty(L, S, Hq, d, dtype=torch.float32, device=dev)
    log("decode plan: %s" % plan)

    def step(ev=None):
        for l in range(L):
            if args.unfused:
                kvq.quantize_pack(g, Knew[l], Vnew[l], cur, ones32, src_new, 1, kbits[l], ksig[l], vsig[l],
                                  cache[l], off)
                kvq.decode_partials(g, Qall[l], cache[l], off, seq_len, max_len, kbits[l], ksig[l], vsig[l],
                                    partials[l], kernel=kern, tiles_per_split=args.tiles_per_split)
            else:  # append inside the attention kernel
                kvq.decode_step_partials(g, Qall[l], Knew[l], Vnew[l], cache[l], off, seq_len, max_len, kbits[l],
                                         ksig[l], vsig[l], partials[l], kernel=kern,
                                         tiles_per_split=args.tiles_per_split)
            kvq.merge_partials(S, Hq, n_split, partials[l], out[l])
        cur.add_(1)
        seq_len.add_(1)

    def seq_bytes():
        # algorithmic bytes of one step at the current lengths (cache read + q + out + append)
        ln = seq_len.cpu().numpy().astype(np.int64)
        attn = int(ln.sum()) * H * bytes_per_token_head + S * Hq * d * (2 + 4)
        app = S * H * (2 * d * 2 + bytes_per_token_head)
        return L * attn, L * app

    # warm-up (eager) then capture
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s_cap):
            with torch.cuda.graph(graph, stream=s_cap):
                step()
        torch.cuda.current_stream().wait_stream(s_cap)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
    # untimed steps that bring the clocks to their steady state (the first ~50 ms of
    # load run a few percent slower), beyond the requested warm-up
    for _ in range(args.ramp):
        if graph is not None:
            graph.replay()
        else:
            step()
    torch.cuda.synchronize()
    attn_b0, app_b0 = seq_bytes()
    # timed region: exactly `steps` steps, synchronised on both sides
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    # an event between consecutive steps as well (recording does not synchronise), for
    # the per-step spread
    sev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    w0 = time.perf_counter()
    e0.record()
    sev[0].record()
    for i in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
        sev[i + 1].record()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / args.steps
    per_step = np.array([sev[i].elapsed_time(sev[i + 1]) for i in range(args.steps)])
    step_pct = {"p10": round(float(np.percentile(per_step, 10)), 5), "p50": round(float(np.percentile(per_step, 50)), 5),
                "p90": round(float(np.percentile(per_step, 90)), 5)}
    attn_b1, app_b1 = seq_bytes()
    step_bytes = 0.5 * (attn_b0 + attn_b1) + app_b0
    value = step_bytes / (ms_step / 1e3) / 1e9
    log("timed %d steps: %.4f ms/step (wall %.4f ms/step), %.1f GB/s = %.1f%% of HBM peak"
        % (args.steps, ms_step, wall * 1e3 / args.steps, value, 100 * value / HBM_PEAK_GBPS))
    # then `reps` more steps timed one by one (each step reads far more than the
    # memory-side cache holds: 36 layers of distinct caches, so no flush is needed)
    median = None
    if args.reps > 0:
        rms = time_reps(graph.replay if graph is not None else step, args.reps)
        attn_b2, _ = seq_bytes()
        mbytes = 0.5 * (attn_b1 + attn_b2) + app_b0
        mmed = float(np.median(rms))
        median = {"reps": args.reps, "ms_per_step_median": round(mmed, 5), "ms_per_step_percentiles": pct(rms),
                  "value_at_median": round(mbytes / (mmed / 1e3) / 1e9, 2), "mall_flushed": False,
                  "step_bytes": int(mbytes)}
        log("median of %d steps timed one by one: %.4f ms/step (p10 %.4f, p90 %.4f)"
            % (args.reps, mmed, median["ms_per_step_percentiles"]["p10"], median["ms_per_step_percentiles"]["p90"]))

    # ------------------------------------------------------------ dominant kernel: back-to-back launches
    # One event pair brackets the 36 layers' split-phase launches, enqueued while a
    # spin holds the GPU, so the span is the kernels' own time.  Fused, these are the
    # next step's launches (its appends write the same bytes on every repetition).
    ksteps = min(args.steps, 10)
    durs = []
    kd0 = torch.cuda.Event(enable_timing=True)
    kd1 = torch.cuda.Event(enable_timing=True)
    for _ in range(ksteps):
        torch.cuda._sleep(20_000_000)
        kd0.record()
        for l in range(L):
            if args.unfused:
                kvq.decode_partials(g, Qall[l], cache[l], off, seq_len, max_len, kbits[l], ksig[l], vsig[l],
                                    partials[l], kernel=kern, tiles_per_split=args.tiles_per_split)
            else:
                kvq.decode_step_partials(g, Qall[l], Knew[l], Vnew[l], cache[l], off, seq_len, max_len, kbits[l],
                                         ksig[l], vsig[l], partials[l], kernel=kern,
                                         tiles_per_split=args.tiles_per_split)
        kd1.record()
        torch.cuda.synchronize()
        durs.append(kd0.elapsed_time(kd1) / 1e3 / L)
    kdur = float(np.mean(durs))
    ln = seq_len.cpu().numpy().astype(np.int64)
    launch_bytes = float(ln.sum()) * H * bytes_per_token_head
    if not args.unfused:  # the appended token: fp16 K and V read, packed bytes written
        launch_bytes += S * H * (2 * d * 2 + bytes_per_token_head)
    achieved = launch_bytes / kdur / 1e9
    kernel_name = "decode_mfma_kernel" if plan["kernel"] == kvq.DECODE_MFMA else "decode_generic_kernel"
    log("%s: %.2f us/launch avg over %d launches, %.1f GB/s algorithmic (%.1f%% of peak)"
        % (kernel_name, kdur * 1e6, len(durs) * L, achieved, 100 * achieved / HBM_PEAK_GBPS))

    # ------------------------------------------------------------ the fp16 recent-window variant
    # The newest W tokens of each (layer, sequence, head) sit binary16 in a ring, the
    # rest in the packed cache; one window step packs the token leaving the window
    # inside the attention launch, then merges with exact attention over the window
    # and writes the new token to the ring.  Lengths stay fixed over the repetitions
    # (every step evicts and inserts at the same rows: identical work).
    wres = None
    if args.window > 0:
        W = args.window
        win_k = torch.empty(L, S, H, W, d, dtype=torch.float16, device=dev)
        win_v = torch.empty_like(win_k)
        for s_ in range(S):
            t = torch.arange(max(lens[s_] - W, 0), lens[s_], device=dev)
            src = int(row0[s_]) + t
            win_k[:, s_, :, t % W] = Kall[:, src].permute(0, 2, 1, 3)
            win_v[:, s_, :, t % W] = Vall[:, src].permute(0, 2, 1, 3)
        wlen = seq_len.clone()
        wmax = int(wlen.max())
        wws_n = kvq.window_workspace_bytes(g, W, Hq, S, wmax, kern, args.tiles_per_split) // 4
        wws = torch.empty(L, wws_n, dtype=torch.float32, device=dev)
        wout = torch.empty(L, S, Hq, d, dtype=torch.float32, device=dev)

        def wstep():
            for l in range(L):
                kvq.window_decode_step(g, W, Qall[l], Knew[l], Vnew[l], win_k[l], win_v[l], cache[l], off, wlen,
                                       wmax, kbits[l], ksig[l], vsig[l], wout[l], wws[l], kernel=kern,
                                       tiles_per_split=args.tiles_per_split)

        for _ in range(max(1, args.warmup)):
            wstep()
        torch.cuda.synchronize()
        wgraph = None
        if not args.no_graph:
            s_cap = torch.cuda.Stream()
            s_cap.wait_stream(torch.cuda.current_stream())
            wgraph = torch.cuda.CUDAGraph()
            with torch.cuda.stream(s_cap):
                with torch.cuda.graph(wgraph, stream=s_cap):
                    wstep()
            torch.cuda.current_stream().wait_stream(s_cap)
            torch.cuda.synchronize()
            for _ in range(args.warmup):
                wgraph.replay()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            if wgraph is not None:
                wgraph.replay()
            else:
                wstep()
        e1.record()
        torch.cuda.synchronize()
        wms = e0.elapsed_time(e1) / args.steps
        wl_ = wlen.cpu().numpy().astype(np.int64)
        npk = np.maximum(wl_ - W, 0)
        nwin = np.minimum(wl_, W)
        wbytes = L * (int(npk.sum()) * H * bytes_per_token_head + int(nwin.sum()) * H * 2 * d * 2
                      + S * Hq * d * (2 + 4) + S * H * (2 * d * 2 + bytes_per_token_head) + S * H * 2 * d * 2)
        wval = wbytes / (wms / 1e3) / 1e9
        log("window step (W=%d): %.4f ms/step, %.1f GB/s = %.1f%% of HBM peak" % (W, wms, wval,
                                                                              100 * wval / HBM_PEAK_GBPS))
        wres = {"window": W, "ms_per_step": round(wms, 5), "value": round(wval, 2), "unit": "GB/s",
                "pct_hbm_peak": round(100 * wval / HBM_PEAK_GBPS, 2), "step_bytes": int(wbytes),
                "entry_point": "kvq_window_decode_step"}

    # ------------------------------------------------------------ chunked prefill attention
    # Each sequence's last C tokens as one chunk of queries (positions n - C .. n - 1)
    # attending its whole packed context causally, every layer once per repetition.
    # Algorithmic work: 4 d flops per (query head, attended key) (QK and PV, multiply
    # and add); the kernel issues twice that on the matrix cores (hi + lo operand
    # splits of q and of the softmax weights).
    pres = None
    if args.prefill_chunk > 0:
        C_ = args.prefill_chunk
        qstart = [max(n - C_, 0) for n in lens]
        nqs = [n - a for n, a in zip(lens, qstart)]
        max_q = max(nqs)
        pq = torch.zeros(L, S, max_q, Hq, d, dtype=torch.float16, device=dev)
        for l in range(L):
            for s_ in range(S):
                pq[l, s_, :nqs[s_]] = synth.gen_chunk_queries(wl, s_, l, qstart[s_], nqs[s_], seed=args.seed,
                                                              device=dev)
        pqs = torch.tensor(qstart, dtype=torch.int32, device=dev)
        pns = torch.tensor(nqs, dtype=torch.int32, device=dev)
        pmax = max(lens)
        pplan = kvq.prefill_plan(g, Hq, S, max_q, pmax, args.prefill_split)
        pws = torch.empty(max(pplan["workspace"] // 4, 4), dtype=torch.float32, device=dev)
        pout = torch.empty(S, max_q, Hq, d, dtype=torch.float32, device=dev)

        def pstep():
            for l in range(L):
                kvq.packed_prefill_attn(g, pq[l], cache[l], off, pqs, pns, pmax, kbits[l], ksig[l], vsig[l], pout,
                                        pws, n_split=args.prefill_split)

        pstep()
        torch.cuda.synchronize()
        preps = 2
        e0.record()
        for _ in range(preps):
            pstep()
        e1.record()
        torch.cuda.synchronize()
        pms = e0.elapsed_time(e1) / (preps * L)
        pairs = sum(Hq * (n_ * a + n_ * (n_ + 1) // 2) for a, n_ in zip(qstart, nqs))
        pflops = 4 * d * pairs
        ptf = pflops / (pms / 1e3) / 1e12
        # the chunk's own quantize + pack (its K/V rows are already resident)
        qfirst = torch.tensor(qstart, dtype=torch.int64, device=dev)
        qsrc = torch.tensor([int(r0) + a for r0, a in zip(row0, qstart)], dtype=torch.int64, device=dev)
        chunk_cache = torch.zeros_like(cache[0])
        kvq.quantize_pack(g, Kall[0], Vall[0], qfirst, pns, qsrc, max_q, kbits[0], ksig[0], vsig[0], chunk_cache, off)
        torch.cuda.synchronize()
        e0.record()
        for l in range(L):
            kvq.quantize_pack(g, Kall[l], Vall[l], qfirst, pns, qsrc, max_q, kbits[l], ksig[l], vsig[l],
                              chunk_cache, off)
        e1.record()
        torch.cuda.synchronize()
        qms = e0.elapsed_time(e1) / L
        log("prefill chunk (%d queries per sequence, n_split %d): attention %.3f ms per layer = %.1f TFLOP/s "
            "(%.1f%% of the fp16 MFMA peak), chunk quantize %.4f ms per layer"
            % (C_, pplan["n_split"], pms, ptf, 100 * ptf / MFMA_F16_PEAK_TFLOPS, qms))
        pres = {"chunk": C_, "entry_point": "kvq_packed_prefill_attn", "n_split": pplan["n_split"],
                "ms_per_layer": round(pms, 5), "tflops": round(ptf, 2), "peak_tflops": MFMA_F16_PEAK_TFLOPS,
                "frac": round(ptf / MFMA_F16_PEAK_TFLOPS, 4), "flops_per_layer": int(pflops),
                "issued_mfma_tflops": round(2 * ptf, 2), "quantize_chunk_ms_per_layer": round(qms, 5)}

    traffic = None
    src_hash = kernel_source_hash("mfma" if kernel_name == "decode_mfma_kernel" else "generic")
    if os.path.exists(TRAFFIC_FILE):
        try:
            tf = json.load(open(TRAFFIC_FILE))
            ent = tf.get(wl.name, {})
            if ent.get("kernel") == kernel_name and ent.get("source_sha256_16") == src_hash:
                traffic = ent.get("hbm_bytes_per_launch")
        except Exception:
            traffic = None

    # ------------------------------------------------------------ layer-batched capability
    # Not a model-realistic step (layer l+1's query depends on layer l): the 36 layers'
    # caches are consecutive, so the same decode kernel can attend all of them in one
    # launch as one geometry of L * H_kv KV heads -- the kernel's throughput with the
    # per-launch cost amortised.  Labelled as such; never the headline.
    batched = None
    if S == 1:
        gb = kvq.geom(L * H, wl.k_budget, wl.v_bits, cap)
        qb_ = Qall.view(1, L * Hq, d)
        bplan = kvq.decode_plan(gb, L * Hq, 1, max_len, kern, 0)
        bpart = torch.empty(bplan["workspace"] // 4, dtype=torch.float32, device=dev)
        bk, bs, bv = kbits.view(L * H, d // 2), ksig.view(L * H, d // 2), vsig.view(L * H, d // 2)

        def bstep():
            kvq.decode_partials(gb, qb_, cache.view(-1), off[:1], seq_len, max_len, bk, bs, bv, bpart, kernel=kern)

        bstep()
        torch.cuda.synchronize()
        bdur = []
        for _ in range(5):
            torch.cuda._sleep(20_000_000)
            kd0.record()
            bstep()
            kd1.record()
            torch.cuda.synchronize()
            bdur.append(kd0.elapsed_time(kd1))
        bms = float(np.median(bdur))
        bbytes = L * int(seq_len[0].item()) * H * bytes_per_token_head
        bgbps = bbytes / (bms / 1e3) / 1e9
        batched = {"label": "kernel capability: all %d layers in one launch (not a model step)" % L,
                   "entry_point": "kvq_decode_partials", "n_split": bplan["n_split"],
                   "tiles_per_split": bplan["tiles_per_split"], "launch_us": round(bms * 1e3, 2),
                   "bytes": bbytes, "GBps": round(bgbps, 1), "frac": round(bgbps / HBM_PEAK_GBPS, 4)}
        log("layer-batched capability: %d layers in one launch %.1f us = %.0f GB/s (%.1f%% of HBM peak)"
            % (L, bms * 1e3, bgbps, 100 * bgbps / HBM_PEAK_GBPS))

    # ------------------------------------------------------------ achievable read bandwidth
    # A plain streaming read of 4 GiB (far beyond the 256 MB MALL) with the library's
    # probe kernel (eight 128-bit loads in flight per thread, many workgroups) is the
    # read ceiling a simple kernel reaches here; the decode figures are also given
    # against it.
    probe = None
    if args.read_probe_gib > 0:
        nprobe = int(args.read_probe_gib * (1 << 30)) // 16 * 16
        pbuf = torch.ones(nprobe // 4, dtype=torch.float32, device=dev)
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        best = None
        for per_cu in (8, 16, 32):
            nb = cus * per_cu
            sink = torch.empty(nb, dtype=torch.int32, device=dev)
            kvq.read_probe(pbuf, sink, nb)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(5):
                kvq.read_probe(pbuf, sink, nb)
            e1.record()
            torch.cuda.synchronize()
            gbps = nprobe / (e0.elapsed_time(e1) / 5 / 1e3) / 1e9
            if best is None or gbps > best[0]:
                best = (gbps, nb)
        del pbuf
        torch.cuda.empty_cache()
        pgbps = best[0]
        # the same read over each layer's packed cache, 36 launches back to back as the
        # decode issues them: what a plain kernel needs per layer-sized launch
        lbytes = cache[0].numel()
        lus, nbl = None, 0
        for per_cu in (2, 4, 8, 16, 32):
            nb = cus * per_cu
            sink = torch.empty(nb, dtype=torch.int32, device=dev)
            ldur = []
            for _ in range(3):
                torch.cuda._sleep(20_000_000)
                kd0.record()
                for l in range(L):
                    kvq.read_probe(cache[l], sink, nb)
                kd1.record()
                torch.cuda.synchronize()
                ldur.append(kd0.elapsed_time(kd1) / L)
            t = 1e3 * float(np.median(ldur))
            if lus is None or t < lus:
                lus, nbl = t, nb
        probe = {"kind": "kvq_read_probe (plain 128-bit streaming read)", "bytes": nprobe, "workgroups": best[1],
                 "GBps": round(pgbps, 1), "pct_hbm_peak": round(100 * pgbps / HBM_PEAK_GBPS, 2),
                 "decode_kernel_pct_of_probe": round(100 * achieved / pgbps, 2),
                 "step_pct_of_probe": round(100 * value / pgbps, 2),
                 "per_layer_read": {"bytes": lbytes, "avg_launch_us": round(lus, 3), "workgroups": nbl,
                                    "GBps": round(lbytes / (lus / 1e6) / 1e9, 1)}}
        log("read probe: %.0f GB/s (%.1f%% of HBM peak, %d workgroups); decode kernel at %.1f%% of it; "
            "a plain read of one layer's %.1f MB cache takes %.2f us per launch back to back"
            % (pgbps, 100 * pgbps / HBM_PEAK_GBPS, best[1], 100 * achieved / pgbps, lbytes / 1e6, lus))

    if args.copy_probe_mib:
        n = args.copy_probe_mib * (1 << 20) // 4
        a = torch.empty(n, dtype=torch.float32, device=dev).normal_()
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy probe: %d MiB copied 3x" % args.copy_probe_mib)

    # ------------------------------------------------------------ CPU baseline: the oracle on a bounded sample
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, Kall, Vall, Qall, lens, row0, bytes_per_token_head)

    # ------------------------------------------------------------ labelled lines on the other workloads
    others = {}
    keys = [k for k in args.extra.split(",") if k]
    if keys:
        flush = MallFlush(dev)
        for k in keys:
            if k == "c3-konly":
                others[k] = workload_line(args, "c3", "auto", v_bits=16, reps=args.reps or 60, flush=flush,
                                          label="K-only value mode (V16) at the 128K Qwen2.5-3B shape")
            elif k == "c3-rot":
                others[k] = rot_line(args, reps=args.reps or 60)
            elif k == "c3-generic":
                others[k] = workload_line(args, "c3", "generic", reps=args.reps or 60, flush=flush,
                                          label="the generic decode kernel at the headline workload")
            else:
                others[k] = workload_line(args, k, args.kernel, reps=args.reps or 60, flush=flush)
        del flush
        torch.cuda.empty_cache()

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xf16->f32 (mfma)" if kernel_name == "decode_mfma_kernel" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "layers": L, "q_heads": Hq, "kv_heads": H, "head_dim": d,
                   "batch": S, "context": lens if S > 1 else lens[0], "k_budget": wl.k_budget,
                   "v_bits": wl.v_bits, "capacity": cap, "graph": graph is not None,
                   "split_chunks": n_split, "kernel": kernel_name, "append": "separate launch" if args.unfused else "inside the attention kernel"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "step_bytes": int(step_bytes),
        "wall_ms_per_step": round(wall * 1e3 / args.steps, 5),
        "ms_per_step_percentiles": step_pct,
        "median_of_reps": median,
        "read_probe": probe,
        "quantize_tokens_per_s": round(rows / t_quant, 1),
        "prefill": {"energy_ms": round(t_energy * 1e3, 4), "energy_GBps": round(energy_bytes / t_energy / 1e9, 1),
                    "allocate_ms": round(t_alloc * 1e3, 4), "quantize_ms": round(t_quant * 1e3, 4),
                    "quantize_GBps": round(quant_bytes / t_quant / 1e9, 1), "total_ms": round(t_prefill * 1e3, 4),
                    "tokens": rows, "token_heads": tok_heads},
        "roofline": {"kernel": kernel_name, "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "avg_launch_us": round(kdur * 1e6, 3),
                     "algorithmic_bytes_per_launch": int(launch_bytes),
                     "bytes_per_token_head": bytes_per_token_head},
        "cpu_baseline": cpu,
        "window_step": wres,
        "prefill_chunk": pres,
        "layer_batched": batched,
        "other_workloads": others or None,
    }
    print(json.dumps(result), flush=True)


def cpu_baseline(wl, Kall, Vall, Qall, lens, row0, bytes_per_token_head, budget_s=12.0):
    """Oracle (CPU, fp64) on a bounded sample: sequence 0 at its full length, layer
    after layer until about budget_s seconds of oracle work: exact energies,
    allocation, quantize+pack, then decode attention of the layer's queries.
    Reports the packed bytes its decode attention processes per second."""
    import numpy as np
    import oracle
    # threads: OMP_NUM_THREADS when set (the GPU hosts here give each GPU 16 cores and
    # set it to 16), else every core of the host
    host_cores = os.cpu_count() or 1
    n_threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or host_cores
    n_threads = oracle.set_threads(n_threads)
    n = lens[0]
    H = wl.n_kv_heads
    t_prep = t_attn = 0.0
    layers = 0
    while layers < wl.n_layers and t_prep + t_attn < budget_s:
        K = Kall[layers, int(row0[0]):int(row0[0]) + n].cpu().numpy()
        V = Vall[layers, int(row0[0]):int(row0[0]) + n].cpu().numpy()
        q = Qall[layers, 0].cpu().numpy()
        t0 = time.perf_counter()
        eK = oracle.block_energy(K)
        eV = oracle.block_energy(V)
        kb, ks = oracle.allocate(eK, wl.k_budget)
        _, vs = oracle.allocate(eV, wl.v_bits * 64, oracle.UNIFORM)
        geom = oracle.Geometry(H, wl.k_budget, wl.v_bits, ((n + 63) // 64) * 64)
        region = np.zeros(geom.seq_bytes, np.uint8)
        oracle.quantize_pack(geom, region, K, V, 0, kb, ks, vs)
        t1 = time.perf_counter()
        oracle.decode_attention(geom, region, q, n, kb, ks, vs)
        t2 = time.perf_counter()
        t_prep += t1 - t0
        t_attn += t2 - t1
        layers += 1
    attn_bytes = layers * n * H * bytes_per_token_head
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    # one thread, one layer: the same work without OpenMP (layer 0 of sequence 0)
    oracle.set_threads(1)
    K = Kall[0, int(row0[0]):int(row0[0]) + n].cpu().numpy()
    V = Vall[0, int(row0[0]):int(row0[0]) + n].cpu().numpy()
    q = Qall[0, 0].cpu().numpy()
    t0 = time.perf_counter()
    eK = oracle.block_energy(K)
    eV = oracle.block_energy(V)
    kb, ks = oracle.allocate(eK, wl.k_budget)
    _, vs = oracle.allocate(eV, wl.v_bits * 64, oracle.UNIFORM)
    geom = oracle.Geometry(H, wl.k_budget, wl.v_bits, ((n + 63) // 64) * 64)
    region = np.zeros(geom.seq_bytes, np.uint8)
    oracle.quantize_pack(geom, region, K, V, 0, kb, ks, vs)
    t1 = time.perf_counter()
    oracle.decode_attention(geom, region, q, n, kb, ks, vs)
    t2 = time.perf_counter()
    oracle.set_threads(n_threads)
    one = {"threads": 1, "layers": 1, "prepare_s": round(t1 - t0, 3), "attention_s": round(t2 - t1, 3),
           "attention_GBps": round(n * H * bytes_per_token_head / (t2 - t1) / 1e9, 5),
           "quantize_tokens_per_s": round(n / (t1 - t0), 1)}
    return {"value": round(attn_bytes / t_attn / 1e9, 5), "unit": "GB/s", "cores": n_threads,
            "host_cores": host_cores, "kind": "oracle", "cpu": cpu_model, "one_thread": one,
            "sample": "sequence 0 (%d tokens), layers 0..%d, %d KV heads, %d query heads: decode attention "
                      "(fp64) %.2f s; energy+allocation+quantize of the same layers %.2f s (%.0f tokens/s)"
                      % (n, layers - 1, H, wl.n_q_heads, t_attn, t_prep, layers * n / t_prep),
            "quantize_tokens_per_s": round(layers * n / t_prep, 1)}


if __name__ == "__main__":
    main()
