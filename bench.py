#!/usr/bin/env python3
"""Decode-step benchmark of the int4 group-wise (g=64) compressed layer.

One step = one decode step of one OPT-shaped layer for the whole block of
B = g*m sequences, entirely in HBM:
  fgq_kv_append (the step's K and V rows into the compressed cache)
  fgq_decode_attn_q4kv (attend over prompt + t positions)
  fgq_dequant_gemm x 4 (Wq|Wk|Wv as one [h][3h] matrix, since the three
  projections share their input; Wout; W1; W2), one weight read per block.
Decode step t cycles through 1..32 (the pages' 32 generated tokens), so the
attended length runs from prompt+1 to prompt+32.  Inputs are seeded synthetic
draws (synth), already resident in HBM when the timed region starts.

Prints one JSON line.  The steps are timed twice: an eager pass with HIP
events recorded on the launch stream around every call (the per-kernel
durations and the roofline come from it), then the same steps replayed as HIP
graphs, one per (decode step, layer instance), which gives value and
ms_per_step (--no-graph: the eager pass gives them).  The CPU baseline is the
oracle on a bounded sample of one step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402
from int4_group_quantized_fgq_amd import accounting as acc  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFLOPS = 2516.6  # MI355X dense fp16 matrix peak, TFLOP/s
METRIC = "q4-KV decode attn + dequant-GEMM: tokens/s/layer, % HBM BW, % MFMA peak"


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=96)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--config", default="opt-175b", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--rotate", type=int, default=0,
                    help="layer instances cycled through (0: at least 3, and enough to exceed the 256 MB "
                         "last-level cache three times over)")
    ap.add_argument("--no-stream", action="store_true",
                    help="skip the weight-streaming measurement (packed weights from pinned host memory)")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the eager launches only (default: the step is also replayed as HIP graphs, "
                         "and that pass gives value and ms_per_step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gqa", action="store_true", help="skip the grouped-query attention line")
    ap.add_argument("--gqa-only", action="store_true",
                    help="only run the grouped-query attention line (for profiling that kernel)")
    ap.add_argument("--no-gqa-sweep", action="store_true", help="skip the K/V-head sweep of the grouped line")
    ap.add_argument("--summarize-gqa-trace", metavar="DIR",
                    help="only summarise a rocprofv3 --kernel-trace --stats folder of a --gqa-only run")
    ap.add_argument("--cpu-sample-seqs", type=int, default=4)
    ap.add_argument("--cpu-sample-cols", type=int, default=256)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 10 plain device copies of MIB MiB (HBM counter calibration under rocprofv3)")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("KERNEL_FETCH", "KERNEL_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="only summarise four rocprofv3 --pmc output folders (FETCH_SIZE / WRITE_SIZE of the "
                         "bench and of --calibrate-copy) into the HBM-traffic profile text")
    ap.add_argument("--kernel", default="dq_gemm_kernel", help="kernel summarised by --summarize-pmc")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="only summarise a rocprofv3 --kernel-trace --stats output folder of this bench: the "
                         "kernel statistics and the steady-state duration of every launch of a step")
    return ap.parse_args()


# Source files whose text defines each timed kernel: a committed counter
# summary applies only while their hash is unchanged.
KERNEL_SOURCES = {
    "dq_gemm_kernel": ("gemm.hip", "common.h"),
    "attn_gqa_kernel": ("gqa_attention.hip", "common.h"),
    "attn_split_kernel": ("attention.hip", "common.h"),
    "attn_topk_wave_kernel": ("topk_attention.hip", "common.h"),
}


def source_hash(kernel: str) -> str:
    """SHA-256 of the kernel's source code with // comments, trailing blanks
    and empty lines removed (a comment edit does not invalidate a measurement)."""
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "int4_group_quantized_fgq_amd", "csrc", f)) as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update((code + "\n").encode())
    return h.hexdigest()


def committed_traffic(kernel: str, config: str):
    """HBM bytes per launch measured by rocprofv3 counters (a 'traffic-json:'
    line of a summary under profiles/), or None when there is none for this
    kernel and workload or the kernel's source has changed since."""
    import glob
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as fh:
            for line in fh:
                if line.startswith("traffic-json: "):
                    d = json.loads(line[len("traffic-json: "):])
                    if d.get("kernel") == kernel and d.get("config") == config and \
                            d.get("source_sha256") == source_hash(kernel):
                        return d
    return None


def read_pmc(folder: str, counter: str):
    """{dispatch id: (kernel name, summed counter value)} from a rocprofv3 --pmc CSV folder."""
    import csv
    import glob
    out = {}
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under " + folder)
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                d = int(r["Dispatch_Id"])
                name, v = out.get(d, (r["Kernel_Name"], 0.0))
                out[d] = (name, v + float(r["Counter_Value"]))
    return out


def summarize_pmc(args):
    """Text of the HBM-traffic profile: counter KiB per dispatch of the kernel,
    scaled by what the same counters read for a copy of known size."""
    kf, kw, cf, cw = args.summarize_pmc
    copy_bytes = None
    fac = {}
    for counter, folder in (("FETCH_SIZE", cf), ("WRITE_SIZE", cw)):
        vals = [v for name, v in read_pmc(folder, counter).values() if "opy" in name or "elementwise" in name]
        big = max(vals)   # the copy dispatches (fills and small helpers read less)
        per = [v for v in vals if v > 0.5 * big]
        copy_bytes = args.calibrate_copy * 2 ** 20 if args.calibrate_copy else None
        fac[counter] = copy_bytes / (np.mean(per) * 1024.0) if copy_bytes else None
    res = {}
    for counter, folder in (("FETCH_SIZE", kf), ("WRITE_SIZE", kw)):
        vals = [v for name, v in read_pmc(folder, counter).values() if args.kernel in name]
        res[counter] = (len(vals), float(np.mean(vals)) if vals else 0.0)
    return fac, res


def measured_ceilings(torch) -> dict:
    """Achievable rates on this GPU next to the spec peaks: a 1 GiB device
    copy (HBM read + write) and a library fp16 GEMM (hipBLASLt, 8192^3)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a = torch.empty(2 ** 28, dtype=torch.float32, device="cuda").uniform_()
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 10 * 2 * a.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    n = 8192
    x = torch.randn(n, n, device="cuda").half()
    y = torch.randn(n, n, device="cuda").half()
    z = x @ y
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        z = x @ y
    e1.record()
    torch.cuda.synchronize()
    gemm_tf = 10 * 2.0 * n ** 3 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del x, y, z
    torch.cuda.empty_cache()
    return {"device_copy_GB_per_s": round(copy_gbs, 1), "hipblaslt_f16_gemm_8192_TFLOP_per_s": round(gemm_tf, 1),
            "spec_hbm_GB_per_s": HBM_PEAK_GBS, "spec_mfma_f16_TFLOP_per_s": MFMA_F16_PEAK_TFLOPS,
            "gpu": torch.cuda.get_device_name(0), "hip": torch.version.hip}


def calibrate_copy(torch, mib: int) -> None:
    a = torch.empty(mib * 2 ** 18, dtype=torch.float32, device="cuda").uniform_()
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(10):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_mib": mib, "copies": 10, "bytes_read_per_copy": mib * 2 ** 20,
                      "bytes_written_per_copy": mib * 2 ** 20}), flush=True)


class Layer:
    """One layer instance: packed weights and a compressed KV cache in HBM."""

    def __init__(self, torch, fgq, w, inst, host_weights, prompt_chunks):
        B, H, D, cap = w.batch, w.heads, w.head_dim, w.capacity
        dev = "cuda"
        # zero-filled: a position not yet appended reconstructs to 0 (min 0, step 0)
        self.k_codes = torch.zeros((B, H, cap, D // 2), dtype=torch.uint8, device=dev)
        self.v_codes = torch.zeros_like(self.k_codes)
        self.k_meta = torch.zeros((B, H, cap, D // 64), dtype=torch.int32, device=dev)
        self.v_meta = torch.zeros_like(self.k_meta)
        self.kv = fgq.kv_struct(self.k_codes, self.v_codes, self.k_meta, self.v_meta, B, H, D, cap)
        for b0, nb, kd, vd in prompt_chunks:
            sub = fgq.kv_struct(self.k_codes[b0:b0 + nb], self.v_codes[b0:b0 + nb], self.k_meta[b0:b0 + nb],
                                self.v_meta[b0:b0 + nb], nb, H, D, cap)
            fgq.fgq_kv_append(sub, kd, vd, 0, w.prompt)
        self.packed = [(pc.clone(), pm.clone()) for pc, pm in host_weights]


def launch_plan(w):
    """The step's GEMM launches as (name, K, N, weight indices).  Weights whose
    projections read the same input (Wq, Wk, Wv of an OPT layer: the first
    three square matrices) are concatenated along N into one launch; groups of
    64 output channels never straddle two matrices, so the fused matrix's
    codes and metadata are the three matrices' side by side."""
    ws = list(w.weights)
    if len(ws) == 6 and ws[0] == ws[1] == ws[2] and ws[0][0] == ws[0][1]:
        K = ws[0][0]
        return [("qkv", K, 3 * K, (0, 1, 2)), ("out", ws[3][0], ws[3][1], (3,)),
                ("ffn1", ws[4][0], ws[4][1], (4,)), ("ffn2", ws[5][0], ws[5][1], (5,))]
    return [("w%d" % i, K, N, (i,)) for i, (K, N) in enumerate(ws)]


def build_weights(torch, fgq, w):
    """Quantise and pack every weight of the layer once (offline step)."""
    out = []
    for name, K, N, idx in launch_plan(w):
        t0 = time.time()
        wd = torch.cat([torch.from_numpy(synth.weight(w, i)).to("cuda") for i in idx], dim=1).contiguous()
        codes = torch.empty((K, N // 2), dtype=torch.uint8, device="cuda")
        meta = torch.empty((K, N // 64), dtype=torch.int32, device="cuda")
        fgq.fgq_quantize_g64(wd, K, N, N, codes, meta)
        pc = torch.empty(K * N // 8, dtype=torch.int32, device="cuda")
        pm = torch.empty(fgq.fgq_pack_weight_meta_words(K, N), dtype=torch.int32, device="cuda")
        fgq.fgq_pack_weight_g64(codes, meta, K, N, pc, pm)
        torch.cuda.synchronize()
        del wd, codes, meta
        out.append((pc, pm))
        log("weight %s (%dx%d) quantised+packed in %.1fs" % (name, K, N, time.time() - t0))
    return out


def prompt_chunks(torch, w, chunk=8):
    for b0 in range(0, w.batch, chunk):
        nb = min(chunk, w.batch - b0)
        kd = torch.from_numpy(synth.prompt_kv(w, "k", b0=b0, nb=nb)).to("cuda")
        vd = torch.from_numpy(synth.prompt_kv(w, "v", b0=b0, nb=nb)).to("cuda")
        yield b0, nb, kd, vd


def cpu_baseline(w, args):
    """The oracle (never tuned) on a bounded sample of one decode step (t = 1),
    scaled to the whole step: a few sequences of append and attention, a few
    256-column slices of every weight GEMM with all g*m rows."""
    import oracle
    S = min(args.cpu_sample_seqs, w.batch)
    H, D = w.heads, w.head_dim
    t = 1
    secs = {}
    # append + attention on S sequences (their prompt is appended untimed)
    ref = oracle.KVCache(S, H, D, w.capacity)
    oracle.kv_append(ref, synth.prompt_kv(w, "k", nb=S), synth.prompt_kv(w, "v", nb=S), 0)
    sk, sv = synth.step_kv(w, "k", t)[:S], synth.step_kv(w, "v", t)[:S]
    q = synth.step_q(w, t)[:S]
    t0 = time.perf_counter()
    oracle.kv_append(ref, sk, sv, w.prompt + t - 1)
    secs["append"] = (time.perf_counter() - t0) * w.batch / S
    t0 = time.perf_counter()
    oracle.decode_attn(ref, q, w.kv_len(t))
    secs["attention"] = (time.perf_counter() - t0) * w.batch / S
    gemm_s = 0.0
    cols = args.cpu_sample_cols
    for i, (K, N) in enumerate(w.weights):
        ncol = min(cols, N)
        wt = synth.weight(w, i)[:, :ncol]
        c, m = oracle.quantize_g64(np.ascontiguousarray(wt))
        x = synth.gemm_x(w, i, t)
        t0 = time.perf_counter()
        oracle.dequant_gemm(x, w.g, w.m, c, m)
        gemm_s += (time.perf_counter() - t0) * N / ncol
    secs["gemm"] = gemm_s
    total = sum(secs.values())
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    return {
        "value": w.batch / total,
        "unit": "tokens/s/layer",
        "cores": cores,
        "kind": "oracle",
        "sample": "decode step t=1 of %s: append+attention on %d of %d sequences, every weight GEMM on a "
                  "%d-column slice with all %d rows; each part scaled to the full step" %
                  (w.name, S, w.batch, cols, w.batch),
        "seconds_per_step": {k: round(v, 4) for k, v in secs.items()},
    }


def short_name(kernel_name: str) -> str:
    n = kernel_name.replace("(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0].replace("fgq::", "").strip()


def summarize_trace(folder: str, w, steps: int) -> None:
    """Markdown: rocprofv3's kernel statistics, then the mean duration of each
    launch of a step over the last `steps` steps (a step starts with the KV
    append; the split-K reduction is listed with the GEMM launch it ends)."""
    import csv
    import glob

    def one(pattern):
        f = glob.glob(os.path.join(folder, "**", pattern), recursive=True)
        if not f:
            raise SystemExit("no %s under %s" % (pattern, folder))
        with open(f[0]) as fh:
            return list(csv.DictReader(fh))

    stats = one("*kernel_stats.csv")
    print("| kernel | calls | average us | total ms | % of GPU time |")
    print("|---|---|---|---|---|")
    for r in stats[:12]:
        print("| %s | %s | %.1f | %.2f | %.1f |" % (short_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
                                                  float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    trace = sorted(one("*kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    names = ["append", "attention"] + ["gemm_" + p[0] for p in launch_plan(w)]
    stepl = []
    cur = None
    for r in trace:
        n = short_name(r["Kernel_Name"])
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if n.startswith("kv_append_kernel") and int(r["Grid_Size_X"]) == w.batch * w.hidden // 4:
            cur = {"ops": [], "kernels": {}}
            stepl.append(cur)
            cur["ops"].append(["append", d])
        elif cur is None:
            continue
        elif n.startswith("attn_split_kernel"):
            cur["ops"].append(["attention", d])
        elif n.startswith("attn_merge_kernel"):
            cur["ops"][-1][1] += d
        elif n.startswith("dq_gemm_kernel"):
            cur["ops"].append([names[len(cur["ops"])] if len(cur["ops"]) < len(names) else "?", d])
        elif n.startswith("splitk_reduce_kernel"):
            cur["ops"][-1][1] += d
    good = [st for st in stepl if [o[0] for o in st["ops"]] == names][-steps:]
    print()
    print("Steady state, mean of the last %d steps (us per launch; a GEMM launch includes its split-K "
          "reduction, attention its merge):" % len(good))
    print()
    print("| launch | us |")
    print("|---|---|")
    tot = 0.0
    for i, nm in enumerate(names):
        v = float(np.mean([st["ops"][i][1] for st in good])) if good else float("nan")
        tot += v
        print("| %s | %.1f |" % (nm, v))
    print("| step (sum) | %.1f |" % tot)


def summarize_gqa_trace(folder: str) -> None:
    """Markdown for a rocprofv3 run of `bench.py --gqa-only`: the kernel
    statistics, then the mean duration of the grouped attention launches of
    the decode steps (the grid of the workload's split plan) and of their
    split merges."""
    import csv
    import glob

    def one(pattern):
        f = glob.glob(os.path.join(folder, "**", pattern), recursive=True)
        if not f:
            raise SystemExit("no %s under %s" % (pattern, folder))
        with open(f[0]) as fh:
            return list(csv.DictReader(fh))

    stats = one("*kernel_stats.csv")
    print("| kernel | calls | average us | total ms | % of GPU time |")
    print("|---|---|---|---|---|")
    for r in stats[:10]:
        print("| %s | %s | %.1f | %.2f | %.1f |" % (short_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
                                                  float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    trace = sorted(one("*kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    by_grid = {}
    merge = []
    prev = None
    for r in trace:
        n = short_name(r["Kernel_Name"])
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        if n.startswith("attn_gqa_kernel"):
            by_grid.setdefault((n, int(r["Grid_Size_X"])), []).append(d)
            prev = (n, int(r["Grid_Size_X"]))
        elif n.startswith("attn_gqa_merge_kernel") and prev is not None:
            merge.append((prev, d))
    print()
    print("Grouped attention launches by grid (the decode steps are the most frequent grid):")
    print()
    print("| kernel | grid (threads) | launches | mean us | split merge mean us |")
    print("|---|---|---|---|---|")
    for key, ds in sorted(by_grid.items(), key=lambda kv: -len(kv[1])):
        ms = [d for k, d in merge if k == key]
        print("| %s | %d | %d | %.1f | %s |" % (key[0], key[1], len(ds), float(np.mean(ds)),
                                              "%.1f" % float(np.mean(ms)) if ms else "-"))


def algorithmic_bytes_per_launch(kernel: str, w, n_steps: int = 0, warmup: int = 0) -> float:
    """Mean algorithmic HBM bytes of one launch of the kernel over the first
    n_steps bench steps (0: one full cycle of decode steps); the top-K kernel
    runs min(warmup, 8) untimed launches and then one per timed step."""
    if kernel == "dq_gemm_kernel":
        plan = launch_plan(w)
        return float(np.mean([acc.gemm_bytes(w.batch, K, N) for _, K, N, _ in plan]))
    if kernel == "attn_gqa_kernel":
        g = synth.WORKLOADS["gqa"]
        n = n_steps or g.steps
        ts = [i % g.steps + 1 for i in range(n)]
        return float(np.mean([acc.gqa_attention_bytes(g.batch, g.heads, g.n_kv_heads, g.head_dim, g.kv_len(t))
                              for t in ts]))
    if kernel == "attn_topk_wave_kernel":
        n = n_steps or w.steps
        ts = [i % w.steps + 1 for i in range(min(warmup, 8))] + \
            [(warmup + i) % w.steps + 1 for i in range(n - warmup)]
        return float(np.mean([acc.topk_attention_bytes(w.batch, w.hidden, w.kv_len(t), -(-w.kv_len(t) // 10))
                              for t in ts]))
    ts = [i % w.steps + 1 for i in range(n_steps or w.steps)]
    return float(np.mean([acc.attention_bytes(w.batch, w.hidden, w.kv_len(t)) for t in ts]))


def weight_streaming(torch, fgq, w, layers, plan, steps_in, attn_out, ys, attn_ws, attn_ws_b, gemm_ws, gemm_ws_b,
                     stream, args):
    """The layer step with the layer's packed weights arriving from pinned host
    memory each step (the offloading setting compression was made for): two
    device buffers, the next step's weights copied on a second stream while
    this step computes; the KV cache stays in HBM.  Also times the plain
    host-to-device copy of the same bytes and of the fp16 weights they replace."""
    B = w.batch
    host = [(pc.cpu().pin_memory(), pm.cpu().pin_memory()) for pc, pm in layers[0].packed]
    nbytes = sum(a.numel() * 4 + b.numel() * 4 for a, b in host)
    bufs = [[(torch.empty_like(pc), torch.empty_like(pm)) for pc, pm in layers[0].packed] for _ in range(2)]
    cstream = torch.cuda.Stream()
    ch = stream.cuda_stream
    copied = [torch.cuda.Event() for _ in range(2)]
    freed = [torch.cuda.Event() for _ in range(2)]
    L = layers[0]
    n = 8

    def copy(i):
        k = i % 2
        with torch.cuda.stream(cstream):
            cstream.wait_event(freed[k])
            for (hc, hm), (dc, dm) in zip(host, bufs[k]):
                dc.copy_(hc, non_blocking=True)
                dm.copy_(hm, non_blocking=True)
            copied[k].record(cstream)

    def step(i):
        k = i % 2
        t = i % w.steps + 1
        d = steps_in[t - 1]
        stream.wait_event(copied[k])
        fgq.fgq_kv_append(L.kv, d["k"], d["v"], w.prompt + t - 1, 1, ch)
        fgq.fgq_decode_attn_q4kv(L.kv, d["q"], w.prompt + t, 0.0, attn_out, fgq.FGQ_DTYPE_F32, attn_ws, attn_ws_b, ch)
        for wi, (_, K, N, _) in enumerate(plan):
            dc, dm = bufs[k][wi]
            fgq.fgq_dequant_gemm(d["x"][wi], w.g, w.m, K, N, dc, dm, ys[wi], fgq.FGQ_DTYPE_F32, gemm_ws, gemm_ws_b, ch)
        freed[k].record(stream)

    for k in range(2):
        freed[k].record(stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    copy(0)
    e0.record(stream)
    for i in range(n):
        if i + 1 < n:
            copy(i + 1)
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    # the plain copy of the packed bytes, and of fp16 weights of the same matrices
    f16 = torch.empty(sum(K * N for _, K, N, _ in plan), dtype=torch.float16).pin_memory()
    dev16 = torch.empty_like(f16, device="cuda")
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    g0.record(stream)
    dev16.copy_(f16, non_blocking=True)
    g1.record(stream)
    torch.cuda.synchronize()
    f16_ms = g0.elapsed_time(g1)
    del dev16, f16, bufs, host
    return {"steps": n, "packed_bytes_per_step": nbytes, "ms_per_step": ms,
            "tokens_per_s_per_layer": B / (ms * 1e-3), "h2d_GB_per_s": nbytes / (ms * 1e-3) / 1e9,
            "fp16_weights_copy_ms": f16_ms, "fp16_over_packed_bytes": 2.0 * sum(K * N for _, K, N, _ in plan) / nbytes}


def gqa_attention_line(torch, fgq, stream, steps: int, warmup: int, sweep_heads=(32, 16, 8, 4, 2, 1)) -> dict:
    """Grouped-query decode attention over the compressed cache at the grouped
    workload's shape (16 sequences, 16K cached positions, 32 query heads over
    8 K/V heads): the prompt bulk-compressed into the cache, then decode steps
    of one appended K/V token and attention over prompt + t positions, the
    attention timed with HIP events on the launch stream.  The K/V-head sweep
    reuses that cache: its first heads for fewer K/V heads, its heads
    repeated for more (same seeded values; the timing does not depend on them)."""
    w = synth.WORKLOADS["gqa"]
    B, Hq, Hkv, D, cap = w.batch, w.heads, w.n_kv_heads, w.head_dim, w.capacity
    sh = stream.cuda_stream

    def alloc(hk):
        kc = torch.zeros((B, hk, cap, D // 2), dtype=torch.uint8, device="cuda")
        km = torch.zeros((B, hk, cap, D // 64), dtype=torch.int32, device="cuda")
        return kc, torch.zeros_like(kc), km, torch.zeros_like(km)

    kc, vc, km, vm = alloc(Hkv)
    for b0 in range(0, B, 4):
        nb = min(4, B - b0)
        sub = fgq.kv_struct(kc[b0:b0 + nb], vc[b0:b0 + nb], km[b0:b0 + nb], vm[b0:b0 + nb], nb, Hkv, D, cap)
        kd = torch.from_numpy(synth.prompt_kv(w, "k", b0=b0, nb=nb)).to("cuda")
        vd = torch.from_numpy(synth.prompt_kv(w, "v", b0=b0, nb=nb)).to("cuda")
        fgq.fgq_kv_append(sub, kd, vd, 0, w.prompt, sh)
        torch.cuda.synchronize()
        del kd, vd
    kv = fgq.kv_struct(kc, vc, km, vm, B, Hkv, D, cap)
    st = [{"k": torch.from_numpy(synth.step_kv(w, "k", t)).to("cuda"),
           "v": torch.from_numpy(synth.step_kv(w, "v", t)).to("cuda"),
           "q": torch.from_numpy(synth.step_q(w, t)).to("cuda")} for t in range(1, w.steps + 1)]
    out = torch.empty((B, Hq * D), dtype=torch.float32, device="cuda")
    wsb = max(fgq.fgq_decode_attn_gqa_ws_bytes(B, Hq, Hkv, D, L) for L in range(w.prompt + 1, cap + 1))
    wsb_all = max(fgq.fgq_decode_attn_gqa_ws_bytes(B, Hq, hk, D, cap) for hk in (1, 2, 4, 8, 16, 32))
    ws = torch.empty(max(wsb, wsb_all, 16), dtype=torch.uint8, device="cuda")

    def step(i, ev=None):
        t = i % w.steps + 1
        d = st[t - 1]
        fgq.fgq_kv_append(kv, d["k"], d["v"], w.prompt + t - 1, 1, sh)
        if ev is not None:
            ev[0].record(stream)
        fgq.fgq_decode_attn_gqa_q4kv(kv, d["q"], Hq, w.prompt + t, 0.0, out, fgq.FGQ_DTYPE_F32, ws, ws.numel(), sh)
        if ev is not None:
            ev[1].record(stream)

    for i in range(warmup):
        step(i)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(warmup + i, evs[i])
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs)
    ts = [(warmup + i) % w.steps + 1 for i in range(steps)]
    byts = sum(acc.gqa_attention_bytes(B, Hq, Hkv, D, w.kv_len(t)) for t in ts)
    fl = sum(acc.gqa_attention_flops(B, Hq, D, w.kv_len(t)) for t in ts)
    line = {"workload": "gqa: %d sequences, %d query heads over %d K/V heads x %d, prompt %d + %d decode steps"
                        % (B, Hq, Hkv, D, w.prompt, w.steps),
            "us_per_launch": 1e3 * ms / steps, "GB_per_s": byts / (ms * 1e-3) / 1e9,
            "frac_hbm_peak": byts / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "TFLOP_per_s": fl / (ms * 1e-3) / 1e12}

    # K/V-head sweep at kv_len = capacity (the cache now holds every decode step)
    sweep = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    q = st[-1]["q"]
    for hk in sweep_heads:
        if hk == Hkv:
            arrs = (kc, vc, km, vm)
        elif hk < Hkv:
            arrs = tuple(a[:, :hk].contiguous() for a in (kc, vc, km, vm))
        else:
            arrs = tuple(a.repeat_interleave(hk // Hkv, dim=1) for a in (kc, vc, km, vm))
        kvs = fgq.kv_struct(*arrs, B, hk, D, cap)
        for _ in range(3):
            fgq.fgq_decode_attn_gqa_q4kv(kvs, q, Hq, cap, 0.0, out, fgq.FGQ_DTYPE_F32, ws, ws.numel(), sh)
        torch.cuda.synchronize()
        reps = 10
        e0.record(stream)
        for _ in range(reps):
            fgq.fgq_decode_attn_gqa_q4kv(kvs, q, Hq, cap, 0.0, out, fgq.FGQ_DTYPE_F32, ws, ws.numel(), sh)
        e1.record(stream)
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / reps
        b = acc.gqa_attention_bytes(B, Hq, hk, D, cap)
        sweep["kv_heads_%d" % hk] = {"group": Hq // hk, "us_per_launch": us, "GB_per_s": b / us / 1e3,
                                     "frac_hbm_peak": b / us / 1e3 / HBM_PEAK_GBS,
                                     "TFLOP_per_s": acc.gqa_attention_flops(B, Hq, D, cap) / us / 1e6}
        del arrs, kvs
    tr = committed_traffic("attn_gqa_kernel", "gqa")
    if tr is not None:
        line["traffic_bytes_per_launch"] = tr["bytes_per_launch"]
        line["traffic_vs_algorithmic"] = tr["ratio"]
    if sweep:
        line["kv_head_sweep_at_kv_len_%d" % cap] = sweep
    del kc, vc, km, vm, st
    torch.cuda.empty_cache()
    return line


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, synth.WORKLOADS[args.config], args.steps)
        return
    if args.summarize_gqa_trace:
        summarize_gqa_trace(args.summarize_gqa_trace)
        return
    if args.summarize_pmc:
        w = synth.WORKLOADS[args.config]
        fac, res = summarize_pmc(args)
        n_f, fetch_kib = res["FETCH_SIZE"]
        n_w, write_kib = res["WRITE_SIZE"]
        per_launch = fetch_kib * 1024.0 * fac["FETCH_SIZE"] + write_kib * 1024.0 * fac["WRITE_SIZE"]
        alg = algorithmic_bytes_per_launch(args.kernel, w, args.warmup + args.steps, args.warmup)
        d = {"kernel": args.kernel, "config": w.name, "source_sha256": source_hash(args.kernel),
             "dispatches": [n_f, n_w], "fetch_kib_per_dispatch": round(fetch_kib, 1),
             "write_kib_per_dispatch": round(write_kib, 1), "fetch_factor": round(fac["FETCH_SIZE"], 4),
             "write_factor": round(fac["WRITE_SIZE"], 4), "bytes_per_launch": round(per_launch),
             "algorithmic_bytes_per_launch": round(alg), "ratio": round(per_launch / alg, 4)}
        print("| counter | dispatches | KiB per dispatch | copy calibration factor | bytes per launch |")
        print("|---|---|---|---|---|")
        print("| FETCH_SIZE | %d | %.1f | %.4f | %.4g |" % (n_f, fetch_kib, fac["FETCH_SIZE"],
                                                           fetch_kib * 1024 * fac["FETCH_SIZE"]))
        print("| WRITE_SIZE | %d | %.1f | %.4f | %.4g |" % (n_w, write_kib, fac["WRITE_SIZE"],
                                                           write_kib * 1024 * fac["WRITE_SIZE"]))
        print()
        print("HBM traffic per launch %.4g B; algorithmic %.4g B; ratio %.3f" % (per_launch, alg, per_launch / alg))
        print()
        print("traffic-json: " + json.dumps(d))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the kernels shard by "
              "sequence/head and by weight column; see DESIGN.md). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import int4_group_quantized_fgq_amd as fgq
    fgq.load()   # fails loudly when the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        calibrate_copy(torch, args.calibrate_copy)
        return
    if args.gqa_only:
        line = gqa_attention_line(torch, fgq, torch.cuda.current_stream(), args.steps, args.warmup,
                                  () if args.no_gqa_sweep else (32, 16, 8, 4, 2, 1))
        print(json.dumps({"gqa_attention": line}), flush=True)
        return
    w = synth.WORKLOADS[args.config]
    B, H, D, h = w.batch, w.heads, w.head_dim, w.hidden
    M = B

    # ---------------- setup (untimed): weights, caches, per-step inputs
    t_setup = time.time()
    plan = launch_plan(w)
    weights = build_weights(torch, fgq, w)
    per_layer = acc.packed_bytes(sum(K * N for K, N in w.weights)) + \
        2 * acc.packed_bytes(B * h * w.capacity)
    R = args.rotate or max(3, min(8, int(np.ceil(3 * 256e6 / per_layer))))
    layers = []
    for inst in range(R):
        layers.append(Layer(torch, fgq, w, inst, weights, prompt_chunks(torch, w)))
        log("layer instance %d ready (%.1fs)" % (inst, time.time() - t_setup))
    del weights
    steps_in = []
    for t in range(1, w.steps + 1):
        d = {
            "k": torch.from_numpy(synth.step_kv(w, "k", t)).to("cuda"),
            "v": torch.from_numpy(synth.step_kv(w, "v", t)).to("cuda"),
            "q": torch.from_numpy(synth.step_q(w, t)).to("cuda"),
            "x": [torch.from_numpy(synth.gemm_x(w, idx[0], t)).to("cuda") for _, _, _, idx in plan],
        }
        steps_in.append(d)
    attn_out = torch.empty((B, h), dtype=torch.float32, device="cuda")
    ys = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _, _, N, _ in plan]
    attn_ws_b = max(fgq.fgq_decode_attn_ws_bytes(B, H, D, L) for L in range(w.prompt + 1, w.capacity + 1))
    gemm_ws_b = max([fgq.fgq_dequant_gemm_ws_bytes(M, K, N) for _, K, N, _ in plan] + [0])
    attn_ws = torch.empty(max(attn_ws_b, 16), dtype=torch.uint8, device="cuda")
    gemm_ws = torch.empty(max(gemm_ws_b, 16), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    log("setup %.1fs, %d layer instance(s), %.2f GB per instance" % (time.time() - t_setup, R, per_layer / 1e9))

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    ops = ["append", "attention"] + ["gemm_" + p[0] for p in plan]

    def run_step(i, ev=None, sh=sh):
        t = i % w.steps + 1
        L = layers[i % R]
        d = steps_in[t - 1]
        if ev is not None:
            ev[0].record(stream)
        fgq.fgq_kv_append(L.kv, d["k"], d["v"], w.prompt + t - 1, 1, sh)
        if ev is not None:
            ev[1].record(stream)
        fgq.fgq_decode_attn_q4kv(L.kv, d["q"], w.prompt + t, 0.0, attn_out, fgq.FGQ_DTYPE_F32, attn_ws,
                                 attn_ws_b, sh)
        if ev is not None:
            ev[2].record(stream)
        for wi, (_, K, N, _) in enumerate(plan):
            pc, pm = L.packed[wi]
            fgq.fgq_dequant_gemm(d["x"][wi], w.g, w.m, K, N, pc, pm, ys[wi], fgq.FGQ_DTYPE_F32, gemm_ws,
                                 gemm_ws_b, sh)
            if ev is not None:
                ev[3 + wi].record(stream)

    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()

    n_ev = 3 + len(plan)
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        run_step(args.warmup + i, events[i])
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(stop)

    # ---------------- the same steps as HIP graphs: one graph per (decode step,
    # layer instance), captured once, replayed with every input already in place
    graph_ms = None
    if not args.no_graph:
        graphs = {}
        cap = torch.cuda.Stream()      # capture needs a stream other than the default one
        for i in range(args.warmup + args.steps):
            key = (i % w.steps, i % R)
            if key not in graphs:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=cap):
                    run_step(i, sh=cap.cuda_stream)
                graphs[key] = g
        torch.cuda.synchronize()
        for i in range(args.warmup):
            graphs[(i % w.steps, i % R)].replay()
        torch.cuda.synchronize()
        gstart = torch.cuda.Event(enable_timing=True)
        gstop = torch.cuda.Event(enable_timing=True)
        wall0 = time.perf_counter()
        gstart.record(stream)
        for i in range(args.steps):
            j = args.warmup + i
            graphs[(j % w.steps, j % R)].replay()
        gstop.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        graph_ms = gstart.elapsed_time(gstop)
        log("%d graphs captured; graph pass %.3f ms/step, eager pass %.3f ms/step" %
            (len(graphs), graph_ms / args.steps, total_ms / args.steps))

    op_ms = {o: 0.0 for o in ops}
    for ev in events:
        op_ms["append"] += ev[0].elapsed_time(ev[1])
        op_ms["attention"] += ev[1].elapsed_time(ev[2])
        for wi, p in enumerate(plan):
            op_ms["gemm_" + p[0]] += ev[2 + wi].elapsed_time(ev[3 + wi])

    # ---------------- accounting
    K_steps = args.steps
    ts = [(args.warmup + i) % w.steps + 1 for i in range(K_steps)]
    attn_bytes = sum(acc.attention_bytes(B, h, w.kv_len(t)) for t in ts)
    attn_flops = sum(acc.attention_flops(B, h, w.kv_len(t)) for t in ts)
    app_bytes = K_steps * acc.append_bytes(B, h)
    gemm_flops = K_steps * acc.layer_gemm_flops(M, w.weights)
    gemm_bytes = K_steps * sum(acc.gemm_bytes(M, K, N) for _, K, N, _ in plan)
    gemm_ms = sum(op_ms["gemm_" + p[0]] for p in plan)
    attn_gbs = attn_bytes / (op_ms["attention"] * 1e-3) / 1e9
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12 if gemm_ms > 0 else 0.0
    step_total_ms = total_ms if graph_ms is None else graph_ms
    ms_per_step = step_total_ms / K_steps
    value = B * K_steps / (step_total_ms * 1e-3)

    kernels = {
        "append": {"us_per_launch": 1e3 * op_ms["append"] / K_steps,
                   "GB_per_s": app_bytes / (op_ms["append"] * 1e-3) / 1e9},
        "attention": {"us_per_launch": 1e3 * op_ms["attention"] / K_steps, "GB_per_s": attn_gbs,
                      "frac_hbm_peak": attn_gbs / HBM_PEAK_GBS,
                      "TFLOP_per_s": attn_flops / (op_ms["attention"] * 1e-3) / 1e12},
    }
    for name, K, N, _ in plan:
        ms = op_ms["gemm_" + name]
        f = K_steps * acc.gemm_flops(M, K, N)
        kernels["gemm_%s_%dx%d" % (name, K, N)] = {
            "us_per_launch": 1e3 * ms / K_steps,
            "TFLOP_per_s": f / (ms * 1e-3) / 1e12,
            "frac_mfma_peak": f / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
            "GB_per_s": K_steps * acc.gemm_bytes(M, K, N) / (ms * 1e-3) / 1e9,
        }

    # prompt bulk compression (the prefill side of the cache, reported beside the
    # decode step): the first 8 sequences' prompt K and V rewritten into layer 0
    nb = min(8, B)
    kd = torch.from_numpy(synth.prompt_kv(w, "k", nb=nb)).to("cuda")
    vd = torch.from_numpy(synth.prompt_kv(w, "v", nb=nb)).to("cuda")
    L0 = layers[0]
    sub = fgq.kv_struct(L0.k_codes[:nb], L0.v_codes[:nb], L0.k_meta[:nb], L0.v_meta[:nb], nb, H, D, w.capacity)
    fgq.fgq_kv_append(sub, kd, vd, 0, w.prompt, sh)
    torch.cuda.synchronize()
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    b0.record(stream)
    for _ in range(reps):
        fgq.fgq_kv_append(sub, kd, vd, 0, w.prompt, sh)
    b1.record(stream)
    torch.cuda.synchronize()
    bulk_us = 1e3 * b0.elapsed_time(b1) / reps
    # prefill attention over the same sequences' fp16 prompt (causal), which
    # precedes that compression in a prefill step
    qd = torch.from_numpy(synth.prompt_q(w, nb=nb)).to("cuda")
    pf_out = torch.empty((nb, w.prompt, h), dtype=torch.float32, device="cuda")
    fgq.fgq_prefill_attn_f16(qd, kd, vd, nb, w.prompt, H, D, 0.0, pf_out, fgq.FGQ_DTYPE_F32, sh)
    torch.cuda.synchronize()
    b0.record(stream)
    for _ in range(reps):
        fgq.fgq_prefill_attn_f16(qd, kd, vd, nb, w.prompt, H, D, 0.0, pf_out, fgq.FGQ_DTYPE_F32, sh)
    b1.record(stream)
    torch.cuda.synchronize()
    pf_us = 1e3 * b0.elapsed_time(b1) / reps
    pf_flops = acc.prefill_attention_flops(nb, h, w.prompt)
    kernels["prefill_attention"] = {
        "sequences": nb, "tokens_per_sequence": w.prompt, "us_per_launch": pf_us,
        "TFLOP_per_s": pf_flops / (pf_us * 1e-6) / 1e12,
        "frac_mfma_peak": pf_flops / (pf_us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS,
        "us_whole_block_estimate": pf_us * B / nb}
    del kd, vd, qd, pf_out
    kernels["prompt_bulk_append"] = {
        "sequences": nb, "tokens_per_sequence": w.prompt, "us_per_launch": bulk_us,
        "GB_per_s": acc.append_bytes(nb, h, w.prompt) / (bulk_us * 1e-6) / 1e9,
        "frac_hbm_peak": acc.append_bytes(nb, h, w.prompt) / (bulk_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
        "us_whole_block_estimate": bulk_us * B / nb}

    # top-K sparse attention (the pages' optional approximation: keep the top
    # tenth of the positions, read only their V rows), over the same decode steps
    tk_out = torch.empty((B, h), dtype=torch.float32, device="cuda")

    def topk_launch(i):
        t = i % w.steps + 1
        L_t = w.prompt + t
        fgq.fgq_decode_attn_topk_q4kv(layers[i % R].kv, steps_in[t - 1]["q"], L_t, -(-L_t // 10), 0.0, tk_out,
                                      fgq.FGQ_DTYPE_F32, None, sh)

    for i in range(min(args.warmup, 8)):
        topk_launch(i)
    tk_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K_steps)]
    torch.cuda.synchronize()
    for i in range(K_steps):
        tk_ev[i][0].record(stream)
        topk_launch(args.warmup + i)
        tk_ev[i][1].record(stream)
    torch.cuda.synchronize()
    tk_ms = sum(a.elapsed_time(b) for a, b in tk_ev)
    tk_bytes = sum(acc.topk_attention_bytes(B, h, w.kv_len(t), -(-w.kv_len(t) // 10)) for t in ts)
    kernels["topk_attention"] = {
        "kept": "ceil(kv_len/10)", "us_per_launch": 1e3 * tk_ms / K_steps,
        "GB_per_s": tk_bytes / (tk_ms * 1e-3) / 1e9,
        "frac_hbm_peak": tk_bytes / (tk_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "time_vs_dense_attention": tk_ms / op_ms["attention"]}
    tk_tr = committed_traffic("attn_topk_wave_kernel", w.name)
    if tk_tr is not None and w.kv_len(w.steps) <= 2048:
        kernels["topk_attention"]["traffic_bytes_per_launch"] = tk_tr["bytes_per_launch"]
        kernels["topk_attention"]["traffic_vs_algorithmic"] = tk_tr["ratio"]

    if not args.no_gqa:
        t0 = time.time()
        kernels["gqa_attention"] = gqa_attention_line(torch, fgq, stream, 32, 8,
                                                      () if args.no_gqa_sweep else (32, 16, 8, 4, 2, 1))
        log("gqa attention line %.1fs" % (time.time() - t0))

    if w.weights and not args.no_stream:
        kernels["weight_streaming"] = weight_streaming(torch, fgq, w, layers, plan, steps_in, attn_out, ys, attn_ws,
                                                       attn_ws_b, gemm_ws, gemm_ws_b, stream, args)

    if w.weights and gemm_ms >= op_ms["attention"]:
        kname = "dq_gemm_kernel"
        roof = {"bound": "mfma", "kernel": kname + " (all %d weight GEMM launches of the step)" % len(plan),
                "achieved": gemm_tflops, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": gemm_tflops / MFMA_F16_PEAK_TFLOPS, "traffic": None,
                "algorithmic_per_launch": "2*M*K*N flops, M=%d; mean algorithmic bytes per launch %.4g" %
                                          (M, algorithmic_bytes_per_launch(kname, w))}
    else:
        kname = "attn_split_kernel"
        roof = {"bound": "hbm", "kernel": kname, "achieved": attn_gbs, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": attn_gbs / HBM_PEAK_GBS, "traffic": None,
                "algorithmic_per_launch": "1.125*hidden*kv_len bytes per sequence (+q, out); mean %.4g" %
                                          algorithmic_bytes_per_launch(kname, w)}
    tr = committed_traffic(kname, w.name)
    if tr is not None:
        roof["traffic"] = tr["bytes_per_launch"]
        roof["traffic_source"] = "rocprofv3 FETCH_SIZE + WRITE_SIZE per launch, copy-calibrated (profiles/)"

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": K_steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded Philox draws: KV and activations N(0,1), weights N(0,0.02))",
        "config": {"workload": w.name, "batch_g_x_m": "%dx%d" % (w.g, w.m), "global_batch": B,
                   "heads": H, "head_dim": D, "hidden": h, "prompt": w.prompt, "decode_steps": w.steps,
                   "weights": ["%dx%d" % kn for kn in w.weights],
                   "gemm_launches": ["%s %dx%d" % (p[0], p[1], p[2]) for p in plan], "layer_instances": R,
                   "parallelism": "single GPU"},
        "roofline": roof,
        "hbm_roofline_attention": {"achieved": attn_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": attn_gbs / HBM_PEAK_GBS},
        "mfma_roofline_gemm": {"achieved": gemm_tflops, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                               "frac": gemm_tflops / MFMA_F16_PEAK_TFLOPS,
                               "GB_per_s": gemm_bytes / (gemm_ms * 1e-3) / 1e9 if gemm_ms else 0.0},
        "step_launch": "eager" if graph_ms is None else "hip-graph replay (one graph per decode step and layer "
                                                           "instance)",
        "eager_ms_per_step": total_ms / K_steps,
        "kernels": kernels,
        "wall_s_timed_region": wall,
        "context": "pages' end-to-end FlexGen 4-bit OPT-175B on one T4 with offloading: 1.12 token/s "
                   "(all 96 layers, prefill included) - not comparable to this per-layer in-HBM rate",
    }
    result["measured_ceilings"] = measured_ceilings(torch)
    if not args.no_cpu_baseline:
        t0 = time.time()
        result["cpu_baseline"] = cpu_baseline(w, args)
        log("cpu baseline %.1fs" % (time.time() - t0))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
