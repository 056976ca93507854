#!/usr/bin/env python3
"""Decode-step benchmark of the int4 group-wise (g=64) compressed layer.

One step = one decode step of one OPT-shaped layer for the whole block of
B = g*m sequences, entirely in HBM, with the layer's real data flow (each
launch reads what the previous one wrote, fp16 hand-offs):
  Y  = X0 * [Wq|Wk|Wv]               fgq_dequant_gemm (one [h][3h] launch: the
                                      three projections share their input)
  fgq_kv_append_ld                    K and V of Y into the compressed cache
  A  = fgq_decode_attn_q4kv_ld        q of Y over prompt + t positions
  A * Wout, then * W1, then * W2      fgq_dequant_gemm x 3
The weights are read once per block; the layer's norms, residual sums and
FFN activation are not part of the compressed path and are not applied.
Decode step t cycles through 1..32 (the pages' 32 generated tokens), so the
attended length runs from prompt+1 to prompt+32.  Inputs are seeded
synthetic draws (synth), already resident in HBM when the timed region
starts.

Prints one JSON line.  Each timed pass starts after a warm-up of at least
--warmup steps and at least --min-warmup-ms of steady work (the clock of a
short burst runs lower).  The steps are timed twice: an eager pass with HIP
events recorded on the launch stream around every call (per-kernel
durations and the rooflines), then the same steps replayed as HIP graphs,
one per (decode step, layer instance), which gives value and ms_per_step
(--no-graph: the eager pass gives them).  The GEMM runs over the offline
packed weight layout (--gemm-layout packed, the default) or straight from
the quantiser's codes (canonical); both are timed.  The other workloads get
a graph-replayed step each (side entries), and the CPU baseline is the
oracle on a bounded sample of the step.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import threading
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
SIDE_CONFIGS = ("tiny", "opt-6.7b", "opt-30b", "opt-175b", "long-t3")


def log(msg: str) -> None:
    print("[bench] " + msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=96)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--min-warmup-ms", type=float, default=400.0,
                    help="each timed pass starts after at least this much warm-up work")
    ap.add_argument("--config", default="opt-175b", choices=sorted(synth.WORKLOADS))
    ap.add_argument("--gemm-layout", default="packed", choices=("packed", "canonical"),
                    help="weight layout of the headline step (the other one is timed beside it)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="layer instances cycled through (0: at least 3, and enough to exceed the 256 MB "
                         "last-level cache three times over)")
    ap.add_argument("--no-side-configs", action="store_true", help="skip the other workloads' step lines")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the lines beside the step (prefill, bulk append, top-K, grouped-query, streaming)")
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
    ap.add_argument("--prefill-only", action="store_true",
                    help="only time causal prefill attention (OPT-175B heads: 8 x 512 and 1 x 4096 tokens; "
                         "for profiling that kernel)")
    ap.add_argument("--summarize-gqa-trace", metavar="DIR",
                    help="only summarise a rocprofv3 --kernel-trace --stats folder of a --gqa-only run")
    ap.add_argument("--cpu-sample-seqs", type=int, default=4)
    ap.add_argument("--cpu-sample-cols", type=int, default=256)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 10 plain device copies of MIB MiB (HBM counter calibration under rocprofv3)")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("KERNEL_FETCH", "KERNEL_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="only summarise four rocprofv3 --pmc output folders (FETCH_SIZE / WRITE_SIZE of the "
                         "bench and of --calibrate-copy) into the HBM-traffic profile text")
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR",
                    help="only summarise rocprofv3 --pmc folders of this bench (any mix of SQ/GRBM counters) "
                         "into per-kernel unit-utilisation figures")
    ap.add_argument("--kernel", default="dq_gemm_kernel", help="kernel summarised by --summarize-pmc")
    ap.add_argument("--kernel-variant", default="",
                    help="regular expression the kernel's full name must also match (e.g. the packed layout's "
                         "template arguments), for --summarize-pmc")
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


def committed_traffic(kernel: str, config: str, variant: str = ""):
    """HBM bytes per launch measured by rocprofv3 counters (a 'traffic-json:'
    line of a summary under profiles/), or None when there is none for this
    kernel, variant and workload or the kernel's source has changed since."""
    import glob
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        with open(path) as fh:
            for line in fh:
                if line.startswith("traffic-json: "):
                    d = json.loads(line[len("traffic-json: "):])
                    if d.get("kernel") == kernel and d.get("config") == config and \
                            d.get("variant", "") == variant and d.get("source_sha256") == source_hash(kernel):
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
    import re
    res = {}
    for counter, folder in (("FETCH_SIZE", kf), ("WRITE_SIZE", kw)):
        vals = [v for name, v in read_pmc(folder, counter).values()
                if args.kernel in name and re.search(args.kernel_variant, name)]
        res[counter] = (len(vals), float(np.mean(vals)) if vals else 0.0)
    return fac, res


def library_gemm_same_shapes(torch, M: int, shapes) -> dict:
    """The library's plain fp16 GEMM (torch matmul, hipBLASLt) on the step's
    own weight shapes with uncompressed fp16 weights: X [M][K] @ W [K][N],
    fp16 out.  It reads 2 bytes per weight element against 0.5625 for the
    compressed ones, so it is a same-shape yardstick, not a ceiling."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out, tot_us, tot_fl = {}, 0.0, 0.0
    for name, K, N in shapes:
        x = torch.randn(M, K, device="cuda").half()
        wt = (torch.randn(K, N, device="cuda") * 0.02).half()
        for _ in range(3):
            y = x @ wt
        torch.cuda.synchronize()
        e0.record()
        for _ in range(20):
            y = x @ wt
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 20
        fl = 2.0 * M * K * N
        out["%s %dx%d" % (name, K, N)] = {"us_per_launch": round(us, 1), "TFLOP_per_s": round(fl / us * 1e-6, 1),
                                          "GB_per_s": round((2.0 * K * N + 2.0 * M * (K + N)) / us * 1e-3, 1)}
        tot_us += us
        tot_fl += fl
        del x, wt, y
    torch.cuda.empty_cache()
    out["all"] = {"us": round(tot_us, 1), "TFLOP_per_s": round(tot_fl / tot_us * 1e-6, 1), "rows": M}
    return out


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


def layer_input(w, t: int) -> np.ndarray:
    """The layer input of decode step t: fp16 [B][hidden] ~ N(0, 1)."""
    key = synth.stream_key(w.cid, synth.T_GEMM_X, 0, t)
    return synth.to_f16(synth.normal(key, w.batch * w.hidden)).reshape(w.batch, w.hidden)


def rotation(w, layouts) -> int:
    """Layer instances cycled through: at least 3, and enough that one cycle
    moves three times the 256 MB last-level cache (capped at 8)."""
    per_layer = acc.packed_bytes(sum(K * N for K, N in w.weights)) * len(layouts) + \
        2 * acc.packed_bytes(w.batch * w.hidden * w.capacity)
    return max(3, min(8, int(np.ceil(3 * 256e6 / per_layer)))), per_layer


class Chain:
    """R instances of one layer of workload w in HBM (the weights in each
    requested layout, a compressed cache holding the prompt) and the
    buffers of the chained decode step.  Instance 0 is built from the
    seeded draws; the others are device copies of it (separate memory, so
    no cache level serves one instance's bytes to the next)."""

    def __init__(self, torch, fgq, w, layouts, R):
        self.torch, self.fgq, self.w, self.R = torch, fgq, w, R
        B, H, D, h, cap = w.batch, w.heads, w.head_dim, w.hidden, w.capacity
        dev = "cuda"
        self.plan = launch_plan(w)
        self.opt = len(self.plan) == 4 and self.plan[0][0] == "qkv"
        t0 = time.time()
        base = []
        for name, K, N, idx in self.plan:
            wd = torch.cat([torch.from_numpy(synth.weight(w, i)).to(dev) for i in idx], dim=1).contiguous()
            codes = torch.empty((K, N // 2), dtype=torch.uint8, device=dev)
            meta = torch.empty((K, N // 64), dtype=torch.int32, device=dev)
            fgq.fgq_quantize_g64(wd, K, N, N, codes, meta)
            entry = {"canonical": (codes, meta)}
            if "packed" in layouts:
                pc = torch.empty(K * N // 8, dtype=torch.int32, device=dev)
                pm = torch.empty(fgq.fgq_pack_weight_meta_words(K, N), dtype=torch.int32, device=dev)
                fgq.fgq_pack_weight_g64(codes, meta, K, N, pc, pm)
                entry["packed"] = (pc, pm)
            if "canonical" not in layouts:
                del entry["canonical"]
            torch.cuda.synchronize()
            del wd
            base.append(entry)
        self.weights = [base] + [[{k: (a.clone(), b.clone()) for k, (a, b) in e.items()} for e in base]
                                 for _ in range(R - 1)]
        # caches: zero-filled (a position not yet appended reconstructs to 0)
        self.caches = []
        k0 = torch.zeros((B, H, cap, D // 2), dtype=torch.uint8, device=dev)
        v0 = torch.zeros_like(k0)
        km0 = torch.zeros((B, H, cap, D // 64), dtype=torch.int32, device=dev)
        vm0 = torch.zeros_like(km0)
        for b0 in range(0, B, 8):
            nb = min(8, B - b0)
            sub = fgq.kv_struct(k0[b0:b0 + nb], v0[b0:b0 + nb], km0[b0:b0 + nb], vm0[b0:b0 + nb], nb, H, D, cap)
            kd = torch.from_numpy(synth.prompt_kv(w, "k", b0=b0, nb=nb)).to(dev)
            vd = torch.from_numpy(synth.prompt_kv(w, "v", b0=b0, nb=nb)).to(dev)
            fgq.fgq_kv_append(sub, kd, vd, 0, w.prompt)
            torch.cuda.synchronize()
            del kd, vd
        for r in range(R):
            arrs = (k0, v0, km0, vm0) if r == 0 else tuple(a.clone() for a in (k0, v0, km0, vm0))
            self.caches.append((arrs, fgq.kv_struct(*arrs, B, H, D, cap)))
        # inputs of the decode steps
        self.inp = []
        for t in range(1, w.steps + 1):
            if self.opt:
                self.inp.append({"x0": torch.from_numpy(layer_input(w, t)).to(dev)})
            else:
                self.inp.append({"k": torch.from_numpy(synth.step_kv(w, "k", t)).to(dev),
                                 "v": torch.from_numpy(synth.step_kv(w, "v", t)).to(dev),
                                 "q": torch.from_numpy(synth.step_q(w, t)).to(dev)})
        f16 = torch.float16
        self.qkv = torch.empty((B, 3 * h), dtype=f16, device=dev) if self.opt else None
        self.attn = torch.empty((B, h), dtype=f16 if self.plan else torch.float32, device=dev)
        self.ys = [torch.empty((B, N), dtype=f16, device=dev) for _, _, N, _ in self.plan]
        aws = max(fgq.fgq_decode_attn_ws_bytes(B, H, D, L) for L in range(w.prompt + 1, cap + 1))
        gws = max([fgq.fgq_dequant_gemm_ws_bytes(B, K, N) for _, K, N, _ in self.plan] + [0])
        self.aws = torch.empty(max(aws, 16), dtype=torch.uint8, device=dev)
        self.gws = torch.empty(max(gws, 16), dtype=torch.uint8, device=dev)
        if self.opt:
            self.ops = ["gemm_qkv", "append", "attention", "gemm_out", "gemm_ffn1", "gemm_ffn2"]
        else:
            self.ops = ["append", "attention"] + ["gemm_" + p[0] for p in self.plan]
        torch.cuda.synchronize()
        log("%s: %d layer instance(s) ready in %.1fs" % (w.name, R, time.time() - t0))

    def gemm(self, inst, wi, layout, x, y, sh):
        w, fgq = self.w, self.fgq
        _, K, N, _ = self.plan[wi]
        a, b = self.weights[inst][wi][layout]
        f = fgq.fgq_dequant_gemm if layout == "canonical" else fgq.fgq_dequant_gemm_packed
        f(x, w.g, w.m, K, N, a, b, y, fgq.FGQ_DTYPE_F16, self.gws, self.gws.numel(), sh)

    def enqueue(self, i, layout, sh, ev=None, stream=None):
        """Decode step i % steps + 1 on layer instance i % R; with ev, HIP
        events are recorded on `stream` around every launch."""
        w, fgq = self.w, self.fgq
        t = i % w.steps + 1
        inst = i % self.R
        d = self.inp[t - 1]
        kv = self.caches[inst][1]
        h = w.hidden
        L = w.prompt + t
        n = [0]

        def rec():
            if ev is not None:
                ev[n[0]].record(stream)
                n[0] += 1
        rec()
        if self.opt:
            self.gemm(inst, 0, layout, d["x0"], self.qkv, sh)
            rec()
            fgq.fgq_kv_append_ld(kv, self.qkv[:, h:2 * h], self.qkv[:, 2 * h:], 3 * h, L - 1, 1, sh)
            rec()
            fgq.fgq_decode_attn_q4kv_ld(kv, self.qkv, 3 * h, L, 0.0, self.attn, fgq.FGQ_DTYPE_F16, self.aws,
                                        self.aws.numel(), sh)
            rec()
            x = self.attn
            for wi in (1, 2, 3):
                self.gemm(inst, wi, layout, x, self.ys[wi], sh)
                x = self.ys[wi]
                rec()
        else:
            fgq.fgq_kv_append(kv, d["k"], d["v"], L - 1, 1, sh)
            rec()
            fgq.fgq_decode_attn_q4kv(kv, d["q"], L, 0.0, self.attn,
                                     fgq.FGQ_DTYPE_F16 if self.plan else fgq.FGQ_DTYPE_F32, self.aws,
                                     self.aws.numel(), sh)
            rec()
            x = self.attn
            for wi in range(len(self.plan)):
                self.gemm(inst, wi, layout, x, self.ys[wi], sh)
                x = self.ys[wi]
                rec()

    def free(self):
        del self.weights, self.caches, self.inp, self.qkv, self.attn, self.ys, self.aws, self.gws
        self.torch.cuda.empty_cache()


class ClockSampler:
    """Samples the GPU's current graphics clock (MHz, via torch/amdsmi) every
    few ms from a background thread.  It never runs inside a timed region:
    its queries cost throughput (a 20-step region of the OPT-175B step read
    1-6% slower with the sampler running, even when it only sampled after
    every launch was queued), so the clock is read in an untimed window of
    the same work right after.  Entering returns after the first sample."""

    def __init__(self, torch):
        self.torch, self.samples, self._stop = torch, [], threading.Event()
        self._first = threading.Event()
        try:
            torch.cuda.clock_rate(0)
            self.ok = True
        except Exception:   # no SMI library on this machine
            self.ok = False

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(float(self.torch.cuda.clock_rate(0)))
            except Exception:
                self._first.set()
                return
            self._first.set()
            time.sleep(0.002)

    def __enter__(self):
        if self.ok:
            self._thr = threading.Thread(target=self._run, daemon=True)
            self._thr.start()
            self._first.wait(timeout=5.0)
        return self

    def __exit__(self, *a):
        self._stop.set()
        if self.ok:
            self._thr.join()

    def summary(self):
        s = [v for v in self.samples if v > 0]
        if not s:
            return None
        return {"median_MHz": float(np.median(s)), "min_MHz": float(np.min(s)), "max_MHz": float(np.max(s)),
                "samples": len(s)}


def warm_up(torch, run, first: int, min_steps: int, min_ms: float) -> tuple:
    """Runs steps first, first+1, ... (in batches of 8, synchronising after
    each) until at least min_steps ran and at least min_ms of wall time
    passed; returns (steps run, ms)."""
    t0 = time.perf_counter()
    n = 0
    while n < min_steps or (time.perf_counter() - t0) * 1e3 < min_ms:
        for _ in range(8):
            run(first + n)
            n += 1
        torch.cuda.synchronize()
    return n, (time.perf_counter() - t0) * 1e3


def eager_pass(torch, ch, layout, steps, warmup, min_ms, first=0):
    """Warm-up, then `steps` eager steps with HIP events on the launch stream
    around every launch; returns per-op ms, the total ms, the decode steps
    timed and the warm-up actually run."""
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    nw, wms = warm_up(torch, lambda i: ch.enqueue(i, layout, sh), first, warmup, min_ms)
    n_ev = len(ch.ops) + 1
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(steps):
        ch.enqueue(first + nw + i, layout, sh, ev=events[i], stream=stream)
    stop.record(stream)
    torch.cuda.synchronize()
    op_ms = {o: 0.0 for o in ch.ops}
    for ev in events:
        for j, o in enumerate(ch.ops):
            op_ms[o] += ev[j].elapsed_time(ev[j + 1])
    ts = [(first + nw + i) % ch.w.steps + 1 for i in range(steps)]
    return {"op_ms": op_ms, "total_ms": start.elapsed_time(stop), "ts": ts, "warmup_steps": nw,
            "warmup_ms": wms}


def graph_pass(torch, ch, layout, steps, warmup, min_ms):
    """The same steps captured as HIP graphs (one per decode step and layer
    instance, through the same C-ABI calls on a capture stream) and replayed;
    returns the timed ms, the warm-up run and the clock samples."""
    stream = torch.cuda.current_stream()
    cap = torch.cuda.Stream()      # capture needs a stream other than the default one
    graphs = {}
    n_keys = int(np.lcm(ch.w.steps, ch.R))
    for i in range(n_keys):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            ch.enqueue(i, layout, cap.cuda_stream)
        graphs[i] = g
    torch.cuda.synchronize()
    nw, wms = warm_up(torch, lambda i: graphs[i % n_keys].replay(), 0, warmup, min_ms)
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    g0.record(stream)
    for i in range(steps):
        graphs[(nw + i) % n_keys].replay()
    g1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = g0.elapsed_time(g1)
    # the clock under the same load: the next replays, untimed, sampled while they run
    for i in range(max(steps, 32)):
        graphs[(nw + steps + i) % n_keys].replay()
    clock = ClockSampler(torch)
    with clock:
        torch.cuda.synchronize()
    ts = [(nw + i) % ch.w.steps + 1 for i in range(steps)]
    del graphs
    return {"total_ms": ms, "wall_s": wall, "ts": ts, "warmup_steps": nw, "warmup_ms": wms,
            "clock": clock.summary(), "graphs": n_keys}


def kernel_lines(ch, ep, steps) -> dict:
    """Per-launch durations and rates of one eager pass."""
    w = ch.w
    B, h = w.batch, w.hidden
    op = ep["op_ms"]
    ts = ep["ts"]
    out = {}
    attn_bytes = sum(acc.attention_bytes(B, h, w.kv_len(t), out_bytes=2 if ch.plan else 4) for t in ts)
    gbs = attn_bytes / (op["attention"] * 1e-3) / 1e9
    out["append"] = {"us_per_launch": 1e3 * op["append"] / steps,
                     "GB_per_s": steps * acc.append_bytes(B, h) / (op["append"] * 1e-3) / 1e9}
    out["attention"] = {"us_per_launch": 1e3 * op["attention"] / steps, "GB_per_s": gbs,
                        "frac_hbm_peak": gbs / HBM_PEAK_GBS,
                        "TFLOP_per_s": sum(acc.attention_flops(B, h, w.kv_len(t)) for t in ts) /
                        (op["attention"] * 1e-3) / 1e12}
    for name, K, N, _ in ch.plan:
        ms = op["gemm_" + name]
        f = steps * acc.gemm_flops(B, K, N)
        by = steps * acc.gemm_bytes(B, K, N, y_bytes=2)
        out["gemm_%s_%dx%d" % (name, K, N)] = {
            "us_per_launch": 1e3 * ms / steps, "TFLOP_per_s": f / (ms * 1e-3) / 1e12,
            "frac_mfma_peak": f / (ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
            "GB_per_s": by / (ms * 1e-3) / 1e9, "frac_hbm_peak": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    return out


def gemm_totals(ch, ep, steps):
    """All GEMM launches of the eager pass together: ms, TFLOP/s, GB/s."""
    w = ch.w
    ms = sum(ep["op_ms"]["gemm_" + p[0]] for p in ch.plan)
    fl = steps * sum(acc.gemm_flops(w.batch, K, N) for _, K, N, _ in ch.plan)
    by = steps * sum(acc.gemm_bytes(w.batch, K, N, y_bytes=2) for _, K, N, _ in ch.plan)
    return ms, (fl / (ms * 1e-3) / 1e12 if ms else 0.0), (by / (ms * 1e-3) / 1e9 if ms else 0.0)


def side_config_line(torch, fgq, name, layout, args) -> dict:
    """A graph-replayed chained step of another workload and its per-launch
    rates (one full generation of 32 decode steps timed)."""
    w = synth.WORKLOADS[name]
    R, per_layer = rotation(w, (layout,))
    ch = Chain(torch, fgq, w, (layout,), R)
    steps = 32
    ep = eager_pass(torch, ch, layout, steps, 8, args.min_warmup_ms)
    line = {"workload": w.name, "batch": w.batch, "heads_x_head_dim": "%dx%d" % (w.heads, w.head_dim),
            "prompt": w.prompt, "layer_instances": R, "gemm_layout": layout, "steps_timed": steps,
            "eager_ms_per_step": ep["total_ms"] / steps}
    if not args.no_graph:
        gp = graph_pass(torch, ch, layout, steps, 8, args.min_warmup_ms)
        line["ms_per_step"] = gp["total_ms"] / steps
        line["gpu_clock"] = gp["clock"]
    else:
        line["ms_per_step"] = ep["total_ms"] / steps
    line["tokens_per_s_per_layer"] = w.batch / (line["ms_per_step"] * 1e-3)
    if w.name == "tiny":
        line["us_per_step"] = 1e3 * line["ms_per_step"]
    line["kernels"] = kernel_lines(ch, ep, steps)
    if ch.plan:
        ms, tf, gbs = gemm_totals(ch, ep, steps)
        line["gemm_all"] = {"TFLOP_per_s": tf, "frac_mfma_peak": tf / MFMA_F16_PEAK_TFLOPS, "GB_per_s": gbs,
                            "frac_hbm_peak": gbs / HBM_PEAK_GBS}
    ch.free()
    del ch
    torch.cuda.empty_cache()
    return line


def cpu_info() -> dict:
    """Host CPU model, sockets and threads (lscpu), for the baseline line."""
    import subprocess
    info = {}
    try:
        out = subprocess.run(["lscpu"], stdout=subprocess.PIPE, stderr=subprocess.DEVNULL, text=True).stdout
        for line in out.splitlines():
            k, _, v = line.partition(":")
            if k.strip() in ("Model name", "Socket(s)", "Thread(s) per core", "Core(s) per socket", "CPU(s)"):
                info[k.strip()] = v.strip()
    except OSError:
        pass
    info["threads_available"] = len(os.sched_getaffinity(0))
    return info


def _omp_threads(n: int) -> None:
    import ctypes
    try:
        ctypes.CDLL("libgomp.so.1").omp_set_num_threads(int(n))
    except OSError:
        pass


def cpu_baseline(w, args):
    """The oracle (never tuned) on a bounded sample of the chained decode step
    at t = 1 and t = 32: append + attention on a few sequences, every weight
    GEMM on a 256-column slice with all g*m rows; each part scaled to the
    full step.  Also the OPT-6.7B attention of one step on a single core."""
    import oracle
    S = min(args.cpu_sample_seqs, w.batch)
    H, D, h = w.heads, w.head_dim, w.hidden
    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    _omp_threads(cores)
    # the GEMM slices do not depend on t: time them once per t anyway (same work)
    slices = []
    for i, (K, N) in enumerate(w.weights):
        ncol = min(args.cpu_sample_cols, N)
        c, m = oracle.quantize_g64(np.ascontiguousarray(synth.weight(w, i)[:, :ncol]))
        slices.append((i, K, N, ncol, c, m))
    ref = oracle.KVCache(S, H, D, w.capacity)
    oracle.kv_append(ref, synth.prompt_kv(w, "k", nb=S), synth.prompt_kv(w, "v", nb=S), 0)
    for t in range(1, w.steps):       # positions of the earlier decode steps (untimed)
        oracle.kv_append(ref, synth.step_kv(w, "k", t)[:S], synth.step_kv(w, "v", t)[:S], w.prompt + t - 1)
    per_t = {}
    for t in (1, w.steps):
        secs = {}
        sk, sv = synth.step_kv(w, "k", t)[:S], synth.step_kv(w, "v", t)[:S]
        q = synth.step_q(w, t)[:S]
        t0 = time.perf_counter()
        oracle.kv_append(ref, sk, sv, w.prompt + t - 1)
        secs["append"] = (time.perf_counter() - t0) * w.batch / S
        t0 = time.perf_counter()
        oracle.decode_attn(ref, q, w.kv_len(t))
        secs["attention"] = (time.perf_counter() - t0) * w.batch / S
        g = 0.0
        for i, K, N, ncol, c, m in slices:
            x = synth.gemm_x(w, i, t)
            t0 = time.perf_counter()
            oracle.dequant_gemm(x, w.g, w.m, c, m)
            g += (time.perf_counter() - t0) * N / ncol
        secs["gemm"] = g
        tot = sum(secs.values())
        per_t["t=%d" % t] = {"tokens_per_s_per_layer": w.batch / tot,
                             "seconds_per_step": {k: round(v, 4) for k, v in secs.items()}}
    # OPT-6.7B attention (B = 64, 32 heads, kv_len 513) on one core, 8 sequences scaled to 64
    w2 = synth.WORKLOADS["opt-6.7b"]
    S2 = 8
    ref2 = oracle.KVCache(S2, w2.heads, w2.head_dim, w2.capacity)
    oracle.kv_append(ref2, synth.prompt_kv(w2, "k", nb=S2), synth.prompt_kv(w2, "v", nb=S2), 0)
    oracle.kv_append(ref2, synth.step_kv(w2, "k", 1)[:S2], synth.step_kv(w2, "v", 1)[:S2], w2.prompt)
    _omp_threads(1)
    t0 = time.perf_counter()
    oracle.decode_attn(ref2, synth.step_q(w2, 1)[:S2], w2.kv_len(1))
    one_core = (time.perf_counter() - t0) * w2.batch / S2
    _omp_threads(cores)
    mean_step = float(np.mean([sum(v["seconds_per_step"].values()) for v in per_t.values()]))
    return {
        "value": w.batch / mean_step,
        "unit": "tokens/s/layer",
        "cores": cores,
        "kind": "oracle",
        "sample": "decode steps t=1 and t=%d of %s (value: their mean step time): append+attention on %d of %d "
                  "sequences, every weight GEMM on a %d-column slice with all %d rows; each part scaled to the "
                  "full step" % (w.steps, w.name, S, w.batch, args.cpu_sample_cols, w.batch),
        "per_step": per_t,
        "opt67b_attention_one_core": {"seconds_per_step": round(one_core, 4),
                                      "GB_per_s": acc.attention_bytes(w2.batch, w2.hidden, w2.kv_len(1)) /
                                      one_core / 1e9,
                                      "sample": "8 of 64 sequences, kv_len 513, scaled"},
        "cpu": cpu_info(),
    }


def prefill_and_bulk_lines(torch, fgq, w, ch, stream) -> dict:
    """Prompt-side launches beside the decode step: the bulk compression of 8
    sequences' prompt K and V into layer instance 0, and causal prefill
    attention over the same sequences' fp16 prompt (fp16 output), which
    precedes it; each timed after a warm-up of at least 100 ms."""
    B, H, D, h = w.batch, w.heads, w.head_dim, w.hidden
    sh = stream.cuda_stream
    nb = min(8, B)
    kd = torch.from_numpy(synth.prompt_kv(w, "k", nb=nb)).to("cuda")
    vd = torch.from_numpy(synth.prompt_kv(w, "v", nb=nb)).to("cuda")
    (kc, vc, km, vm), _ = ch.caches[0]
    sub = fgq.kv_struct(kc[:nb], vc[:nb], km[:nb], vm[:nb], nb, H, D, w.capacity)
    warm_up(torch, lambda i: fgq.fgq_kv_append(sub, kd, vd, 0, w.prompt, sh), 0, 8, 100.0)
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    b0.record(stream)
    for _ in range(reps):
        fgq.fgq_kv_append(sub, kd, vd, 0, w.prompt, sh)
    b1.record(stream)
    torch.cuda.synchronize()
    bulk_us = 1e3 * b0.elapsed_time(b1) / reps
    qd = torch.from_numpy(synth.prompt_q(w, nb=nb)).to("cuda")
    # fp16 output: the hand-off to the out projection, as in the decode step
    pf_out = torch.empty((nb, w.prompt, h), dtype=torch.float16, device="cuda")
    warm_up(torch, lambda i: fgq.fgq_prefill_attn_f16(qd, kd, vd, nb, w.prompt, H, D, 0.0, pf_out,
                                                       fgq.FGQ_DTYPE_F16, sh), 0, 8, 100.0)
    b0.record(stream)
    for _ in range(reps):
        fgq.fgq_prefill_attn_f16(qd, kd, vd, nb, w.prompt, H, D, 0.0, pf_out, fgq.FGQ_DTYPE_F16, sh)
    b1.record(stream)
    torch.cuda.synchronize()
    pf_us = 1e3 * b0.elapsed_time(b1) / reps
    pf_flops = acc.prefill_attention_flops(nb, h, w.prompt)
    ab = acc.append_bytes(nb, h, w.prompt)
    del kd, vd, qd, pf_out
    return {
        "prefill_attention": {"sequences": nb, "tokens_per_sequence": w.prompt, "us_per_launch": pf_us,
                              "TFLOP_per_s": pf_flops / (pf_us * 1e-6) / 1e12,
                              "frac_mfma_peak": pf_flops / (pf_us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS,
                              "us_whole_block_estimate": pf_us * B / nb},
        "prompt_bulk_append": {"sequences": nb, "tokens_per_sequence": w.prompt, "us_per_launch": bulk_us,
                               "GB_per_s": ab / (bulk_us * 1e-6) / 1e9,
                               "frac_hbm_peak": ab / (bulk_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                               "us_whole_block_estimate": bulk_us * B / nb}}


def prefill_only_lines(torch, fgq, stream, reps: int) -> dict:
    """Causal prefill attention alone at OPT-175B's heads (96 x 128), on the
    seeded prompt recipe: 8 sequences of 512 tokens (the short-prompt launch) and
    one of 4096 (the long-prompt launch), reps launches each after a warm-up."""
    w = synth.WORKLOADS["opt-175b"]
    H, D, h = w.heads, w.head_dim, w.hidden
    sh = stream.cuda_stream
    lines = {}
    for nb, S in ((8, 512), (1, 4096)):
        rng = np.random.default_rng(S)
        qd, kd, vd = (torch.from_numpy(rng.standard_normal((nb, S, h)).astype(np.float16)).to("cuda")
                      for _ in range(3))
        out = torch.empty((nb, S, h), dtype=torch.float16, device="cuda")

        def run(_i=0):
            fgq.fgq_prefill_attn_f16(qd, kd, vd, nb, S, H, D, 0.0, out, fgq.FGQ_DTYPE_F16, sh)
        warm_up(torch, run, 0, 8, 200.0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / reps
        fl = acc.prefill_attention_flops(nb, h, S)
        lines["%dx%d" % (nb, S)] = {"us_per_launch": us, "TFLOP_per_s": fl / (us * 1e-6) / 1e12,
                                    "frac_mfma_peak": fl / (us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFLOPS}
        del qd, kd, vd, out
    return lines


def topk_line(torch, fgq, w, ch, stream, steps, warmup) -> dict:
    """Top-K sparse attention (keep the top tenth of the positions, read only
    their V rows) over the same caches and decode steps, queries drawn per
    step."""
    B, h = w.batch, w.hidden
    sh = stream.cuda_stream
    tk_out = torch.empty((B, h), dtype=torch.float32, device="cuda")
    qs = [torch.from_numpy(synth.step_q(w, t)).to("cuda") for t in range(1, w.steps + 1)]

    def launch(i):
        t = i % w.steps + 1
        L_t = w.prompt + t
        fgq.fgq_decode_attn_topk_q4kv(ch.caches[i % ch.R][1], qs[t - 1], L_t, -(-L_t // 10), 0.0, tk_out,
                                      fgq.FGQ_DTYPE_F32, None, sh)

    nw, _ = warm_up(torch, launch, 0, min(warmup, 8), 100.0)   # >= 100 ms: the clock of a short burst runs lower
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        ev[i][0].record(stream)
        launch(nw + i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in ev)
    ts = [(nw + i) % w.steps + 1 for i in range(steps)]
    by = sum(acc.topk_attention_bytes(B, h, w.kv_len(t), -(-w.kv_len(t) // 10)) for t in ts)
    line = {"kept": "ceil(kv_len/10)", "us_per_launch": 1e3 * ms / steps, "GB_per_s": by / (ms * 1e-3) / 1e9,
            "frac_hbm_peak": by / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    tr = committed_traffic("attn_topk_wave_kernel", w.name)
    if tr is not None and w.kv_len(w.steps) <= 2048:
        line["traffic_bytes_per_launch"] = tr["bytes_per_launch"]
        line["traffic_vs_algorithmic"] = tr["ratio"]
    del qs, tk_out
    return line


def weight_streaming(torch, fgq, ch, stream) -> dict:
    """The chained step with the layer's packed weights arriving from pinned
    host memory every step (the offloading setting compression was made
    for): two device buffers, the next step's weights copied on a second
    stream (default priority) while this step computes; the KV cache stays
    in HBM.  Also times the plain host-to-device copy of the same bytes and
    of the fp16 weights they replace."""
    w = ch.w
    B = w.batch
    src = [e["packed"] for e in ch.weights[0]]
    host = [(pc.cpu().pin_memory(), pm.cpu().pin_memory()) for pc, pm in src]
    nbytes = sum(a.numel() * 4 + b.numel() * 4 for a, b in host)
    bufs = [[{"packed": (torch.empty_like(pc), torch.empty_like(pm))} for pc, pm in src] for _ in range(2)]
    cstream = torch.cuda.Stream()
    sh = stream.cuda_stream
    copied = [torch.cuda.Event() for _ in range(2)]
    freed = [torch.cuda.Event() for _ in range(2)]
    n = 8
    saved_w, saved_r = ch.weights, ch.R

    def copy(i):
        k = i % 2
        with torch.cuda.stream(cstream):
            cstream.wait_event(freed[k])
            for (hc, hm), e in zip(host, bufs[k]):
                dc, dm = e["packed"]
                dc.copy_(hc, non_blocking=True)
                dm.copy_(hm, non_blocking=True)
            copied[k].record(cstream)

    for k in range(2):
        freed[k].record(stream)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ch.weights, ch.R = bufs, 2        # instance k of the chain = device buffer k (cache of instance 0 or 1)
    copy(0)
    e0.record(stream)
    for i in range(n):
        if i + 1 < n:
            copy(i + 1)
        stream.wait_event(copied[i % 2])
        ch.enqueue(i, "packed", sh)
        freed[i % 2].record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ch.weights, ch.R = saved_w, saved_r
    ms = e0.elapsed_time(e1) / n
    nel = sum(K * N for _, K, N, _ in ch.plan)
    f16 = torch.empty(nel, dtype=torch.float16).pin_memory()
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
            "fp16_weights_copy_ms": f16_ms, "fp16_over_packed_bytes": 2.0 * nel / nbytes}


def short_name(kernel_name: str) -> str:
    n = kernel_name.replace("(anonymous namespace)::", "").replace("void ", "")
    return n.split("(")[0].replace("fgq::", "").strip()


def _read_csvs(folder: str, pattern: str):
    import csv
    import glob
    files = glob.glob(os.path.join(folder, "**", pattern), recursive=True)
    if not files:
        raise SystemExit("no %s under %s" % (pattern, folder))
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def summarize_trace(folder: str, w, steps: int) -> None:
    """Markdown: rocprofv3's kernel statistics, then the mean duration of each
    launch of the chained step over the last `steps` steps of the headline
    layout (a GEMM launch includes its split-K reduction, attention its
    merge).  A step is located by its decode-time KV append: the GEMM launch
    before it is the Q/K/V product, and attention and the other products
    follow it."""
    stats = _read_csvs(folder, "*kernel_stats.csv")
    print("| kernel | calls | average us | total ms | % of GPU time |")
    print("|---|---|---|---|---|")
    for r in stats[:14]:
        print("| %s | %s | %.1f | %.2f | %.1f |" % (short_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
                                                  float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    trace = sorted(_read_csvs(folder, "*kernel_trace.csv"), key=lambda r: int(r["Start_Timestamp"]))
    recs = [(short_name(r["Kernel_Name"]), (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3,
             int(r["Grid_Size_X"])) for r in trace]
    # merge each split-K reduction / split merge into the launch before it
    ops = []
    for n, d, g in recs:
        if (n.startswith("splitk_reduce_kernel") or n.startswith("attn_merge_kernel")) and ops:
            ops[-1][1] += d
        else:
            ops.append([n, d, g])
    names = ["gemm_qkv", "append", "attention", "gemm_out", "gemm_ffn1", "gemm_ffn2"]
    want = ["dq_gemm_kernel", "kv_append_kernel", "attn_split_kernel", "dq_gemm_kernel", "dq_gemm_kernel",
            "dq_gemm_kernel"]
    stepl = []
    for a in range(1, len(ops) - 4):
        if ops[a][0].startswith("kv_append_kernel") and ops[a][2] == w.batch * w.hidden // 4:
            seq = ops[a - 1:a + 5]
            if [s[0].split("<")[0] for s in seq] == want:
                stepl.append(seq)
    layout_steps = [st for st in stepl if "false" in st[0][0]] or stepl
    good = layout_steps[-steps:]
    print()
    print("Steady state, mean of the last %d chained steps of the packed layout (us per launch; a GEMM launch "
          "includes its split-K reduction, attention its merge):" % len(good))
    print()
    print("| launch | kernel | us |")
    print("|---|---|---|")
    tot = 0.0
    for i, nm in enumerate(names):
        v = float(np.mean([st[i][1] for st in good])) if good else float("nan")
        tot += v
        print("| %s | %s | %.1f |" % (nm, good[0][i][0] if good else "?", v))
    print("| step (sum) | | %.1f |" % tot)


# Unit-utilisation figures from raw counters.  rocprofv3 reports each counter
# per dispatch summed over its dimensions; the GRBM counters run once per XCD,
# so their per-XCD value (rocprof's reduce(..., max)) is the sum / 8 on
# MI355X.  rocprofv3's own derived-metric formulas:
#   MfmaUtil  = 100 * SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE * SIMD_NUM)
#   VALUBusy  = 100 * SQ_ACTIVE_INST_VALU / CU_NUM / GRBM_GUI_ACTIVE
#   Occupancy = 400 * SQ_WAVE_CYCLES / GRBM_GUI_ACTIVE / CU_NUM / 32   (% of 32 wave slots per CU)
#   LdsBankConflict (% of LDS-active cycles stalled) = 100 * SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE
#   LdsUtil   = 100 * SQ_LDS_IDX_ACTIVE / (GRBM_GUI_ACTIVE * CU_NUM)
#   SIMD_UTILIZATION = SQ_BUSY_CU_CYCLES / GRBM_COUNT / CU_NUM  (GUI_ACTIVE used when GRBM_COUNT is absent)
CU_NUM, SIMD_NUM, XCD_NUM = 256, 1024, 8


def summarize_counters(folders, kernels) -> None:
    """Markdown of per-kernel counter figures from rocprofv3 --pmc folders of
    this bench (one folder per counter pass)."""
    per = {}
    durs = {}
    for folder in folders:
        for r in _read_csvs(folder, "*counter_collection.csv"):
            name = short_name(r["Kernel_Name"])
            key = (folder, int(r["Dispatch_Id"]))
            d = per.setdefault(name, {}).setdefault(key, {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if "Start_Timestamp" in r and r.get("End_Timestamp"):
                durs.setdefault(name, {})[key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    print("| kernel | dispatches | GUI_ACTIVE cycles | MFMA busy % | CU busy % | VALU busy % | VALU insts per MFMA | "
          "LDS insts per MFMA | occupancy % of 32 slots | LDS util % | LDS bank-conflict % of LDS-active | "
          "MFMA-VALU co-issue % | wave-cycles waiting to issue % | waiting on LDS % |")
    print("|---|---|---|---|---|---|---|---|---|---|---|---|---|---|")
    out = {}
    for name in sorted(per):
        if kernels and not any(k in name for k in kernels):
            continue
        disp = per[name]
        tot = {}
        cnt = {}
        for vals in disp.values():
            for c, v in vals.items():
                tot[c] = tot.get(c, 0.0) + v
                cnt[c] = cnt.get(c, 0) + 1
        m = {c: tot[c] / cnt[c] for c in tot}      # mean per dispatch

        def g(c):
            return m.get(c)

        def pct(a, b, f=1.0):
            return "%.1f" % (100.0 * f * a / b) if a is not None and b else "-"
        gui = g("GRBM_GUI_ACTIVE")
        gui = gui / XCD_NUM if gui else gui
        mf = g("SQ_INSTS_MFMA")
        valu = g("SQ_INSTS_VALU")
        row = {
            "dispatches": max(cnt.values()),
            "gui_active": gui,
            "mfma_busy": pct(g("SQ_VALU_MFMA_BUSY_CYCLES"), gui and gui * SIMD_NUM),
            "mfma_cycles_per_inst": "%.1f" % (g("SQ_VALU_MFMA_BUSY_CYCLES") / mf)
            if g("SQ_VALU_MFMA_BUSY_CYCLES") is not None and mf else "-",
            "valu_busy": pct(g("SQ_ACTIVE_INST_VALU"), gui and gui * CU_NUM),
            "valu_per_mfma": "%.2f" % ((valu - mf) / mf) if valu is not None and mf else "-",
            "lds_per_mfma": "%.2f" % (g("SQ_INSTS_LDS") / mf) if g("SQ_INSTS_LDS") is not None and mf else "-",
            "occupancy": pct(g("SQ_WAVE_CYCLES"), gui and gui * CU_NUM * 32, 4.0),
            "lds_util": pct(g("SQ_LDS_IDX_ACTIVE"), gui and gui * CU_NUM),
            "lds_conflict": pct(g("SQ_LDS_BANK_CONFLICT"), g("SQ_LDS_IDX_ACTIVE")),
            "coexec": pct(g("SQ_VALU_MFMA_COEXEC_CYCLES"), g("SQ_VALU_MFMA_BUSY_CYCLES")),
            "cu_busy": pct(g("SQ_BUSY_CU_CYCLES"), gui and gui * CU_NUM),
            "wait_issue": pct(g("SQ_WAIT_INST_ANY"), g("SQ_WAVE_CYCLES")),
            "wait_lds": pct(g("SQ_WAIT_INST_LDS"), g("SQ_WAVE_CYCLES")),
        }
        out[name] = row
        print("| %s | %d | %s | %s | %s | %s | %s | %s | %s | %s | %s | %s | %s | %s |" % (
            name, row["dispatches"], "%.4g" % gui if gui else "-", row["mfma_busy"], row["cu_busy"], row["valu_busy"],
            row["valu_per_mfma"], row["lds_per_mfma"], row["occupancy"], row["lds_util"], row["lds_conflict"],
            row["coexec"], row["wait_issue"], row["wait_lds"]))
        dd = durs.get(name)
        if dd and gui:
            mean_us = float(np.mean(list(dd.values())))
            print("|  (%s: mean %.1f us per dispatch under counters, %.2f GHz from GUI_ACTIVE) |" %
                  (name, mean_us, gui / (mean_us * 1e3)))
    print()
    print("counters-json: " + json.dumps(out))


def algorithmic_bytes_per_launch(kernel: str, w, n_steps: int = 0, warmup: int = 0) -> float:
    """Mean algorithmic HBM bytes of one launch of the kernel over the
    chained step (fp16 hand-offs) or the grouped workload."""
    if kernel == "dq_gemm_kernel":
        plan = launch_plan(w)
        return float(np.mean([acc.gemm_bytes(w.batch, K, N, y_bytes=2) for _, K, N, _ in plan]))
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
    return float(np.mean([acc.attention_bytes(w.batch, w.hidden, w.kv_len(t), out_bytes=2 if w.weights else 4)
                          for t in ts]))


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

    # at least `warmup` steps and 100 ms of them, as for the sweep below: the
    # clock of a short burst runs lower
    nw, _ = warm_up(torch, step, 0, warmup, 100.0)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(nw + i, evs[i])
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs)
    ts = [(nw + i) % w.steps + 1 for i in range(steps)]
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
        warm_up(torch, lambda i: fgq.fgq_decode_attn_gqa_q4kv(kvs, q, Hq, cap, 0.0, out, fgq.FGQ_DTYPE_F32, ws,
                                                              ws.numel(), sh), 0, 8, 100.0)
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
        if hk == Hq:
            # top-K (a tenth of the positions kept) over the same multi-head cache: 16416 + 1642 positions of
            # fp32 scores and kept list fit the workgroup kernel's LDS bound (19840)
            kk = -(-cap // 10)
            tk_out = torch.empty_like(out)
            warm_up(torch, lambda i: fgq.fgq_decode_attn_topk_q4kv(kvs, q, cap, kk, 0.0, tk_out, fgq.FGQ_DTYPE_F32,
                                                                   None, sh), 0, 8, 100.0)
            e0.record(stream)
            for _ in range(reps):
                fgq.fgq_decode_attn_topk_q4kv(kvs, q, cap, kk, 0.0, tk_out, fgq.FGQ_DTYPE_F32, None, sh)
            e1.record(stream)
            torch.cuda.synchronize()
            tus = 1e3 * e0.elapsed_time(e1) / reps
            tb = acc.topk_attention_bytes(B, Hq * D, cap, kk)
            line["topk_attention_at_kv_len_%d" % cap] = {
                "heads": Hq, "kept": kk, "us_per_launch": tus, "GB_per_s": tb / tus / 1e3,
                "frac_hbm_peak": tb / tus / 1e3 / HBM_PEAK_GBS, "time_vs_dense_attention": tus / us}
            del tk_out
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
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, ("dq_gemm_kernel", "attn_split_kernel", "attn_merge_kernel",
                                                     "kv_append_kernel", "splitk_reduce_kernel",
                                                     "prefill_attn_kernel", "attn_gqa_kernel",
                                                     "attn_gqa_merge_kernel"))
        return
    if args.summarize_pmc:
        w = synth.WORKLOADS[args.config]
        fac, res = summarize_pmc(args)
        n_f, fetch_kib = res["FETCH_SIZE"]
        n_w, write_kib = res["WRITE_SIZE"]
        per_launch = fetch_kib * 1024.0 * fac["FETCH_SIZE"] + write_kib * 1024.0 * fac["WRITE_SIZE"]
        alg = algorithmic_bytes_per_launch(args.kernel, w, args.warmup + args.steps, args.warmup)
        d = {"kernel": args.kernel, "variant": args.kernel_variant, "config": w.name,
             "source_sha256": source_hash(args.kernel),
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
        print("bench.py measures one GPU: the library has no multi-GPU path (the work would shard by "
              "sequence and head, and the weights by column group). Run with --gpus 1.", file=sys.stderr)
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
    if args.prefill_only:
        print(json.dumps({"prefill_attention": prefill_only_lines(torch, fgq, torch.cuda.current_stream(),
                                                                  args.steps)}), flush=True)
        return
    w = synth.WORKLOADS[args.config]
    B, H, D, h = w.batch, w.heads, w.head_dim, w.hidden
    other = "canonical" if args.gemm_layout == "packed" else "packed"
    layouts = (args.gemm_layout, other) if w.weights else (args.gemm_layout,)
    R, per_layer = rotation(w, layouts)
    R = args.rotate or R
    ch = Chain(torch, fgq, w, layouts, R)
    stream = torch.cuda.current_stream()
    K_steps = args.steps

    # ---------------- the chained step, each layout: eager (per-launch events), then HIP graphs
    passes = {}
    for layout in layouts:
        ep = eager_pass(torch, ch, layout, K_steps, args.warmup, args.min_warmup_ms)
        gp = None if args.no_graph else graph_pass(torch, ch, layout, K_steps, args.warmup, args.min_warmup_ms)
        passes[layout] = (ep, gp)
        log("%s layout: eager %.4f ms/step%s (warm-up %d steps, %.0f ms)" % (
            layout, ep["total_ms"] / K_steps, "" if gp is None else ", graphs %.4f ms/step" %
            (gp["total_ms"] / K_steps), ep["warmup_steps"], ep["warmup_ms"]))
    ep, gp = passes[args.gemm_layout]
    kernels = kernel_lines(ch, ep, K_steps)
    step_ms = ep["total_ms"] if gp is None else gp["total_ms"]
    ms_per_step = step_ms / K_steps
    value = B * K_steps / (step_ms * 1e-3)
    attn_gbs = kernels["attention"]["GB_per_s"]
    gemm_ms, gemm_tflops, gemm_gbs = gemm_totals(ch, ep, K_steps) if w.weights else (0.0, 0.0, 0.0)
    if w.weights:
        ep2, gp2 = passes[other]
        k2 = kernel_lines(ch, ep2, K_steps)
        ms2, tf2, gb2 = gemm_totals(ch, ep2, K_steps)
        kernels["gemm_%s_layout" % other] = {
            "what": "the same chained step with fgq_dequant_gemm%s" % ("" if other == "canonical" else "_packed"),
            "ms_per_step": (ep2["total_ms"] if gp2 is None else gp2["total_ms"]) / K_steps,
            "gemm_TFLOP_per_s": tf2, "gemm_frac_mfma_peak": tf2 / MFMA_F16_PEAK_TFLOPS,
            "launches": {k: v for k, v in k2.items() if k.startswith("gemm_")}}

    if not args.no_extras:
        kernels.update(prefill_and_bulk_lines(torch, fgq, w, ch, stream))
        kernels["topk_attention"] = topk_line(torch, fgq, w, ch, stream, K_steps, args.warmup)
        kernels["topk_attention"]["time_vs_dense_attention"] = \
            kernels["topk_attention"]["us_per_launch"] / kernels["attention"]["us_per_launch"]
        if w.weights and "packed" in layouts and not args.no_stream:
            kernels["weight_streaming"] = weight_streaming(torch, fgq, ch, stream)
    ch.free()
    del ch
    torch.cuda.empty_cache()
    if not args.no_extras and not args.no_gqa:
        t0 = time.time()
        kernels["gqa_attention"] = gqa_attention_line(torch, fgq, stream, 32, 8,
                                                      () if args.no_gqa_sweep else (32, 16, 8, 4, 2, 1))
        log("gqa attention line %.1fs" % (time.time() - t0))

    if w.weights and gemm_ms >= 1e-3 * kernels["attention"]["us_per_launch"] * K_steps:
        kname = "dq_gemm_kernel"
        roof = {"bound": "mfma", "kernel": kname + " (all %d weight GEMM launches of the step, %s layout)" %
                (len(launch_plan(w)), args.gemm_layout),
                "achieved": gemm_tflops, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": gemm_tflops / MFMA_F16_PEAK_TFLOPS, "traffic": None,
                "algorithmic_per_launch": "2*M*K*N flops, M=%d; mean algorithmic bytes per launch %.4g" %
                                          (B, algorithmic_bytes_per_launch(kname, w))}
    else:
        kname = "attn_split_kernel"
        roof = {"bound": "hbm", "kernel": kname, "achieved": attn_gbs, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": attn_gbs / HBM_PEAK_GBS, "traffic": None,
                "algorithmic_per_launch": "1.125*hidden*kv_len bytes per sequence (+q, out); mean %.4g" %
                                          algorithmic_bytes_per_launch(kname, w)}
    tr = committed_traffic(kname, w.name, ("false>" if args.gemm_layout == "packed" else "true>")
                           if kname == "dq_gemm_kernel" else "")
    if tr is not None:
        roof["traffic"] = tr["bytes_per_launch"]
        roof["traffic_source"] = "rocprofv3 FETCH_SIZE + WRITE_SIZE per launch, copy-calibrated (profiles/)"

    side = {}
    if not args.no_side_configs:
        for name in SIDE_CONFIGS:
            if name == w.name:
                continue
            t0 = time.time()
            side[name] = side_config_line(torch, fgq, name, args.gemm_layout, args)
            log("side config %s: %.4f ms/step (%.1fs)" % (name, side[name]["ms_per_step"], time.time() - t0))

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
        "data": "synthetic (seeded Philox draws: prompt KV and layer input N(0,1), weights N(0,0.02))",
        "config": {"workload": w.name, "batch_g_x_m": "%dx%d" % (w.g, w.m), "global_batch": B,
                   "heads": H, "head_dim": D, "hidden": h, "prompt": w.prompt, "decode_steps": w.steps,
                   "weights": ["%dx%d" % kn for kn in w.weights],
                   "step": "chained: Q|K|V product -> KV append -> attention -> Wout -> W1 -> W2, fp16 hand-offs"
                   if w.weights else "append -> attention",
                   "gemm_launches": ["%s %dx%d" % (p[0], p[1], p[2]) for p in launch_plan(w)],
                   "gemm_layout": args.gemm_layout, "layer_instances": R, "parallelism": "single GPU"},
        "roofline": roof,
        "hbm_roofline_attention": {"achieved": attn_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                   "frac": attn_gbs / HBM_PEAK_GBS},
        "mfma_roofline_gemm": {"achieved": gemm_tflops, "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                               "frac": gemm_tflops / MFMA_F16_PEAK_TFLOPS, "GB_per_s": gemm_gbs},
        "step_launch": "eager" if gp is None else "hip-graph replay (one graph per decode step and layer instance)",
        "eager_ms_per_step": ep["total_ms"] / K_steps,
        "warmup_run": {"eager": {"steps": ep["warmup_steps"], "ms": round(ep["warmup_ms"], 1)},
                       "graph": None if gp is None else {"steps": gp["warmup_steps"], "ms": round(gp["warmup_ms"], 1)}},
        "gpu_clock_same_work_after_timed_steps": None if gp is None else gp["clock"],
        "kernels": kernels,
        "configs": side,
        "wall_s_timed_region": None if gp is None else gp["wall_s"],
        "context": "pages' end-to-end FlexGen 4-bit OPT-175B on one T4 with offloading: 1.12 token/s "
                   "(all 96 layers, prefill included) - not comparable to this per-layer in-HBM rate",
    }
    result["measured_ceilings"] = measured_ceilings(torch)
    if w.weights:
        result["measured_ceilings"]["library_f16_gemm_same_shapes"] = library_gemm_same_shapes(
            torch, B, [(p[0], p[1], p[2]) for p in launch_plan(w)])
    if not args.no_cpu_baseline and w.weights:
        t0 = time.time()
        result["cpu_baseline"] = cpu_baseline(w, args)
        log("cpu baseline %.1fs" % (time.time() - t0))
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
