"""Benchmark of the causal GQA attention forward on one MI355X.

One step is one pass of the whole hot path over resident inputs: one
attn_fwd call on the dense causal GQA prefill (B=4, Hq=32, Hkv=8, Q=K=4096,
D=Dv=128: the bf16 MFMA prefill kernel) and one attn_fwd call on the batched
long-context decode (B=64, Hq=64, Hkv=8, Q=1, int32 KV lengths log-uniform in
[1024, 32768] padded to 32768, D=Dv=128: split-KV decode + log-sum-exp
combine).  Inputs are seeded N(0,1) rounded to bf16 (Philox, seed 1234).

Before any timing the step runs untimed for at least --settle-s seconds of
GPU time (whatever --warmup says): the chip runs the prefill at its power
limit and its clock settles over about a second of sustained load.

Reported: prefill TFLOP/s (2*(D+Dv) per legal (row, key) pair) and decode KV
GB/s (K_b*Hkv*(D+Dv)*2 bytes summed over sequences), each against its
roofline (bf16 dense MFMA 2.5 PFLOP/s, HBM 8 TB/s).  `value` is the whole
step's fraction of roofline: the time the step would take at both peaks
divided by the measured step time, in percent.  The other three
configurations (the variable-length windowed prefill, the short decode with
a ragged tail, the tiny fp32 case) are timed separately after the step and
reported in `roofline_by_call`.

The fp64 oracle is timed on the host cores as a reported CPU baseline (never
the target): whole runs of the two small configurations, bounded samples of
rows of the three large ones.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 (and fp16) MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "causal GQA attn fwd: prefill TFLOP/s + decode KV GB/s, % of roofline"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma.json")
PEAK_FP32_VALU_TFLOPS = 157.3  # MI355X fp32 vector (the fp32 path's VALU kernel)
KERNEL_SOURCES = ["attn_internal.h", "prefill_bf16.hip", "decode_bf16.hip"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_digest() -> str:
    h = hashlib.sha1()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "attention_attn_fwd_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, digest: str):
    """HBM bytes per launch from the committed counter summary, or None when the
    kernel sources changed since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(kernel)
    if not ent or ent.get("kernel_digest") != digest:
        return None
    return ent.get("bytes_per_launch")


def measured_mfma(kernel: str, digest: str):
    """MFMA busy fraction and shader clock of a kernel from the committed
    counter summary, or (None, None) when the kernel sources changed since."""
    try:
        with open(MFMA_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None, None
    ent = rec.get("kernels", {}).get(kernel)
    if not ent or ent.get("kernel_digest") != digest:
        return None, None
    return ent.get("mfma_busy_frac"), ent.get("sclk_ghz")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def stats(ts):
    """mean / median / min of a list of seconds, in microseconds."""
    a = np.asarray(ts) * 1e6
    return {"us_per_call": float(np.mean(a)), "us_median": float(np.median(a)), "us_min": float(np.min(a))}


class Problem:
    def __init__(self, w, torch):
        from attention_attn_fwd_amd import inputs  # noqa: F401
        t0 = time.time()
        self.w = w
        q = w.gen_q()
        k = w.gen_k(padding="zero")
        v = w.gen_v(padding="zero")
        dev = "cuda:0"
        as_dev = (lambda a: torch.from_numpy(a).to(dev).view(torch.bfloat16)) if w.dtype == "bf16" else \
            (lambda a: torch.from_numpy(a).to(dev))
        self.q, self.k, self.v = as_dev(q), as_dev(k), as_dev(v)
        self.host = (q, k, v)  # kept for the CPU baseline
        self.seq = None if w.seqlens is None else torch.from_numpy(np.asarray(w.seqlens, np.int32)).to(dev)
        self.o = torch.empty(w.o_shape(), dtype={"bf16": torch.bfloat16, "f16": torch.float16,
                                                 "f32": torch.float32}[w.dtype], device=dev)
        self.lse = torch.empty((w.B, w.Hq, w.Q), dtype=torch.float32, device=dev)
        self.pairs = w.legal_pairs()
        self.flops = 2.0 * (w.D + w.Dv) * self.pairs
        self.kv_bytes = float(w.kv_tokens()) * (w.D + w.Dv) * (4 if w.dtype == "f32" else 2)
        log(f"[bench] {w.name}: inputs ready in {time.time() - t0:.1f}s "
            f"(pairs {self.pairs}, flops {self.flops:.4e}, kv bytes {self.kv_bytes:.4e})")

    def paginate(self, page, torch):
        """Move K/V into a paged cache: every page of a sequence's first K_b keys,
        in a seeded random order; the calls then go through attn_fwd_paged."""
        w = self.w
        q, k, v = self.host
        rng = np.random.default_rng(1234)
        pps = w.K // page
        used = [(b, j) for b in range(w.B) for j in range(pps) if j * page < w.kb(b)]
        order = rng.permutation(len(used))
        kp = np.zeros((len(used), w.Hkv, page, w.D), dtype=k.dtype)
        vp = np.zeros((len(used), w.Hkv, page, w.Dv), dtype=v.dtype)
        table = np.zeros((w.B, pps), dtype=np.int32)
        for i, (b, j) in enumerate(used):
            pg = int(order[i])
            table[b, j] = pg
            kp[pg] = k[b, :, j * page:(j + 1) * page]
            vp[pg] = v[b, :, j * page:(j + 1) * page]
        as_dev = (lambda a: torch.from_numpy(a).to("cuda:0").view(torch.bfloat16)) if w.dtype == "bf16" else \
            (lambda a: torch.from_numpy(a).to("cuda:0"))
        self.k, self.v = as_dev(kp), as_dev(vp)
        self.table = torch.from_numpy(table).to("cuda:0")
        self.page, self.num_pages = page, len(used)
        self.host = None

    def make_backward(self, af, torch):
        """Turn the call into the backward: O and LSE from one forward call, a
        seeded dO, and gradient buffers.  Algorithmic work: the four products
        dV, dP (over Dv), dQ, dK (over D) and the recomputed S (over D) per
        legal pair, 2 * (3D + 2Dv) flop."""
        from attention_attn_fwd_amd import inputs
        w = self.w
        self.call(af, torch.cuda.current_stream())
        dout = inputs.normal(w.o_shape(), 7, w.seed, w.dtype)
        self.dout = torch.from_numpy(dout).to("cuda:0")
        if w.dtype == "bf16":
            self.dout = self.dout.view(torch.bfloat16)
        self.dq, self.dk, self.dv = torch.empty_like(self.q), torch.empty_like(self.k), torch.empty_like(self.v)
        self.flops = 2.0 * (3 * w.D + 2 * w.Dv) * self.pairs
        self.backward = True

    def call(self, af, stream):
        w = self.w
        if getattr(self, "backward", False):
            flags = (af.ATTN_FWD_FP16 if w.dtype == "f16" else 0) | (0 if w.causal else af.ATTN_FWD_NONCAUSAL)
            st = af.attn_bwd(self.q, self.k, self.v, self.o, self.lse, self.dout, self.dq, self.dk, self.dv, w.B, w.Hq,
                             w.Hkv, w.Q, w.K, w.D, w.Dv, self.seq, w.window, w.scale, flags, stream)
        elif getattr(self, "page", None):
            flags = (af.ATTN_FWD_FP16 if w.dtype == "f16" else 0) | (0 if w.causal else af.ATTN_FWD_NONCAUSAL)
            st = af.attn_fwd_paged(self.q, self.k, self.v, self.o, self.lse, w.B, w.Hq, w.Hkv, w.Q, w.D, w.Dv,
                                   self.table, w.K // self.page, self.page, self.num_pages, self.seq, w.window,
                                   w.scale, flags, stream)
        elif w.dtype == "f32":
            st = af.attn_fwd_f32(self.q, self.k, self.v, self.o, self.lse, w.B, w.Hq, w.Hkv, w.Q, w.K, w.D, w.Dv,
                                 self.seq, w.window, w.scale, stream)
        elif w.dtype == "bf16" and w.causal:
            st = af.attn_fwd(self.q, self.k, self.v, self.o, self.lse, w.B, w.Hq, w.Hkv, w.Q, w.K, w.D, w.Dv,
                             self.seq, w.window, w.scale, stream)
        else:
            flags = (af.ATTN_FWD_FP16 if w.dtype == "f16" else 0) | (0 if w.causal else af.ATTN_FWD_NONCAUSAL)
            st = af.attn_fwd_ex(self.q, self.k, self.v, self.o, self.lse, w.B, w.Hq, w.Hkv, w.Q, w.K, w.D, w.Dv,
                                self.seq, w.window, w.scale, flags, stream)
        if st != af.ATTN_OK:
            raise RuntimeError(f"attn_fwd failed on {w.name}: {af.strerror(st)}")


def _sample_pairs(w, rows):
    """Legal (row, key) pairs of the given flat rows of a causal workload."""
    kb = np.array([w.kb(b) for b in range(w.B)])
    b = rows // (w.Hq * w.Q)
    qi = rows % w.Q
    p = qi + kb[b] - w.Q
    hi = np.minimum(kb[b] - 1, p)
    lo = np.zeros_like(hi) if w.window <= 0 else np.maximum(0, p - w.window + 1)
    return float(np.maximum(hi - lo + 1, 0).sum())


def cpu_baseline(probs, budget_s: float):
    """Time the fp64 oracle on the host cores: the whole of each small
    configuration, a bounded random sample of rows of each large one (its
    share of budget_s).  Rates: oracle GFLOP/s (2*(D+Dv) per legal pair) for
    the prefill-shaped configurations, oracle KV GB/s (the bytes of K/V rows
    the rows read, K_b*Hkv*(D+Dv)*element size per sequence) for the decodes."""
    from oracle import attn_oracle
    from attention_attn_fwd_amd import inputs
    orc = attn_oracle.load()
    threads = inputs.host_threads()
    large = [t for t, pr in probs if pr.w.B * pr.w.Hq * pr.w.Q > 4096]
    out = {}
    for tag, pr in probs:
        w = pr.w
        q, k, v = pr.host
        esz = 4 if w.dtype == "f32" else 2
        if tag not in large:
            t0 = time.perf_counter()
            orc.fwd(q, k, v, seqlens=w.seqlens, window=w.window, scale=w.scale, threads=threads)
            sec = time.perf_counter() - t0
            rows, pairs, sample = w.B * w.Hq * w.Q, float(pr.pairs), "whole configuration"
        else:
            rng = np.random.default_rng(7)
            rows, pairs, sec = 0, 0.0, 0.0
            batch = 256 if w.Q > 1 else 64
            while sec < budget_s / max(len(large), 1):
                rr = rng.integers(0, w.B * w.Hq * w.Q, size=batch).astype(np.int64)
                t0 = time.perf_counter()
                orc.rows(q, k, v, rr, seqlens=w.seqlens, window=w.window, scale=w.scale, threads=threads)
                sec += time.perf_counter() - t0
                rows += len(rr)
                pairs += _sample_pairs(w, rr)
            sample = f"{rows} random rows of {w.B * w.Hq * w.Q}"
        flops = 2.0 * (w.D + w.Dv) * pairs
        # K/V bytes the sampled rows read: each row reads its sequence's legal keys.
        kv_bytes = pairs / max(pr.pairs, 1) * float(w.kv_tokens()) * (w.D + w.Dv) * esz if w.Q == 1 else None
        rec = {"workload": w.name, "sample": sample, "seconds": sec, "rows": rows,
               "oracle_gflops": flops / sec / 1e9}
        if kv_bytes is not None:
            rec["oracle_kv_gbs"] = kv_bytes / sec / 1e9
        # Time the oracle would take for the whole configuration at this rate.
        rec["seconds_whole"] = sec * float(pr.pairs) / max(pairs, 1.0)
        out[tag] = rec
    return out, threads


def run_options(args, torch, af, inputs):
    """attn_fwd_ex / attn_fwd_paged options on the step's two shapes, each call
    timed alone: fp16 storage (causal prefill, decode), the non-causal mode
    (bf16 prefill, every key legal for every row), a paged K/V cache (pages of
    256 keys for the prefill, 128 for the decode, in random order), and two
    chunked-prefill shapes (short query runs against a long cache), heads of
    256 channels on the step's two shapes and of 512 on the prefill shape, the
    backward at the prefill shape, and the varlen windowed prefill and short
    decode configurations."""
    import dataclasses
    c3, c5 = inputs.config(3), inputs.config(5)
    cases = [
        ("prefill_f16", dataclasses.replace(c3, name="c3_shape_f16_causal_prefill", dtype="f16")),
        ("prefill_noncausal", dataclasses.replace(c3, name="c3_shape_bf16_noncausal_prefill", causal=False)),
        ("decode_f16", dataclasses.replace(c5, name="c5_shape_f16_decode", dtype="f16")),
    ]
    cases += [("prefill_paged", dataclasses.replace(c3, name="c3_paged256_prefill")),
              ("decode_paged", dataclasses.replace(c5, name="c5_paged128_decode"))]
    # Chunked prefill against a long cache, with the step's head layout: a
    # 64-row chunk (packed tiles of 4 heads, K/V range split 8 ways; K/V bytes
    # bound it) and a 512-row chunk at batch 1 (per-head tiles split 4 ways).
    cases += [("prefill_chunk64", inputs.Workload("chunk64_ctx16k_b4_prefill", 4, 32, 8, 64, 16384, 128, 128)),
              ("prefill_chunk512", inputs.Workload("chunk512_ctx32k_b1_prefill", 1, 32, 8, 512, 32768, 128, 128))]
    # Heads of 256 (the 8-wave kernel form), on the step's two shapes.
    cases += [("prefill_d256", dataclasses.replace(c3, name="c3_shape_d256_prefill", D=256, Dv=256)),
              ("decode_d256", dataclasses.replace(c5, name="c5_shape_d256_decode", D=256, Dv=256)),
              ("prefill_d512", dataclasses.replace(c3, name="c3_shape_d512_prefill", D=512, Dv=512))]
    # The backward (attn_bwd) at the dense prefill shape.
    cases += [("backward", dataclasses.replace(c3, name="c3_shape_bf16_backward")),
              ("backward_d256", dataclasses.replace(c3, name="c3_shape_d256_backward", D=256, Dv=256))]
    # The remaining configurations, reported beside the step: the
    # variable-length windowed prefill (legal pairs from the realised lengths
    # and the window) and the short decode with a ragged tail (latency-bound,
    # its GB/s for information).
    cases += [("prefill_varlen_window", inputs.config(4)), ("decode_tail", inputs.config(2))]
    hbm_bound = {"prefill_chunk64"}
    pages = {"prefill_paged": 256, "decode_paged": 128}
    stream = torch.cuda.current_stream()
    parts = {}
    for tag, w in cases:
        pr = Problem(w, torch)
        if tag in pages:
            pr.paginate(pages[tag], torch)
        if tag.startswith("backward"):
            pr.make_backward(af, torch)
        for _ in range(args.warmup):
            pr.call(af, stream)
        settle([lambda pr=pr: pr.call(af, stream)], 0.5, torch)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        for i in range(args.steps):
            ev[i].record(stream)
            pr.call(af, stream)
        ev[args.steps].record(stream)
        torch.cuda.synchronize()
        t = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])) * 1e-3
        if (tag.startswith("prefill") or tag.startswith("backward")) and tag not in hbm_bound:
            achieved, peak, unit, bound = pr.flops / t / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
        else:
            achieved, peak, unit, bound = pr.kv_bytes / t / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
        parts[tag] = {"workload": w.name, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                      "frac": achieved / peak, "us_per_call": 1e6 * t}
        log(f"[bench] {tag}: {1e6 * t:.1f} us/call, {achieved:.1f} {unit} = {100 * achieved / peak:.1f}% of peak")
        del pr
        torch.cuda.empty_cache()
    print(json.dumps({"metric": "options: fp16 storage, non-causal mode, paged K/V cache, chunked prefill, "
                                "head dim 256 and 512, backward, % of roofline",
                      "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
                      "data": "synthetic: seeded N(0,1) rounded to the storage type (Philox-4x32-10, seed 1234)",
                      "calls": parts, "kernel_digest": kernel_digest()}), flush=True)


def settle(calls, seconds: float, torch):
    """Run the calls untimed until `seconds` of wall time have passed (the GPU
    is kept busy throughout: the queue never drains between rounds)."""
    t0 = time.perf_counter()
    n = 0
    while True:
        for c in calls:
            c()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                return n


def time_calls(pr, af, torch, stream, reps: int):
    """Per-call durations of `reps` back-to-back calls, HIP events on the
    stream the kernels run on."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    for i in range(reps):
        ev[i].record(stream)
        pr.call(af, stream)
    ev[reps].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) * 1e-3 for i in range(reps)]


def run_mfma_cal(args, torch):
    """A kernel of known MFMA count: calibrates SQ_INSTS_MFMA,
    SQ_VALU_MFMA_BUSY_CYCLES and GRBM_GUI_ACTIVE (profiled by rocprofv3)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "attention_attn_fwd_amd", "libattn_calib.so"))
    lib.attn_calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.attn_calib_mfma_count.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.attn_calib_mfma_count.restype = ctypes.c_int64
    blocks, iters = 2048, 2048
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    times = []
    for _ in range(args.warmup + args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        assert lib.attn_calib_mfma(out.data_ptr(), blocks, iters, ctypes.c_void_p(stream.cuda_stream)) == 0
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    n = lib.attn_calib_mfma_count(blocks, iters)
    t = float(np.median(times[args.warmup:]))
    print(json.dumps({"calibration": "mfma 16x16x32 bf16", "mfma_per_dispatch": n, "blocks": blocks,
                      "iters": iters, "dispatches": args.warmup + args.steps, "us_median": 1e6 * t,
                      "tflops": n * 16384 / t / 1e12}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20, help="untimed steps before the settle and the timed steps")
    ap.add_argument("--settle-s", type=float, default=2.0,
                    help="seconds of untimed steps before timing, whatever --warmup says: the clock settles "
                         "under sustained load")
    ap.add_argument("--workload", choices=["step", "prefill", "decode", "copy", "options", "mfma_cal"],
                    default="step",
                    help="time the whole step (default), one of its two calls alone (for profiling), a "
                         "plain 1 GiB device copy (to calibrate the HBM byte counters), a kernel of known MFMA "
                         "count (to calibrate the MFMA counters), or the options (fp16 storage, non-causal, "
                         "paged, wide heads, backward, ...) each call timed alone")
    ap.add_argument("--cpu-budget", type=float, default=24.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the three other configurations timed after the step")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "this attention forward has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import attention_attn_fwd_amd as af
    from attention_attn_fwd_amd import inputs

    af.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.workload == "copy":
        # A plain copy of known size: FETCH_SIZE / WRITE_SIZE of this dispatch calibrate the counters.
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read_per_dispatch": nbytes,
                          "bytes_written_per_dispatch": nbytes, "dispatches": args.warmup + args.steps}))
        return
    if args.workload == "mfma_cal":
        run_mfma_cal(args, torch)
        return
    if args.workload == "options":
        run_options(args, torch, af, inputs)
        return
    prefill_w, decode_w = inputs.config(3), inputs.config(5)
    probs = []
    if args.workload in ("step", "prefill"):
        probs.append(("prefill", Problem(prefill_w, torch)))
    if args.workload in ("step", "decode"):
        probs.append(("decode", Problem(decode_w, torch)))
    stream = torch.cuda.current_stream()

    step_calls = [(lambda pr=pr: pr.call(af, stream)) for _, pr in probs]
    for _ in range(args.warmup):
        for c in step_calls:
            c()
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    n_settle = settle(step_calls, args.settle_s, torch)
    t_settle = time.perf_counter() - t_settle
    log(f"[bench] warmup {args.warmup} steps, then settled {t_settle:.2f}s ({n_settle} steps)")

    # Events on the stream every kernel is launched on: one before each call and one after the last.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(probs) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    for s in range(args.steps):
        for i, (_, pr) in enumerate(probs):
            ev[s][i].record(stream)
            pr.call(af, stream)
        ev[s][len(probs)].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    per_call = {name: [ev[s][i].elapsed_time(ev[s][i + 1]) * 1e-3 for s in range(args.steps)]
                for i, (name, _) in enumerate(probs)}
    step_times = [ev[s][0].elapsed_time(ev[s][len(probs)]) * 1e-3 for s in range(args.steps)]
    ms_per_step = 1e3 * float(np.mean(step_times))
    log(f"[bench] timed {args.steps} steps: {ms_per_step:.3f} ms/step (median {1e3 * np.median(step_times):.3f}, "
        f"wall {1e3 * wall / args.steps:.3f} ms/step)")

    digest = kernel_digest()
    parts, ideal, measured = {}, 0.0, 0.0
    for name, pr in probs:
        st = stats(per_call[name])
        t = st["us_per_call"] * 1e-6
        measured += t
        if name == "prefill":
            achieved = pr.flops / t / 1e12
            peak, unit, bound = PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
            ideal += pr.flops / (PEAK_BF16_TFLOPS * 1e12)
            kern = "prefill_bf16_kernel"
        else:
            achieved = pr.kv_bytes / t / 1e9
            peak, unit, bound = PEAK_HBM_GBS, "GB/s", "hbm"
            ideal += pr.kv_bytes / (PEAK_HBM_GBS * 1e9)
            kern = "decode_split_kernel"
        busy, sclk = measured_mfma(kern, digest)
        parts[name] = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                       "frac": achieved / peak, "traffic": measured_traffic(kern, digest),
                       "mfma_util": busy, "sclk_ghz": sclk, **st, "workload": pr.w.name}
        log(f"[bench] {name}: {st['us_per_call']:.1f} us/call (median {st['us_median']:.1f}, min {st['us_min']:.1f}), "
            f"{achieved:.1f} {unit} = {100 * achieved / peak:.1f}% of peak")
    frac = ideal / measured
    dominant = max(parts, key=lambda n: parts[n]["us_per_call"])
    roof = {k: parts[dominant][k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic",
                                            "mfma_util", "sclk_ghz")}

    # The other three configurations, each timed alone after the step.
    others = []
    if args.workload == "step" and not args.no_configs:
        for idx, tag, reps in ((4, "varlen_window_prefill", 20), (2, "decode_tail", 200), (1, "fp32_tiny", 200)):
            pr = Problem(inputs.config(idx), torch)
            settle([lambda pr=pr: pr.call(af, stream)], 0.3, torch)
            st = stats(time_calls(pr, af, torch, stream, reps))
            t = st["us_per_call"] * 1e-6
            if idx == 4:
                achieved, peak, unit, bound = pr.flops / t / 1e12, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma"
            elif idx == 2:
                achieved, peak, unit, bound = pr.kv_bytes / t / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
            else:
                achieved, peak, unit, bound = pr.flops / t / 1e12, PEAK_FP32_VALU_TFLOPS, "TFLOP/s", "alu"
            parts[tag] = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit, "frac": achieved / peak,
                          **st, "workload": pr.w.name}
            log(f"[bench] {tag}: {st['us_per_call']:.1f} us/call (median {st['us_median']:.1f}), "
                f"{achieved:.3f} {unit} = {100 * achieved / peak:.2f}% of peak")
            others.append((tag, pr))

    cpu = None
    if not args.no_cpu_baseline:
        by_cfg, threads = cpu_baseline([(n, pr) for n, pr in probs] + others, args.cpu_budget)
        t_cpu = sum(by_cfg[n]["seconds_whole"] for n, _ in probs)
        desc = "; ".join(f"{n}: {by_cfg[n]['sample']} ({by_cfg[n]['seconds']:.1f}s)" for n, _ in probs)
        cpu = {"value": 100.0 * ideal / t_cpu, "unit": "% of roofline", "cores": threads, "kind": "oracle",
               "sample": desc + "; step time extrapolated from each workload's sampled rate",
               "seconds_per_step": t_cpu, "cpu_model": cpu_model(), "by_config": by_cfg}
        for n, r in by_cfg.items():
            log(f"[bench] cpu oracle {n}: {r['oracle_gflops']:.2f} GFLOP/s"
                + (f", {r['oracle_kv_gbs']:.3f} KV GB/s" if "oracle_kv_gbs" in r else "") + f" ({r['sample']})")

    w3, w5 = prefill_w, decode_w
    workload = []
    if "prefill" in parts:
        workload.append(f"dense causal GQA prefill B={w3.B},Hq={w3.Hq},Hkv={w3.Hkv},Q=K={w3.K},D=Dv={w3.D}")
    if "decode" in parts:
        workload.append(f"batched long-context decode B={w5.B},Hq={w5.Hq},Hkv={w5.Hkv},Q=1,"
                        f"K_b log-uniform [1024,32768] padded to {w5.K},D=Dv={w5.D}")
    rec = {
        "metric": METRIC,
        "value": 100.0 * frac,
        "unit": "% of roofline",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": round(t_settle, 3),
        "ms_per_step": ms_per_step,
        "ms_per_step_median": 1e3 * float(np.median(step_times)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) rounded to bf16 (Philox-4x32-10, seed 1234)",
        "config": {"workload": " + ".join(workload), "seed": 1234, "parallelism": "single GPU"},
        "prefill_tflops": parts.get("prefill", {}).get("achieved"),
        "decode_kv_gbs": parts.get("decode", {}).get("achieved"),
        "roofline": roof,
        "roofline_by_call": parts,
        "realised_seqlens": {"c4_varlen_window_prefill": [int(x) for x in inputs.config(4).seqlens],
                             "c5_batched_long_decode": [int(x) for x in decode_w.seqlens]},
        "kernel_digest": digest,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
