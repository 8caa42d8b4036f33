"""Benchmark of the decode hot path on one MI355X.

Default workload (one "step" = one call of entro_decode_dequant):
  16 distinct device copies of a 4096 x 4096 float32 tensor w ~ Laplace(0, 0.015),
  quantized per tensor to unsigned 4-bit codes, canonical-Huffman coded (lengths
  <= 12) in 8192-code chunks of 32 interleaved lanes, decoded and dequantized
  to bf16 in one batched call.  16 copies put the working set (about 590 MB)
  well above the 256 MB last-level cache, so the timed data comes from HBM.

Other workloads (``--workload``): tensor_2048 (8-bit asymmetric, 4096-code
chunks, decode to codes and to bf16), smollm_stack / smollm_stack_u8 (decode
all 169 tensors in one call), phi3_stack / mistral_stack (per token: fused
decode + GEMV, or with ``--path ahead`` each matrix decoded to bf16 on a side
stream just ahead of the stock linear kernel, or with ``--path dense`` the
stock kernel on resident bf16 weights; ``--graph`` replays the token as one
HIP graph).  ``--coder rans`` runs the tensor workloads on interleaved-rANS
streams of the same codes instead (entro_rans_decode[_dequant]).

The encoder used to produce the inputs is the library's own (host C++), not
the oracle; the oracle is only timed in the CPU-baseline leg.

Output: one JSON line (rank 0).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MAX_TENSORS_PER_LAUNCH = 32   # the library batches up to 32 tensors per kernel launch
METRIC = "decoded Gsym/s + effective HBM GB/s (% of peak); fused decode+GEMV ms/token"
KERNEL_SOURCES = ["entropy_coded_weight_canonical_amd/csrc/entro_decode.hip",
                  "entropy_coded_weight_canonical_amd/csrc/entro_device.h",
                  "entropy_coded_weight_canonical_amd/csrc/entro_internal.h"]


# The five workloads as stated, and the layout readings where the statement
# gives none (chunk C, lanes W).  Every stream is encoded refilling ahead with
# a refill decision every two steps.  GEMV workloads use row-aligned chunks of
# about `chunk_target` weights.  The GPU parity tests run the same settings.
REFILL_STEPS = 2
REFILL_AHEAD = True
WORKLOADS = {
    "tensor_2048": {"config": 1, "bits": 8, "scheme": "asymmetric", "chunk": 4096, "lanes": 32, "replicas": 64},
    "tensor_4096": {"config": 2, "bits": 4, "scheme": "unsigned", "chunk": 8192, "lanes": 32, "replicas": 16},
    "smollm_stack": {"config": 3, "bits": 8, "scheme": "mixed", "chunk": 4096, "lanes": 32},
    "phi3_stack": {"config": 4, "bits": 4, "scheme": "mixed", "chunk_target": 4096, "lanes": 64, "clip_sigma": 0.0},
    "mistral_stack": {"config": 5, "bits": 4, "scheme": "unsigned", "chunk_target": 4096, "lanes": 64,
                      "clip_sigma": None},   # None: synth.MISTRAL_CLIP_SIGMA (3.90 bits per weight)
}


def gemv_chunk(cols: int, chunk_target: int) -> int:
    """Row-aligned chunk: the whole rows nearest to chunk_target weights (at least one)."""
    return cols * max(1, round(chunk_target / cols))

def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_src_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(name: str, config: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None
    if the kernel source changed since the counters were taken or the summary
    was taken on another configuration (lanes, chunk, refill options, replicas)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_src_sha") != kernel_src_sha() or kv.get("config") != config:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def traffic_config(chunk, lanes, args, replicas) -> str:
    """The configuration a traffic summary applies to (recorded in it)."""
    return f"C={chunk} W={lanes} refill_steps={args.refill_steps} ahead={int(args.refill_ahead)} replicas={replicas}"


# --------------------------------------------------------------------------
# inputs (library encoder)
# --------------------------------------------------------------------------

class Coded:
    def __init__(self, q, scale, zp, scheme, bits, max_len, chunk, lanes, rows, cols, refill_steps, ahead=False):
        import entropy_coded_weight_canonical_amd as ent

        self.rows, self.cols = rows, cols
        self.bits, self.max_len, self.chunk, self.lanes = bits, max_len, chunk, lanes
        self.scale, self.zp, self.scheme = scale, zp, scheme
        self.refill_steps, self.ahead = refill_steps, bool(ahead)
        self.n = int(q.size)
        self.lengths = ent.code_lengths(q, bits, max_len)
        self.words, self.offs = ent.encode(q, self.lengths, bits, chunk, lanes, refill_steps=refill_steps,
                                           ahead=self.ahead)
        self.lut = ent.lut_build(self.lengths, bits, max_len, scale, zp)
        self.n_chunks = int(self.offs.size - 1)

    @property
    def in_bytes(self) -> int:
        return 4 * int(self.words.size) + 8 * (self.n_chunks + 1)

    @property
    def coded_bits_per_weight(self) -> float:
        return 8.0 * self.in_bytes / self.n


def code_tensor(spec, bits, scheme, chunk, lanes, refill_steps, clip_sigma=0.0, ahead=False):
    import entropy_coded_weight_canonical_amd as ent
    from synth import weights

    w = weights(spec)
    clip = float(clip_sigma * np.std(w, dtype=np.float64)) if clip_sigma else 0.0
    q, s, zp, chosen = ent.quantize(w, bits, scheme, clip=clip)
    return Coded(q, s, zp, chosen, bits, 16 if bits == 8 else 12, chunk, lanes, spec.rows, spec.cols, refill_steps,
                 ahead)


# --------------------------------------------------------------------------
# CPU baseline: the oracle, as it stands
# --------------------------------------------------------------------------

def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(coded: Coded, budget_s: float = 12.0, single_budget_s: float = 4.0):
    """The oracle's C decoder over host threads (the chunk-parallel CPU decode
    of EntroLLM), plus numpy dequant; also one thread alone."""
    from oracle import ccodec
    from oracle.dequant import dequant_bf16

    def rate(threads, budget):
        n_done, reps, t_dec = 0, 0, 0.0
        t0 = time.perf_counter()
        while True:
            ta = time.perf_counter()
            q = ccodec.decode(coded.words, coded.offs, coded.lengths, coded.n, coded.chunk, coded.lanes,
                              threads=threads, refill_steps=coded.refill_steps, ahead=coded.ahead)
            t_dec += time.perf_counter() - ta
            dequant_bf16(q, coded.scale, coded.zp)
            n_done += coded.n
            reps += 1
            if time.perf_counter() - t0 >= budget:
                break
        dt = time.perf_counter() - t0
        return n_done / dt / 1e9, n_done / t_dec / 1e9, reps, dt

    threads = min(16, os.cpu_count() or 1)
    v, vd, reps, dt = rate(threads, budget_s)
    v1, vd1, reps1, dt1 = rate(1, single_budget_s)
    return {"value": round(v, 4), "unit": "Gsym/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} x one {coded.rows}x{coded.cols} tensor ({coded.n} codes): bit-serial C decode "
                      f"over {threads} host threads + numpy bf16 dequant (one thread), {dt:.1f} s wall",
            "decode_only_value": round(vd, 4),
            "single_thread_value": round(v1, 4), "single_thread_decode_only_value": round(vd1, 4),
            "single_thread_sample": f"{reps1} x the same tensor with the decode on 1 thread, {dt1:.1f} s wall",
            "nproc": os.cpu_count(), "cpu_model": cpu_model()}


# --------------------------------------------------------------------------
# GPU timing helpers
# --------------------------------------------------------------------------

def time_steps(step, steps, warmup):
    """Warm-up, then the timed region: `steps` steps back to back between two
    events on the launch stream, synchronized on both sides (-> total ms; its
    average per launch is what the roofline uses).  Then the same number of
    steps again, each between its own event pair, for the spread of single
    launches (p10/p50/p90): events between launches keep the next launch from
    starting right behind the previous one and add a few microseconds each,
    so they stay out of the timed region."""
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = ev0.elapsed_time(ev1)
    per = []
    for _ in range(steps):
        e_a = torch.cuda.Event(enable_timing=True)
        e_b = torch.cuda.Event(enable_timing=True)
        e_a.record(stream)
        step()
        e_b.record(stream)
        per.append((e_a, e_b))
    torch.cuda.synchronize()
    per_ms = [a.elapsed_time(b) for a, b in per]
    return total_ms, per_ms, wall


def flush_mall(torch):
    """Evict the last-level cache between measurements (writes 512 MB)."""
    buf = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    return buf


def launch_pct(per_ms):
    p10, p50, p90 = np.percentile(np.asarray(per_ms, dtype=np.float64), [10, 50, 90])
    return {"launch_ms_p10": round(float(p10), 5), "launch_ms_p50": round(float(p50), 5),
            "launch_ms_p90": round(float(p90), 5)}


def device_info(torch):
    """GPU name, CU count (torch) and the agent's maximum clock (rocminfo)."""
    props = torch.cuda.get_device_properties(0)
    info = {"name": torch.cuda.get_device_name(0), "compute_units": int(props.multi_processor_count),
            "arch": getattr(props, "gcnArchName", "")}
    try:
        import subprocess

        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
        gpu, clk = False, None
        for line in out.splitlines():
            t = line.strip()
            if t.startswith("Name:") and "gfx" in t:
                gpu = True
            if gpu and t.startswith("Max Clock Freq. (MHz):"):
                clk = int(t.split(":", 1)[1].split()[0])
                break
        info["max_clock_mhz"] = clk
    except Exception as e:   # rocminfo missing or slow: the clock is context only
        info["max_clock_mhz"] = None
        info["clock_error"] = type(e).__name__
    return info


def device_copy_gbps(torch, nbytes=256 << 20, reps=10):
    """A plain device-to-device copy of nbytes (read + write counted), median."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(5)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return 2.0 * nbytes / (float(np.median(ts)) * 1e-3) / 1e9


def single_call_us(torch, step, reps=20):
    """Latency of one call (median of reps, data warm in cache)."""
    step()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        step()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return round(float(np.median(ts)) * 1e3, 2)


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

def bench_decode(args, workload, bits, scheme, chunk, lanes, replicas, mode):
    import torch

    import entropy_coded_weight_canonical_amd as ent
    from synth import tensor_specs

    spec = tensor_specs(workload)[0]
    log(f"encoding {workload} ({spec.rows}x{spec.cols}, {bits}-bit {scheme}, C={chunk}, W={lanes})")
    coded = code_tensor(spec, bits, scheme, chunk, lanes, args.refill_steps, ahead=args.refill_ahead)
    log(f"coded {coded.coded_bits_per_weight:.3f} bits/weight; uploading {replicas} replicas")
    dts = [ent.DeviceTensor.upload(coded.lut, coded.words, coded.offs, coded.n, chunk, lanes, bits,
                                   coded.max_len, refill_steps=args.refill_steps, ahead=coded.ahead)
           for _ in range(replicas)]
    odt = torch.uint8 if mode == "u8" else torch.int16
    outs = [torch.empty(coded.n, dtype=odt, device="cuda") for _ in range(replicas)]
    status = torch.zeros(replicas, dtype=torch.int32, device="cuda")
    descs = [d.desc for d in dts]
    ptrs = [o.data_ptr() for o in outs]
    fn = ent.decode if mode == "u8" else ent.decode_dequant

    def step():
        fn(descs, ptrs, status.data_ptr())

    step()
    torch.cuda.synchronize()
    if int(status.abs().sum().item()) != 0:
        raise SystemExit(f"stream flags set: {status.cpu().numpy()}")
    # spot check: replica 0 decodes to the library encoder's input codes
    log(f"timing {args.steps} steps after {args.warmup} warm-up")
    _keep = flush_mall(torch)
    total_ms, per_ms, wall = time_steps(step, args.steps, args.warmup)
    ms = total_ms / args.steps
    n_sym = coded.n * replicas
    out_b = coded.n * (1 if mode == "u8" else 2)
    bytes_step = replicas * (coded.in_bytes + out_b)
    launches = -(-replicas // MAX_TENSORS_PER_LAUNCH)
    launch_ms = ms / launches   # the timed region's average launch
    achieved = (bytes_step / launches) / (launch_ms * 1e-3) / 1e9   # per launch
    traffic = read_traffic(f"{workload}_{mode}", traffic_config(chunk, lanes, args, replicas))
    res = {
        "metric": METRIC,
        "value": round(n_sym / (ms * 1e-3) / 1e9, 3),
        "unit": "Gsym/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if mode == "bf16" else "u8",
        "data": "synthetic",
        "config": {"workload": f"{workload}: {spec.rows}x{spec.cols} {scheme} {bits}-bit, C={chunk}, W={lanes}, "
                               f"refill every {args.refill_steps} step(s){', ahead' if coded.ahead else ''}, "
                               f"x{replicas} replicas, "
                               f"decode{'+dequant->bf16' if mode == 'bf16' else '->u8'}",
                   "global_batch": replicas, "symbols_per_step": n_sym,
                   "coded_bits_per_weight": round(coded.coded_bits_per_weight, 4),
                   "parallelism": "single GPU"},
        "eff_GBps": round(bytes_step / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(bytes_step / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": None if traffic is None else round(traffic / (launch_ms * 1e-3) / 1e9, 1)},
        "kernel": {"name": "ecw_decode_kernel", "launches_per_step": launches, "avg_launch_ms": round(launch_ms, 5),
                   **{"event_bracketed_" + k.replace("launch_", "step_"): v for k, v in launch_pct(per_ms).items()},
                   "algorithmic_bytes_per_launch": bytes_step // launches, "src_sha": kernel_src_sha()},
    }
    if args.single_latency:   # extra launches of the same kernel: kept out of the default (profiled) run
        res["single_tensor_us"] = single_call_us(torch, lambda: fn(descs[:1], ptrs[:1], status.data_ptr()))
    return res, coded



class RansCoded:
    """One tensor coded with the library's rANS encoder (ECR v1)."""

    def __init__(self, q, scale, zp, bits, chunk, lanes, rows, cols):
        import entropy_coded_weight_canonical_amd as ent

        self.q = np.ascontiguousarray(q, dtype=np.uint8).ravel()
        self.rows, self.cols, self.bits, self.chunk, self.lanes = rows, cols, bits, chunk, lanes
        self.scale, self.zp, self.n = scale, zp, int(self.q.size)
        self.freqs = ent.rans_freqs(np.bincount(self.q, minlength=1 << bits).astype(np.uint64))
        self.units, self.offs = ent.rans_encode(self.q, self.freqs, bits, chunk, lanes)
        self.table = ent.rans_table_build(self.freqs, bits, scale, zp)
        self.n_chunks = int(self.offs.size - 1)

    @property
    def in_bytes(self) -> int:
        return 2 * int(self.units.size) + 8 * (self.n_chunks + 1)

    @property
    def coded_bits_per_weight(self) -> float:
        return 8.0 * self.in_bytes / self.n


def cpu_baseline_rans(rc: RansCoded, budget_s: float = 12.0):
    """The rANS oracle (pure Python, one thread) on the tensor's first chunks."""
    from oracle import rans
    from oracle.dequant import dequant_bf16

    k = min(rc.n_chunks, 2)
    n = min(rc.n, k * rc.chunk)
    offs = rc.offs[: k + 1]
    units = rc.units[: int(offs[-1])]
    freqs = rc.freqs.astype(np.int64)
    n_done, reps = 0, 0
    t0 = time.perf_counter()
    while True:
        q = rans.decode(units, offs, freqs, n, rc.chunk, rc.lanes)
        dequant_bf16(q, rc.scale, rc.zp)
        n_done += n
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": round(n_done / dt / 1e9, 6), "unit": "Gsym/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} x the first {k} chunks ({n} codes) of one {rc.rows}x{rc.cols} tensor: "
                      f"pure-Python rANS decode + numpy bf16 dequant, {dt:.1f} s wall"}


def bench_decode_rans(args, workload, bits, scheme, chunk, lanes, replicas, mode):
    """The same tensors and call shape as bench_decode, coded with interleaved
    rANS instead of canonical Huffman."""
    import torch

    import entropy_coded_weight_canonical_amd as ent
    from synth import tensor_specs, weights

    spec = tensor_specs(workload)[0]
    log(f"rANS-encoding {workload} ({spec.rows}x{spec.cols}, {bits}-bit {scheme}, C={chunk}, W={lanes})")
    q, s, zp, chosen = ent.quantize(weights(spec), bits, scheme)
    rc = RansCoded(q, s, zp, bits, chunk, lanes, spec.rows, spec.cols)
    huff = Coded(q, s, zp, chosen, bits, 16 if bits == 8 else 12, chunk, lanes, spec.rows, spec.cols,
                 args.refill_steps, args.refill_ahead)
    log(f"rANS {rc.coded_bits_per_weight:.3f} bits/weight (Huffman {huff.coded_bits_per_weight:.3f}); "
        f"uploading {replicas} replicas")
    dts = [ent.DeviceRansTensor.upload(rc.table, rc.units, rc.offs, rc.n, chunk, lanes, bits) for _ in range(replicas)]
    odt = torch.uint8 if mode == "u8" else torch.int16
    outs = [torch.empty(rc.n, dtype=odt, device="cuda") for _ in range(replicas)]
    status = torch.zeros(replicas, dtype=torch.int32, device="cuda")
    descs = [d.desc for d in dts]
    ptrs = [o.data_ptr() for o in outs]
    fn = ent.rans_decode if mode == "u8" else ent.rans_decode_dequant

    def step():
        fn(descs, ptrs, status.data_ptr())

    step()
    torch.cuda.synchronize()
    if int(status.abs().sum().item()) != 0:
        raise SystemExit(f"stream flags set: {status.cpu().numpy()}")
    log(f"timing {args.steps} steps after {args.warmup} warm-up")
    _keep = flush_mall(torch)
    total_ms, per_ms, wall = time_steps(step, args.steps, args.warmup)
    ms = total_ms / args.steps
    n_sym = rc.n * replicas
    bytes_step = replicas * (rc.in_bytes + rc.n * (1 if mode == "u8" else 2))
    launches = -(-replicas // MAX_TENSORS_PER_LAUNCH)
    launch_ms = ms / launches   # the timed region's average launch
    achieved = (bytes_step / launches) / (launch_ms * 1e-3) / 1e9   # per launch
    res = {
        "metric": METRIC,
        "value": round(n_sym / (ms * 1e-3) / 1e9, 3),
        "unit": "Gsym/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if mode == "bf16" else "u8",
        "data": "synthetic",
        "config": {"workload": f"{workload}: {spec.rows}x{spec.cols} {scheme} {bits}-bit, interleaved rANS "
                               f"(M=4096, 16-bit units), C={chunk}, W={lanes}, x{replicas} replicas, "
                               f"decode{'+dequant->bf16' if mode == 'bf16' else '->u8'}",
                   "global_batch": replicas, "symbols_per_step": n_sym,
                   "coded_bits_per_weight": round(rc.coded_bits_per_weight, 4),
                   "huffman_coded_bits_per_weight": round(huff.coded_bits_per_weight, 4),
                   "parallelism": "single GPU"},
        "eff_GBps": round(bytes_step / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(bytes_step / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": None},
        "kernel": {"name": "ecr_kernel", "launches_per_step": launches, "avg_launch_ms": round(launch_ms, 5),
                   **{"event_bracketed_" + k.replace("launch_", "step_"): v for k, v in launch_pct(per_ms).items()},
                   "algorithmic_bytes_per_launch": bytes_step // launches, "src_sha": kernel_src_sha()},
    }
    if args.single_latency:
        res["single_tensor_us"] = single_call_us(torch, lambda: fn(descs[:1], ptrs[:1], status.data_ptr()))
    return res, rc


def bench_gemv(args, workload, batch, clip_sigma=0.0):
    """Per-token fused decode+GEMV over the whole stack, one call per group of
    matrices sharing an input (q/k/v, o, gate/up, down) per layer."""
    import torch

    import entropy_coded_weight_canonical_amd as ent
    from synth import activations_bf16, tensor_specs

    specs = tensor_specs(workload)
    layers = max(s.layer for s in specs) + 1
    # every layer has the same shapes; encode layer 0 and layer 1, and give the
    # other layers distinct device copies of them (same bytes, other addresses)
    n_distinct = min(args.distinct_layers, layers)
    log(f"{workload}: encoding {n_distinct} distinct layer(s) of {layers}")
    coded_layers = []
    for L in range(n_distinct):
        row = []
        for s in (x for x in specs if x.layer == L):
            chunk = s.cols * max(1, round(args.gemv_chunk / s.cols))
            row.append((s, code_tensor(s, 4, "unsigned" if clip_sigma else "mixed", chunk, 64, args.refill_steps,
                                       clip_sigma, ahead=args.refill_ahead)))
        coded_layers.append(row)
    groups = []   # per layer: list of (descs, items)
    keep = []
    mats = []     # (DeviceTensor, rows, cols, x) in token order, for the unfused paths
    n_sym = 0
    in_bytes = 0
    for L in range(layers):
        row = coded_layers[L % n_distinct]
        by_group = {}
        for s, c in row:
            by_group.setdefault(s.group, []).append((s, c))
        for gname, members in by_group.items():
            cols = members[0][0].cols
            x = torch.from_numpy(activations_bf16(workload, len(groups), cols, batch).view(np.int16)).cuda()
            descs, items = [], []
            for s, c in members:
                dt = ent.DeviceTensor.upload(c.lut, c.words, c.offs, c.n, c.chunk, c.lanes, c.bits, c.max_len,
                                             refill_steps=c.refill_steps, ahead=c.ahead)
                y = torch.empty((batch, s.rows), dtype=torch.float32, device="cuda")
                keep += [dt, y]
                descs.append(dt.desc)
                items.append(ent.GemvItem(s.rows, s.cols, x.data_ptr(), y.data_ptr()))
                mats.append((dt, s.rows, s.cols, x))
                n_sym += c.n
                in_bytes += c.in_bytes + 2 * batch * s.cols + 4 * batch * s.rows
            keep.append(x)
            groups.append((descs, items))
    status = torch.zeros(64, dtype=torch.int32, device="cuda")
    path = args.path
    hbm_bytes = in_bytes   # algorithmic HBM bytes per token of the chosen path

    if path == "fused":
        def step():
            for descs, items in groups:
                ent.decode_gemv(descs, items, batch, status.data_ptr())

        def flags():
            return status
    elif path == "gemm":
        # prompt processing: all `batch` tokens at once through the decode +
        # GEMM entry point (every weight decoded once, products on MFMA)
        def step():
            for descs, items in groups:
                ent.decode_gemm(descs, items, batch, status.data_ptr())

        def flags():
            return status
    elif path == "ahead":
        # decode-ahead streaming: each matrix decoded to bf16 on a side stream
        # just before the stock linear kernel reads it
        from entropy_coded_weight_canonical_amd.ahead import DecodeAhead

        da = DecodeAhead([m[0] for m in mats], [(m[1], m[2]) for m in mats], depth=args.ahead_depth,
                         block_elems=args.ahead_block or None)
        xs_bf = [m[3].view(torch.bfloat16) for m in mats]
        hbm_bytes = sum(m[0].desc.n_words * 4 + 2 * m[1] * m[2] * 2 + 2 * batch * m[2] + 2 * batch * m[1]
                        for m in mats)

        def step():
            da.run(xs_bf)

        def flags():
            return da.status
    else:
        # dense bf16 baseline: every matrix decoded once to its own resident bf16
        # copy, then only the stock linear kernel per token
        import torch.nn.functional as F

        dense = []
        for dt, r, c, x in mats:
            wbuf = torch.empty((r, c), dtype=torch.bfloat16, device="cuda")
            ent.decode_dequant([dt.desc], [wbuf.data_ptr()], status.data_ptr())
            dense.append((wbuf, x.view(torch.bfloat16)))
        hbm_bytes = sum(2 * w.numel() + 2 * batch * w.shape[1] + 2 * batch * w.shape[0] for w, _ in dense)

        def step():
            for w, x in dense:
                F.linear(x, w)

        def flags():
            return status

    step()
    torch.cuda.synchronize()
    if int(flags().abs().sum().item()) != 0:
        raise SystemExit(f"stream flags set: {flags().cpu().numpy()}")
    if args.graph:
        # the whole token as one HIP graph (warm-up on a side stream first)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        step = graph.replay
        step()
        torch.cuda.synchronize()
        if int(flags().abs().sum().item()) != 0:
            raise SystemExit(f"stream flags set in graph replay: {flags().cpu().numpy()}")
    _keep = flush_mall(torch)
    total_ms, per_ms, wall = time_steps(step, args.steps, args.warmup)
    ms = total_ms / args.steps
    bits = np.mean([c.coded_bits_per_weight for row in coded_layers for _, c in row])
    per_token = ms / batch if path == "gemm" else ms
    res = {
        "metric": METRIC,
        "value": round(per_token, 4),
        "unit": "ms/token",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{workload}: {len(specs)} matrices, 4-bit "
                               f"{'unsigned clip %.2f sigma' % clip_sigma if clip_sigma else 'mixed'}, "
                               f"row-aligned chunks, W=64, " + {
                                   "fused": f"fused decode+dequant+GEMV batch {batch}",
                                   "ahead": f"decode-ahead to bf16 (depth {args.ahead_depth}, blocks of "
                                            f"{args.ahead_block or 'whole'} weights) + stock matmul, "
                                            f"batch {batch}",
                                   "dense": f"dense bf16 weights (decoded once) + stock linear kernel, "
                                            f"batch {batch}",
                                   "gemm": f"fused decode+dequant+GEMM (MFMA) over a {batch}-token prompt, "
                                           f"value per token"}[path],
                   "path": path, "hip_graph": bool(args.graph), "chunk_target": args.gemv_chunk,
                   "refill_ahead": bool(args.refill_ahead),
                   "global_batch": batch, "symbols_per_token": n_sym, "launch_groups": len(groups),
                   "distinct_layers": n_distinct, "coded_bits_per_weight": round(float(bits), 4),
                   "parallelism": "single GPU"},
        "decoded_Gsym_per_s": round(n_sym / (ms * 1e-3) / 1e9, 3),
        "matmul_TFLOPs": round(2.0 * batch * n_sym / (ms * 1e-3) / 1e12, 2),
        "hbm_bytes_per_token": int(hbm_bytes),
        "eff_GBps": round(hbm_bytes / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(hbm_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "step_ms_pct": {k.replace("launch_", "step_"): v for k, v in launch_pct(per_ms).items()},
    }
    return res


def bench_stack_decode(args, workload, mode):
    """Decode a whole stack in one call (all tensors, batched by the library
    into launches of up to 32 tensors): 8-bit mixed codes, C 4096, W 32."""
    import torch

    import entropy_coded_weight_canonical_amd as ent
    from synth import tensor_specs

    specs = tensor_specs(workload)
    layers = max(s.layer for s in specs) + 1
    n_distinct = min(args.distinct_layers, layers)
    lanes = args.lanes or 32
    log(f"{workload}: encoding {n_distinct} distinct layer(s) of {layers} and the unlayered tensors")
    coded = {}
    for s in specs:
        key = (s.layer % n_distinct, s.name.split(".", 1)[-1]) if s.layer >= 0 else ("x", s.name)
        if key not in coded:
            coded[key] = code_tensor(s, 8, "mixed", 4096, lanes, args.refill_steps, ahead=args.refill_ahead)
    dts, outs, keep = [], [], []
    n_sym = 0
    bytes_step = 0
    odt = torch.uint8 if mode == "u8" else torch.int16
    for s in specs:
        key = (s.layer % n_distinct, s.name.split(".", 1)[-1]) if s.layer >= 0 else ("x", s.name)
        c = coded[key]
        dts.append(ent.DeviceTensor.upload(c.lut, c.words, c.offs, c.n, c.chunk, c.lanes, c.bits, c.max_len,
                                           refill_steps=c.refill_steps, ahead=c.ahead))
        outs.append(torch.empty(c.n, dtype=odt, device="cuda"))
        n_sym += c.n
        bytes_step += c.in_bytes + c.n * (1 if mode == "u8" else 2)
    status = torch.zeros(len(specs), dtype=torch.int32, device="cuda")
    descs = [d.desc for d in dts]
    ptrs = [o.data_ptr() for o in outs]
    fn = ent.decode if mode == "u8" else ent.decode_dequant

    def step():
        fn(descs, ptrs, status.data_ptr())

    step()
    torch.cuda.synchronize()
    if int(status.abs().sum().item()) != 0:
        raise SystemExit(f"stream flags set: {status.cpu().numpy()}")
    _keep = flush_mall(torch)
    total_ms, per_ms, wall = time_steps(step, args.steps, args.warmup)
    ms = total_ms / args.steps
    call_ms = ms   # one call per step: the timed region's average call
    launches = -(-len(specs) // MAX_TENSORS_PER_LAUNCH)   # one lane count in the stack
    bits = 8.0 * sum(c.in_bytes for c in coded.values()) / sum(c.n for c in coded.values())
    res = {
        "metric": METRIC,
        "value": round(n_sym / (ms * 1e-3) / 1e9, 3),
        "unit": "Gsym/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if mode == "bf16" else "u8",
        "data": "synthetic",
        "config": {"workload": f"{workload}: {len(specs)} tensors, 8-bit mixed, C=4096, W={lanes}, "
                               f"refill every {args.refill_steps} step(s){', ahead' if args.refill_ahead else ''}, "
                               f"decode all "
                               f"{'+dequant->bf16' if mode == 'bf16' else '->u8'} in one call",
                   "global_batch": 1, "symbols_per_step": n_sym, "distinct_layers": n_distinct,
                   "coded_bits_per_weight": round(bits, 4), "parallelism": "single GPU"},
        "eff_GBps": round(bytes_step / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(bytes_step / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "achieved": round(bytes_step / (call_ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(bytes_step / (call_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None},
        "kernel": {"name": "ecw_decode_kernel", "launches_per_step": launches, "avg_call_ms": round(call_ms, 5),
                   **{"event_bracketed_" + k.replace("launch_", "call_"): v for k, v in launch_pct(per_ms).items()},
                   "algorithmic_bytes_per_step": bytes_step, "src_sha": kernel_src_sha()},
    }
    return res


def calibrate_copy(nbytes=256 << 20):
    """A plain device copy of known size, for scaling HBM byte counters."""
    import torch

    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(3)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"calibration copy: {nbytes} bytes read + {nbytes} written per launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="tensor_4096",
                    choices=["tensor_4096", "tensor_2048", "tensor_2048_u8", "smollm_stack", "smollm_stack_u8",
                             "phi3_stack", "mistral_stack"])
    ap.add_argument("--replicas", type=int, default=0)
    ap.add_argument("--lanes", type=int, default=0)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--clip-sigma", type=float, default=0.0)
    ap.add_argument("--distinct-layers", type=int, default=2)
    ap.add_argument("--refill-steps", type=int, default=2, choices=[1, 2],
                    help="steps per refill decision of the encoded streams")
    ap.add_argument("--refill-ahead", type=int, default=1, choices=[0, 1],
                    help="encode the streams refilling ahead (same words, fetch order for early decoding)")
    ap.add_argument("--path", default="fused", choices=["fused", "ahead", "dense", "gemm"],
                    help="GEMV workloads: fused decode+GEMV, decode-ahead + stock linear, dense bf16, or "
                         "fused decode+GEMM over a prompt of --batch tokens")
    ap.add_argument("--ahead-depth", type=int, default=2, help="staging buffers of the decode-ahead path")
    ap.add_argument("--ahead-block", type=int, default=0,
                    help="weights per decode-ahead block (whole chunks; 0 = whole matrices)")
    ap.add_argument("--graph", action="store_true", help="GEMV workloads: replay each token as one HIP graph")
    ap.add_argument("--gemv-chunk", type=int, default=4096,
                    help="GEMV workloads: target chunk size in weights (rounded to whole rows)")
    ap.add_argument("--coder", default="huffman", choices=["huffman", "rans"],
                    help="tensor workloads: canonical Huffman (ECW v1) or interleaved rANS (ECR v1) streams")
    ap.add_argument("--single-latency", action="store_true",
                    help="tensor workloads: also time one call on a single tensor (median of 20, warm)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU only; --gpus must be 1"}))
        raise SystemExit(2)
    import torch

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs the GPU")
    import entropy_coded_weight_canonical_amd as ent

    ent.load()
    if args.calibrate_copy:
        calibrate_copy()
    coded = None
    if args.coder == "rans" and not args.workload.startswith("tensor_"):
        raise SystemExit("--coder rans applies to the single-tensor workloads")
    tensor_bench = bench_decode_rans if args.coder == "rans" else bench_decode
    if args.workload == "tensor_4096":
        res, coded = tensor_bench(args, "tensor_4096", 4, "unsigned", 8192, args.lanes or 32,
                                  args.replicas or 16, "bf16")
    elif args.workload in ("tensor_2048", "tensor_2048_u8"):
        res, coded = tensor_bench(args, "tensor_2048", 8, "asymmetric", 4096, args.lanes or 32,
                                  args.replicas or 64, "u8" if args.workload.endswith("u8") else "bf16")
    elif args.workload in ("phi3_stack", "mistral_stack"):
        res = bench_gemv(args, args.workload, args.batch, args.clip_sigma)
    elif args.workload in ("smollm_stack", "smollm_stack_u8"):
        res = bench_stack_decode(args, "smollm_stack", "u8" if args.workload.endswith("u8") else "bf16")
    else:
        raise SystemExit(f"unknown workload {args.workload}")
    res["gpu"] = torch.cuda.get_device_name(0)
    res["device"] = device_info(torch)
    copy = device_copy_gbps(torch)
    res["device_copy_GBps"] = round(copy, 1)
    ach = res.get("roofline", {}).get("achieved") or res.get("eff_GBps")
    if ach:
        res["frac_of_device_copy"] = round(float(ach) / copy, 4)
    if coded is not None and not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline_rans(coded) if args.coder == "rans" else cpu_baseline(coded)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
