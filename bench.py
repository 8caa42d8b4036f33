"""Benchmark of the hot path on one MI355X: decoded Gsym/s and effective HBM
GB/s for decoding, ms per token for the fused decode + GEMV.

Default run (``python bench.py``): the headline is the largest stated
workload, the Mistral-shaped stack (32 layers x {q, k, v, o, gate, up, down},
Student-t(4) weights) with unsigned 4-bit codes clipped so that the stream
takes 3.90 bits per weight, decoded and multiplied on the fly (fused decode +
dequant + GEMV) for one token at batch 1; ``value`` is ms per token.  The
same JSON line carries every other stated workload as a sub-record
(``configs``), each with its own roofline and CPU-oracle baseline:

* mistral_stack at batch 8;
* phi3_stack: fused decode + GEMV, batch 1;
* smollm_stack: 169 tensors, mixed 8-bit; decode all to bf16 in one call;
* tensor_2048: 2048 x 2048 N(0, 0.02), asymmetric 8-bit, 4096-code chunks;
  decode to bf16 and to u8, 64 replicas per call;
* tensor_4096: 4096 x 4096 Laplace(0, 0.015), unsigned 4-bit, 8192-code
  chunks of 32 lanes; decode + dequant to bf16, 16 replicas per call.

``--workload NAME`` runs one workload alone (the profiles under profiles/
are taken that way).  GEMV workloads also take ``--path ahead`` (each matrix
decoded to bf16 on a side stream just ahead of the stock linear kernel),
``--path dense`` (the stock kernel on resident bf16 weights), ``--path gemm``
(decode + GEMM on the matrix cores over a prompt of --batch tokens) and
``--graph`` (the token replayed as one HIP graph).  ``--coder rans`` runs the
single-tensor workloads on interleaved-rANS streams of the same codes.

Inputs are encoded by the library's own host encoder, not the oracle; every
workload is checked before timing (decoded codes bit-exact against the
encoder's input codes, bf16 bit-exact against torch's rounding of
scale * (q - zp), GEMV outputs within 1e-2 of a float64 product on those
weights).  The oracle is only timed, in the CPU-baseline leg.

Output: one JSON line.
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
# VALU roof: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (a wave64 instruction
# occupies a SIMD for 4 cycles)
VALU_PEAK_GLANE_OPS = 256 * 4 * 16 * 2.4
MAX_TENSORS_PER_LAUNCH = 32   # the library batches up to 32 tensors per kernel launch
METRIC = "decoded Gsym/s + effective HBM GB/s (% of peak); fused decode+GEMV ms/token"
KERNEL_SOURCES = ["entropy_coded_weight_canonical_amd/csrc/entro_decode.hip",
                  "entropy_coded_weight_canonical_amd/csrc/entro_device.h",
                  "entropy_coded_weight_canonical_amd/csrc/entro_internal.h"]

# The five workloads as stated, and the layout readings where the statement
# gives none (chunk C, lanes W: 64 wherever no lane count is stated, the
# faster layout on this GPU).  Every stream is encoded refilling ahead with a
# refill decision every two steps.  GEMV workloads use row-aligned chunks of
# about `chunk_target` weights.  The GPU parity tests run the same settings.
REFILL_STEPS = 2
REFILL_AHEAD = True
WORKLOADS = {
    "tensor_2048": {"config": 1, "bits": 8, "scheme": "asymmetric", "chunk": 4096, "lanes": 64, "replicas": 64},
    "tensor_4096": {"config": 2, "bits": 4, "scheme": "unsigned", "chunk": 8192, "lanes": 32, "replicas": 16},
    "smollm_stack": {"config": 3, "bits": 8, "scheme": "mixed", "chunk": 4096, "lanes": 64},
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


def read_profile(kind: str, name: str, config: str):
    """Fields of profiles/<kind>_<name>.txt (``key: value`` lines), or None if
    the kernel sources changed since it was taken or it was taken on another
    configuration."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{name}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.split("#", 1)[0].strip()
    if kv.get("kernel_src_sha") != kernel_src_sha() or kv.get("config") != config:
        return None
    return kv


def read_traffic(name: str, config: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, or None."""
    kv = read_profile("traffic", name, config)
    try:
        return None if kv is None else float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def traffic_config(chunk, lanes, args, replicas) -> str:
    """The configuration a decode traffic summary applies to (recorded in it)."""
    return f"C={chunk} W={lanes} refill_steps={args.refill_steps} ahead={int(args.refill_ahead)} replicas={replicas}"


# --------------------------------------------------------------------------
# inputs (library encoder)
# --------------------------------------------------------------------------

class Coded:
    def __init__(self, q, scale, zp, scheme, bits, max_len, chunk, lanes, rows, cols, refill_steps, ahead=False):
        import entropy_coded_weight_canonical_amd as ent

        self.q = np.ascontiguousarray(q, dtype=np.uint8).ravel()
        self.rows, self.cols = rows, cols
        self.bits, self.max_len, self.chunk, self.lanes = bits, max_len, chunk, lanes
        self.scale, self.zp, self.scheme = scale, zp, scheme
        self.refill_steps, self.ahead = refill_steps, bool(ahead)
        self.n = int(self.q.size)
        self.lengths = ent.code_lengths(self.q, bits, max_len)
        self.words, self.offs = ent.encode(self.q, self.lengths, bits, chunk, lanes, refill_steps=refill_steps,
                                           ahead=self.ahead)
        self.lut = ent.lut_build(self.lengths, bits, max_len, scale, zp)
        self.n_chunks = int(self.offs.size - 1)

    @property
    def in_bytes(self) -> int:
        return 4 * int(self.words.size) + 8 * (self.n_chunks + 1)

    @property
    def coded_bits_per_weight(self) -> float:
        return 8.0 * self.in_bytes / self.n

    def upload(self):
        import entropy_coded_weight_canonical_amd as ent

        return ent.DeviceTensor.upload(self.lut, self.words, self.offs, self.n, self.chunk, self.lanes, self.bits,
                                       self.max_len, refill_steps=self.refill_steps, ahead=self.ahead)


def code_tensor(spec, bits, scheme, chunk, lanes, refill_steps, clip_sigma=0.0, ahead=False):
    import entropy_coded_weight_canonical_amd as ent
    from synth import weights

    w = weights(spec)
    clip = float(clip_sigma * np.std(w, dtype=np.float64)) if clip_sigma else 0.0
    q, s, zp, chosen = ent.quantize(w, bits, scheme, clip=clip)
    return Coded(q, s, zp, chosen, bits, 16 if bits == 8 else 12, chunk, lanes, spec.rows, spec.cols, refill_steps,
                 ahead)


def stream_bits(coded) -> float:
    """Coded bits per weight of a set of tensors (weighted by their sizes)."""
    coded = list(coded)
    return 8.0 * sum(c.in_bytes for c in coded) / sum(c.n for c in coded)


# --------------------------------------------------------------------------
# checks before timing: the library's outputs against the encoder's input
# codes (torch does the reference arithmetic; no oracle involved)
# --------------------------------------------------------------------------

def torch_dequant(torch, q_dev, scale, zp):
    """bf16 bits of f32(scale) * f32(q - zp), rounded to nearest even (torch's
    float32 -> bfloat16 conversion), as int16."""
    v = (q_dev.to(torch.int32) - int(zp)).to(torch.float32) * torch.tensor(float(np.float32(scale)),
                                                                          dtype=torch.float32, device=q_dev.device)
    return v.to(torch.bfloat16).view(torch.int16)


def check_decoded(torch, coded, out, mode, what):
    """out (device) must equal coded.q (u8) or its bf16 dequantization."""
    q = torch.from_numpy(coded.q).cuda()
    exp = q if mode == "u8" else torch_dequant(torch, q, coded.scale, coded.zp)
    if not torch.equal(out[: coded.n], exp):
        raise SystemExit(f"check failed: {what} does not decode to its input codes ({mode})")


# --------------------------------------------------------------------------
# CPU baselines: the oracle, as it stands
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


def cpu_threads() -> int:
    return min(16, os.cpu_count() or 1)


def oracle_decode(coded, threads):
    from oracle import ccodec

    return ccodec.decode(coded.words, coded.offs, coded.lengths, coded.n, coded.chunk, coded.lanes, threads=threads,
                         refill_steps=coded.refill_steps, ahead=coded.ahead)


def cpu_baseline(coded: Coded, budget_s: float = 8.0, single_budget_s: float = 3.0, dequant: bool = True):
    """The oracle's C decoder over host threads (the chunk-parallel CPU decode
    of EntroLLM), plus numpy dequant; also one thread alone."""
    from oracle.dequant import dequant_bf16

    def rate(threads, budget):
        n_done, reps, t_dec = 0, 0, 0.0
        t0 = time.perf_counter()
        while True:
            ta = time.perf_counter()
            q = oracle_decode(coded, threads)
            t_dec += time.perf_counter() - ta
            if dequant:
                dequant_bf16(q, coded.scale, coded.zp)
            n_done += coded.n
            reps += 1
            if time.perf_counter() - t0 >= budget:
                break
        dt = time.perf_counter() - t0
        return n_done / dt / 1e9, n_done / t_dec / 1e9, reps, dt

    threads = cpu_threads()
    v, vd, reps, dt = rate(threads, budget_s)
    v1, vd1, reps1, dt1 = rate(1, single_budget_s)
    what = "bit-serial C decode" + (" + numpy bf16 dequant (one thread)" if dequant else "")
    return {"value": round(v, 4), "unit": "Gsym/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} x one {coded.rows}x{coded.cols} tensor ({coded.n} codes): {what}, decode "
                      f"over {threads} host threads, {dt:.1f} s wall",
            "decode_only_value": round(vd, 4),
            "single_thread_value": round(v1, 4), "single_thread_decode_only_value": round(vd1, 4),
            "single_thread_sample": f"{reps1} x the same tensor with the decode on 1 thread, {dt1:.1f} s wall",
            "nproc": os.cpu_count(), "cpu_model": cpu_model()}


def cpu_baseline_stack(sample, mode, n_total, budget_s: float = 8.0):
    """The oracle's C decode (over host threads) of a sample of a stack's
    tensors, plus numpy dequant for bf16; Gsym/s, and the stack's time at
    that rate."""
    from oracle.dequant import dequant_bf16

    threads = cpu_threads()
    n_done, reps = 0, 0
    t0 = time.perf_counter()
    while True:
        for c in sample:
            q = oracle_decode(c, threads)
            if mode == "bf16":
                dequant_bf16(q, c.scale, c.zp)
            n_done += c.n
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    rate = n_done / dt / 1e9
    return {"value": round(rate, 4), "unit": "Gsym/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} x {len(sample)} tensors of the stack ({sum(c.n for c in sample)} codes): bit-serial "
                      f"C decode over {threads} host threads" + (" + numpy bf16 dequant (one thread)"
                                                                  if mode == "bf16" else "") + f", {dt:.1f} s wall",
            "stack_seconds_at_this_rate": round(n_total / (rate * 1e9), 2),
            "nproc": os.cpu_count(), "cpu_model": cpu_model()}


def cpu_baseline_gemv(layer, batch, workload, layers, n_token):
    """The oracle on one layer of a GEMV stack: C decode over host threads,
    numpy bf16 dequant, numpy float64 product; ms per token extrapolated to
    the whole stack."""
    from oracle.dequant import dequant_bf16
    from oracle.gemv import gemv_f64
    from synth import activations_bf16

    threads = cpu_threads()
    t0 = time.perf_counter()
    t_dec = 0.0
    n = 0
    for i, (s, c) in enumerate(layer):
        x = activations_bf16(workload, i, s.cols, batch)
        ta = time.perf_counter()
        q = oracle_decode(c, threads)
        t_dec += time.perf_counter() - ta
        gemv_f64(dequant_bf16(q, c.scale, c.zp).reshape(s.rows, s.cols), x)
        n += c.n
    dt = time.perf_counter() - t0
    ms_token = dt * 1e3 * n_token / n
    return {"value": round(ms_token, 1), "unit": "ms/token", "cores": threads, "kind": "oracle",
            "sample": f"one layer ({len(layer)} matrices, {n} weights): bit-serial C decode over {threads} host "
                      f"threads, numpy bf16 dequant, numpy float64 GEMV at batch {batch} (numpy's BLAS threads), "
                      f"{dt:.1f} s wall, scaled to the {layers}-layer token",
            "decode_only_Gsym_per_s": round(n / t_dec / 1e9, 4),
            "nproc": os.cpu_count(), "cpu_model": cpu_model()}


# --------------------------------------------------------------------------
# GPU timing helpers
# --------------------------------------------------------------------------

def time_steps(step, steps, warmup):
    """Warm-up, then the timed region: `steps` steps back to back between two
    events on the launch stream, synchronized on both sides (-> total ms; its
    average per launch is what the roofline uses).  Then the same number of
    steps again, each between its own event pair, for the spread of single
    steps (p10/p50/p90): events between steps keep the next one from starting
    right behind the previous one, so they stay out of the timed region."""
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


def hbm_roofline(bytes_per_launch, launch_ms, traffic_bytes):
    ach = bytes_per_launch / (launch_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBPS, 4),
            "traffic": None if traffic_bytes is None else round(traffic_bytes / (launch_ms * 1e-3) / 1e9, 1)}


def record(value, unit, ms, args, higher, dtype, config, **extra):
    return {"metric": METRIC, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms, 5), "higher_is_better": higher, "scaling": "weak", "vs_baseline": None,
            "dtype": dtype, "data": "synthetic", "config": config, **extra}


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

def bench_decode(args, workload, mode, lanes=None, replicas=None):
    """One tensor, `replicas` distinct device copies decoded in one call."""
    import torch

    import entropy_coded_weight_canonical_amd as ent
    from synth import tensor_specs

    cfg = WORKLOADS[workload]
    bits, scheme, chunk = cfg["bits"], cfg["scheme"], cfg["chunk"]
    lanes = lanes or cfg["lanes"]
    replicas = replicas or cfg["replicas"]
    spec = tensor_specs(workload)[0]
    log(f"{workload}: encoding ({spec.rows}x{spec.cols}, {bits}-bit {scheme}, C={chunk}, W={lanes})")
    coded = code_tensor(spec, bits, scheme, chunk, lanes, args.refill_steps, ahead=args.refill_ahead)
    dts = [coded.upload() for _ in range(replicas)]
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
    check_decoded(torch, coded, outs[0], mode, f"{workload} replica 0")
    check_decoded(torch, coded, outs[-1], mode, f"{workload} replica {replicas - 1}")
    log(f"{workload}: {coded.coded_bits_per_weight:.3f} bits/weight, checked; timing {args.steps} steps")
    _keep = flush_mall(torch)
    total_ms, per_ms, wall = time_steps(step, args.steps, args.warmup)
    ms = total_ms / args.steps
    n_sym = coded.n * replicas
    out_b = coded.n * (1 if mode == "u8" else 2)
    bytes_step = replicas * (coded.in_bytes + out_b)
    launches = -(-replicas // MAX_TENSORS_PER_LAUNCH)
    launch_ms = ms / launches   # the timed region's average launch
    traffic = read_traffic(f"{workload}_{mode}", traffic_config(chunk, lanes, args, replicas))
    res = record(round(n_sym / (ms * 1e-3) / 1e9, 3), "Gsym/s", ms, args, True, "bf16" if mode == "bf16" else "u8",
                 {"workload": f"{workload}: {spec.rows}x{spec.cols} {scheme} {bits}-bit, C={chunk}, W={lanes}, "
                              f"refill every {args.refill_steps} step(s){', ahead' if coded.ahead else ''}, "
                              f"x{replicas} replicas, decode{'+dequant->bf16' if mode == 'bf16' else '->u8'}",
                  "stated_config": cfg["config"], "global_batch": replicas, "symbols_per_step": n_sym,
                  "coded_bits_per_weight": round(coded.coded_bits_per_weight, 4), "parallelism": "single GPU"},
                 eff_GBps=round(bytes_step / (ms * 1e-3) / 1e9, 1),
                 hbm_frac=round(bytes_step / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                 roofline=hbm_roofline(bytes_step / launches, launch_ms, traffic),
                 kernel={"name": "ecw_kernel", "launches_per_step": launches, "avg_launch_ms": round(launch_ms, 5),
                         **{"event_bracketed_" + k.replace("launch_", "step_"): v for k, v in launch_pct(per_ms).items()},
                         "algorithmic_bytes_per_launch": bytes_step // launches, "src_sha": kernel_src_sha()})
    if args.single_latency:   # extra launches of the same kernel: kept out of the default (profiled) run
        res["single_tensor_us"] = single_call_us(torch, lambda: fn(descs[:1], ptrs[:1], status.data_ptr()))
    if not args.no_cpu_baseline:
        log(f"{workload}: cpu baseline (oracle)")
        res["cpu_baseline"] = cpu_baseline(coded, dequant=(mode == "bf16"))
    return res, coded


def stack_key(s, n_distinct):
    return (s.layer % n_distinct, s.name.split(".", 1)[-1]) if s.layer >= 0 else ("x", s.name)


def bench_stack_decode(args, workload, mode):
    """Decode a whole stack in one call (all tensors, batched by the library
    into launches of up to 32 tensors)."""
    import torch

    import entropy_coded_weight_canonical_amd as ent
    from synth import tensor_specs

    cfg = WORKLOADS[workload]
    specs = tensor_specs(workload)
    layers = max(s.layer for s in specs) + 1
    n_distinct = min(args.distinct_layers, layers)
    lanes = args.lanes or cfg["lanes"]
    log(f"{workload}: encoding {n_distinct} distinct layer(s) of {layers} and the unlayered tensors")
    coded = {}
    for s in specs:
        key = stack_key(s, n_distinct)
        if key not in coded:
            coded[key] = code_tensor(s, cfg["bits"], cfg["scheme"], cfg["chunk"], lanes, args.refill_steps,
                                     ahead=args.refill_ahead)
    dts, outs, keys = [], [], []
    n_sym = 0
    bytes_step = 0
    odt = torch.uint8 if mode == "u8" else torch.int16
    for s in specs:
        c = coded[stack_key(s, n_distinct)]
        dts.append(c.upload())
        outs.append(torch.empty(c.n, dtype=odt, device="cuda"))
        keys.append(stack_key(s, n_distinct))
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
    seen = set()
    for key, o in zip(keys, outs):   # every distinct tensor once
        if key not in seen:
            check_decoded(torch, coded[key], o, mode, f"{workload} {key}")
            seen.add(key)
    bits = stream_bits(coded.values())
    log(f"{workload}: {bits:.3f} bits/weight, {len(seen)} distinct tensors checked; timing {args.steps} steps")
    _keep = flush_mall(torch)
    total_ms, per_ms, wall = time_steps(step, args.steps, args.warmup)
    ms = total_ms / args.steps
    launches = -(-len(specs) // MAX_TENSORS_PER_LAUNCH)   # one lane count in the stack
    res = record(round(n_sym / (ms * 1e-3) / 1e9, 3), "Gsym/s", ms, args, True, "bf16" if mode == "bf16" else "u8",
                 {"workload": f"{workload}: {len(specs)} tensors, {cfg['bits']}-bit {cfg['scheme']}, "
                              f"C={cfg['chunk']}, W={lanes}, refill every {args.refill_steps} step(s)"
                              f"{', ahead' if args.refill_ahead else ''}, decode all "
                              f"{'+dequant->bf16' if mode == 'bf16' else '->u8'} in one call",
                  "stated_config": cfg["config"], "global_batch": 1, "symbols_per_step": n_sym,
                  "distinct_layers": n_distinct, "coded_bits_per_weight": round(bits, 4),
                  "parallelism": "single GPU"},
                 eff_GBps=round(bytes_step / (ms * 1e-3) / 1e9, 1),
                 hbm_frac=round(bytes_step / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                 # the step's launches run back to back: their average is the step over the launch count
                 roofline=hbm_roofline(bytes_step / launches, ms / launches,
                                       read_traffic(f"{workload}_{mode}", f"W={lanes} launches={launches}")),
                 kernel={"name": "ecw_kernel", "launches_per_step": launches, "avg_launch_ms": round(ms / launches, 5),
                         **{"event_bracketed_" + k.replace("launch_", "step_"): v for k, v in launch_pct(per_ms).items()},
                         "algorithmic_bytes_per_launch": bytes_step // launches, "src_sha": kernel_src_sha()})
    if not args.no_cpu_baseline:
        log(f"{workload}: cpu baseline (oracle)")
        sample = [coded[k] for k in coded if k[0] == 0]
        res["cpu_baseline"] = cpu_baseline_stack(sample, mode, n_sym)
    return res


class GemvStack:
    """A GEMV stack on the device: every layer's matrices (distinct_layers of
    them encoded, the others device copies of those bytes at their own
    addresses), grouped by shared input as a transformer layer uses them."""

    def __init__(self, args, workload, clip_sigma):
        from synth import MISTRAL_CLIP_SIGMA, tensor_specs

        cfg = WORKLOADS[workload]
        if clip_sigma is None:
            clip_sigma = cfg.get("clip_sigma")
            if clip_sigma is None:
                clip_sigma = MISTRAL_CLIP_SIGMA
        self.workload, self.clip_sigma = workload, float(clip_sigma)
        self.scheme = "unsigned" if clip_sigma else "mixed"
        self.specs = tensor_specs(workload)
        self.layers = max(s.layer for s in self.specs) + 1
        self.n_distinct = min(args.distinct_layers, self.layers)
        self.chunk_target = args.gemv_chunk or cfg["chunk_target"]
        log(f"{workload}: encoding {self.n_distinct} distinct layer(s) of {self.layers}")
        self.coded_layers = []
        for L in range(self.n_distinct):
            self.coded_layers.append([(s, code_tensor(s, 4, self.scheme, gemv_chunk(s.cols, self.chunk_target),
                                                      cfg["lanes"], args.refill_steps, self.clip_sigma,
                                                      ahead=args.refill_ahead))
                                      for s in self.specs if s.layer == L])
        self.bits = stream_bits(c for row in self.coded_layers for _, c in row)
        self.mats = []     # per layer: list of (group, [(spec, coded, DeviceTensor)])
        for L in range(self.layers):
            by_group = {}
            for s, c in self.coded_layers[L % self.n_distinct]:
                by_group.setdefault(s.group, []).append((s, c, c.upload()))
            self.mats.append(list(by_group.items()))
        self.n_sym = sum(c.n for L in range(self.layers) for _, c in self.coded_layers[L % self.n_distinct])
        self.in_bytes = sum(c.in_bytes for L in range(self.layers) for _, c in self.coded_layers[L % self.n_distinct])

    def describe(self):
        q = (f"unsigned 4-bit clip {self.clip_sigma:.4f} sigma" if self.clip_sigma else "mixed 4-bit (min-max)")
        return f"{self.workload}: {len(self.specs)} matrices, {q}, {self.bits:.3f} bits/weight"


def check_gemv(torch, stack, groups, batch, tol=1e-2):
    """The first layer of each distinct layer: the codes through the
    standalone decode, and the fused outputs against a float64 product on
    bf16 weights that torch dequantizes from the input codes."""
    import entropy_coded_weight_canonical_amd as ent

    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    worst = 0.0
    gi = 0
    for L in range(stack.n_distinct):
        for gname, members in stack.mats[L]:
            x, ys = groups[gi][2], groups[gi][3]
            gi += 1
            xf = x.view(torch.bfloat16).double().view(batch, -1)
            for (s, c, dt), y in zip(members, ys):
                qd = torch.from_numpy(c.q).cuda()
                out = torch.empty(c.n, dtype=torch.uint8, device="cuda")
                ent.decode([dt.desc], [out.data_ptr()], st.data_ptr())
                torch.cuda.synchronize()
                if int(st.item()) or not torch.equal(out, qd):
                    raise SystemExit(f"check failed: {s.name} does not decode to its input codes")
                w = torch_dequant(torch, qd, c.scale, c.zp).view(torch.bfloat16).view(s.rows, s.cols).double()
                ref = xf @ w.t()
                den = torch.maximum(ref.abs(), 1e-3 * ref.abs().amax(dim=1, keepdim=True))
                err = float(((y.double() - ref).abs() / den).max().item())
                worst = max(worst, err)
                del w, ref, den
                if err > tol:
                    raise SystemExit(f"check failed: {s.name} GEMV error {err:.3g} > {tol}")
    return worst


def gemv_roofline(key, config, sym_per_s, bytes_per_token, ms):
    """VALU roof (lane-ops per symbol from the committed counter summary of
    the same kernel sources and configuration) and the HBM fraction."""
    kv = read_profile("counters", key, config)
    ops = float(kv["valu_lane_ops_per_symbol"]) if kv and "valu_lane_ops_per_symbol" in kv else None
    tr = read_profile("traffic", key, config)
    traffic = float(tr["hbm_bytes_per_token"]) if tr and "hbm_bytes_per_token" in tr else None
    hbm = bytes_per_token / (ms * 1e-3) / 1e9
    ach = None if ops is None else sym_per_s / 1e9 * ops
    return {"bound": "alu", "achieved": None if ach is None else round(ach, 1), "peak": round(VALU_PEAK_GLANE_OPS, 1),
            "unit": "Glane-op/s", "frac": None if ach is None else round(ach / VALU_PEAK_GLANE_OPS, 4),
            "traffic": None if traffic is None else round(traffic / (ms * 1e-3) / 1e9, 1),
            "valu_lane_ops_per_symbol": ops,
            "peak_derivation": "256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz (a wave64 VALU instruction takes 4 cycles)",
            "hbm": {"achieved": round(hbm, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(hbm / HBM_PEAK_GBPS, 4)}}


def bench_gemv(args, workload, batch, path="fused", stack=None):
    """Per-token fused decode+GEMV over the whole stack, one call per group of
    matrices sharing an input (q/k/v, o, gate/up, down) per layer."""
    import torch

    import entropy_coded_weight_canonical_amd as ent
    from synth import activations_bf16

    cfg = WORKLOADS[workload]
    stack = stack or GemvStack(args, workload, args.clip_sigma)
    status = torch.zeros(64, dtype=torch.int32, device="cuda")
    groups = []   # (layer, group, x, [y], [desc], [item])
    for L in range(stack.layers):
        for gname, members in stack.mats[L]:
            cols = members[0][0].cols
            x = torch.from_numpy(activations_bf16(workload, len(groups), cols, batch).view(np.int16)).cuda()
            ys = [torch.empty((batch, s.rows), dtype=torch.float32, device="cuda") for s, _, _ in members]
            items = [ent.GemvItem(s.rows, s.cols, x.data_ptr(), y.data_ptr()) for (s, _, _), y in zip(members, ys)]
            groups.append((L, gname, x, ys, [dt.desc for _, _, dt in members], items))
    hbm_bytes = stack.in_bytes + sum(2 * batch * s.cols + 4 * batch * s.rows
                                     for L in range(stack.layers) for _, m in stack.mats[L] for s, _, _ in m)
    launches = len(groups)
    if path == "fused":
        calls = [ent.GemvCall(g[4], g[5], batch, status.data_ptr()) for g in groups]

        def step():
            for c in calls:
                c()

        def flags():
            return status
    elif path == "gemm":
        def step():
            for g in groups:
                ent.decode_gemm(g[4], g[5], batch, status.data_ptr())

        def flags():
            return status
    elif path == "ahead":
        from entropy_coded_weight_canonical_amd.ahead import DecodeAhead

        mats = [(dt, s.rows, s.cols, g[2]) for g in groups for (s, _, dt) in dict(stack.mats[g[0]])[g[1]]]
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
        import torch.nn.functional as F

        dense = []
        for g in groups:
            for (s, _, dt) in dict(stack.mats[g[0]])[g[1]]:
                wbuf = torch.empty((s.rows, s.cols), dtype=torch.bfloat16, device="cuda")
                ent.decode_dequant([dt.desc], [wbuf.data_ptr()], status.data_ptr())
                dense.append((wbuf, g[2].view(torch.bfloat16).view(batch, -1)))
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
    err = check_gemv(torch, stack, groups, batch) if path in ("fused", "gemm") else None
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
    log(f"{stack.describe()}; checked (worst GEMV error {err}); timing {args.steps} steps at batch {batch}")
    _keep = flush_mall(torch)
    total_ms, per_ms, wall = time_steps(step, args.steps, args.warmup)
    ms = total_ms / args.steps
    per_token = ms / batch if path == "gemm" else ms
    sym_per_s = stack.n_sym / (ms * 1e-3)
    key = f"{workload}_gemv_b{batch}"
    prof_config = f"{stack.scheme} clip={stack.clip_sigma:.4f} chunk_target={stack.chunk_target} W=64 " \
                  f"refill_steps={args.refill_steps} ahead={int(args.refill_ahead)} batch={batch} path={path}"
    res = record(round(per_token, 4), "ms/token", ms, args, False, "bf16",
                 {"workload": f"{stack.describe()}, row-aligned chunks of about {stack.chunk_target} weights, W=64, "
                              f"refill every {args.refill_steps} step(s){', ahead' if args.refill_ahead else ''}; " + {
                                  "fused": f"fused decode+dequant+GEMV batch {batch}",
                                  "ahead": f"decode-ahead to bf16 (depth {args.ahead_depth}, blocks of "
                                           f"{args.ahead_block or 'whole'} weights) + stock matmul, batch {batch}",
                                  "dense": f"dense bf16 weights (decoded once) + stock linear kernel, batch {batch}",
                                  "gemm": f"fused decode+dequant+GEMM (MFMA) over a {batch}-token prompt, "
                                          f"value per token"}[path],
                  "stated_config": cfg["config"], "path": path, "hip_graph": bool(args.graph),
                  "global_batch": batch, "symbols_per_token": stack.n_sym, "launch_groups": launches,
                  "distinct_layers": stack.n_distinct, "coded_bits_per_weight": round(stack.bits, 4),
                  "parallelism": "single GPU"},
                 decoded_Gsym_per_s=round(sym_per_s / 1e9, 3),
                 matmul_TFLOPs=round(2.0 * batch * stack.n_sym / (ms * 1e-3) / 1e12, 2),
                 hbm_bytes_per_token=int(hbm_bytes),
                 eff_GBps=round(hbm_bytes / (ms * 1e-3) / 1e9, 1),
                 hbm_frac=round(hbm_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                 step_ms_pct={k.replace("launch_", "step_"): v for k, v in launch_pct(per_ms).items()})
    if path == "fused":
        res["roofline"] = gemv_roofline(key, prof_config, sym_per_s, hbm_bytes, ms)
        res["kernel"] = {"name": "ecw_gemv_stream_kernel", "launches_per_step": launches,
                         "avg_launch_ms": round(ms / launches, 5),
                         "algorithmic_bytes_per_launch": int(hbm_bytes // launches), "src_sha": kernel_src_sha(),
                         "profile_config": prof_config}
        res["check_max_rel_err"] = err
    if not args.no_cpu_baseline and path == "fused":
        log(f"{workload}: cpu baseline (oracle), batch {batch}")
        res["cpu_baseline"] = cpu_baseline_gemv(stack.coded_layers[0], batch, workload, stack.layers, stack.n_sym)
    return res, stack


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="default",
                    choices=["default", "tensor_4096", "tensor_2048", "tensor_2048_u8", "smollm_stack",
                             "smollm_stack_u8", "phi3_stack", "mistral_stack"],
                    help="default: the Mistral-shaped stack at batch 1 with every other workload as a sub-record")
    ap.add_argument("--no-sub", action="store_true", help="default run: the headline only")
    ap.add_argument("--replicas", type=int, default=0)
    ap.add_argument("--lanes", type=int, default=0)
    ap.add_argument("--batch", type=int, default=1)
    ap.add_argument("--clip-sigma", type=float, default=None,
                    help="GEMV workloads: clip factor of the unsigned 4-bit codes (0: min-max mixed codes; "
                         "default: the workload's own)")
    ap.add_argument("--distinct-layers", type=int, default=2)
    ap.add_argument("--refill-steps", type=int, default=REFILL_STEPS, choices=[1, 2],
                    help="steps per refill decision of the encoded streams")
    ap.add_argument("--refill-ahead", type=int, default=int(REFILL_AHEAD), choices=[0, 1],
                    help="encode the streams refilling ahead (same words, fetch order for early decoding)")
    ap.add_argument("--path", default="fused", choices=["fused", "ahead", "dense", "gemm"],
                    help="GEMV workloads: fused decode+GEMV, decode-ahead + stock linear, dense bf16, or "
                         "fused decode+GEMM over a prompt of --batch tokens")
    ap.add_argument("--ahead-depth", type=int, default=2, help="staging buffers of the decode-ahead path")
    ap.add_argument("--ahead-block", type=int, default=0,
                    help="weights per decode-ahead block (whole chunks; 0 = whole matrices)")
    ap.add_argument("--graph", action="store_true", help="GEMV workloads: replay each token as one HIP graph")
    ap.add_argument("--gemv-chunk", type=int, default=0,
                    help="GEMV workloads: target chunk size in weights, rounded to whole rows (0: the workload's)")
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
    if args.coder == "rans" and not args.workload.startswith("tensor_"):
        raise SystemExit("--coder rans applies to the single-tensor workloads")
    w = args.workload
    if w == "default":
        res, stack = bench_gemv(args, "mistral_stack", 1)
        if not args.no_sub:
            subs = [bench_gemv(args, "mistral_stack", 8, stack=stack)[0]]
            del stack
            import gc

            gc.collect()
            torch.cuda.empty_cache()
            subs.append(bench_gemv(args, "phi3_stack", 1)[0])
            gc.collect()
            torch.cuda.empty_cache()
            subs.append(bench_stack_decode(args, "smollm_stack", "bf16"))
            gc.collect()
            torch.cuda.empty_cache()
            subs.append(bench_decode(args, "tensor_2048", "bf16", args.lanes or None)[0])
            subs.append(bench_decode(args, "tensor_2048", "u8", args.lanes or None)[0])
            subs.append(bench_decode(args, "tensor_4096", "bf16", args.lanes or None)[0])
            res["configs"] = subs
    elif w in ("tensor_4096", "tensor_2048", "tensor_2048_u8"):
        base = w.replace("_u8", "")
        mode = "u8" if w.endswith("u8") else "bf16"
        cfg = WORKLOADS[base]
        if args.coder == "rans":
            res, _ = bench_decode_rans(args, base, cfg["bits"], cfg["scheme"], cfg["chunk"], args.lanes or cfg["lanes"],
                                       args.replicas or cfg["replicas"], mode)
        else:
            res, _ = bench_decode(args, base, mode, args.lanes or None, args.replicas or None)
    elif w in ("phi3_stack", "mistral_stack"):
        res, _ = bench_gemv(args, w, args.batch, args.path)
    else:
        res = bench_stack_decode(args, "smollm_stack", "u8" if w.endswith("u8") else "bf16")
    res["gpu"] = torch.cuda.get_device_name(0)
    res["device"] = device_info(torch)
    copy = device_copy_gbps(torch)
    res["device_copy_GBps"] = round(copy, 1)
    ach = res.get("roofline", {}).get("achieved") if res.get("roofline", {}).get("unit") == "GB/s" else None
    if ach:
        res["frac_of_device_copy"] = round(float(ach) / copy, 4)
    print(json.dumps(res), flush=True)


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


if __name__ == "__main__":
    main()
