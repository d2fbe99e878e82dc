#!/usr/bin/env python3
"""Benchmark of the k-quant prefill MMQ hot path on one MI355X.

One step = one pass of the hot path over one batch of synthetic input at the
q-projection shape (od = id = 3584, nt = 512): one q4_K and one q6_K GEMM,
each after the quantization of its own activations into the tiled plane:
    quantize_q8_tiled(x4) -> mmq_q4k_staged_q8t (W4 as a staged buffer)
    quantize_q8_tiled(x6) -> mmq_q6k_limbs_q8t (W6 as a limb buffer)
Inputs are resident in HBM before timing.  Registration-time forms of the
weights (the staged and limb buffers, the dense plane, the prepared
buffers) are built once beforehand and timed separately.  Every other arm --
both types on raw blocks, q6_K on the dense plane (the paths the workloads
name), the prepared buffers, and the pad40 activation plane -- is timed per
kernel after the step.

Before the W warmup steps the step runs back to back for --spinup-s seconds
(untimed), so that a short --warmup does not time a GPU that is still ramping
its clock; the shader clock under the step's load is then measured with a
one-wave cycle-count spin on a second stream.

Prints one JSON line: value = int8 TOPS of the whole step (2 GEMMs x
2*nt*od*id ops / step time), the per-kernel average durations from HIP
events recorded on the launch stream (K launches queued back to back
behind a spin kernel, so that a kernel shorter than the host's launch time
is still timed on the GPU), per-launch medians and minima over --launches
launches each, warm and cold (a 512 MiB write before each launch), a roofline entry for the dominant kernel against
the int8 MFMA peak (also at the measured clock) and against HBM, and the CPU
oracle timed on the host cores.

``--summarize-profiles DIR`` writes the profiles/ summaries from rocprofv3
outputs instead (see summarize_profiles).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MMQ int8 TOPS + µs/GEMM, q4_K & q6_K 3584×3584×nt512; % of int8 MFMA peak"
PEAK_INT8_TOPS = 5000.0       # MI355X dense int8 MFMA, published
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E, published
NT, OD, ID = 512, 3584, 3584
SEED4, SEED6 = 20261, 20262   # seed base + workload index


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    # about 40 ms of steps: a shorter warmup leaves the GPU below its steady
    # clocks and measured up to ~10% slow, depending on what ran first
    p.add_argument("--warmup", type=int, default=300)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--workload", choices=["proj", "ffn", "layer", "layer_q6v", "down", "kv"], default="proj",
                   help="proj: the q4_K and q6_K 3584x3584 nt=512 GEMMs (the headline); ffn: the 7B-class "
                        "FFN GEMMs at nt=512; layer: all seven GEMMs of a 7B-class layer at nt=2630; down: "
                        "the layer's q6_K down projection alone (3584x18944, nt=2630); kv: the layer's k and v "
                        "projections; layer_q6v: the layer with a q6_K v projection")
    p.add_argument("--activations", choices=["tiled", "pad40"], default="tiled",
                   help="ffn / layer workloads: activation plane of the timed step")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 256 MiB device copy 3x (outside the timed region) so that "
                        "HBM counters taken over this run can be scaled by a kernel of known traffic")
    p.add_argument("--spinup-s", type=float, default=0.3,
                   help="seconds of back-to-back steps before the warmup steps, so that the GPU is at its "
                        "steady clock whatever --warmup is")
    p.add_argument("--launches", type=int, default=100,
                   help="launches per kernel for the per-launch medians (warm, and cold after a 512 MiB write)")
    p.add_argument("--summarize-profiles", metavar="DIR",
                   help="instead of benchmarking: turn the rocprofv3 outputs under DIR (trace/, and for proj and "
                        "down fetch/, write/, sqA/, sqB/) of the --workload run into the summaries under profiles/")
    return p.parse_args()


KERNEL_SOURCES = ("mmq.hip", "qig_device.h", "qig_launch.h", "qig_quant.h")


def kernel_source_digest() -> str:
    """sha256 of the GEMM kernel's code (mmq.hip and the headers it includes,
    comments and blank space removed): HBM-traffic figures recorded from
    counters are only reported while the code they were taken on is unchanged."""
    import hashlib
    import re
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "quant_integer_gemm_amd", "csrc", name)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        src = "\n".join(" ".join(line.split()) for line in src.splitlines() if line.strip())
        h.update(name.encode() + b"\0" + src.encode() + b"\0")
    return h.hexdigest()


def recorded_counter(kernel: str, field: str = "bytes_per_launch"):
    """A per-launch figure of `kernel` from the counter summary kept under
    profiles/: HBM bytes (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy) or
    VALU instructions (SQ_INSTS_VALU - SQ_INSTS_MFMA, wave instructions), or
    None when there is none or the kernel source changed since it was
    taken."""
    path = os.path.join(ROOT, "profiles", "mmq_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_code_sha256") != kernel_source_digest():
        return None
    v = rec.get(field, {}).get(kernel)
    return None if v is None else int(v)


def recorded_traffic(kernel: str):
    return recorded_counter(kernel, "bytes_per_launch")


# fp32 VALU rate of MI355X: 256 CUs x 4 SIMDs x 32 lanes per clock at
# 2.4 GHz, in lane operations (one fma per lane) per second, 10^12: the
# published 157.3 TFLOP/s.  Probe kernels on the device reach it with the
# unpacked VOP3 v_fma_f32 (about 2 cycles per wave instruction per SIMD) once
# 4 waves share a SIMD.  A wave issues at most one instruction per 4 cycles,
# so at 2 waves per SIMD, the occupancy of these kernels, independent fmas
# reach 2.7 cycles per wave instruction: VALU_CEIL_2W of the peak.
PEAK_VALU_TLANEOPS = 256 * 4 * 32 * 2.4e9 / 1e12
VALU_CEIL_2W = 0.74


def valu_roofline(kernel, us, clock_mhz):
    """The kernel against the VALU rate, the bound of its epilogue: VALU wave
    instructions per launch (recorded counters) x 64 lanes over its average
    duration, against PEAK_VALU_TLANEOPS, against the ceiling at 2 waves per
    SIMD, and against the peak at the measured clock.  None without recorded
    counters for the current code."""
    n = recorded_counter(kernel, "valu_insts_per_launch")
    if n is None:
        return None
    achieved = n * 64 / (us * 1e-6) / 1e12
    out = {"insts_per_launch": n, "achieved": round(achieved, 2), "peak": PEAK_VALU_TLANEOPS,
           "unit": "T lane-op/s", "frac": round(achieved / PEAK_VALU_TLANEOPS, 4),
           "frac_of_2wave_ceiling": round(achieved / (VALU_CEIL_2W * PEAK_VALU_TLANEOPS), 4)}
    if clock_mhz:
        out["frac_at_clock"] = round(achieved / (PEAK_VALU_TLANEOPS * clock_mhz / 2400.0), 4)
    return out


def smi_clock_mhz():
    """Graphics clock of GPU 0 in MHz as the SMI library reports it, or None."""
    try:
        import torch
        mhz = torch.cuda.clock_rate(0)
        return int(mhz) if mhz else None
    except Exception:
        return None


def shader_clock_mhz(step, busy_steps):
    """Shader clock under load: while `busy_steps` steps run on the current
    stream, a one-wave kernel on a second stream spins for a fixed count of
    shader-clock cycles (s_memtime); its duration between HIP events gives
    the clock the GPU ran at meanwhile.  Median of three."""
    import torch
    side = torch.cuda.Stream()
    cycles = 1 << 21
    out = []
    for _ in range(3):
        for _ in range(busy_steps):
            step()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(side):
            e0.record()
            torch.cuda._sleep(cycles)
            e1.record()
        torch.cuda.synchronize()
        out.append(cycles / (e0.elapsed_time(e1) * 1e3))
    out.sort()
    return round(out[1])


def spin_up(step, seconds):
    """Run `step` back to back for `seconds` of wall time (untimed), so that
    the timed steps do not start on a GPU still ramping its clock.  Returns
    the number of steps run and the clocks: the shader clock measured under
    the step's load, and the SMI's reading taken with steps queued."""
    import torch
    t_end = time.perf_counter() + seconds
    n, burst, smi = 0, 20, []
    while time.perf_counter() < t_end:
        t0 = time.perf_counter()
        for _ in range(burst):
            step()
        n += burst
        mhz = smi_clock_mhz()
        if mhz:
            smi.append(mhz)
        torch.cuda.synchronize()
        if time.perf_counter() - t0 < 0.02 and burst < 640:
            burst *= 2   # keep about 20 ms of work queued per burst
    smi.sort()
    return n, {"shader_mhz": shader_clock_mhz(step, burst),
               "smi_mhz": smi[len(smi) // 2] if smi else None}


def queue_ahead(host_seconds):
    """Occupy the launch stream for about 1.5x `host_seconds` with a spin
    kernel, so that launches the host queues meanwhile run back to back once
    it ends: HIP events around them then time the GPU, not the host's launch
    rate (a short kernel finishes before the host has queued the next)."""
    import torch
    torch.cuda._sleep(int(1.5 * host_seconds * 2.6e9) + (1 << 16))


def gpu_avg_us(fn, n):
    """Average duration of fn over n launches queued back to back behind a
    spin kernel, between one pair of HIP events on the launch stream."""
    import torch
    fn()
    torch.cuda.synchronize()
    t = time.perf_counter()
    for _ in range(n):
        fn()
    host = time.perf_counter() - t
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    queue_ahead(host)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / n


def per_launch_us(fn, n, flush=None):
    """Median and minimum of n launches of fn, each between its own pair of
    HIP events on the launch stream, all queued behind a spin kernel; with
    `flush`, a write of 512 MiB (which evicts the L2s and the 256 MB Infinity
    Cache) runs before each launch, outside its events."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]

    def batch():
        for k, (e0, e1) in enumerate(evs):
            if flush is not None:
                flush(k)
            e0.record()
            fn()
            e1.record()
    torch.cuda.synchronize()
    t = time.perf_counter()
    batch()
    host = time.perf_counter() - t
    torch.cuda.synchronize()
    queue_ahead(host)
    batch()
    torch.cuda.synchronize()
    ts = sorted(e0.elapsed_time(e1) * 1e3 for e0, e1 in evs)
    return {"median": round(ts[len(ts) // 2], 3), "min": round(ts[0], 3)}


def oracle_single_thread(W4, x4, W6, x6, sample_tokens=128):
    """The oracle on one thread: workload 0 in full, and the q4_K / q6_K
    projection GEMMs (workloads 1 and 2) on their first `sample_tokens`
    tokens, scaled to all 512."""
    import oracle
    from quant_integer_gemm_amd import inputs
    g0 = inputs.WORKLOADS[0][0]
    W0, x0 = inputs.make_gemm_inputs(g0, inputs.SEED_BASE)
    oracle.set_num_threads(1)
    try:
        t = time.perf_counter()
        q80 = oracle.quantize_q8_pad40(x0)
        oracle.mmq_q6k(W0, 224, g0.od, g0.id, q80, g0.nt)
        c0 = time.perf_counter() - t
        k = sample_tokens
        t = time.perf_counter()
        oracle.mmq_q4k(W4, OD, ID, oracle.quantize_q8_pad40(np.ascontiguousarray(x4[:k])), k)
        c1 = (time.perf_counter() - t) * NT / k
        t = time.perf_counter()
        oracle.mmq_q6k(W6, 224, OD, ID, oracle.quantize_q8_pad40(np.ascontiguousarray(x6[:k])), k)
        c2 = (time.perf_counter() - t) * NT / k
    finally:
        oracle.set_num_threads(0)
    return {"threads": 1, "workload0_ms": round(c0 * 1e3, 2),
            "q4k_3584x3584_nt512_ms": round(c1 * 1e3, 1), "q6k_3584x3584_nt512_ms": round(c2 * 1e3, 1),
            "sample": f"workload 0 in full; the nt=512 GEMMs (quantization included) on their first {k} "
                      f"tokens, scaled to 512"}


def cpu_baseline(W4, x4, W6, x6):
    """The oracle as it stands, on the host cores: the step's arithmetic (both
    quantizations, the q4_K and the q6_K GEMM), repeated until ~10 s; also the
    mean time of each part, and single-thread times."""
    import oracle
    ops = 2 * 2.0 * NT * OD * ID
    reps, total = 0, 0.0
    parts = {"quantize_x4": 0.0, "mmq_q4k": 0.0, "quantize_x6": 0.0, "mmq_q6k": 0.0}
    while total < 10.0 and reps < 200:
        t = [time.perf_counter()]
        q84 = oracle.quantize_q8_pad40(x4)
        t.append(time.perf_counter())
        oracle.mmq_q4k(W4, OD, ID, q84, NT)
        t.append(time.perf_counter())
        q86 = oracle.quantize_q8_pad40(x6)
        t.append(time.perf_counter())
        oracle.mmq_q6k(W6, 224, OD, ID, q86, NT)
        t.append(time.perf_counter())
        for k, name in enumerate(parts):
            parts[name] += t[k + 1] - t[k]
        total += t[-1] - t[0]
        reps += 1
    return {
        "value": round(ops * reps / total / 1e12, 4),
        "unit": "TOPS",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"the full step (2 quantizations, the q4_K and q6_K GEMMs, nt={NT}, od=id={ID}) "
                  f"repeated {reps}x in {total:.1f} s",
        "parts_ms": {k: round(v / reps * 1e3, 1) for k, v in parts.items()},
        "single_thread": oracle_single_thread(W4, x4, W6, x6),
    }


# GEMM sets of the FFN and layer workloads: (GEMM name, quant type, od, id, the
# input it reads).  GEMMs that read the same input share one quantization.
GEMM_SETS = {
    "ffn": {"nt": 512, "xscale": 2.0, "gemms": [
        ("ffn_gate", "q4_K", 18944, 3584, "x_ffn"), ("ffn_up", "q4_K", 18944, 3584, "x_ffn"),
        ("ffn_down", "q6_K", 3584, 18944, "x_down")]},
    "layer": {"nt": 2630, "xscale": 1.0, "gemms": [
        ("attn_q", "q4_K", 3584, 3584, "x_attn"), ("attn_k", "q4_K", 512, 3584, "x_attn"),
        ("attn_v", "q4_K", 512, 3584, "x_attn"), ("attn_o", "q4_K", 3584, 3584, "x_o"),
        ("ffn_gate", "q4_K", 18944, 3584, "x_ffn"), ("ffn_up", "q4_K", 18944, 3584, "x_ffn"),
        ("ffn_down", "q6_K", 3584, 18944, "x_down")]},
    "down": {"nt": 2630, "xscale": 1.0, "gemms": [("ffn_down", "q6_K", 3584, 18944, "x_down")]},
    # the layer with its v projection stored as q6_K, as the pages' model keeps it in some layers
    "layer_q6v": {"nt": 2630, "xscale": 1.0, "gemms": [
        ("attn_q", "q4_K", 3584, 3584, "x_attn"), ("attn_k", "q4_K", 512, 3584, "x_attn"),
        ("attn_v", "q6_K", 512, 3584, "x_attn"), ("attn_o", "q4_K", 3584, 3584, "x_o"),
        ("ffn_gate", "q4_K", 18944, 3584, "x_ffn"), ("ffn_up", "q4_K", 18944, 3584, "x_ffn"),
        ("ffn_down", "q6_K", 3584, 18944, "x_down")]},
    "kv": {"nt": 2630, "xscale": 1.0, "gemms": [
        ("attn_k", "q4_K", 512, 3584, "x_attn"), ("attn_v", "q4_K", 512, 3584, "x_attn")]},
}


def run_gemm_set(args):
    """The FFN, layer, down or k/v workload: one quantization per distinct
    input (tiled plane, or pad40), then its GEMMs: with the tiled plane q4_K
    on the staged buffer and q6_K on the limb buffer, with pad40 both on raw
    blocks; the stream-K workspace is passed to every GEMM and used where the
    tile count calls for it.  With the tiled plane each GEMM is also timed,
    outside the step, on raw blocks (q6_K also on the dense plane; q4_K also
    quantizing its own activations)."""
    import torch
    import quant_integer_gemm_amd as qig
    from quant_integer_gemm_amd import inputs
    spec = GEMM_SETS[args.workload]
    nt = spec["nt"]
    dev = torch.device("cuda:0")
    tiled = args.activations == "tiled"
    ws = qig.new_workspace(dev)
    xs, qs, Ws, ys, host, limbs, wexps, staged = {}, {}, {}, {}, {}, {}, {}, {}
    registration_us = {}
    for i, (name, qt, od, id_, xin) in enumerate(spec["gemms"]):
        W, x = inputs.make_gemm_inputs(inputs.Gemm(name, qt, od, id_, nt, spec["xscale"]),
                                       inputs.SEED_BASE + 500 + i)
        Ws[name] = torch.from_numpy(W).to(dev)
        host[name] = W
        if qt == "q4_K" and tiled:
            staged[name] = torch.empty(qig.q4k_staged_bytes(od, id_), dtype=torch.uint8, device=dev)
            torch.cuda.synchronize()
            t = time.perf_counter()
            qig.prepare_q4k_staged(Ws[name], od, id_, out=staged[name])
            torch.cuda.synchronize()
            registration_us["prepare_q4k_staged:" + name] = round((time.perf_counter() - t) * 1e6, 1)
        if qt == "q6_K" and tiled:
            limbs[name] = torch.empty(qig.q6k_limbs_bytes(od, id_), dtype=torch.uint8, device=dev)
            wexps[name] = torch.empty((od, id_), dtype=torch.int8, device=dev)
            torch.cuda.synchronize()
            t = time.perf_counter()
            qig.prepare_q6k_limbs(Ws[name], 224, od, id_, out=limbs[name])
            torch.cuda.synchronize()
            registration_us["prepare_q6k_limbs:" + name] = round((time.perf_counter() - t) * 1e6, 1)
            qig.expand_q6k_dense(Ws[name], 224, od, id_, out=wexps[name])
        if xin not in xs:
            xs[xin] = torch.from_numpy(x).to(dev)
            host[xin] = x
            nbytes = qig.q8_tiled_bytes(nt, id_) if tiled else qig.q8_pad40_bytes(nt, id_)
            qs[xin] = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        ys[name] = torch.empty((nt, od), dtype=torch.float32, device=dev)

    def quant(xin):
        if tiled:
            return lambda: qig.quantize_q8_tiled(xs[xin], out=qs[xin])
        return lambda: qig.quantize_q8_pad40(xs[xin], out=qs[xin])

    def gemm(name, qt, od, id_, xin, arm="registered"):
        W, q8, y = Ws[name], qs[xin], ys[name]
        if qt == "q4_K":
            if tiled and arm == "raw":
                return lambda: qig.mmq_q4k_q8t(W, od, id_, q8, nt, y=y, ldy=od, ws=ws)
            if tiled:
                Wst = staged[name]
                return lambda: qig.mmq_q4k_staged_q8t(Wst, od, id_, q8, nt, y=y, ldy=od, ws=ws)
            return lambda: qig.mmq_q4k_streamk(W, od, id_, q8, nt, y=y, ldy=od, ws=ws)
        if not tiled:
            return lambda: qig.mmq_q6k_streamk(W, 224, od, id_, q8, nt, y=y, ldy=od, ws=ws)
        if arm == "registered":
            Wl = limbs[name]
            return lambda: qig.mmq_q6k_limbs_q8t(Wl, od, id_, q8, nt, y=y, ldy=od, ws=ws)
        if arm == "wexp":
            We = wexps[name]
            return lambda: qig.mmq_q6k_q8t(W, 224, od, id_, q8, nt, W_exp=We, y=y, ldy=od, ws=ws)
        return lambda: qig.mmq_q6k_q8t(W, 224, od, id_, q8, nt, y=y, ldy=od, ws=ws)

    names, calls, done = [], [], set()
    extra = {}
    for (name, qt, od, id_, xin) in spec["gemms"]:
        if xin not in done:
            names.append("quantize_" + xin)
            calls.append(quant(xin))
            done.add(xin)
        names.append(name)
        calls.append(gemm(name, qt, od, id_, xin))
        if qt == "q6_K" and tiled:
            extra[name + "[raw]"] = gemm(name, qt, od, id_, xin, "raw")
            extra[name + "[wexp]"] = gemm(name, qt, od, id_, xin, "wexp")
        if qt == "q4_K" and tiled:
            extra[name + "[raw]"] = gemm(name, qt, od, id_, xin, "raw")
            # the same GEMM quantizing its own activations (no q8 plane)
            extra[name + "[xf32]"] = (lambda W=Ws[name], x=xs[xin], y=ys[name], od=od, id_=id_:
                                      qig.mmq_q4k_xf32(W, od, id_, x, y=y, ldy=od, ws=ws))

    def step():
        for fn in calls:
            fn()

    spun, clocks = spin_up(step, args.spinup_s)
    clock_mhz = clocks["shader_mhz"]
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) / args.steps * 1e3

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    per = {n: gpu_avg_us(fn, args.steps) for n, fn in list(zip(names, calls)) + list(extra.items())}
    ops = {name: 2.0 * nt * od * id_ for (name, qt, od, id_, xin) in spec["gemms"]}
    for n in extra:
        ops[n] = ops[n.split("[")[0]]
    total_ops = sum(2.0 * nt * od * id_ for (name, qt, od, id_, xin) in spec["gemms"])   # the step's GEMMs
    gemms = [g[0] for g in spec["gemms"]]
    dom = max(gemms, key=lambda n: per[n])
    achieved = ops[dom] / (per[dom] * 1e-6) / 1e12
    out = {
        "metric": METRIC,
        "value": round(total_ops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": {"ffn": "7B-class FFN GEMMs at nt=512: q4_K gate/up 18944x3584, q6_K down 3584x18944",
                         "layer": "7B-class layer at nt=2630: q4_K q, k, v, o, gate, up and q6_K down, one "
                                  "quantization per distinct input",
                         "down": "7B-class layer's q6_K down projection 3584x18944 at nt=2630, after its "
                                 "activation quantization",
                         "kv": "7B-class layer's q4_K k and v projections 512x3584 at nt=2630 after one "
                               "shared activation quantization",
                         "layer_q6v": "7B-class layer at nt=2630 with a q6_K v projection: q4_K q, k, o, gate, "
                                      "up and q6_K v and down"}[args.workload],
            "weights": "q4_K staged buffer, q6_K limb buffer" if tiled else "raw blocks",
            "activations": args.activations, "nt": nt,
            "gemms": {g[0]: f"{g[1]} {g[2]}x{g[3]}" for g in spec["gemms"]},
        },
        "per_kernel_us": {k: round(v, 3) for k, v in per.items()},
        "summed_us": round(sum(per[n] for n in names), 2),
        "per_gemm_tops": {n: round(ops[n] / (per[n] * 1e-6) / 1e12, 1) for n in gemms + list(extra)},
        "registration_us": registration_us,
        "spinup": {"seconds": args.spinup_s, "steps": spun},
        "clocks_mhz": clocks,
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_INT8_TOPS,
            "unit": "TOP/s",
            "frac": round(achieved / PEAK_INT8_TOPS, 4),
            "traffic": None,
            "clock_mhz": clock_mhz,
            "frac_at_clock": None if clock_mhz is None else round(achieved / (PEAK_INT8_TOPS * clock_mhz / 2400.0), 4),
        },
    }
    if not args.no_cpu_baseline:
        # the whole step on all tokens, once (the layer: about 14 s on 16
        # cores), with the time of each quantization and GEMM
        import oracle
        parts = {}
        t_all = time.perf_counter()
        qh = {}
        for (name, qt, od, id_, xin) in spec["gemms"]:
            if xin not in qh:
                t = time.perf_counter()
                qh[xin] = oracle.quantize_q8_pad40(host[xin])
                parts["quantize_" + xin] = time.perf_counter() - t
            t = time.perf_counter()
            if qt == "q4_K":
                oracle.mmq_q4k(host[name], od, id_, qh[xin], nt)
            else:
                oracle.mmq_q6k(host[name], 224, od, id_, qh[xin], nt)
            parts[name] = time.perf_counter() - t
        total = time.perf_counter() - t_all
        out["cpu_baseline"] = {
            "value": round(total_ops / total / 1e12, 4), "unit": "TOPS",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the whole step, all {nt} tokens through every quantization and GEMM, once, in {total:.1f} s",
            "parts_ms": {k: round(v * 1e3, 1) for k, v in parts.items()},
        }
    print(json.dumps(out), flush=True)


# rocprofv3 kernel names -> the names bench.py reports
PROFILE_NAMES = {
    "qig::mmq_kernel<4, 0, 0, 0>": "mmq_q4k", "qig::mmq_kernel<6, 0, 0, 0>": "mmq_q6k_raw",
    "qig::mmq_kernel<6, 1, 0, 0>": "mmq_q6k_wexp", "qig::mmq_kernel<4, 2, 0, 0>": "mmq_q4k_prepared",
    "qig::mmq_kernel<6, 2, 0, 0>": "mmq_q6k_prepared", "qig::mmq_kernel<4, 0, 0, 1>": "mmq_q4k_q8t",
    "qig::mmq_kernel<6, 0, 0, 1>": "mmq_q6k_raw_q8t", "qig::mmq_kernel<6, 1, 0, 1>": "mmq_q6k_wexp_q8t",
    "qig::mmq_kernel<4, 2, 0, 1>": "mmq_q4k_prepared_q8t", "qig::mmq_kernel<6, 2, 0, 1>": "mmq_q6k_prepared_q8t",
    "qig::mmq_limbs_kernel<2>": "mmq_q6k_limbs_q8t", "qig::mmq_limbs_kernel<3>": "mmq_q6k_limbs_q8t (3 per CU)",
    "qig::mmq_kernel<4, 0, 0, 2>": "mmq_q4k_xf32", "qig::mmq_kernel<4, 4, 0, 1>": "mmq_q4k_staged_q8t",
    "qig::prepare_q4k_staged_kernel": "prepare_q4k_staged",
    "qig::prepare_q4k_kernel": "prepare_q4k", "qig::prepare_q6k_scales_kernel": "prepare_q6k (scales)",
    "qig::prepare_q6k_limbs_kernel": "prepare_q6k_limbs",
    "qig::quantize_kernel": "quantize_q8_pad40", "qig::quantize_tiled_kernel<1>": "quantize_q8_tiled",
    "qig::quantize_tiled_kernel<2>": "quantize_q8_tiled (2 tokens per group)",
    "qig::expand_q6k_kernel": "expand_q6k_dense", "qig::clear_counters_kernel": "clear_counters",
    "__amd_rocclr_copyBuffer": "copy_256MiB (calibration)",
}
# shapes (nt, od, id) and titles of the profiled workloads
PROFILE_WORKLOADS = {
    "proj": (512, 3584, 3584, "mmq_3584x3584_nt512",
             "q4_K / q6_K MMQ at od=id=3584, nt=512 (bench.py default run)"),
    "down": (2630, 3584, 18944, "mmq_q6k_down_3584x18944_nt2630",
             "q6_K down projection MMQ at od=3584, id=18944, nt=2630 (bench.py --workload down)"),
    "layer": (2630, None, None, "mmq_layer_nt2630",
              "the seven GEMMs of a 7B-class layer at nt=2630 (bench.py --workload layer)"),
}


def _algorithmic_bytes(nt=NT, od=OD, id_=ID):
    """(read, write) bytes of one launch of each kernel at the given shape:
    each input and output once."""
    nsb, q8 = id_ // 256, nt * (id_ // 32) * 40
    y = nt * od * 4
    raw4, raw6 = od * nsb * 144, od * nsb * 224
    wexp = od * id_ + od * nsb * 18
    prep4, prep6 = od * id_ // 2 + od * nsb * 64, od * id_ + od * nsb * 64
    limbs = 2 * od * id_ + od * nsb * 4
    gemm = {"mmq_q4k": raw4, "mmq_q6k_raw": raw6, "mmq_q6k_wexp": wexp, "mmq_q4k_prepared": prep4,
            "mmq_q6k_prepared": prep6}
    alg = {}
    for k, w in gemm.items():
        alg[k] = alg[k + "_q8t"] = (w + q8, y)
    alg["mmq_q6k_limbs_q8t"] = (limbs + q8, y)
    alg["mmq_q4k_xf32"] = (raw4 + nt * id_ * 4, y)
    staged = (od + 63) // 64 * nsb * 14336
    alg["mmq_q4k_staged_q8t"] = (staged + q8, y)
    alg["prepare_q4k_staged"] = (raw4, staged)
    alg["quantize_q8_pad40"] = alg["quantize_q8_tiled"] = (nt * id_ * 4, q8)
    alg["expand_q6k_dense"] = (od * nsb * 210, od * id_)
    alg["prepare_q6k_limbs"] = (od * nsb * 210, limbs)
    alg["copy_256MiB (calibration)"] = (256 << 20, 256 << 20)
    return alg


COUNTER_SETS = [
    ("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE"),
    ("sqA", "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT "
            "SQ_WAIT_ANY SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE"),
    ("sqB", "SQ_INSTS_VALU_MFMA_MOPS_I8 SQ_WAIT_INST_ANY SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS SQ_INSTS_SALU "
            "SQ_WAIT_INST_LDS SQ_LDS_ADDR_CONFLICT SQ_LDS_IDX_ACTIVE"),
]
PROFILE_BENCH = {
    "proj": "python3 /root/repo/bench.py --steps 5 --warmup 2 --launches 5 --no-cpu-baseline --copy-calibration",
    "down": "python3 /root/repo/bench.py --workload down --steps 5 --warmup 2 --no-cpu-baseline "
            "--copy-calibration",
}
PROFILE_TRACE = {
    "proj": "python3 /root/repo/bench.py",
    "down": "python3 /root/repo/bench.py --workload down --no-cpu-baseline",
    "layer": "python3 /root/repo/bench.py --workload layer --no-cpu-baseline",
}


def summarize_profiles(src_dir, workload="proj", out_dir=None):
    """Write profiles/<tag>_{kernel_trace,counters}.md (and, for the proj
    workload, profiles/mmq_traffic.json) from rocprofv3 outputs under src_dir:
    trace/t_kernel_trace.csv (kernel trace of the PROFILE_TRACE run, whose
    bench line is trace/bench.json) and {fetch,write,sqA,sqB}/p_counter_collection.csv
    (one counter run each, of PROFILE_BENCH)."""
    import collections
    import csv

    def short(k):
        return k.replace("(anonymous namespace)", "{anon}").replace("void ", "").split("(")[0]

    nt, od, id_, tag, title = PROFILE_WORKLOADS[workload]
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    # --- kernel trace
    disp = collections.defaultdict(list)
    for r in csv.DictReader(open(os.path.join(src_dir, "trace", "t_kernel_trace.csv"))):
        wg = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
        disp[(short(r["Kernel_Name"]), wg)].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in disp.values())
    tl = [f"# Kernel trace: {title}", "",
          "Command, from /tmp (`cd /tmp && export TMPDIR=/tmp`):", "```",
          "timeout -k 10 300 rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/prof/trace -o t "
          f"-- {PROFILE_TRACE[workload]}", "```", "",
          ("Per-dispatch durations of every launch in the run: the spin-up and warmup steps, the timed steps, "
           "the back-to-back launches behind bench.py's per-kernel averages, and 100 warm and 100 cold (after a "
           "512 MiB write) launches per step kernel. The median is the steady warm figure; `mean` includes the "
           "cold launches and the clock ramp at the start." if workload == "proj" else
           "Per-dispatch durations of every launch in the run: the spin-up and warmup steps, the timed steps, "
           "and the back-to-back launches behind bench.py's per-kernel averages, which also time the q6_K GEMM "
           "on raw blocks and on the dense plane. The median is the steady figure."), "",
          "Dispatches are grouped by kernel and workgroup count (GEMMs of different shapes, and whole-tile "
          "and split launches, differ in it).", "",
          "| kernel | workgroups | calls | median us | mean us | p10 us | min us | max us | share of GPU time |",
          "|---|---|---|---|---|---|---|---|---|"]
    for (k, wg), d in sorted(disp.items(), key=lambda kv: -sum(kv[1])):
        d = sorted(d)
        n = PROFILE_NAMES.get(k, k)
        tl.append(f"| {n} | {wg} | {len(d)} | {d[len(d) // 2]:.2f} | {sum(d) / len(d):.2f} | "
                  f"{d[len(d) // 10]:.2f} | {d[0]:.2f} | {d[-1]:.2f} | {100 * sum(d) / total:.1f}% |")
    bj = os.path.join(src_dir, "trace", "bench.json")
    if os.path.exists(bj):
        tl += ["", "The same run's bench.py line (per-kernel figures from HIP events on the launch stream):", "```",
               open(bj).read().strip(), "```"]
    with open(os.path.join(out_dir, f"{tag}_kernel_trace.md"), "w") as f:
        f.write("\n".join(tl) + "\n")
    # --- counters
    if od is None:
        return
    cnt = collections.defaultdict(dict)
    for sub, _ in COUNTER_SETS:
        path = os.path.join(src_dir, sub, "p_counter_collection.csv")
        if not os.path.exists(path):
            continue
        agg = collections.defaultdict(lambda: collections.defaultdict(list))
        for r in csv.DictReader(open(path)):
            agg[short(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
        for k, dd in agg.items():
            for c, v in dd.items():
                cnt[k][c] = sum(v) / len(v)
    copy = cnt.get("__amd_rocclr_copyBuffer", {})
    if "FETCH_SIZE" not in copy or "WRITE_SIZE" not in copy:
        return
    fs = copy["FETCH_SIZE"] * 1024 / (256 << 20)
    wsc = copy["WRITE_SIZE"] * 1024 / (256 << 20)
    alg = _algorithmic_bytes(nt, od, id_)
    lines = [f"# HBM traffic and SQ counters: {title}", "",
             "Each counter set is its own run, from /tmp (`cd /tmp && export TMPDIR=/tmp`):", "```"]
    for sub, cs in COUNTER_SETS:
        lines.append(f"timeout -s KILL 120 rocprofv3 --pmc {cs} --output-format csv -d gpurun_out/prof/{sub} -o p "
                     f"-- {PROFILE_BENCH[workload]}")
    lines += ["```", "",
              f"Calibration: a plain 256 MiB device copy reads FETCH_SIZE = {copy['FETCH_SIZE']:.0f} KiB and "
              f"WRITE_SIZE = {copy['WRITE_SIZE']:.0f} KiB per dispatch against 262144 KiB moved each way, so HBM "
              f"bytes = FETCH_SIZE x 1024 / {fs:.4f} + WRITE_SIZE x 1024 / {wsc:.4f}.", "",
              "| kernel | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB (scaled) | HBM write MB | algorithmic read MB "
              "| algorithmic write MB | read / algorithmic |",
              "|---|---|---|---|---|---|---|---|"]
    traffic = {}
    for k, n in PROFILE_NAMES.items():
        c = cnt.get(k)
        if not c or "FETCH_SIZE" not in c or "WRITE_SIZE" not in c or n not in alg:
            continue
        rb, wb = c["FETCH_SIZE"] * 1024 / fs, c["WRITE_SIZE"] * 1024 / wsc
        ar, aw = alg[n]
        traffic[n] = int(round(rb + wb))
        lines.append(f"| {n} | {c['FETCH_SIZE']:.1f} | {c['WRITE_SIZE']:.1f} | {rb / 1e6:.2f} | {wb / 1e6:.2f} | "
                     f"{ar / 1e6:.2f} | {aw / 1e6:.2f} | {rb / ar:.2f} |")
    cols = ["SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_MFMA_MOPS_I8", "SQ_VALU_MFMA_BUSY_CYCLES",
            "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE",
            "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_VALU", "SQ_INSTS_SALU"]
    lines += ["", "SQ counters per dispatch (means over the run's dispatches; SQ_* summed over the chip):", "",
              "| kernel | " + " | ".join(cols) + " |", "|---" * (len(cols) + 1) + "|"]
    for k, n in PROFILE_NAMES.items():
        c = cnt.get(k)
        if not c or "SQ_INSTS_VALU" not in c:
            continue
        lines.append(f"| {n} | " + " | ".join(f"{c[x]:.0f}" if x in c else "—" for x in cols) + " |")
    with open(os.path.join(out_dir, f"{tag}_counters.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    if workload != "proj":
        return
    valu = {}
    for k, n in PROFILE_NAMES.items():
        c = cnt.get(k)
        if n.startswith("mmq") and c and "SQ_INSTS_VALU" in c and "SQ_INSTS_MFMA" in c:
            valu[n] = int(round(c["SQ_INSTS_VALU"] - c["SQ_INSTS_MFMA"]))
    rec = {"kernel_code_sha256": kernel_source_digest(), "fetch_scale": round(fs, 5), "write_scale": round(wsc, 5),
           "source": f"profiles/{tag}_counters.md",
           "bytes_per_launch": {k: v for k, v in traffic.items() if k.startswith("mmq")},
           "valu_insts_per_launch": valu}
    with open(os.path.join(out_dir, "mmq_traffic.json"), "w") as f:
        json.dump(rec, f, indent=1)


def main():
    args = parse()
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is described, not built).", file=sys.stderr)
        sys.exit(2)

    import torch
    import quant_integer_gemm_amd as qig
    from quant_integer_gemm_amd import inputs

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    qig.load()
    if args.workload != "proj":
        run_gemm_set(args)
        return
    dev = torch.device("cuda:0")
    g4 = inputs.WORKLOADS[1][0]
    g6 = inputs.WORKLOADS[2][0]
    W4, x4 = inputs.make_gemm_inputs(g4, SEED4)
    W6, x6 = inputs.make_gemm_inputs(g6, SEED6)
    W4d = torch.from_numpy(W4).to(dev)
    W6d = torch.from_numpy(W6).to(dev)
    x4d = torch.from_numpy(x4).to(dev)
    x6d = torch.from_numpy(x6).to(dev)
    nb = qig.q8_pad40_bytes(NT, ID)
    q84 = torch.empty(nb, dtype=torch.uint8, device=dev)
    q86 = torch.empty(nb, dtype=torch.uint8, device=dev)
    t84 = torch.empty(qig.q8_tiled_bytes(NT, ID), dtype=torch.uint8, device=dev)
    t86 = torch.empty(qig.q8_tiled_bytes(NT, ID), dtype=torch.uint8, device=dev)
    y4 = torch.empty((NT, OD), dtype=torch.float32, device=dev)
    y6 = torch.empty((NT, OD), dtype=torch.float32, device=dev)
    wexp = torch.empty((OD, ID), dtype=torch.int8, device=dev)
    W4p = torch.empty(qig.prepared_bytes("q4_K", OD, ID), dtype=torch.uint8, device=dev)
    W6p = torch.empty(qig.prepared_bytes("q6_K", OD, ID), dtype=torch.uint8, device=dev)
    W6l = torch.empty(qig.q6k_limbs_bytes(OD, ID), dtype=torch.uint8, device=dev)
    W4s = torch.empty(qig.q4k_staged_bytes(OD, ID), dtype=torch.uint8, device=dev)

    # registration-time work, each timed on its own
    def time_us(fn, reps=10):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    registration_us = {
        "expand_q6k_dense": time_us(lambda: qig.expand_q6k_dense(W6d, 224, OD, ID, out=wexp)),
        "prepare_q4k": time_us(lambda: qig.prepare_q4k(W4d, OD, ID, out=W4p)),
        "prepare_q6k": time_us(lambda: qig.prepare_q6k(W6d, 224, OD, ID, out=W6p)),
        "prepare_q6k_limbs": time_us(lambda: qig.prepare_q6k_limbs(W6d, 224, OD, ID, out=W6l)),
        "prepare_q4k_staged": time_us(lambda: qig.prepare_q4k_staged(W4d, OD, ID, out=W4s)),
    }

    # The step: one q4_K and one q6_K GEMM at the q-projection shape, each after
    # its activation quantization (tiled plane), each on the fastest
    # registration-time form of its weights: q4_K on the staged buffer, q6_K on
    # the limb buffer.  Every other arm (raw blocks among them) and
    # activation form is timed after it, per kernel.
    steps = {
        "quantize_tiled_x4": lambda: qig.quantize_q8_tiled(x4d, out=t84),
        "mmq_q4k_staged_q8t": lambda: qig.mmq_q4k_staged_q8t(W4s, OD, ID, t84, NT, y=y4, ldy=OD),
        "quantize_tiled_x6": lambda: qig.quantize_q8_tiled(x6d, out=t86),
        "mmq_q6k_limbs_q8t": lambda: qig.mmq_q6k_limbs_q8t(W6l, OD, ID, t86, NT, y=y6, ldy=OD),
    }
    arms = {
        "mmq_q4k_q8t": lambda: qig.mmq_q4k_q8t(W4d, OD, ID, t84, NT, y=y4, ldy=OD),
        "mmq_q4k_xf32": lambda: qig.mmq_q4k_xf32(W4d, OD, ID, x4d, y=y4, ldy=OD),
        "mmq_q6k_raw_q8t": lambda: qig.mmq_q6k_q8t(W6d, 224, OD, ID, t86, NT, y=y6, ldy=OD),
        "mmq_q6k_wexp_q8t": lambda: qig.mmq_q6k_q8t(W6d, 224, OD, ID, t86, NT, W_exp=wexp, y=y6, ldy=OD),
        "mmq_q6k_prepared_q8t": lambda: qig.mmq_q6k_prepared_q8t(W6p, OD, ID, t86, NT, y=y6, ldy=OD),
        "mmq_q4k_prepared_q8t": lambda: qig.mmq_q4k_prepared_q8t(W4p, OD, ID, t84, NT, y=y4, ldy=OD),
        "quantize_x4": lambda: qig.quantize_q8_pad40(x4d, out=q84),
        "quantize_x6": lambda: qig.quantize_q8_pad40(x6d, out=q86),
        "mmq_q4k": lambda: qig.mmq_q4k(W4d, OD, ID, q84, NT, y=y4, ldy=OD),
        "mmq_q6k_raw": lambda: qig.mmq_q6k(W6d, 224, OD, ID, q86, NT, y=y6, ldy=OD),
        "mmq_q6k_wexp": lambda: qig.mmq_q6k(W6d, 224, OD, ID, q86, NT, W_exp=wexp, y=y6, ldy=OD),
        "mmq_q4k_prepared": lambda: qig.mmq_q4k_prepared(W4p, OD, ID, q84, NT, y=y4, ldy=OD),
        "mmq_q6k_prepared": lambda: qig.mmq_q6k_prepared(W6p, OD, ID, q86, NT, y=y6, ldy=OD),
    }
    names = list(steps)
    calls = list(steps.values())

    def step():
        for fn in calls:
            fn()

    spun, clocks = spin_up(step, args.spinup_s)
    clock_mhz = clocks["shader_mhz"]
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # timed region: K whole steps back to back
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3

    # per-kernel durations: each call launched K times back to back, queued
    # behind a spin kernel, between one pair of HIP events recorded on the
    # launch stream (an event pair around every single launch would add the
    # event's own latency to each figure)
    per = {n: gpu_avg_us(fn, args.steps) for n, fn in list(steps.items()) + list(arms.items())}
    # per-launch distributions of the step's kernels: warm (back to back) and
    # cold (a 512 MiB write before each launch, outside its events), against
    # the same event pair around a one-element kernel
    tiny = torch.zeros(1, dtype=torch.float32, device=dev)
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    event_overhead = per_launch_us(lambda: tiny.add_(1.0), args.launches)
    per_launch = {}
    for n, fn in steps.items():
        per_launch[n] = {"warm": per_launch_us(fn, args.launches),
                         "cold": per_launch_us(fn, args.launches, flush=lambda k: flush_buf.fill_(k & 255))}
    del flush_buf

    gemm_ops = 2.0 * NT * OD * ID
    value = 2 * gemm_ops / (ms_per_step * 1e-3) / 1e12
    gemms = [n for n in names if n.startswith("mmq")]
    all_gemms = gemms + [n for n in arms if n.startswith("mmq")]
    dom = max(gemms, key=lambda n: per[n])
    achieved = gemm_ops / (per[dom] * 1e-6) / 1e12
    # algorithmic bytes per launch of each GEMM: its weight form (raw blocks; the
    # dense plane plus d and the 16 scales of each block; a prepared or limb
    # buffer) + the activation plane + fp32 y, once each (the tiled plane has
    # the pad40 plane's size at this nt)
    nsb = ID // 256
    wb = {"mmq_q4k": OD * nsb * 144, "mmq_q6k_raw": OD * nsb * 224, "mmq_q6k_wexp": OD * ID + OD * nsb * 18,
          "mmq_q4k_prepared": qig.prepared_bytes("q4_K", OD, ID), "mmq_q6k_prepared": qig.prepared_bytes("q6_K", OD, ID),
          "mmq_q6k_limbs": qig.q6k_limbs_bytes(OD, ID), "mmq_q4k_xf32": OD * nsb * 144,
          "mmq_q4k_staged": qig.q4k_staged_bytes(OD, ID)}
    wbytes = {n: wb[n.replace("_q8t", "")] for n in all_gemms}
    abytes = nb + NT * OD * 4
    # the fused GEMM reads the fp32 activations in place of a q8 plane
    gbytes = {n: wbytes[n] + (NT * ID * 4 + NT * OD * 4 if n.endswith("xf32") else abytes) for n in all_gemms}
    dom_bytes = gbytes[dom]
    clock_frac = None if clock_mhz is None else round(achieved / (PEAK_INT8_TOPS * clock_mhz / 2400.0), 4)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {
            "workload": "q4_K GEMM and q6_K GEMM, od=id=3584, nt=512, each after its activation quantization "
                        "(tiled plane); q4_K on the registration-time staged buffer, q6_K on the limb buffer; "
                        "the raw-block, dense-plane and prepared arms timed per kernel",
            "nt": NT, "od": OD, "id": ID, "seeds": [SEED4, SEED6],
        },
        "per_kernel_us": {k: round(v, 3) for k, v in per.items()},
        "per_gemm_tops": {n: round(gemm_ops / (per[n] * 1e-6) / 1e12, 1) for n in all_gemms},
        "per_gemm_pct_int8_peak": {n: round(100 * gemm_ops / (per[n] * 1e-6) / 1e12 / PEAK_INT8_TOPS, 2)
                                   for n in all_gemms},
        "per_gemm_hbm_gbs": {n: round(gbytes[n] / (per[n] * 1e-6) / 1e9, 1) for n in all_gemms},
        "registration_us": {k: round(v, 3) for k, v in registration_us.items()},
        "per_launch_us": per_launch,
        "event_overhead_us": event_overhead,
        "spinup": {"seconds": args.spinup_s, "steps": spun},
        "clocks_mhz": clocks,
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_INT8_TOPS,
            "unit": "TOP/s",
            "frac": round(achieved / PEAK_INT8_TOPS, 4),
            "traffic": recorded_traffic(dom),
            "clock_mhz": clock_mhz,
            "frac_at_clock": clock_frac,
            "hbm_algorithmic_bytes": dom_bytes,
            "hbm_achieved_gbs": round(dom_bytes / (per[dom] * 1e-6) / 1e9, 1),
            "hbm_peak_gbs": PEAK_HBM_GBS,
            "hbm_frac": round(dom_bytes / (per[dom] * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "valu": valu_roofline(dom, per[dom], clock_mhz),
        },
        "roofline_frac_per_arm": {n: round(gemm_ops / (per[n] * 1e-6) / 1e12 / PEAK_INT8_TOPS, 4)
                                  for n in all_gemms},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(W4, x4, W6, x6)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
