"""Benchmark of one MoE expert-FFN layer forward on one MI355X.

A step is one call of moe_layer_forward (router -> permute -> grouped SwiGLU FFN -> combine)
over one batch of T synthetic tokens, with every input already resident in HBM. The default run
measures every workload of the layer's configurations and prints one JSON line: the headline is
the prefill-sized DeepSeek-V3-shaped layer (the largest single-GPU workload, the one the metric's
MFMA half is quoted on), and a "configs" block holds the same record for the other four (the tiny
fp32 layer and the three decode layers). Each record has the whole-step tokens/s, the layer's
algorithmic HBM GB/s and TFLOP/s, the dominant kernel's roofline fraction (its duration measured
with HIP events on the launch stream) and the CPU oracle timed on a bounded sample of the same
workload.

    python bench.py [--config all|c1..c5|...] [--steps K] [--warmup W] [--gpus 1] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA TFLOP/s (prefill)"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3, "int8": 5000.0}
HEADLINE = "c5"
BLOCK = ("c1", "c2", "c3", "c4")
WORKLOADS = ("c1", "c2", "c3", "c4", "c5", "v4p", "v4p-w4a8", "v4p-mx", "v3-int8", "c4-w4a8", "c4-mx", "c3-int8")
# HBM bytes per launch of the dominant kernel, from two rocprofv3 --pmc runs of this script
# (FETCH_SIZE, then WRITE_SIZE), each scaled by what the same counter reads for the plain copy
# kernel of known size that --calib-copy appends. Keyed by workload; an entry holds only while
# the kernel sources it was measured on are unchanged (hash of their code).
TRAFFIC = {
    # gate/up decode kernel
    "c1": {"sha": "10b97aefda9c717d", "bytes": 2390482},
    "c2": {"sha": "10b97aefda9c717d", "bytes": 3176729742},
    "c3": {"sha": "10b97aefda9c717d", "bytes": 14043819466},
    "c4": {"sha": "10b97aefda9c717d", "bytes": 3662068654},
    # gate/up prefill kernel
    "c5": {"sha": "a4d75bc69100650b", "bytes": 16302908956},
    # the W4A8 gate/up stage: x to MXFP8 + routed W4A8 GEMM + shared bf16 GEMM
    "v4p-w4a8": {"sha": "b631906a8dfde38d", "bytes": 10146152314},
    # the hybrid gate/up stage: x to MXFP8 + routed W4A8 GEMM + shared W8A8 MXFP8 GEMM
    "v4p-mx": {"sha": "b631906a8dfde38d", "bytes": 9802442640},
    # the int8 gate/up stage: x to int8 + Int8 W8A8 GEMM
    "v3-int8": {"sha": "b631906a8dfde38d", "bytes": 17093371508},
}
CSRC = os.path.join(ROOT, "expert_ffn_layer_amd", "csrc")
KERNEL_SOURCES = {"decode": ("gemm_decode.hip", "common.h", "kernels.h"),
                  "prefill": ("gemm_prefill.hip", "common.h", "kernels.h"),
                  "w4a8": ("gemm_prefill.hip", "quant.hip", "common.h", "kernels.h"),
                  "int8": ("gemm_prefill.hip", "quant.hip", "common.h", "kernels.h")}
# bounded CPU-oracle samples (first tokens of the layer): about 10-30 s of oracle work on the host's
# threads; and the single-thread samples of the small layers
CPU_TOKENS = {"c1": 16, "c2": 64, "c3": 160, "c4": 32, "c5": 64, "v4p": 16, "v4p-w4a8": 16, "v4p-mx": 16,
              "v3-int8": 32, "c4-w4a8": 32, "c4-mx": 32, "c3-int8": 64}
CPU_TOKENS_1T = {"c1": 16, "c2": 32}


def kernel_sha(path: str) -> str:
    """Hash of the code of the kernel sources (comments and blank lines left out: they cannot
    change what the kernel does)."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[path]:
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(l.rstrip() for l in text.splitlines() if l.strip()).encode())
    return h.hexdigest()[:16]


def measured_traffic(config: str, path: str):
    t = TRAFFIC.get(config)
    if t is None or t["sha"] != kernel_sha(path):
        return None
    return t["bytes"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def host_cpu():
    """(model, threads the oracle runs on): lscpu's model name with its CPU family, model and
    stepping numbers, CPU count and hypervisor (a virtual machine may report only a family name);
    the threads this process may run on (its affinity mask), capped by OMP_NUM_THREADS when set."""
    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        f = {l.split(":", 1)[0].strip(): l.split(":", 1)[1].strip() for l in out.splitlines() if ":" in l}
        model = f.get("Model name")
        if model:
            model += " (CPU family %s, model %s, stepping %s; %s CPUs%s)" % (
                f.get("CPU family", "?"), f.get("Model", "?"), f.get("Stepping", "?"), f.get("CPU(s)", "?"),
                "; %s guest" % f["Hypervisor vendor"] if "Hypervisor vendor" in f else "")
    except (OSError, subprocess.SubprocessError):
        pass
    if not model:
        try:
            with open("/proc/cpuinfo") as fh:
                model = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), None)
        except OSError:
            pass
    n = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    if omp and omp.isdigit() and int(omp) > 0:
        n = min(n, int(omp))
    return model, max(n, 1)


def ceilings(args, dev):
    """The measured ceilings beside the published peaks: a plain streaming read of 4 GiB (the
    achievable HBM read rate) and register-only MFMA bursts (2 waves per SIMD, operands rotating
    over random register sets) of each instruction kind the GEMMs issue."""
    import torch

    from measure import ceilings as M
    if args.no_ceiling:
        return None, None
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    M.stream_read(buf, sink)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(5):
        M.stream_read(buf, sink)
    c1.record()
    torch.cuda.synchronize()
    hbm = round(5 * buf.numel() / (c0.elapsed_time(c1) * 1e-3) / 1e9, 1)
    del buf
    mfma = {}
    for kind, name in ((0, "bf16 16x16x32"), (1, "fp4 x fp8 16x16x128"), (2, "fp8 x fp8 16x16x128"),
                       (3, "int8 16x16x64")):
        iters = 2048 if kind else 8192
        M.mfma_burst(kind, iters, 512, sink)
        m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        m0.record()
        fl = sum(M.mfma_burst(kind, iters, 512, sink) for _ in range(5))
        m1.record()
        torch.cuda.synchronize()
        mfma[name] = round(fl / (m0.elapsed_time(m1) * 1e-3) / 1e12, 1)
    return hbm, mfma


def measure(name, args, dev, hbm_ceiling, mfma_ceiling, cpu_info):
    """Generate the workload on the device, time K layer steps (after W warm-up steps), the same K
    steps replayed from a HIP graph and through the per-stage timed entry point; price the dominant
    kernel against its roofline; time the oracle on a bounded sample. Returns the record."""
    import numpy as np
    import torch

    from expert_ffn_layer_amd import native as N
    from expert_ffn_layer_amd import perfmodel as pm
    from expert_ffn_layer_amd.layer import PackedLayer
    from inputgen import gpu as G
    from inputgen import layers as L

    spec = L.workload(name)
    log("bench: generating %s on the device" % spec.name)
    lay = G.layer_on_device(spec, dev)
    pl = PackedLayer(spec, lay["Wr"], lay["routed"], lay["shared"], path=args.path)
    x = lay["x"] if spec.act == "f32" else lay["x"].view(torch.bfloat16)
    act_dt = torch.float32 if spec.act == "f32" else torch.bfloat16
    y = torch.empty((spec.T, spec.H), dtype=act_dt, device=dev)
    idx = torch.empty((spec.T, spec.k), dtype=torch.int32, device=dev)
    w = torch.empty((spec.T, spec.k), dtype=torch.float32, device=dev)
    bias = lay["bias"]

    def step():
        N.moe_layer_forward(pl.shape, x, pl.Wr, bias, pl.routed, pl.shared, y, idx, w, pl.ws)

    log("bench: %s warmup %d" % (name, args.warmup))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=spec.E)
    traffic = pm.layer_traffic(spec, counts)

    log("bench: %s timing %d steps" % (name, args.steps))
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record()
    for _ in range(args.steps):
        step()
    t1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / args.steps

    # The same forward captured once in a HIP graph and replayed K times: one host launch per layer
    # instead of one per kernel (the plan lives on the device, so nothing is read back).
    graph_ms = None
    try:
        gs = torch.cuda.Stream()
        gs.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(gs):
            step()
        torch.cuda.current_stream().wait_stream(gs)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(args.steps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_ms = round(g0.elapsed_time(g1) / args.steps, 4)
        del graph
    except RuntimeError as e:  # reported, not fatal: the eager loop above is the measurement
        log("bench: graph capture failed: %s" % e)

    # Per-kernel durations, live: the same K steps again through the timed entry point, which
    # records HIP events on the launch stream between the kernels of each forward (one event
    # set per step, no synchronisation inside the region).
    names = ["route", "permute", "plan", "gate_up", "down", "combine"]
    evsets = [[torch.cuda.Event(enable_timing=True) for _ in range(N.TIMED_EVENTS)] for _ in range(args.steps)]
    for evs in evsets:
        for e in evs:
            e.record()  # creates the underlying HIP events before the region
    torch.cuda.synchronize()
    for evs in evsets:
        N.moe_layer_forward_timed(pl.shape, x, pl.Wr, bias, pl.routed, pl.shared, y, evs, idx, w, pl.ws)
    torch.cuda.synchronize()
    acc = np.zeros(len(names))
    for evs in evsets:
        acc += [evs[i].elapsed_time(evs[i + 1]) for i in range(len(names))]
    stage_ms = acc / args.steps
    timed_ms = sum(evs[0].elapsed_time(evs[-1]) for evs in evsets) / args.steps

    # roofline of the dominant kernel (the gate/up grouped GEMM, or the W4A8 gate/up stage), against
    # the roof that binds it: its algorithmic FLOPs at the MFMA peak of its instruction kinds, or its
    # algorithmic bytes at the HBM peak, whichever takes longer
    H, I, T, k = spec.H, spec.I, spec.T, spec.k
    R = T * k + (T if spec.shared else 0)
    ab = 4 if spec.act == "f32" else 2
    a8 = spec.w_routed == "mxfp4a8"
    i8 = spec.w_routed == "int8"
    mx = a8 and spec.shared and spec.w_shared == "mxfp8a8"
    w_bytes = (traffic["active_experts"] * 2 * pm.matrix_bytes(H, I, spec.w_routed)
               + (2 * pm.matrix_bytes(H, I, spec.w_shared) if spec.shared else 0))
    if a8:
        q = 1 + 1 / 32  # MXFP8 bytes per element (E4M3 code + an e8m0 byte per 32)
        # x read once as bf16, its MXFP8 form written and read once; h written as MXFP8 (routed rows,
        # and the shared rows in the hybrid scheme) or bf16 (a bf16 shared expert)
        gu_bytes = int(w_bytes + T * H * ab + 2 * T * H * q + T * k * I * q
                       + (T * I * (q if mx else ab) if spec.shared else 0))
    elif i8:
        # x read once as bf16, its int8 copy (and a scale per token) written and read once, h in bf16
        gu_bytes = w_bytes + T * H * ab + 2 * (T * H + 4 * T) + R * I * ab
    else:
        gu_bytes = w_bytes + T * H * ab + R * I * ab
    gu_flops = 4 * H * I * R
    gu_ms = stage_ms[names.index("gate_up")]
    prefill = a8 or i8 or (T * k) / spec.E >= 64
    traffic_b = measured_traffic(name, "w4a8" if a8 else "int8" if i8 else "prefill" if prefill else "decode")
    hbm_ach = gu_bytes / (gu_ms * 1e-3) / 1e9
    hbm_roof = {"bound": "hbm", "achieved": round(hbm_ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(hbm_ach / HBM_PEAK_GBPS, 4),
                "frac_of_read_ceiling": round(hbm_ach / hbm_ceiling, 4) if hbm_ceiling else None}
    if a8:
        # W4A8: the gate/up stage is the x quantisation, the routed fp4 x fp8 GEMM (fp8 peak) and
        # the shared expert's GEMM: bf16 (bf16 peak), or W8A8 MXFP8 in the hybrid scheme (fp8 peak);
        # the stage's MFMA peak is the FLOP-weighted blend, i.e. its FLOPs over the time both GEMMs
        # would take at their own peaks
        fr, fs = 4 * H * I * T * k, 4 * H * I * (T if spec.shared else 0)
        t_peak = fr / (MFMA_PEAK_TFLOPS["fp8"] * 1e12) + fs / (MFMA_PEAK_TFLOPS["fp8" if mx else "bf16"] * 1e12)
        peak = round(gu_flops / t_peak / 1e12, 1)
        kernel = ("gate/up stage: x to MXFP8, W4A8 routed GEMM and W8A8 MXFP8 shared GEMM (fp8 peak 5000)"
                  if mx else "gate/up stage: x to MXFP8, W4A8 routed GEMM (fp8 peak 5000), bf16 shared GEMM "
                             "(bf16 peak 2500)")
        per_launch = {"flops": gu_flops, "routed_flops": fr, "shared_flops": fs, "bytes": gu_bytes,
                      "ms": round(gu_ms, 4)}
    elif i8:
        peak = MFMA_PEAK_TFLOPS["int8"]
        kernel = "gate/up stage: x to int8 per token, Int8 W8A8 grouped GEMM (int8 peak 5000 TOP/s)"
        per_launch = {"ops": gu_flops, "bytes": gu_bytes, "ms": round(gu_ms, 4)}
    else:
        peak = MFMA_PEAK_TFLOPS["bf16" if spec.act == "bf16" else "f32"]
        kernel = "gate/up grouped GEMM"
        per_launch = {"flops": gu_flops, "bytes": gu_bytes, "ms": round(gu_ms, 4)}
    mfma_ach = gu_flops / (gu_ms * 1e-3) / 1e12
    mfma_roof = {"bound": "mfma", "achieved": round(mfma_ach, 1), "peak": peak, "unit": "TOP/s" if i8 else "TFLOP/s",
                 "frac": round(mfma_ach / peak, 4)}
    if mfma_ceiling and prefill:
        if a8:
            # the time both GEMMs would take at the measured sustained rates, over the stage time
            rs = mfma_ceiling["fp8 x fp8 16x16x128" if mx else "bf16 16x16x32"]
            t_meas = fr / (mfma_ceiling["fp4 x fp8 16x16x128"] * 1e12) + fs / (rs * 1e12)
            mfma_roof["frac_of_measured_mfma"] = round(t_meas / (gu_ms * 1e-3), 4)
        else:
            mfma_roof["frac_of_measured_mfma"] = round(mfma_ach / mfma_ceiling["int8 16x16x64" if i8 else "bf16 16x16x32"], 4)
    t_hbm = gu_bytes / (HBM_PEAK_GBPS * 1e9)
    t_mfma = gu_flops / (peak * 1e12)
    binding, other = (mfma_roof, hbm_roof) if prefill and t_mfma >= t_hbm else (hbm_roof, mfma_roof)
    roof = dict(binding)
    roof.update({"traffic": traffic_b, "kernel": kernel, "per_launch": per_launch,
                 "roof_ms": {"hbm": round(t_hbm * 1e3, 4), "mfma": round(t_mfma * 1e3, 4)}, "other_roof": other})

    rec = {
        "workload": name,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "ms_per_step": round(ms, 4),
        "dtype": spec.act,
        "config": {"workload": spec.name, "T": T, "H": H, "E": spec.E, "k": k, "I": I,
                   "shared_expert": spec.shared, "w_routed": spec.w_routed,
                   "w_shared": spec.w_shared if spec.shared else None, "router": spec.router,
                   "zipf_alpha": spec.zipf_alpha or None, "active_experts": traffic["active_experts"],
                   "max_rows_per_expert": int(counts.max())},
        "hbm_GBps": round(traffic["bytes"] / (ms * 1e-3) / 1e9, 1),
        "hbm_frac": round(traffic["bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "tflops": round(traffic["flops"] / (ms * 1e-3) / 1e12, 2),
        "algorithmic": {"bytes": traffic["bytes"], "flops": traffic["flops"]},
        "stages_ms": {n: round(float(v), 4) for n, v in zip(names, stage_ms)},
        "timed_entry_ms_per_step": round(timed_ms, 4),
        "graph_replay_ms_per_step": graph_ms,
        "wall_s_timed": round(wall, 3),
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu:
        S = args.cpu_tokens or CPU_TOKENS[name]
        sample = sample_to_host(spec, lay, max(S, CPU_TOKENS_1T.get(name, 0)))
        rec["cpu_baseline"] = cpu_baseline(spec, sample, S, cpu_info[1], cpu_info[0])
        if name in CPU_TOKENS_1T:
            one = cpu_baseline(spec, sample, CPU_TOKENS_1T[name], 1, cpu_info[0])
            rec["cpu_baseline"]["one_thread"] = {k: one[k] for k in ("value", "unit", "cores", "sample")}
    return rec


def sample_to_host(spec, lay, S):
    """The first S tokens' inputs and the stored weights of the experts they select, copied to the
    host (outside any timed region)."""
    from inputgen import gpu as G
    from oracle import oracle as O

    S = min(S, spec.T)
    x = lay["x_host"][:S]
    idx, _, _ = O.route(x, lay["Wr_host"], lay["bias_host"], spec.k, spec.act)
    need = sorted(set(int(e) for e in idx.reshape(-1)))
    routed = {k: None if v is None else G.to_numpy_stored(v[need]) for k, v in lay["routed"].items()}
    shared = None
    if spec.shared:
        shared = {k: None if v is None else G.to_numpy_stored(v[0]) for k, v in lay["shared"].items()}
    return {"x": x, "Wr": lay["Wr_host"], "bias": lay["bias_host"], "need": need, "routed": routed, "shared": shared}


def cpu_baseline(spec, smp, S, threads, model):
    """The oracle, as it stands, on the first S tokens of the same layer: route, permute, every
    selected expert's SwiGLU on its rows (plus the shared expert on every token), combine. The
    rows' FFNs are independent oracle calls of one row each, spread over `threads` host threads
    (the oracle's own row loop runs one row per call, so each call uses one thread)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    from inputgen.layers import act_to_f64
    from oracle import oracle as O

    S = min(S, spec.T)
    log("bench: CPU oracle on %d tokens, %d threads" % (S, threads))
    x = smp["x"][:S]
    pos = {e: j for j, e in enumerate(smp["need"])}
    t = time.perf_counter()
    idx, wts, _ = O.route(x, smp["Wr"], smp["bias"], spec.k, spec.act)
    off, st, ps = O.permute(idx, spec.E)
    u = act_to_f64(x, spec.act)
    # (row r of the permuted batch, its expert e); the shared expert's rows are (token, -1)
    jobs = [(r, int(e)) for e in range(spec.E) for r in range(off[e], off[e + 1])]
    if spec.shared:
        jobs += [(tk, -1) for tk in range(S)]

    def ffn(job):
        r, e = job
        if e < 0:
            return O.expert_ffn(u[r:r + 1], smp["shared"], spec.w_shared)[0]
        one = {k: None if v is None else v[pos[e]] for k, v in smp["routed"].items()}
        return O.expert_ffn(u[st[r]:st[r] + 1], one, spec.w_routed)[0]

    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            out = list(ex.map(ffn, jobs))
    else:
        out = [ffn(j) for j in jobs]
    res = dict(zip(jobs, out))
    yperm = np.zeros((S * spec.k, spec.H))
    for (r, e), v in res.items():
        if e >= 0:
            yperm[r] = v
    for tk in range(S):
        O.combine_token(wts[tk], yperm[ps[tk * spec.k:(tk + 1) * spec.k]], res[(tk, -1)] if spec.shared else None)
    dt = time.perf_counter() - t
    active = len(set(int(e) for e in idx.reshape(-1)))
    return {"value": round(S / dt, 3), "unit": "tokens/s", "cores": threads, "kind": "oracle", "cpu": model,
            "sample": "first %d of %d tokens of the same layer (route, permute, %d active experts' SwiGLU%s, "
                      "combine), fp64 C oracle, one row per call over %d host thread%s, %.1f s"
                      % (S, spec.T, active, " + shared expert" if spec.shared else "", threads,
                         "s" if threads > 1 else "", dt)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="all", choices=("all",) + WORKLOADS,
                    help="all: the prefill layer (c5) as the headline and c1-c4 in a configs block; c1-c5: one "
                         "workload alone; v4p, v4p-w4a8, v4p-mx: the V4-Pro-shaped layer at a prefill batch with "
                         "MXFP4 / W4A8 routed experts, and in the hybrid MXFP8-MXFP4 scheme (W4A8 routed, W8A8 "
                         "MXFP8 shared); v3-int8: the c5 layer with Int8 W8A8 experts; c4-w4a8, c4-mx: the c4 "
                         "decode layer with W4A8 routed experts, and hybrid; c3-int8: the c3 decode layer with Int8 "
                         "W8A8 experts")
    ap.add_argument("--path", default="auto", choices=["auto", "decode", "prefill"])
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-tokens", type=int, default=None)
    ap.add_argument("--no-ceiling", action="store_true", help="skip the measured ceilings (streaming HBM read, sustained MFMA rate)")
    ap.add_argument("--calib-copy", type=int, default=0, metavar="MiB",
                    help="end with one plain copy kernel of this size (byte-counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the layer would shard "
              "by experts across GPUs, each GPU running this same path on its share). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from expert_ffn_layer_amd import native as N

    N.load()
    dev = torch.device("cuda:0")
    cpu_info = host_cpu()
    hbm_ceiling, mfma_ceiling = ceilings(args, dev)
    names = [HEADLINE, *BLOCK] if args.config == "all" else [args.config]
    recs = {}
    for name in names:
        recs[name] = measure(name, args, dev, hbm_ceiling, mfma_ceiling, cpu_info)
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    if args.calib_copy:
        # one plain copy of known size, the reference that scales the byte counters of a --pmc run
        from measure import ceilings as M
        nb = args.calib_copy << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        M.copy(src, torch.empty_like(src))
        torch.cuda.synchronize()
        log("bench: calibration copy of %d bytes" % nb)

    head = recs[names[0]]
    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
    }
    out.update({k: v for k, v in head.items() if k not in out and k not in ("workload",)})
    out["hbm_read_ceiling_GBps"] = hbm_ceiling
    out["mfma_sustained_TFLOPs"] = mfma_ceiling
    if len(names) > 1:
        out["configs"] = {n: recs[n] for n in names[1:]}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
