"""Benchmark of one MoE expert-FFN layer forward on one MI355X.

A step is one call of moe_layer_forward (router -> permute -> grouped SwiGLU FFN -> combine)
over one batch of T synthetic tokens, with every input already resident in HBM. Prints one
JSON line: whole-step tokens/s, the layer's algorithmic HBM GB/s and TFLOP/s, the dominant
kernel's roofline fraction (its duration measured with HIP events on the launch stream), and
the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--config c2] [--steps K] [--warmup W] [--gpus 1] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s + achieved HBM GB/s (decode) / MFMA TFLOP/s (prefill)"
HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3, "int8": 5000.0}
# HBM bytes per launch of the dominant kernel, from two rocprofv3 --pmc runs of this script
# (FETCH_SIZE, then WRITE_SIZE), each scaled by what the same counter reads for the plain copy
# kernel of known size that --calib-copy appends. Keyed by workload; an entry holds only while
# the kernel sources it was measured on are unchanged (sha256 of those files).
TRAFFIC = {
    # gate/up decode kernel
    "c2": {"sha": "24c0fd2cc318dc45", "bytes": 3176791832},
    "c3": {"sha": "24c0fd2cc318dc45", "bytes": 14695798301},
    "c4": {"sha": "24c0fd2cc318dc45", "bytes": 3676200475},
    # gate/up prefill kernel
    "c5": {"sha": "e0463fd1be82c895", "bytes": 16306116370},
    # the W4A8 gate/up stage: x to MXFP8 + routed W4A8 GEMM + shared bf16 GEMM
    "v4p-w4a8": {"sha": "176a8dd7ef59aeac", "bytes": 10131416530},
    # the hybrid gate/up stage: x to MXFP8 + routed W4A8 GEMM + shared W8A8 MXFP8 GEMM
    "v4p-mx": {"sha": "176a8dd7ef59aeac", "bytes": 9795198467},
    # the int8 gate/up stage: x to int8 + Int8 W8A8 GEMM
    "v3-int8": {"sha": "176a8dd7ef59aeac", "bytes": 17225696545},
}
CSRC = os.path.join(ROOT, "expert_ffn_layer_amd", "csrc")
KERNEL_SOURCES = {"decode": ("gemm_decode.hip", "common.h", "kernels.h"),
                  "prefill": ("gemm_prefill.hip", "common.h", "kernels.h"),
                  "w4a8": ("gemm_prefill.hip", "quant.hip", "common.h", "kernels.h"),
                  "int8": ("gemm_prefill.hip", "quant.hip", "common.h", "kernels.h")}


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


# bounded CPU-oracle samples (tokens): about 10-30 s of oracle work per config
CPU_TOKENS = {"c1": 16, "c2": 64, "c3": 12, "c4": 32, "c5": 4, "v4p": 6, "v4p-w4a8": 6, "v4p-mx": 6, "v3-int8": 4,
              "c4-w4a8": 32, "c4-mx": 32, "c3-int8": 12}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c2",
                    choices=["c1", "c2", "c3", "c4", "c5", "v4p", "v4p-w4a8", "v4p-mx", "v3-int8", "c4-w4a8", "c4-mx", "c3-int8"],
                    help="c1-c5: the layer configurations; v4p, v4p-w4a8, v4p-mx: the V4-Pro-shaped layer at a "
                         "prefill batch with MXFP4 / W4A8 routed experts, and in the hybrid MXFP8-MXFP4 scheme "
                         "(W4A8 routed, W8A8 MXFP8 shared); v3-int8: the c5 layer with Int8 W8A8 experts; "
                         "c4-w4a8, c4-mx: the c4 decode layer with W4A8 routed experts, and hybrid; c3-int8: the c3 "
                         "decode layer with Int8 W8A8 experts")
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

    import numpy as np
    import torch

    from expert_ffn_layer_amd import native as N
    from expert_ffn_layer_amd import perfmodel as pm
    from expert_ffn_layer_amd.layer import PackedLayer
    from inputgen import gpu as G
    from inputgen import layers as L

    N.load()
    dev = torch.device("cuda:0")
    spec = L.workload(args.config)
    log("bench: generating %s on the device" % spec.name)
    lay = G.layer_on_device(spec, dev)
    pl = PackedLayer(spec, lay["Wr"], lay["routed"], lay["shared"], path=args.path)
    # the stored (unpacked) copies are only needed by the CPU baseline; free HBM otherwise
    x = lay["x"] if spec.act == "f32" else lay["x"].view(torch.bfloat16)
    act_dt = torch.float32 if spec.act == "f32" else torch.bfloat16
    y = torch.empty((spec.T, spec.H), dtype=act_dt, device=dev)
    idx = torch.empty((spec.T, spec.k), dtype=torch.int32, device=dev)
    w = torch.empty((spec.T, spec.k), dtype=torch.float32, device=dev)
    bias = lay["bias"]

    def step():
        N.moe_layer_forward(pl.shape, x, pl.Wr, bias, pl.routed, pl.shared, y, idx, w, pl.ws)

    log("bench: warmup %d" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    counts = np.bincount(idx.cpu().numpy().reshape(-1), minlength=spec.E)
    traffic = pm.layer_traffic(spec, counts)

    log("bench: timing %d steps" % args.steps)
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
    log("bench: per-stage timing over %d steps" % args.steps)
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

    ceiling = None
    if not args.no_ceiling:
        # the achievable HBM read rate on this GPU: a plain streaming read of 4 GiB, 5 times
        buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        G.stream_read(buf, sink)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(5):
            G.stream_read(buf, sink)
        c1.record()
        torch.cuda.synchronize()
        ceiling = round(5 * buf.numel() / (c0.elapsed_time(c1) * 1e-3) / 1e9, 1)
        del buf

    mfma_ceiling = None
    a8 = spec.w_routed == "mxfp4a8"
    i8 = spec.w_routed == "int8"
    if not args.no_ceiling and (a8 or i8 or (spec.T * spec.k) / spec.E >= 64):
        # the matrix-core rates this GPU sustains with GEMM-like (changing, random) operands:
        # register-only MFMA bursts of the GEMMs' instruction kinds, 2 waves per SIMD
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
        mfma_ceiling = {}
        kinds = ((0, "bf16 16x16x32"), (1, "fp4 x fp8 16x16x128"), (2, "fp8 x fp8 16x16x128")) if a8 else \
            ((3, "int8 16x16x64"),) if i8 else ((0, "bf16 16x16x32"),)
        for kind, name in kinds:
            iters = 2048 if kind else 8192
            G.mfma_burst(kind, iters, 512, sink)
            m0, m1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            m0.record()
            fl = sum(G.mfma_burst(kind, iters, 512, sink) for _ in range(5))
            m1.record()
            torch.cuda.synchronize()
            mfma_ceiling[name] = round(fl / (m0.elapsed_time(m1) * 1e-3) / 1e12, 1)

    if args.calib_copy:
        # one plain copy of known size, the reference that scales the byte counters of a --pmc run
        nb = args.calib_copy << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        G.copy(src, torch.empty_like(src))
        torch.cuda.synchronize()
        log("bench: calibration copy of %d bytes" % nb)

    # roofline of the dominant kernel (the gate/up grouped GEMM, or the W4A8 gate/up stage), against
    # the roof that binds it: its algorithmic FLOPs at the MFMA peak of its instruction kinds, or its
    # algorithmic bytes at the HBM peak, whichever takes longer
    H, I, T, k = spec.H, spec.I, spec.T, spec.k
    R = T * k + (T if spec.shared else 0)
    ab = 4 if spec.act == "f32" else 2
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
    traffic_b = measured_traffic(args.config, "w4a8" if a8 else "int8" if i8 else "prefill" if prefill else "decode")
    hbm_ach = gu_bytes / (gu_ms * 1e-3) / 1e9
    hbm_roof = {"bound": "hbm", "achieved": round(hbm_ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(hbm_ach / HBM_PEAK_GBPS, 4),
                "frac_of_read_ceiling": round(hbm_ach / ceiling, 4) if ceiling else None}
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

    out = {
        "metric": METRIC,
        "value": round(T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.act,
        "data": "synthetic",
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
        "hbm_read_ceiling_GBps": ceiling,
        "mfma_sustained_TFLOPs": mfma_ceiling,
        "cpu_baseline": None,
    }

    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(spec, lay, args.cpu_tokens or CPU_TOKENS[args.config])
    print(json.dumps(out), flush=True)


def cpu_baseline(spec, lay, S):
    """The oracle, as it stands, on the first S tokens of the same layer (host cores)."""
    import numpy as np

    from inputgen import gpu as G
    from oracle import oracle as O

    S = min(S, spec.T)
    log("bench: CPU oracle on %d tokens" % S)
    x = lay["x_host"][:S]
    idx, wts, _ = O.route(x, lay["Wr_host"], lay["bias_host"], spec.k, spec.act)
    need = sorted(set(idx.reshape(-1).tolist()))
    routed = {k: None if v is None else G.to_numpy_stored(v[need]) for k, v in lay["routed"].items()}
    shared = None
    if spec.shared:
        shared = {k: None if v is None else G.to_numpy_stored(v[0]) for k, v in lay["shared"].items()}
    import os as _os
    cores = int(_os.environ.get("OMP_NUM_THREADS", _os.cpu_count() or 1))
    t = time.perf_counter()
    from inputgen.layers import act_to_f64
    idx, wts, _ = O.route(x, lay["Wr_host"], lay["bias_host"], spec.k, spec.act)
    off, st, ps = O.permute(idx, spec.E)
    u = act_to_f64(x, spec.act)
    yperm = np.zeros((S * spec.k, spec.H))
    for j, e in enumerate(need):
        r0, r1 = off[e], off[e + 1]
        one = {k: None if v is None else v[j] for k, v in routed.items()}
        yperm[r0:r1] = O.expert_ffn(u[st[r0:r1]], one, spec.w_routed)
    ysh = O.expert_ffn(u, shared, spec.w_shared) if spec.shared else None
    for tkn in range(S):
        O.combine_token(wts[tkn], yperm[ps[tkn * spec.k:(tkn + 1) * spec.k]], None if ysh is None else ysh[tkn])
    dt = time.perf_counter() - t
    cpu = None
    try:
        with open("/proc/cpuinfo") as fh:
            cpu = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), None)
    except OSError:
        pass
    return {"value": round(S / dt, 3), "unit": "tokens/s", "cores": cores, "kind": "oracle", "cpu": cpu,
            "sample": "first %d of %d tokens of the same layer (route, permute, %d active experts' SwiGLU%s, "
                      "combine), fp64 C oracle, %.1f s" % (S, spec.T, len(need),
                                                           " + shared expert" if spec.shared else "", dt)}


if __name__ == "__main__":
    main()
