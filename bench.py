"""Throughput of the deterministic MoE layer on one MI355X.

Default workload (the headline): one step = route -> plan -> forward -> backward ->
router backward over one batch of the bf16 workload T=4096, H=7168, I=2048, E=256,
k=8 with a shared expert (I_shared=2048) and Zipf(1.2)-skewed routing; all inputs
are synthetic and already resident in HBM.  Prints ONE JSON line with tokens/s
(from the timed steps alone), the roofline of the dominant kernel and per-kernel
MFMA / HBM / roofline fractions (from HIP events around each launch, recorded in a
second pass of the same number of steps: the events lengthen a step by about 1%),
and the fp64 oracle's throughput on a bounded sample of the same workload on the
host.

`--config` selects another workload of synth.CONFIGS: forward-only configs time
route -> plan -> forward; the MXFP8 ring config times the MX layer with its
weights quantised once before the timed region (the weight conversion runs once
per weight update and is reported on its own); `ep_share_bf16` is one GPU's share
of an expert-parallel layer (4 local experts x 4096 rows), compute-bound.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3, "mxfp8": 5000.0}
# rows from which an expert's bf16 weight gradients run on the 256 x 256 tiles (the
# library's split of the K-grouped wgrads)
WGRAD_HOT_ROWS = 256
# bytes of packed token range from which an expert's MXFP8 weight gradients run on the
# 256 x 256 tiles
MX_WGRAD_HOT_BYTES = 256
METRIC = "MoE layer tokens/s fwd+bwd @H7168 I2048 E256 top8, 1 GPU; % MFMA/HBM peak"


def kernel_work(name, sh, counts_mb, es=2):
    """Algorithmic (bytes, flops) of kernel `name` summed over its launches in one
    step, for the realised routing (counts_mb: per-minibatch expert row counts).

    Bytes count every operand once per launch: weights of the touched experts,
    activation rows read and written, gradients written; flops count 2 per
    multiply-add.  MXFP8 operands are 1 byte per element plus one scale byte per
    32."""
    T, H, I, E, k, Is = sh.T, sh.H, sh.I, sh.E, sh.k, sh.I_shared
    q = 1 + 1 / 32  # MXFP8 bytes per element with its scale
    mbs = [(sum(c), sum(1 for v in c if v > 0)) for c in counts_mb]  # (R_m, Et_m)
    n_mb = len(mbs)
    Tm = [min(sh.T_minibatch or T, T - m * (sh.T_minibatch or T)) for m in range(n_mb)]
    R = sum(r for r, _ in mbs)
    union = [sum(c[e] for c in counts_mb) for e in range(E)]
    Et = sum(1 for v in union if v > 0)
    # bf16 wgrads: experts with >= WGRAD_HOT_ROWS rows go to the 256-tile kernel when H
    # and I are multiples of 256; the 128-tile kernel keeps the rest and the zero
    # gradients of the experts without rows
    hot_split = es == 2 and H % 256 == 0 and I % 256 == 0 and not sh.T_minibatch
    Eh = sum(1 for v in union if v >= WGRAD_HOT_ROWS) if hot_split else 0
    Rh = sum(v for v in union if v >= WGRAD_HOT_ROWS) if hot_split else 0
    # MXFP8 wgrads: experts whose packed token range (their rows of all minibatches,
    # padded to 32) has >= MX_WGRAD_HOT_BYTES bytes go to the 256-tile kernel
    packed = [-(-union[e] // 32) * 32 for e in range(E)]
    mx_hot = [e for e in range(E) if packed[e] >= MX_WGRAD_HOT_BYTES] \
        if H % 256 == 0 and I % 256 == 0 else []
    Emx = len(mx_hot)
    Rmx = sum(union[e] for e in mx_hot)

    def over_mb(f, replayed=False):
        # replayed: the launch runs once more in the backward for every minibatch but
        # the last when the activations are replayed instead of kept
        b = fl = 0.0
        for m, ((Rm, Etm), tm) in enumerate(zip(mbs, Tm)):
            x, y = f(Rm, Etm, tm)
            n = 2 if replayed and sh.replay and m < n_mb - 1 else 1
            b += n * x
            fl += n * y
        return int(b), int(fl)

    w = {
        "route": lambda: (T * E * 4 + T * k * 8, 0),
        "route_backward": lambda: (T * k * 12 + T * E * 4, 0),
        "plan_hist": lambda: over_mb(lambda Rm, Etm, tm: (Rm * 4, 0)),
        "plan_scan": lambda: over_mb(lambda Rm, Etm, tm: (E * 12, 0)),
        "plan_scatter": lambda: over_mb(lambda Rm, Etm, tm: (Rm * 16, 0)),
        "dg_reduce": lambda: over_mb(lambda Rm, Etm, tm: (Rm * (I // 128) * 4 + Rm * 8, 0)),
        # X and dYu replays: each source row is read once and written to its k rows,
        # (1 + k) H b bytes per token, plus the pull list
        "gather_rows": lambda: (2 * ((T + R) * H * es + R * 4), 0),
        "combine_bf16": lambda: over_mb(lambda Rm, Etm, tm: (Rm * H * 2 + 2 * tm * H * 2 + tm * k * 8, 0)),
        "reverse_dispatch_bf16": lambda: over_mb(lambda Rm, Etm, tm: (Rm * H * 2 + 2 * tm * H * 2, 0)),
        # saved pre-activations Z are fp32 (4 bytes), h in the layer's dtype
        "gemm_up_swiglu": lambda: (Et * 2 * I * H * es + R * H * es + R * 2 * I * 4 + R * I * es,
                                   2 * R * H * 2 * I),
        "gemm_down": lambda: (Et * H * I * es + R * I * es + R * H * es, 2 * R * I * H),
        # the persistent forward: routed and shared GEMM1 + SwiGLU and GEMM2, combine
        "gemm_forward_fused": lambda: tuple(map(sum, zip(*(
            kernel_work(n, sh, counts_mb, es)
            for n in ("gemm_up_swiglu", "gemm_down", "combine_bf16")
            + (("gemm_up_swiglu_shared", "gemm_down_shared") if Is else ()))))),
        "fused_zero": lambda: (0, 0),
        "gemm_dgrad_down": lambda: (Et * H * I * es + R * H * es + R * 2 * I * 4 + R * 3 * I * es
                                    + R * (I // 128) * 4, 2 * R * H * I),
        # the wgrads also store the zero gradients of the E - Et experts without rows
        "gemm_wgrad_down": lambda: ((R - Rh) * (H + I) * es + (E - Eh) * H * I * es,
                                    2 * (R - Rh) * H * I),
        "gemm_wgrad_down_hot": lambda: (Rh * (H + I) * es + Eh * H * I * es, 2 * Rh * H * I),
        "gemm_dgrad_up": lambda: (Et * 2 * I * H * es + R * 2 * I * es + R * H * es, 2 * R * 2 * I * H),
        "gemm_wgrad_up": lambda: ((R - Rh) * (2 * I + H) * es + (E - Eh) * 2 * I * H * es,
                                  2 * (R - Rh) * 2 * I * H),
        "gemm_wgrad_up_hot": lambda: (Rh * (2 * I + H) * es + Eh * 2 * I * H * es,
                                      2 * Rh * 2 * I * H),
        "gemm_up_swiglu_shared": lambda: (2 * Is * H * 2 + T * H * 2 + T * 2 * Is * 4 + T * Is * 2,
                                          2 * T * H * 2 * Is),
        "gemm_down_shared": lambda: (Is * H * 2 + T * Is * 2 + T * H * 2, 2 * T * Is * H),
        "gemm_dgrad_down_shared": lambda: (Is * H * 2 + T * H * 2 + T * 2 * Is * 4 + T * 3 * Is * 2,
                                           2 * T * H * Is),
        "gemm_wgrad_down_shared": lambda: (T * H * 2 + T * Is * 2 + H * Is * 2, 2 * T * H * Is),
        "gemm_dgrad_up_shared": lambda: (2 * Is * H * 2 + T * 2 * Is * 2 + T * H * 2, 2 * T * 2 * Is * H),
        "gemm_wgrad_up_shared": lambda: (T * 2 * Is * 2 + T * H * 2 + 2 * Is * H * 2, 2 * T * 2 * Is * H),
        # MXFP8 path (per minibatch unless noted)
        # x (forward) and dy (backward) gathered into the ring and quantised: each
        # source row read once, its k rows written as E4M3 codes with scales
        "mx_quant_rows": lambda: tuple(a + b for a, b in zip(
            over_mb(lambda Rm, Etm, tm: (tm * H * 2 + Rm * H * q + Rm * 4, 0), replayed=True),
            over_mb(lambda Rm, Etm, tm: (tm * H * 2 + Rm * H * q + Rm * 4, 0)))),
        # the wgrad operands of the macro batch, quantised along each expert's tokens:
        # dy and x (bf16 sources read once per token), g h and dZ (fp32 rows), the
        # row maps
        "mx_quant_tokens": lambda: (int(2 * (T * H * 2 + R * H * q) + R * I * (4 + q)
                                        + R * 2 * I * (4 + q) + 4 * R * 4), 0),
        "mb_rows": lambda: (R * 20, 0),
        "mx_gemm_up_swiglu": lambda: over_mb(lambda Rm, Etm, tm: (
            Etm * 2 * I * H * q + Rm * H * q + Rm * 2 * I * 4 + Rm * I * q, 2 * Rm * H * 2 * I),
            replayed=True),
        "mx_gemm_down": lambda: over_mb(lambda Rm, Etm, tm: (
            Etm * H * I * q + Rm * I * q + Rm * H * 2, 2 * Rm * I * H)),
        "mx_gemm_dgrad_down": lambda: over_mb(lambda Rm, Etm, tm: (
            Etm * H * I * q + Rm * H * q + Rm * 2 * I * 4 + Rm * 2 * I * 4 + Rm * I * 4
            + Rm * 2 * I * q + Rm * (I // 128) * 4, 2 * Rm * H * I)),
        "mx_gemm_dgrad_up": lambda: over_mb(lambda Rm, Etm, tm: (
            Etm * 2 * I * H * q + Rm * 2 * I * q + Rm * H * 2, 2 * Rm * 2 * I * H)),
        # the MX wgrads also store the zero gradients of the E - Et experts without rows
        "mx_gemm_wgrad_down": lambda: (int((R - Rmx) * (H + I) * q + (E - Emx) * H * I * 2),
                                       2 * (R - Rmx) * H * I),
        "mx_gemm_wgrad_up": lambda: (int((R - Rmx) * (2 * I + H) * q + (E - Emx) * 2 * I * H * 2),
                                     2 * (R - Rmx) * 2 * I * H),
        "mx_gemm_wgrad_down_hot": lambda: (int(Rmx * (H + I) * q + Emx * H * I * 2), 2 * Rmx * H * I),
        "mx_gemm_wgrad_up_hot": lambda: (int(Rmx * (2 * I + H) * q + Emx * 2 * I * H * 2),
                                         2 * Rmx * 2 * I * H),
        "mx_zero_tail": lambda: ((2 * H + I + 2 * I) * 128, 0),  # both wgrads' operand rows
    }
    f = w.get(name)
    return f() if f else (0, 0)


def kernel_sources_sha256() -> str:
    """Hash of the HIP sources of the library (kernels and their headers) with their
    comments removed and whitespace collapsed, so that editing a comment does not
    invalidate the measurements keyed by it."""
    import hashlib
    import re
    d = os.path.join(ROOT, "mixture_experts_layer_plan_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp")):
            text = open(os.path.join(d, f), encoding="utf-8").read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            text = re.sub(r"//[^\n]*", "", text)
            text = re.sub(r"\s+", " ", text)
            h.update(f.encode())
            h.update(text.encode())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary of this workload, scaled by the copy-kernel calibration;
    None when there is none or the kernel sources changed since it was taken."""
    p = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("kernel_sources_sha256") != kernel_sources_sha256():
        return None
    k = d.get("kernels", {}).get(kernel)
    return None if k is None else int(k["fetch_bytes"] + k["write_bytes"])


def cpu_baseline(sh, inp, n_tokens):
    """The fp64 oracle, as it stands, on the first n_tokens tokens of the workload
    (forward + backward with every expert's weights streamed from the device)."""
    import numpy as np
    import torch

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    sl = slice(0, n_tokens)
    x = inp["x"][sl].cpu()
    logits = inp["logits"][sl].cpu()
    dy = inp["dy"][sl].cpu()
    shared = (inp["s_gate"], inp["s_up"], inp["s_down"]) if "s_gate" in inp else None
    t0 = time.perf_counter()
    c = oracle.layer_forward(x, logits, sh.k, inp["w_gate"], inp["w_up"], inp["w_down"],
                             shared=shared)
    g = oracle.layer_backward(c, dy)
    dt = time.perf_counter() - t0
    assert np.isfinite(g["dx"]).all()
    del torch
    return {"value": n_tokens / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n_tokens} tokens of the same workload, fwd+bwd, fp64 numpy, "
                      f"weights streamed one expert at a time ({dt:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="kimi_bf16_fwdbwd")
    ap.add_argument("--cpu-tokens", type=int, default=32)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one plain 1 GiB device copy first (counter calibration)")
    ap.add_argument("--dump-launches", default=None,
                    help="write the library's launch names of one timed step, in order, to this "
                         "file (to name the kernels of a profiler trace)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the layer; multi-GPU runs are not "
              "implemented (expert-parallel sharding is described in the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from mixture_experts_layer_plan_amd import LayerBuffers, binding, layer
    from mixture_experts_layer_plan_amd.layer import run_layer
    from synth import CONFIGS, make_inputs

    sh = CONFIGS[args.config]
    torch.cuda.set_device(0)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731
    log(f"[bench] generating {args.config} inputs on the device")
    inp = make_inputs(sh, seed=0, device="cuda", with_dy=sh.backward)
    b = LayerBuffers(sh.T, sh.H, sh.I, sh.E, sh.k, sh.I_shared, sh.dtype, backward=sh.backward,
                     router_gemm=sh.router == "gemm", T_minibatch=sh.T_minibatch,
                     replay=sh.replay, fused_forward=sh.fused_forward)
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    stream = torch.cuda.current_stream()
    mx = sh.dtype == "mxfp8"
    quant_ms = None
    if mx:
        # weights change once per optimiser step, not per layer pass: convert them
        # once here and time that conversion on its own
        layer.quantize_weights(b, inp)
        torch.cuda.synchronize()
        q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        q0.record(stream)
        layer.quantize_weights(b, inp)
        q1.record(stream)
        torch.cuda.synchronize()
        quant_ms = q0.elapsed_time(q1)

    def step():
        run_layer(b, inp, backward=sh.backward, quantize=False)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    n_mb = max(1, binding.moe_plan_layout_of(b.s).n_minibatch)
    counts_mb = [binding.plan_views(b.s, b.plan, m)["counts"].cpu().tolist() for m in range(n_mb)]
    counts = [sum(c[e] for c in counts_mb) for e in range(sh.E)]

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev0.elapsed_time(ev1)
    # per-kernel durations: the same steps again with HIP events around every launch
    # (kept out of the timed steps above, whose time they would lengthen)
    log(f"[bench] {args.steps} more steps with per-launch events")
    trace = binding.KernelTrace(capacity=96 * max(args.steps, 1))
    tr0, tr1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    tr0.record(stream)
    with trace:
        for _ in range(args.steps):
            step()
    tr1.record(stream)
    torch.cuda.synchronize()
    ms_total_traced = tr0.elapsed_time(tr1)
    recs = trace.records()
    trace.close()
    if args.dump_launches:
        per_step = len(recs) // max(args.steps, 1)
        with open(args.dump_launches, "w") as f:
            f.write("\n".join(n for n, _ in recs[:per_step]) + "\n")
    ms_per_step = ms_total / max(args.steps, 1)
    tokens_per_s = sh.T / (ms_per_step / 1e3)

    # per-kernel averages over the timed region; work per step from the routing
    es = 4 if sh.dtype == "f32" else 2
    peak_flops = MFMA_PEAK_TFLOPS["mxfp8" if mx else sh.dtype] * 1e12
    agg = {}
    for name, ms in recs:
        a = agg.setdefault(name, [0.0, 0])
        a[0] += ms
        a[1] += 1
    kernels = {}
    for name, (tot, n) in sorted(agg.items(), key=lambda kv: -kv[1][0]):
        byt, flop = kernel_work(name, sh, counts_mb, es)
        pk = peak_flops if name.startswith("mx_gemm") else MFMA_PEAK_TFLOPS[
            "f32" if sh.dtype == "f32" else "bf16"] * 1e12
        t_step = tot / max(args.steps, 1) / 1e3  # seconds per step
        t_roof = max(byt / (HBM_PEAK_GBS * 1e9), flop / pk)
        kernels[name] = {"avg_ms": round(tot / n, 4), "launches_per_step": n // max(args.steps, 1),
                         "share": round(tot / max(ms_total_traced, 1e-9), 4),
                         "GB_s": round(byt / t_step / 1e9, 1) if byt else None,
                         "TFLOP_s": round(flop / t_step / 1e12, 1) if flop else None,
                         "hbm_frac": round(byt / t_step / (HBM_PEAK_GBS * 1e9), 4) if byt else None,
                         "mfma_frac": round(flop / t_step / pk, 4) if flop else None,
                         "roof_frac": round(t_roof / t_step, 4) if t_roof else None}
    dom = max(agg, key=lambda n: agg[n][0])
    byt, flop = kernel_work(dom, sh, counts_mb, es)
    n_launch = agg[dom][1] // max(args.steps, 1)
    byt, flop = byt // max(n_launch, 1), flop // max(n_launch, 1)  # per launch
    avg_s = agg[dom][0] / agg[dom][1] / 1e3
    pk = peak_flops if dom.startswith("mx_gemm") else MFMA_PEAK_TFLOPS[
        "f32" if sh.dtype == "f32" else "bf16"] * 1e12
    t_hbm, t_mfma = byt / (HBM_PEAK_GBS * 1e9), flop / pk
    if t_mfma > t_hbm:
        roof = {"bound": "mfma", "achieved": round(flop / avg_s / 1e12, 2),
                "peak": pk / 1e12, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(byt / avg_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(dom, args.config)
    roof["kernel"] = dom
    roof["algorithmic_bytes"] = byt
    roof["algorithmic_flops"] = flop

    cpu = None
    if not args.no_cpu_baseline and args.config == "kimi_bf16_fwdbwd":
        log(f"[bench] oracle on {args.cpu_tokens} tokens (cpu baseline)")
        cpu = cpu_baseline(sh, inp, args.cpu_tokens)

    passes = "fwd+bwd" if sh.backward else "fwd"
    metric = METRIC if args.config == "kimi_bf16_fwdbwd" else (
        f"MoE layer tokens/s {passes} @H{sh.H} I{sh.I} E{sh.E} top{sh.k}, 1 GPU; "
        f"% MFMA/HBM peak")
    desc = (f"{args.config}: {sh.dtype} MoE layer {passes}, T={sh.T} H={sh.H} I={sh.I} E={sh.E} "
            f"top-{sh.k}" + (f", shared expert I={sh.I_shared}" if sh.I_shared else "")
            + (f", Zipf({sh.zipf_s}) routing" if sh.zipf_s else "")
            + (f", minibatches of {sh.T_minibatch}" if sh.T_minibatch else "")
            + (", activations of all but the last minibatch replayed" if sh.replay else "")
            + (", up/gate and down GEMMs in one persistent launch" if sh.fused_forward else ""))
    out = {
        "metric": metric, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "f32": "f32", "mxfp8": "fp8-e4m3 (MX) + bf16"}[sh.dtype],
        "data": "synthetic",
        "config": {"workload": desc, "T": sh.T, "H": sh.H, "I": sh.I,
                   "E": sh.E, "k": sh.k, "I_shared": sh.I_shared, "parallelism": "single GPU",
                   "experts_touched": int(sum(1 for c in counts if c > 0)),
                   "max_rows_per_expert": int(max(counts))},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "wall_s_timed": round(wall, 3),
        "ms_per_step_with_kernel_events": round(ms_total_traced / max(args.steps, 1), 4),
    }
    if quant_ms is not None:
        out["config"]["T_minibatch"] = sh.T_minibatch
        out["mx_weight_quantisation_ms"] = round(quant_ms, 4)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
