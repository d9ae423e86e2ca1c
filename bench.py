"""Throughput of the deterministic MoE layer (forward + backward) on one MI355X.

One step = route -> plan -> forward -> backward -> router backward over one batch of
the bf16 workload T=4096, H=7168, I=2048, E=256, k=8 with a shared expert
(I_shared=2048) and Zipf(1.2)-skewed routing; all inputs are synthetic and already
resident in HBM.  Prints ONE JSON line with tokens/s, the roofline of the dominant
kernel (timed live with HIP events around each launch over the timed region) and
the fp64 oracle's throughput on a bounded sample of the same workload on the host.
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
METRIC = "MoE layer tokens/s fwd+bwd @H7168 I2048 E256 top8, 1 GPU; % MFMA/HBM peak"


def kernel_work(name, sh, counts, es=2):
    """Algorithmic (bytes, flops) of one launch of kernel `name` for this routing.

    Bytes count every operand once: weights of the touched experts, activation
    rows read and written, gradients written; flops count 2 per multiply-add."""
    T, H, I, E, k, Is = sh.T, sh.H, sh.I, sh.E, sh.k, sh.I_shared
    R = int(sum(counts))
    Et = int(sum(1 for c in counts if c > 0))
    w = {
        "route": (T * E * 4 + T * k * 8, 0),
        "plan_hist": (R * 4, 0), "plan_scan": (E * 12, 0), "plan_scatter": (R * 16, 0),
        # saved pre-activations Z are fp32 (4 bytes), h bf16
        "gemm_up_swiglu": (Et * 2 * I * H * es + R * H * es + R * 2 * I * 4 + R * I * es,
                           2 * R * H * 2 * I),
        "gemm_down": (Et * H * I * es + R * I * es + R * H * es, 2 * R * I * H),
        "gemm_up_swiglu_shared": (2 * Is * H * es + T * H * es + T * 2 * Is * 4 + T * Is * es,
                                  2 * T * H * 2 * Is),
        "gemm_down_shared": (Is * H * es + T * Is * es + T * H * es, 2 * T * Is * H),
        "combine_bf16": (R * H * es + 2 * T * H * es + T * k * 8, 0),
        "gemm_dgrad_down": (Et * H * I * es + R * H * es + R * 2 * I * 4 + R * 3 * I * es
                            + R * (I // 128) * 4, 2 * R * H * I),
        "dg_reduce": (R * (I // 128) * 4 + R * 8, 0),
        "zero_empty_experts": ((E - Et) * 3 * I * H * es, 0),
        # the wgrads also store the zero gradients of the E - Et experts without rows
        "gemm_wgrad_down": (R * H * es + R * I * es + E * H * I * es, 2 * R * H * I),
        "gemm_dgrad_up": (Et * 2 * I * H * es + R * 2 * I * es + R * H * es, 2 * R * 2 * I * H),
        "gemm_wgrad_up": (R * 2 * I * es + R * H * es + E * 2 * I * H * es, 2 * R * 2 * I * H),
        "gemm_dgrad_down_shared": (Is * H * es + T * H * es + T * 2 * Is * 4 + T * 3 * Is * es,
                                   2 * T * H * Is),
        "gemm_wgrad_down_shared": (T * H * es + T * Is * es + H * Is * es, 2 * T * H * Is),
        "gemm_dgrad_up_shared": (2 * Is * H * es + T * 2 * Is * es + T * H * es, 2 * T * 2 * Is * H),
        "gemm_wgrad_up_shared": (T * 2 * Is * es + T * H * es + 2 * Is * H * es, 2 * T * 2 * Is * H),
        "reverse_dispatch_bf16": (R * H * es + 2 * T * H * es, 0),
        "gather_rows": (2 * R * H * es + R * 4, 0),
        "route_backward": (T * k * 12 + T * E * 4, 0),
    }
    return w.get(name, (0, 0))


def kernel_sources_sha256() -> str:
    """Hash of the HIP sources of the library (kernels and their headers)."""
    import hashlib
    d = os.path.join(ROOT, "mixture_experts_layer_plan_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp")):
            h.update(f.encode())
            h.update(open(os.path.join(d, f), "rb").read())
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
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU's share of the layer; runs on more than one GPU are "
              "not part of this build (see the sharding design notes).", file=sys.stderr)
        sys.exit(2)

    import torch

    from mixture_experts_layer_plan_amd import LayerBuffers, binding
    from mixture_experts_layer_plan_amd.layer import run_layer
    from synth import CONFIGS, make_inputs

    sh = CONFIGS[args.config]
    if sh.dtype != "bf16" or not sh.backward:
        raise SystemExit(f"bench config {args.config} is not a bf16 forward+backward workload")
    torch.cuda.set_device(0)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)  # noqa: E731
    log(f"[bench] generating {args.config} inputs on the device")
    inp = make_inputs(sh, seed=0, device="cuda", with_dy=True)
    b = LayerBuffers(sh.T, sh.H, sh.I, sh.E, sh.k, sh.I_shared, "bf16", backward=True)
    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        run_layer(b, inp, backward=True)
    torch.cuda.synchronize()
    counts = b.plan_views()["counts"].cpu().tolist()

    trace = binding.KernelTrace(capacity=64 * max(args.steps, 1))
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    with trace:
        for _ in range(args.steps):
            run_layer(b, inp, backward=True)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev0.elapsed_time(ev1)
    recs = trace.records()
    trace.close()
    ms_per_step = ms_total / max(args.steps, 1)
    tokens_per_s = sh.T / (ms_per_step / 1e3)

    # per-kernel averages over the timed region
    agg = {}
    for name, ms in recs:
        a = agg.setdefault(name, [0.0, 0])
        a[0] += ms
        a[1] += 1
    kernels = {}
    for name, (tot, n) in sorted(agg.items(), key=lambda kv: -kv[1][0]):
        byt, flop = kernel_work(name, sh, counts)
        avg_s = tot / n / 1e3
        kernels[name] = {"avg_ms": round(tot / n, 4), "launches": n,
                         "share": round(tot / max(ms_total, 1e-9), 4),
                         "GB_s": round(byt / avg_s / 1e9, 1) if byt else None,
                         "TFLOP_s": round(flop / avg_s / 1e12, 1) if flop else None}
    dom = max(agg, key=lambda n: agg[n][0])
    byt, flop = kernel_work(dom, sh, counts)
    avg_s = agg[dom][0] / agg[dom][1] / 1e3
    t_hbm, t_mfma = byt / (HBM_PEAK_GBS * 1e9), flop / (MFMA_PEAK_TFLOPS["bf16"] * 1e12)
    if t_mfma > t_hbm:
        roof = {"bound": "mfma", "achieved": round(flop / avg_s / 1e12, 2),
                "peak": MFMA_PEAK_TFLOPS["bf16"], "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": round(byt / avg_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = measured_traffic(dom, args.config)
    roof["kernel"] = dom
    roof["algorithmic_bytes"] = byt
    roof["algorithmic_flops"] = flop

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] oracle on {args.cpu_tokens} tokens (cpu baseline)")
        cpu = cpu_baseline(sh, inp, args.cpu_tokens)

    out = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: bf16 MoE layer fwd+bwd, T={sh.T} H={sh.H} "
                               f"I={sh.I} E={sh.E} top-{sh.k}, shared expert I={sh.I_shared}, "
                               f"Zipf({sh.zipf_s}) routing", "T": sh.T, "H": sh.H, "I": sh.I,
                   "E": sh.E, "k": sh.k, "I_shared": sh.I_shared, "parallelism": "single GPU",
                   "experts_touched": int(sum(1 for c in counts if c > 0)),
                   "max_rows_per_expert": int(max(counts))},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
