"""Benchmark of the tensor-parallel MLP shard step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
tpmlp_fwd (Z_i = X·A_i with the GeLU epilogue, P_i = Y_i·B_i) for all t shards,
tpmlp_reduce_partials (O = Σ P_i), tpmlp_bwd (D_i with the GeLU' epilogue,
dB_i, dA_i, dX_i) and tpmlp_reduce_partials (dX = Σ dX_i).

Workload: the GPT-8.3B-shaped layer, h = 3072, m = 4h = 12288, t = 8, so
A_i is 3072×1536 and B_i 1536×3072; n = b·s = 8·1024 = 8192 tokens; bf16 with
fp32 accumulation; all 8 shards resident on the one GPU and summed locally.
FLOPs per step = 6 GEMMs × 2·n·d·m_i × t = 12·n·d·m_i·t (GeLU math and the
reductions are not counted).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Prints one JSON line.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU × 2.4 GHz × 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
METRIC = "TP-MLP shard fwd+bwd TFLOP/s (bf16) and % of MI355X MFMA peak"
WORKLOAD = "gpt8p3b_t8"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate budget of the oracle timing on the host")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain device copy of 512 MiB (read 512 MiB, write 512 MiB), "
                         "the reference kernel for scaling FETCH_SIZE / WRITE_SIZE counters")
    return ap.parse_args()


def cpu_baseline(inp, t, budget_s):
    """Time the fp64 oracle (forward + backward of whole shards, full n) on the
    host cores until the budget is used; report its FLOP rate."""
    import numpy as np
    import threadpoolctl

    from oracle import mlp as om

    X, G = inp["X"].f64, inp["G"].f64
    A, B = inp["A"].f32, inp["B"].f32
    n, d = X.shape
    mi = A.shape[1] // t
    info = threadpoolctl.threadpool_info()
    threads = max((i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"), default=1)
    shards, t0 = 0, time.perf_counter()
    while shards < 4 * t:  # whole shards, cycling, until the budget is used
        i = shards % t
        Ai = A[:, i * mi:(i + 1) * mi].astype(np.float64)
        Bi = B[i * mi:(i + 1) * mi, :].astype(np.float64)
        Z, Y, P = om.shard_forward(X, Ai, Bi)
        om.shard_backward(X, Ai, Bi, Z, Y, G)
        shards += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    flops = 12.0 * n * d * mi * shards
    return {"value": round(flops / el / 1e12, 4), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{shards} whole-shard passes (of {t} shards), full n={n}: fp64 NumPy forward + "
                      f"backward ({flops:.3e} FLOP in {el:.1f} s); host logical CPUs {os.cpu_count()}, "
                      f"affinity {len(os.sched_getaffinity(0))}"}


def recorded_traffic(kernel_file, summary):
    """HBM bytes per launch recorded from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
    in a profiles/ summary, or None when the summary is missing or the kernel
    source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if ":" in line and line.split(":", 1)[0].strip() in ("source_sha256", "traffic_bytes_per_launch"):
            k, v = line.split(":", 1)
            rec[k.strip()] = v.strip()
    src = open(os.path.join(ROOT, "megatron_tensor_transformer_amd", "csrc", kernel_file), "rb").read()
    if rec.get("source_sha256") != hashlib.sha256(src).hexdigest():
        return None
    try:
        return float(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(every box here has one GPU; the path would shard one TP rank per GPU).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import megatron_tensor_transformer_amd as tp
    from tpmlp_inputs import CONFIGS, config_inputs

    cfg = CONFIGS[WORKLOAD]
    n, d, m, t = cfg["n"], cfg["d"], cfg["m"], cfg["t"]
    mi = m // t
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    inp = config_inputs(WORKLOAD, seed=0)

    def to_dev(T):
        return torch.from_numpy(T.bits.view(np.int16)).view(torch.bfloat16).to(dev)

    X, A, B, G = (to_dev(inp[k]) for k in "XABG")
    A_s = A.reshape(d, t, mi).permute(1, 0, 2).contiguous()
    B_s = B.reshape(t, mi, d).contiguous()
    del A, B
    bf = torch.bfloat16
    Z = torch.empty((t, n, mi), dtype=bf, device=dev)
    Y = torch.empty_like(Z)
    P = torch.empty((t, n, d), dtype=bf, device=dev)
    O = torch.empty((n, d), dtype=bf, device=dev)
    D = torch.empty_like(Z)
    dA = torch.empty((t, d, mi), dtype=torch.float32, device=dev)
    dB = torch.empty((t, mi, d), dtype=torch.float32, device=dev)
    dXp = torch.empty_like(P)
    dX = torch.empty_like(O)
    nb = tp.bwd_workspace_bytes(X, A_s)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev) if nb else None
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        tp.tpmlp_fwd(X, A_s, B_s, Z, Y, P, stream)
        if ev is not None:
            ev[1].record(stream)
        tp.tpmlp_reduce_partials(P, O, stream)
        if ev is not None:
            ev[2].record(stream)
        tp.tpmlp_bwd(X, A_s, B_s, Z, Y, G, D, dA, dB, dXp, ws, stream)
        if ev is not None:
            ev[3].record(stream)
        tp.tpmlp_reduce_partials(dXp, dX, stream)
        if ev is not None:
            ev[4].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # timed region: K whole steps, events around each entry point
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t_wall0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0

    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    r1_ms = [e[1].elapsed_time(e[2]) for e in evs]
    bwd_ms = [e[2].elapsed_time(e[3]) for e in evs]
    r2_ms = [e[3].elapsed_time(e[4]) for e in evs]
    step_ms = [e[0].elapsed_time(e[4]) for e in evs]
    ms = float(np.mean(step_ms))
    flops = 12.0 * n * d * mi * t
    value = flops / (ms * 1e-3) / 1e12
    gemm_ms = float(np.mean(fwd_ms) + np.mean(bwd_ms))
    gemm_tflops = flops / (gemm_ms * 1e-3) / 1e12
    per_launch_flop = 2.0 * n * d * mi * t          # every one of the six GEMMs
    avg_launch_ms = gemm_ms / 6.0
    achieved = per_launch_flop / (avg_launch_ms * 1e-3) / 1e12
    red_bytes = (t + 1) * n * d * 2                 # t bf16 partials read, one bf16 sum written
    red_ms = float(np.mean(r1_ms + r2_ms))
    red_gbs = red_bytes / (red_ms * 1e-3) / 1e9

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weights, N(0,1e-4) grads)",
        "config": {"workload": "GPT-8.3B-shaped TP-MLP layer, h=3072, m=4h=12288, t=8 shards "
                               "resident on one GPU (A_i 3072x1536, B_i 1536x3072), n=b*s=8*1024",
                   "n": n, "d": d, "m": m, "t": t, "m_i": mi, "parallelism": "tp8 simulated on 1 GPU"},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "gemm_only": {"tflops": round(gemm_tflops, 2),
                      "pct_of_peak": round(100.0 * gemm_tflops / PEAK_BF16_TFLOPS, 2),
                      "fwd_ms": round(float(np.mean(fwd_ms)), 4), "bwd_ms": round(float(np.mean(bwd_ms)), 4)},
        "roofline": {"bound": "mfma", "kernel": "gemm_bf16_kernel, average over the 6 launches of a step",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic("gemm_bf16.hip", "gemm_bf16_gpt8p3b_t8_traffic.md"),
                     "flop_per_launch": per_launch_flop, "avg_launch_ms": round(avg_launch_ms, 4)},
        "roofline_reduce": {"bound": "hbm", "kernel": "reduce_vec8_kernel",
                            "achieved": round(red_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(red_gbs / PEAK_HBM_GBS, 4),
                            "traffic": recorded_traffic("reduce.hip", "reduce_gpt8p3b_t8_traffic.md"),
                            "bytes_per_launch": red_bytes, "avg_launch_ms": round(red_ms, 4)},
        "wall_s_timed": round(wall, 3),
        "step_ms_min_max": [round(min(step_ms), 4), round(max(step_ms), 4)],
    }
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(inp, t, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
