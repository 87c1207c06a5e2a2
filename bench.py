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

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-extra]

Prints one JSON line.  The engine clock is sampled from the host during the
timed steps (`sclk_mhz`).  Besides the headline step it reports (unless
--no-extra): the per-rank rate (one shard per launch, t_local = 1, as one TP
rank runs it), the single-shard layer (n = 2048, d = 1024, m = 4096, t = 1),
the GPT-1T-shaped shard (n = 2048, d = 25600, m_i = 12800, one shard), the
sequence-parallel region's memory-bound kernels on the h = 4096 block (LN
forward, reduce + dropout + residual, dropout backward, LN backward with the
fused dU reduce) in GB/s against 8 TB/s, each timed after writing a 512 MiB
scratch buffer so the 256 MiB last-level cache holds none of its inputs, the
whole sequence-parallel block step on that block, the biased layer, the
attention side and the vocabulary-parallel cross-entropy.
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
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 (matrix cores; the vector units' figure is the same)
GEMM_LAUNCHES = 4           # GEMM core launches per step
METRIC = "TP-MLP shard fwd+bwd TFLOP/s (bf16) and % of MI355X MFMA peak"
WORKLOAD = "gpt8p3b_t8"
LEGS = ("biased_step", "per_rank", "c2", "gpt1t_shard", "sp_region", "c5_block", "attention", "vocab_ce",
        "fp32_path")
OPTIONAL_LEGS = ("library_yardsticks",)  # only when named in --legs


TILE_POLICIES = {"auto": 0, "256": 1, "192": 2, "tail": 3, "128": 4}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip every leg besides the headline step")
    ap.add_argument("--legs", default=None,
                    help="comma-separated subset of the extra legs to run (default: all of " + ",".join(LEGS)
                    + "); also " + ",".join(OPTIONAL_LEGS) + " (library kernels on the same shapes, as context)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate budget of the oracle timing on the host")
    ap.add_argument("--cpu-all-configs", action="store_true",
                    help="also time the oracle once on every configuration (3x4 worked example, the "
                         "single-shard layer, the 8.3B-shaped layer, the GPT-1T-shaped shard, the h=4096 "
                         "sequence-parallel block); about a minute of host time")
    ap.add_argument("--gemm-tile-policy", choices=sorted(TILE_POLICIES), default="auto",
                    help="the bf16 GEMMs' tile and schedule policy (tpmlp_set_gemm_tile_policy): auto (the "
                         "library's choice per launch), 256 (256x256 tiles only, no K-split tail), 192 or 128 "
                         "(narrow tiles wherever available), tail (a K-split tail wherever available); for A/B "
                         "timing, the results do not depend on it beyond the tail's fp32 rounding")
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


def cpu_all_configs():
    """The fp64 oracle, forward + backward, once per configuration on the
    host's cores (small ones: median of 5), with the BLAS it ran on."""
    import threadpoolctl

    from oracle import mlp as om
    from oracle import sp_block as osp
    from tpmlp_inputs import CONFIGS, config_inputs

    info = threadpoolctl.threadpool_info()
    blas = [{k: i.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer")}
            for i in info if i.get("user_api") == "blas"]
    out = {"host_logical_cpus": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)), "blas": blas}
    for name in ("worked_example", "single_shard", "gpt8p3b_t8", "gpt1t_t8_shard0", "sp_block_t8"):
        c = CONFIGS[name]
        t0 = time.perf_counter()
        inp = config_inputs(name, seed=0)
        gen_s = time.perf_counter() - t0
        n, d, m, t = c["n"], c["d"], c["m"], c["t"]
        mi = m // t
        if c["kind"] == "sp":
            v = {k: inp[k].f64 for k in ("x", "A", "B", "G", "gamma", "beta")}

            def run():
                f = osp.sp_forward(v["x"], v["gamma"], v["beta"], c["eps"], v["A"], v["B"], t, c["p"],
                                   c["mask_seed"])
                osp.sp_backward(f, v["gamma"], v["A"], v["B"], v["G"], t, c["p"])
            flops = 12.0 * n * d * mi * t
        elif c.get("shards"):
            X, A, B, G = (inp[k].f64 for k in "XABG")

            def run():
                Z, Y, P = om.shard_forward(X, A, B)
                om.shard_backward(X, A, B, Z, Y, G)
            flops = 12.0 * n * d * mi * len(c["shards"])
        else:
            X, A, B, G = (inp[k].f64 for k in "XABG")

            def run():
                f = om.tp_forward(X, A, B, t)
                om.tp_backward(X, A, B, f, G)
            flops = 12.0 * n * d * mi * t
        reps = 5 if flops < 1e12 else 1
        times = []
        for _ in range(reps):
            t0 = time.perf_counter()
            run()
            times.append(time.perf_counter() - t0)
        w = sorted(times)[len(times) // 2]
        out[name] = {"flop": flops, "wall_s": round(w, 6), "gflops": round(flops / w / 1e9, 2),
                     "reps": reps, "input_generation_s": round(gen_s, 2)}
    return out


class ClockSampler:
    """Samples the GPU's engine clock (and socket power) from the host every
    `period` seconds while the timed loop runs, through the AMD SMI library's
    GPU metrics table (per-XCD current gfx clocks), so the result can be read
    against the clock the peak assumes.  Host-side only: it never touches the
    GPU's command queues."""

    def __init__(self, period=0.005):
        import threading
        self.period = period
        self.samples = []   # (mean over XCDs of the current gfx clock in MHz, socket power W or None)
        self.error = None
        self._stop = threading.Event()
        self._thread = None
        self._handle = None
        self._smi = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            self._smi = amdsmi
            self._handle = self._pick(amdsmi, handles)
        except Exception as e:  # no SMI library or no access: report why
            self.error = f"{type(e).__name__}: {e}"

    @staticmethod
    def _pick(amdsmi, handles):
        """The handle of cuda:0, matched by PCI bus id when torch exposes it."""
        import torch
        if len(handles) == 1:
            return handles[0]
        try:
            pr = torch.cuda.get_device_properties(0)
            bus = (int(pr.pci_domain_id), int(pr.pci_bus_id), int(pr.pci_device_id))
            for h in handles:
                bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)  # "dddd:bb:dd.f"
                dom, b, df = bdf.split(":")
                if (int(dom, 16), int(b, 16), int(df.split(".")[0], 16)) == bus:
                    return h
        except Exception:
            pass
        return handles[0]

    def read(self):
        m = self._smi.amdsmi_get_gpu_metrics_info(self._handle)
        clks = m.get("current_gfxclks")
        vals = [c for c in clks if isinstance(c, (int, float)) and 0 < c < 10000] if isinstance(clks, list) else []
        if not vals:
            c = m.get("current_gfxclk")
            vals = [c] if isinstance(c, (int, float)) and 0 < c < 10000 else []
        pw = m.get("current_socket_power")
        if not isinstance(pw, (int, float)) or not 0 < pw < 5000:
            pw = m.get("average_socket_power")
        pw = pw if isinstance(pw, (int, float)) and 0 < pw < 5000 else None
        return (sum(vals) / len(vals) if vals else None), pw

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self.read())
            except Exception as e:
                self.error = f"{type(e).__name__}: {e}"
                return
            self._stop.wait(self.period)

    def start(self):
        import threading
        if self._handle is None:
            return
        self._thread = threading.Thread(target=self._run, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()

    def summary(self):
        import numpy as np
        # the metrics table refreshes on its own schedule: samples before its
        # first refresh repeat the reading taken before the load and are left
        # out (all of them, when it never refreshed)
        first = self.samples[0][0] if self.samples else None
        k = next((i for i, (c, _) in enumerate(self.samples) if c != first), None)
        live = self.samples[k:] if k is not None else []
        clk = [c for c, _ in live if c is not None]
        pw = [p for _, p in live if p is not None]
        out = {"source": "AMD SMI GPU metrics, mean over XCDs of current_gfxclks, sampled every "
                         f"{int(self.period * 1000)} ms",
               "samples": len(self.samples), "samples_after_first_refresh": len(clk)}
        if clk:
            out.update({"median_mhz": round(float(np.median(clk)), 1), "min_mhz": round(float(np.min(clk)), 1),
                        "max_mhz": round(float(np.max(clk)), 1),
                        "frac_of_2400": round(float(np.median(clk)) / 2400.0, 4)})
        if pw:
            out["socket_power_w_median"] = round(float(np.median(pw)), 1)
        if self.error:
            out["error"] = self.error
        return out


def _stats(ms):
    import numpy as np
    return {"median_ms": round(float(np.median(ms)), 4), "min_ms": round(float(np.min(ms)), 4),
            "max_ms": round(float(np.max(ms)), 4)}


def _time_events(fn, reps, before=None):
    """Run fn() reps times on the current stream, each bracketed by events
    (before() runs outside the bracket); returns the per-rep milliseconds."""
    import torch
    out = []
    for _ in range(reps):
        if before is not None:
            before()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        e1.synchronize()
        out.append(e0.elapsed_time(e1))
    return out


def _time_batched(fn, reps, inner):
    """Like _time_events, but each bracket holds `inner` back-to-back calls
    (for steps short enough that the host's launch latency would otherwise
    show); returns the per-call milliseconds of each bracket."""
    import torch
    out = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(inner):
            fn()
        e1.record()
        e1.synchronize()
        out.append(e0.elapsed_time(e1) / inner)
    return out


def leg_mlp_shard(tp, n, d, mi, reps, seed, inner=1):
    """fwd + bwd GEMMs of one shard per launch (t_local = 1) on seeded device
    data of the given shape: the rate one TP rank sees."""
    import torch
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    bf = torch.bfloat16

    def rnd(shape, std):
        return (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * std).to(bf)

    X, G = rnd((n, d), 1.0), rnd((n, d), 0.01)
    A, B = rnd((1, d, mi), 0.02), rnd((1, mi, d), 0.02)
    Z = torch.empty((1, n, mi), dtype=bf, device=dev)
    Y, D = torch.empty_like(Z), torch.empty_like(Z)
    P, dXp = torch.empty((1, n, d), dtype=bf, device=dev), torch.empty((1, n, d), dtype=bf, device=dev)
    dA = torch.empty((1, d, mi), dtype=torch.float32, device=dev)
    dB = torch.empty((1, mi, d), dtype=torch.float32, device=dev)

    wsf = tp.workspace(tp.fwd_workspace_bytes(X, A), dev)
    wsb = tp.workspace(tp.bwd_workspace_bytes(X, A), dev)

    def run():
        tp.tpmlp_fwd(X, A, B, Z, Y, P, wsf)
        tp.tpmlp_bwd(X, A, B, Z, Y, G, D, dA, dB, dXp, wsb)

    for _ in range(3):
        run()
    ms = _time_events(run, reps) if inner == 1 else _time_batched(run, reps, inner)
    import numpy as np
    med = float(np.median(ms))
    flops = 12.0 * n * d * mi
    return {"n": n, "d": d, "m_i": mi, "t_local": 1, "flop": flops, "steps_per_timing": inner,
            "tflops_median": round(flops / (med * 1e-3) / 1e12, 2),
            "pct_of_peak": round(100.0 * flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2), **_stats(ms)}


def leg_fp32(tp, reps):
    """The fp32 path (the single-card numeric-alignment path) on the 8.3B-shaped
    layer: the same step as the headline (8 shards' forward, the partial sum,
    their backward, the partial sum) with fp32 tensors throughout; its GEMMs
    run v_mfma_f32_32x32x2_f32.  TFLOP/s against the fp32 dense peak."""
    import numpy as np
    import torch
    from tpmlp_inputs import CONFIGS
    cfg = CONFIGS["gpt8p3b_t8"]
    n, d, m, t = cfg["n"], cfg["d"], cfg["m"], cfg["t"]
    mi = m // t
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    f32 = torch.float32

    def rnd(shape, std):
        return torch.randn(shape, generator=gen, device=dev, dtype=f32) * std

    X, G = rnd((n, d), 1.0), rnd((n, d), 0.01)
    A, B = rnd((t, d, mi), 0.02), rnd((t, mi, d), 0.02)
    Z, Y, D = (torch.empty((t, n, mi), dtype=f32, device=dev) for _ in range(3))
    P, dXp = (torch.empty((t, n, d), dtype=f32, device=dev) for _ in range(2))
    dA, dB = torch.empty((t, d, mi), dtype=f32, device=dev), torch.empty((t, mi, d), dtype=f32, device=dev)
    O, dX = torch.empty((n, d), dtype=f32, device=dev), torch.empty((n, d), dtype=f32, device=dev)

    def run():
        tp.tpmlp_fwd(X, A, B, Z, Y, P)
        tp.tpmlp_reduce_partials(P, O)
        tp.tpmlp_bwd(X, A, B, Z, Y, G, D, dA, dB, dXp)
        tp.tpmlp_reduce_partials(dXp, dX)

    run()
    torch.cuda.synchronize()
    ms = _time_events(run, reps)
    med = float(np.median(ms))
    flops = 12.0 * n * d * mi * t
    return {"workload": f"fp32 path of the 8.3B-shaped layer: n={n}, d={d}, m_i={mi}, t={t}, fp32 tensors",
            "flop": flops, "tflops_median": round(flops / (med * 1e-3) / 1e12, 2),
            "pct_of_fp32_peak": round(100.0 * flops / (med * 1e-3) / 1e12 / PEAK_FP32_TFLOPS, 2), **_stats(ms)}


def leg_sp(tp, reps):
    """The sequence-parallel region's memory-bound kernels on the h = 4096
    block (s = 4096 tokens, t = 8 shards of 512 rows), each timed alone after
    a cache flush; algorithmic bytes count each tensor read or written once."""
    import numpy as np
    import torch
    from tpmlp_inputs import CONFIGS
    cfg = CONFIGS["sp_block_t8"]
    s, h, t, p = cfg["n"], cfg["d"], cfg["t"], cfg["p"]
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    bf = torch.bfloat16
    x = torch.randn((s, h), generator=gen, device=dev).to(bf)
    gamma = (1 + 0.1 * torch.randn((h,), generator=gen, device=dev)).to(bf)
    beta = (0.1 * torch.randn((h,), generator=gen, device=dev)).to(bf)
    parts = torch.randn((t, s, h), generator=gen, device=dev).to(bf)
    g_out = (0.01 * torch.randn((s, h), generator=gen, device=dev)).to(bf)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def fl():
        flush.zero_()

    U, mean, rstd = tp.sp_ln_fwd(x, gamma, beta, t)
    E = 2 * s * h  # bytes of one [s, h] bf16 tensor
    legs = {
        "ln_fwd": (lambda: tp.sp_ln_fwd(x, gamma, beta, t), 2 * E + 8 * s),
        "reduce_dropout_residual_fwd": (lambda: tp.sp_dropres_fwd(parts, x, p, 0), (t + 2) * E),
        "dropout_bwd": (lambda: tp.sp_dropres_bwd(g_out, t, p, 0), 2 * E),
        "ln_bwd_with_reduce": (lambda: tp.sp_ln_bwd(parts, g_out, x, gamma, mean, rstd), (t + 3) * E + 8 * s),
    }
    out = {}
    for name, (fn, nbytes) in legs.items():
        fn()
        torch.cuda.synchronize()
        ms = _time_events(fn, reps, before=fl)
        med = float(np.median(ms))
        out[name] = {"bytes": nbytes, "gbs_median": round(nbytes / (med * 1e-3) / 1e9, 1),
                     "frac_of_hbm": round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), **_stats(ms)}
    return {"workload": f"sequence-parallel region of the h={h} block: s={s}, t={t}, p={p}, bf16", **out}


def leg_c5_block(tp, reps):
    """The whole sequence-parallel block step on the h = 4096 configuration
    (s = 4096 tokens, h = 4096, m = 4h, t = 8 sequence and tensor shards,
    p = 0.1, bf16): LN forward on every sequence shard (the AllGather is the
    row-block layout of its output), the 8 MLP shards' forward, the sum of the
    partials fused with dropout and the residual add (the ReduceScatter),
    dropout backward, the MLP shards' backward, LN backward with the sum of the
    input-gradient partials and dγ/dβ.  TFLOP/s over the MLP GEMMs,
    12·n·d·m_i per shard ([EFF] FLOPs appendix); the SP kernels' time is
    included."""
    import ctypes

    import numpy as np
    import torch
    from tpmlp_inputs import CONFIGS
    cfg = CONFIGS["sp_block_t8"]
    s, h, m, t, p = cfg["n"], cfg["d"], cfg["m"], cfg["t"], cfg["p"]
    mi = m // t
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(9)
    bf = torch.bfloat16

    def rnd(shape, std, mean=0.0):
        return (mean + torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * std).to(bf)

    x, g_out = rnd((s, h), 1.0), rnd((s, h), 0.01)
    gamma, beta = rnd((h,), 0.1, 1.0), rnd((h,), 0.1)
    A, B = rnd((t, h, mi), 0.02), rnd((t, mi, h), 0.02)
    U, out, dS, dx = (torch.empty((s, h), dtype=bf, device=dev) for _ in range(4))
    mean, rstd = (torch.empty(s, dtype=torch.float32, device=dev) for _ in range(2))
    Z, Y, D = (torch.empty((t, s, mi), dtype=bf, device=dev) for _ in range(3))
    P, dXp = (torch.empty((t, s, h), dtype=bf, device=dev) for _ in range(2))
    dA = torch.empty((t, h, mi), dtype=torch.float32, device=dev)
    dB = torch.empty((t, mi, h), dtype=torch.float32, device=dev)
    dgamma, dbeta = (torch.empty(h, dtype=torch.float32, device=dev) for _ in range(2))
    nb = tp.lib().tpmlp_sp_workspace_bytes(s, h)
    ws = torch.empty(max(nb, 4), dtype=torch.uint8, device=dev)
    wsf = tp.workspace(tp.fwd_workspace_bytes(U, A), dev)
    wsb = tp.workspace(tp.bwd_workspace_bytes(U, A), dev)
    P_ = tp._ptr
    common = dict(dt=tp.BF16, t=t, s=s, h=h, eps=cfg["eps"], p_drop=p, seed=cfg["mask_seed"])
    a_ln = tp.SpArgs(phase=tp.SP_LN_FWD, x=P_(x), gamma=P_(gamma), beta=P_(beta), ln_out=P_(U), mean=P_(mean),
                     rstd=P_(rstd), **common)
    a_dr = tp.SpArgs(phase=tp.SP_DROPRES_FWD, partials=P_(P), x=P_(x), out=P_(out), **common)
    a_db = tp.SpArgs(phase=tp.SP_DROPRES_BWD, g_out=P_(g_out), dS=P_(dS), **common)
    a_lb = tp.SpArgs(phase=tp.SP_LN_BWD, dU_partials=P_(dXp), g_out=P_(g_out), x=P_(x), gamma=P_(gamma),
                     mean=P_(mean), rstd=P_(rstd), dx=P_(dx), dgamma=P_(dgamma), dbeta=P_(dbeta), ws=P_(ws),
                     ws_bytes=nb, **common)
    stream = torch.cuda.current_stream()
    names = ("ln_fwd", "mlp_fwd", "reduce_dropout_residual", "dropout_bwd", "mlp_bwd", "ln_bwd_with_reduce")

    def step(ev=None):
        rec = (lambda k: ev[k].record(stream)) if ev is not None else (lambda k: None)
        rec(0)
        tp.tpmlp_ln_sp(a_ln, stream)
        rec(1)
        tp.tpmlp_fwd(U, A, B, Z, Y, P, wsf, stream)
        rec(2)
        tp.tpmlp_ln_sp(a_dr, stream)
        rec(3)
        tp.tpmlp_ln_sp(a_db, stream)
        rec(4)
        tp.tpmlp_bwd(U, A, B, Z, Y, dS, D, dA, dB, dXp, wsb, stream)
        rec(5)
        tp.tpmlp_ln_sp(a_lb, stream)
        rec(6)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(7)] for _ in range(reps)]
    for k in range(reps):
        step(evs[k])
    torch.cuda.synchronize()
    step_ms = [e[0].elapsed_time(e[6]) for e in evs]
    med = float(np.median(step_ms))
    flops = 12.0 * s * h * mi * t
    parts = {nm: round(float(np.median([e[i].elapsed_time(e[i + 1]) for e in evs])), 4)
             for i, nm in enumerate(names)}
    gemm_ms = parts["mlp_fwd"] + parts["mlp_bwd"]
    _ = ctypes  # the SpArgs structures hold the raw pointers for the calls above
    return {"workload": f"sequence-parallel block step: s={s}, h={h}, m={m}, t={t} sequence and tensor shards "
                        f"resident, p={p}, bf16 (LN -> MLP fwd -> reduce+dropout+residual -> dropout bwd -> "
                        f"MLP bwd -> LN bwd with the dU reduce)",
            "flop": flops, "tflops_median": round(flops / (med * 1e-3) / 1e12, 2),
            "pct_of_peak": round(100.0 * flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "gemm_only_tflops": round(flops / (gemm_ms * 1e-3) / 1e12, 2),
            "median_ms_by_part": parts, **_stats(step_ms)}


def leg_biased(tp, X, A_s, B_s, G, bufs, reps, flops):
    """The same layer with both biases: bias + GeLU in the first GEMM's
    epilogue, the second bias added in the reduce, and the bias gradients
    inside the biased backward (db1_i = Σ_rows D_i from the dgrad-1 GEMM's
    epilogue, db2 = Σ_rows G as a fixed-order column sum).  TFLOP/s counts the
    GEMM flops only (the bias work adds O(n·m) flops)."""
    import numpy as np
    import torch
    Z, Y, P, O, D, dA, dB, dXp, dX = bufs
    t, d, mi = A_s.shape
    n = X.shape[0]
    dev = X.device
    gen = torch.Generator(device=dev)
    gen.manual_seed(3)
    b1 = (0.5 * torch.randn((t, mi), generator=gen, device=dev)).to(torch.bfloat16)
    b2 = (0.5 * torch.randn((d,), generator=gen, device=dev)).to(torch.bfloat16)
    db1 = torch.empty((t, mi), dtype=torch.float32, device=dev)
    db2 = torch.empty((d,), dtype=torch.float32, device=dev)
    wsf = tp.workspace(tp.fwd_workspace_bytes(X, A_s, bias=True), dev)
    wsb = tp.workspace(tp.bwd_bias_workspace_bytes(X, A_s), dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        rec = (lambda k: ev[k].record(stream)) if ev is not None else (lambda k: None)
        rec(0)
        tp.tpmlp_fwd_bias(X, A_s, B_s, b1, Z, Y, P, wsf, stream)
        tp.tpmlp_reduce_partials_bias(P, b2, O, stream)
        rec(1)
        tp.tpmlp_bwd_bias(X, A_s, B_s, Z, Y, G, D, dA, dB, dXp, db1, db2, wsb, stream)
        rec(2)
        tp.tpmlp_reduce_partials(dXp, dX, stream)
        rec(3)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(reps)]
    for k in range(reps):
        step(evs[k])
    torch.cuda.synchronize()
    step_ms = [e[0].elapsed_time(e[3]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    med = float(np.median(step_ms))
    return {"workload": "the 8.3B-shaped layer with both biases (b1 split with A, b2 unsplit); backward "
                        "tpmlp_bwd_bias (db1 fused into the dgrad-1 epilogue, db2 a column sum of G)",
            "tflops_median": round(flops / (med * 1e-3) / 1e12, 2),
            "pct_of_peak": round(100.0 * flops / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "step": _stats(step_ms), "bwd_bias": _stats(bwd_ms)}


def leg_attention(tp, reps):
    """The attention side of the 8.3B-shaped layer: h = 3072, 24 heads of 128,
    t = 8 shards resident, b = 8, s = 1024, causal, bf16.  Forward = QKV GEMM,
    flash-attention core, projection GEMM; backward = dW_proj with dO, the
    core's backward, dW_qkv with dX.  FLOP counts: GEMMs 2·m·n·k each; the
    core 4·b·s²·h forward and 8·b·s²·h backward in the pages' formula (no
    causal discount, [EFF] FLOPs appendix), and also the causal half."""
    import numpy as np
    import torch
    from tpmlp_inputs import CONFIGS
    c = CONFIGS["gpt8p3b_attn_t8"]
    s, b, d, heads, t = c["s"], c["b"], c["d"], c["heads"], c["t"]
    dh = d // heads
    w = d // t
    n = s * b
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(7)
    bf = torch.bfloat16

    def rnd(shape, std):
        return (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * std).to(bf)
    X, G = rnd((n, d), 1.0), rnd((n, d), 0.01)
    Wq, Wp = rnd((t, d, 3 * w), 0.02), rnd((t, w, d), 0.02)
    QKV = torch.empty((t, n, 3 * w), dtype=bf, device=dev)
    O = torch.empty((t, n, w), dtype=bf, device=dev)
    lse = torch.empty((t, b, heads // t, s), dtype=torch.float32, device=dev)
    P = torch.empty((t, n, d), dtype=bf, device=dev)
    dO, dQKV = torch.empty_like(O), torch.empty_like(QKV)
    dWq = torch.empty((t, d, 3 * w), dtype=torch.float32, device=dev)
    dWp = torch.empty((t, w, d), dtype=torch.float32, device=dev)
    dXp = torch.empty_like(P)
    ws = torch.empty(tp.attn_bwd_workspace_bytes(t, s, b, heads // t), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def fwd():
        tp.tpmlp_attn_fwd(X, Wq, Wp, QKV, O, lse, P, s, b, dh, True, stream=stream)

    def core_f():
        tp.tpmlp_attn_core_fwd(QKV, O, lse, s, b, heads // t, dh, True, stream=stream)

    def core_b():
        tp.tpmlp_attn_core_bwd(QKV, O, lse, dO, dQKV, ws, s, b, heads // t, dh, True, stream=stream)

    def bwd():
        tp.tpmlp_attn_bwd(X, Wq, Wp, QKV, O, lse, G, dO, dQKV, dWq, dWp, dXp, ws, s, b, dh, True, stream=stream)

    for _ in range(3):
        fwd()
        bwd()
    torch.cuda.synchronize()
    out = {"workload": f"attention side of the 8.3B-shaped layer: h={d}, {heads} heads of {dh}, t={t} "
                       f"resident, b={b}, s={s}, causal, bf16"}
    gemm_f = 2.0 * n * d * 3 * w * t + 2.0 * n * w * d * t
    core_f_flop = 4.0 * b * s * s * d            # QK^T and A·V over all heads, pages' formula
    # executed work of the causal core: only the s(s+1)/2 visible (query, key)
    # pairs of each sequence and head are computed
    core_f_exec = core_f_flop * (s + 1) / (2.0 * s)
    for name, fn, fl, fx in (("fwd", fwd, gemm_f + core_f_flop, gemm_f + core_f_exec),
                             ("bwd", bwd, 2 * gemm_f + 2 * core_f_flop, 2 * gemm_f + 2 * core_f_exec),
                             ("core_fwd", core_f, core_f_flop, core_f_exec),
                             ("core_bwd", core_b, 2 * core_f_flop, 2 * core_f_exec)):
        ms = _time_events(fn, reps)
        med = float(np.median(ms))
        out[name] = {"flop_executed": fx, "tflops_median": round(fx / (med * 1e-3) / 1e12, 2),
                     "pct_of_peak": round(100.0 * fx / (med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                     "flop_pages_formula": fl, "tflops_pages_formula": round(fl / (med * 1e-3) / 1e12, 2),
                     **_stats(ms)}
    step = out["fwd"]["median_ms"] + out["bwd"]["median_ms"]
    tot_x = 3 * gemm_f + 3 * core_f_exec
    tot_p = 3 * gemm_f + 3 * core_f_flop
    out["step"] = {"median_ms": round(step, 4), "flop_executed": tot_x,
                   "tflops": round(tot_x / (step * 1e-3) / 1e12, 2),
                   "pct_of_peak": round(100.0 * tot_x / (step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                   "tflops_pages_formula": round(tot_p / (step * 1e-3) / 1e12, 2),
                   "note": "tflops counts executed work (the causal core's visible pairs); "
                           "tflops_pages_formula counts 4·b·s²·h for the core regardless of the mask"}
    # the core with a general mask instead: BERT-style padding (lengths drawn
    # from [s/2, s], padded query rows see no key), not causal; the flop count
    # is the pages' unmasked one, so the rate is what the mask leaves of it
    from tpmlp_inputs import attn_mask
    mbytes = torch.from_numpy(attn_mask(b, s, "padding", seed=7)).to(dev)
    visible = float(mbytes.numel() - int(mbytes.sum().item())) / mbytes.numel()
    mask = tp.attn_pack_mask(mbytes)  # once per batch; every layer and pass reads the packed form

    def core_mf():
        tp.tpmlp_attn_core_fwd(QKV, O, lse, s, b, heads // t, dh, False, mask=mask, stream=stream)

    def core_mb():
        tp.tpmlp_attn_core_bwd(QKV, O, lse, dO, dQKV, ws, s, b, heads // t, dh, False, mask=mask, stream=stream)
    core_mf()
    core_mb()
    torch.cuda.synchronize()
    pad = {"mask": "padding (BERT-style), not causal", "visible_fraction": round(visible, 4)}
    for name, fn, fl in (("core_fwd", core_mf, core_f_flop), ("core_bwd", core_mb, 2 * core_f_flop)):
        ms = _time_events(fn, reps)
        med = float(np.median(ms))
        pad[name] = {"tflops_pages_formula": round(fl / (med * 1e-3) / 1e12, 2),
                     "tflops_visible_entries": round(fl * visible / (med * 1e-3) / 1e12, 2), **_stats(ms)}
    out["padding_mask"] = pad
    return out


def leg_library(reps):
    """Library kernels on the shapes measured above, as context for their rates
    (the libraries run as shipped; nothing of this package is involved):
    - hipBLASLt through torch.bmm on the six products of the 8.3B-shaped layer
      (t = 8 shards; each product's operands stored contiguous in the order it
      reads them, so no transposed view reaches the library; bf16 outputs,
      where the GEMM core writes dA_i and dB_i in fp32);
    - torch's scaled_dot_product_attention, restricted to its flash and
      memory-efficient kernels (never its math path), at the 8.3B attention
      shape: b = 8, 24 heads of 128, s = 1024, causal, bf16, [b, heads, s, dh];
      FLOP counted as in the attention leg (executed causal work);
    - torch's device copy of the sequence-parallel kernels' byte counts, each
      after the same 512 MiB cache flush as the sp_region leg."""
    import numpy as np
    import torch
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    bf = torch.bfloat16
    out = {}

    def rnd(shape, std):
        return (torch.randn(shape, generator=gen, device=dev, dtype=torch.float32) * std).to(bf)

    t, n, d, mi = 8, 8192, 3072, 1536
    prods = (("Z=X.A_i", (t, n, d), (t, d, mi)), ("P=Y.B_i", (t, n, mi), (t, mi, d)),
             ("E=G.B_i^T", (t, n, d), (t, d, mi)), ("dA_i=X^T.D_i", (t, d, n), (t, n, mi)),
             ("dB_i=Y_i^T.G", (t, mi, n), (t, n, d)), ("dX_i=D_i.A_i^T", (t, n, mi), (t, mi, d)))
    gem = {}
    total_ms = 0.0
    for name, sa, sb in prods:
        a, b = rnd(sa, 1.0), rnd(sb, 0.02)
        c = torch.empty((t, sa[1], sb[2]), dtype=bf, device=dev)
        fn = lambda: torch.bmm(a, b, out=c)  # noqa: E731
        fn()
        torch.cuda.synchronize()
        ms = _time_events(fn, reps)
        med = float(np.median(ms))
        fl = 2.0 * t * sa[1] * sa[2] * sb[2]
        gem[name] = {"tflops_median": round(fl / (med * 1e-3) / 1e12, 2), **_stats(ms)}
        total_ms += med
        del a, b, c
    flops = 12.0 * n * d * mi * t
    gem["six_products"] = {"median_ms_sum": round(total_ms, 4),
                           "tflops": round(flops / (total_ms * 1e-3) / 1e12, 2),
                           "pct_of_peak": round(100.0 * flops / (total_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)}
    out["hipblaslt_bmm_gpt8p3b_t8"] = gem
    torch.cuda.empty_cache()

    from torch.nn.attention import SDPBackend, sdpa_kernel
    b, heads, s, dh = 8, 24, 1024, 128
    q, k, v = rnd((b, heads, s, dh), 1.0), rnd((b, heads, s, dh), 1.0), rnd((b, heads, s, dh), 1.0)
    go = rnd((b, heads, s, dh), 0.01)
    core_f_exec = 4.0 * b * s * s * heads * dh * (s + 1) / (2.0 * s)
    att = {"shape": f"b={b}, heads={heads}, s={s}, dh={dh}, causal, bf16"}
    for be in (SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION):
        try:
            with sdpa_kernel([be]):
                qq, kk, vv = (x.detach().requires_grad_() for x in (q, k, v))

                def fwd():
                    return torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True)
                o = fwd()

                def bwd():
                    torch.autograd.grad(o, (qq, kk, vv), go, retain_graph=True)
                bwd()
                torch.cuda.synchronize()
                rf, rb = _time_events(fwd, reps), _time_events(bwd, reps)
            rec = {}
            for nm, ms, fl in (("fwd", rf, core_f_exec), ("bwd", rb, 2 * core_f_exec)):
                med = float(np.median(ms))
                rec[nm] = {"tflops_executed": round(fl / (med * 1e-3) / 1e12, 2), **_stats(ms)}
            att[be.name.lower()] = rec
            del o
        except RuntimeError as ex:  # the backend has no kernel for this GPU or shape
            att[be.name.lower()] = {"unavailable": str(ex).splitlines()[0][:200]}
    out["sdpa_attention_core"] = att
    del q, k, v, go
    torch.cuda.empty_cache()

    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    E = 2 * 4096 * 4096  # one [4096, 4096] bf16 tensor
    cp = {}
    for name, nbytes in (("33.5MB", E), ("168MB", 5 * E), ("185MB", 11 * E // 2)):
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(3)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        ms = _time_events(lambda: dst.copy_(src), reps, before=lambda: flush.zero_())
        med = float(np.median(ms))
        cp[name] = {"traffic_bytes": 2 * nbytes, "gbs_median": round(2 * nbytes / (med * 1e-3) / 1e9, 1), **_stats(ms)}
        del src, dst
    del flush
    out["device_copy_after_flush"] = cp
    return out


def leg_vocab(tp, reps):
    """The logit layer and vocabulary-parallel cross-entropy of the 8.3B-shaped
    model: n = 8192 tokens, h = 3072, V = 51200 in t = 8 shards of 6400, bf16,
    g = 1/n.  TFLOP/s over the GEMMs (2·n·h·V forward, twice that backward,
    [EFF] FLOPs appendix), the cross-entropy kernels included in the time: the
    row statistics come from the logit GEMM's epilogue, then a combine over the
    shards; backward: dlogits (logits read and dlogits written once), then the
    two GEMMs."""
    import numpy as np
    import torch
    from tpmlp_inputs import CONFIGS
    c = CONFIGS["gpt8p3b_vocab_t8"]
    n, h, V, t = c["n"], c["d"], c["V"], c["t"]
    vi = V // t
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(11)
    bf = torch.bfloat16
    X = torch.randn((n, h), generator=gen, device=dev).to(bf)
    W = (0.02 * torch.randn((t, vi, h), generator=gen, device=dev)).to(bf)
    tg = torch.randint(0, V, (n,), generator=gen, device=dev, dtype=torch.int32)
    g = torch.full((n,), 1.0 / n, dtype=torch.float32, device=dev)
    logits = torch.empty((t, n, vi), dtype=bf, device=dev)
    loss, rmax, rsum = (torch.empty(n, dtype=torch.float32, device=dev) for _ in range(3))
    ws = torch.empty(tp.lib().tpmlp_vocab_ce_workspace_bytes(t, n, vi), dtype=torch.uint8, device=dev)
    dlogits = torch.empty_like(logits)
    dW = torch.empty((t, vi, h), dtype=torch.float32, device=dev)
    dXp = torch.empty((t, n, h), dtype=bf, device=dev)
    stream = torch.cuda.current_stream()

    def fwd():
        tp.tpmlp_vocab_ce_fwd(X, W, tg, logits, loss, rmax, rsum, ws, 0, stream)

    def bwd():
        tp.tpmlp_vocab_ce_bwd(X, W, tg, logits, rmax, rsum, g, dlogits, dW, dXp, 0, stream)

    for _ in range(3):
        fwd()
        bwd()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for k in range(reps):
        ev[k][0].record(stream)
        fwd()
        ev[k][1].record(stream)
        bwd()
        ev[k][2].record(stream)
    torch.cuda.synchronize()
    f_ms = [e[0].elapsed_time(e[1]) for e in ev]
    b_ms = [e[1].elapsed_time(e[2]) for e in ev]
    fl = 2.0 * n * h * V
    step = float(np.median(f_ms)) + float(np.median(b_ms))
    return {"workload": f"logit layer + vocabulary-parallel cross-entropy: n={n}, h={h}, V={V}, t={t} "
                        f"resident ({vi} per shard), bf16, mean loss",
            "fwd": {"tflops_median": round(fl / (float(np.median(f_ms)) * 1e-3) / 1e12, 2), **_stats(f_ms)},
            "bwd": {"tflops_median": round(2 * fl / (float(np.median(b_ms)) * 1e-3) / 1e12, 2), **_stats(b_ms)},
            "step": {"median_ms": round(step, 4), "tflops": round(3 * fl / (step * 1e-3) / 1e12, 2),
                     "pct_of_peak": round(100.0 * 3 * fl / (step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)},
            "logits_bytes": t * n * vi * 2}


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
              "(a multi-GPU run would place one TP rank per GPU and replace the local "
              "reduction by an all-reduce).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import megatron_tensor_transformer_amd as tp
    from tpmlp_inputs import CONFIGS, config_inputs

    cfg = CONFIGS[WORKLOAD]
    n, d, m, t = cfg["n"], cfg["d"], cfg["m"], cfg["t"]
    mi = m // t
    tp.set_gemm_tile_policy(TILE_POLICIES[args.gemm_tile_policy])
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
    wsf = tp.workspace(tp.fwd_workspace_bytes(X, A_s), dev)
    ws = tp.workspace(tp.bwd_workspace_bytes(X, A_s), dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        tp.tpmlp_fwd(X, A_s, B_s, Z, Y, P, wsf, stream)
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
    clocks = ClockSampler()
    idle_clk = clocks.read()[0] if clocks.error is None else None
    clocks.start()
    t_wall0 = time.perf_counter()
    for k in range(args.steps):
        step(evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    clocks.stop()

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
    # GEMM core launches per step: fwd GEMM1 and GEMM2; bwd dgrad-1, then both
    # weight gradients with dgrad-2 (one launch of three problems)
    per_launch_flop = flops / GEMM_LAUNCHES
    avg_launch_ms = gemm_ms / GEMM_LAUNCHES
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
                   "n": n, "d": d, "m": m, "t": t, "m_i": mi, "parallelism": "tp8 simulated on 1 GPU",
                   "gemm_tile_policy": args.gemm_tile_policy},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "gemm_only": {"tflops": round(gemm_tflops, 2),
                      "pct_of_peak": round(100.0 * gemm_tflops / PEAK_BF16_TFLOPS, 2),
                      "fwd_ms": round(float(np.mean(fwd_ms)), 4), "bwd_ms": round(float(np.mean(bwd_ms)), 4)},
        "roofline": {"bound": "mfma", "kernel": "gemm_bf16_kernel, mean over the 4 launches of a step "
                                                "(the last one runs dA, dB and dX)",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic("gemm_bf16.hip", "gemm_bf16_gpt8p3b_t8_traffic.md"),
                     "flop_per_launch": per_launch_flop, "avg_launch_ms": round(avg_launch_ms, 4)},
        "roofline_reduce": {"bound": "hbm", "kernel": "reduce_vec8_kernel",
                            "achieved": round(red_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(red_gbs / PEAK_HBM_GBS, 4),
                            "traffic": recorded_traffic("reduce.hip", "reduce_gpt8p3b_t8_traffic.md"),
                            "bytes_per_launch": red_bytes, "avg_launch_ms": round(red_ms, 4)},
        "sclk_mhz": {"timed_window": {**clocks.summary(), "before_timed_mhz": idle_clk}},
        "wall_s_timed": round(wall, 3),
        "step_ms_min_max": [round(min(step_ms), 4), round(max(step_ms), 4)],
    }
    rec["gemm_only"].update({"tflops_median": round(flops / (float(np.median(
        np.array(fwd_ms) + np.array(bwd_ms))) * 1e-3) / 1e12, 2)})
    rec["step_ms"] = _stats(step_ms)
    # the clock under sustained load: about two seconds more of the same step,
    # untimed, sampled the same way (the timed steps alone may be too short
    # for the clock to settle)
    soak = ClockSampler()
    soak.start()
    t_soak = time.perf_counter()
    while time.perf_counter() - t_soak < 2.0:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    soak.stop()
    sus = soak.summary()
    # the SMI metrics table refreshes more slowly than a short timed window:
    # when it did not refresh there (no samples after its first refresh),
    # only the soak's figure describes the loaded clock
    rec["sclk_mhz"].update({
        "median_mhz": sus.get("median_mhz"), "max_mhz": sus.get("max_mhz"),
        "frac_of_2400": sus.get("frac_of_2400"), "socket_power_w_median": sus.get("socket_power_w_median"),
        "clock_adjusted_peak_tflops": (round(PEAK_BF16_TFLOPS * sus["median_mhz"] / 2400.0, 1)
                                       if sus.get("median_mhz") else None),
        "sustained_2s": {k: v for k, v in sus.items() if k != "source"},
        "source": "AMD SMI GPU metrics (mean over XCDs of current_gfxclks, socket power), sampled every 5 ms "
                  "over about 2 s of the same step run right after the timed steps, from the table's first "
                  "refresh on"})
    if rec["sclk_mhz"]["clock_adjusted_peak_tflops"]:
        rec["pct_of_clock_adjusted_peak"] = round(100.0 * value / rec["sclk_mhz"]["clock_adjusted_peak_tflops"], 2)
    # the reduce alone, inputs flushed from the last-level cache first
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    red_flushed = _time_events(lambda: tp.tpmlp_reduce_partials(P, O), 10, before=lambda: flush.zero_())
    del flush
    rec["roofline_reduce"]["cache_flushed"] = {
        "gbs_median": round(red_bytes / (float(np.median(red_flushed)) * 1e-3) / 1e9, 1), **_stats(red_flushed)}
    legs = set() if args.no_extra else set(LEGS if args.legs is None else args.legs.split(","))
    unknown = legs - set(LEGS) - set(OPTIONAL_LEGS)
    if unknown:
        print(f"unknown legs: {sorted(unknown)}; known: {LEGS + OPTIONAL_LEGS}", file=sys.stderr)
        sys.exit(2)
    if "biased_step" in legs:
        rec["biased_step"] = leg_biased(tp, X, A_s, B_s, G, (Z, Y, P, O, D, dA, dB, dXp, dX), 10, flops)
    del Z, Y, P, D, dA, dB, dXp, O, dX
    torch.cuda.empty_cache()
    if "per_rank" in legs:
        rec["per_rank"] = {"workload": "one shard of the 8.3B-shaped layer per launch (t_local=1)",
                           **leg_mlp_shard(tp, n, d, mi, 20, seed=1)}
    if "c2" in legs:
        rec["c2"] = {"workload": "single-shard layer: n=b*s=4*512=2048, d=1024, m=4096, t=1 (fwd+bwd, no "
                                 "reduction: with one shard the sum is the partial itself)",
                     **leg_mlp_shard(tp, 2048, 1024, 4096, 20, seed=4, inner=20)}
    if "gpt1t_shard" in legs:
        rec["gpt1t_shard"] = {"workload": "GPT-1T-shaped shard: h=25600, m_i=12800, n=2048 tokens, one shard",
                              **leg_mlp_shard(tp, 2048, 25600, 12800, 10, seed=2)}
    for name, fn in (("sp_region", lambda: leg_sp(tp, 10)), ("c5_block", lambda: leg_c5_block(tp, 10)),
                     ("attention", lambda: leg_attention(tp, 10)), ("vocab_ce", lambda: leg_vocab(tp, 10)),
                     ("fp32_path", lambda: leg_fp32(tp, 5)), ("library_yardsticks", lambda: leg_library(10))):
        if name in legs:
            torch.cuda.empty_cache()
            rec[name] = fn()
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(inp, t, args.cpu_seconds)
    if args.cpu_all_configs:
        rec["cpu_oracle_configs"] = cpu_all_configs()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
