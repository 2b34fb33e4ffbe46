"""Benchmark of the MoE layer forward pass on one MI355X.

One step = one moe_forward call (router -> top-k -> capacity -> dispatch ->
grouped SwiGLU -> combine) over one batch of synthetic, seeded input that is
already resident in HBM.  Prints one JSON line:

  value        tokens/s of the headline layer (Mixtral-shaped prefill, bf16)
               over the K timed steps: T * K / wall time between two device
               synchronisations, with no per-phase instrumentation inside
  roofline     the dominant kernel (gate/up grouped GEMM + SwiGLU): its
               algorithmic FLOPs or bytes per launch divided by its average
               duration, from HIP events recorded on the launch stream at the
               phase boundaries of a second, instrumented pass of K steps
  layer        the whole step against its binding roof, kernel phases, the
               dispatch and combine streaming rates, router statistics
  configs      the same measurements for every layer shape of the suite:
               tiny fp32, Mixtral prefill, DeepSeek-V3 prefill and decode,
               and the skewed Switch layer at capacity factors 1.0 and 1.25
  cpu_baseline the CPU oracle (numpy float64) timed on a bounded token sample
               of the headline workload, on this host's cores

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-configs] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s; % bf16 MFMA peak (prefill), % HBM GB/s peak (decode)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
PEAK_F32_TFLOPS = 157.3        # MI355X fp32 (matrix and vector)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
GEMM_SRC = os.path.join(ROOT, "mixture_experts_layer_47_amd", "csrc", "gemm.hip")

# The layer shapes the report covers, in suite order, and the bound each one
# is judged against: the matrix cores for the Mixtral-shaped prefill (about
# 1000 FLOP per weight byte), HBM for the rest (DeepSeek-V3's ~128 rows per
# expert sit below the bf16 ridge; decode and the capacity-limited Switch
# layer stream weights for a handful of rows).
SUITE = (("c1", "tiny_fp32"), ("c2", "mixtral_prefill"), ("c3", "dsv3_prefill"),
         ("c4", "dsv3_decode"), ("c5_cf1.0", "switch_capacity"),
         ("c5_cf1.25", "switch_capacity_cf125"))


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_hash() -> str:
    """sha256[:16] of gemm.hip's code: comments removed and whitespace
    collapsed, so that an edit of the comments alone keeps the byte counters
    taken with the same code."""
    with open(GEMM_SRC) as f:
        src = f.read()
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return hashlib.sha256(" ".join(src.split()).encode()).hexdigest()[:16]


def weight_elem_bytes(w):
    from mixture_experts_layer_47_amd.workloads import weight_elem_bytes as web
    return web(w)


def es_of(w):
    return 2 if w.dtype == "bf16" else 4


def up_kernel_work(w, counts_kept, n_kept):
    """Algorithmic work of one gate/up launch (real kept rows only).

    FLOPs = 2 * rows * d * 2F (gate and up projections).
    Bytes = W1 + W3 of every expert that has rows (each read once; FP8
            weights: one byte per element plus one fp32 scale per row)
          + the X rows the launch reads (T distinct tokens, each read once)
          + H written (rows * F).
    """
    es = es_of(w)
    ew = weight_elem_bytes(w)
    rows = n_kept + (w.T if w.n_shared else 0)
    touched = int((counts_kept > 0).sum()) + (1 if w.n_shared else 0)
    flops = 4.0 * rows * w.d * w.F
    wbytes = 2.0 * w.F * w.d * ew + (2.0 * w.F * 4 if w.wdtype == "fp8" else 0.0)
    bytes_ = touched * wbytes + w.T * w.d * es + rows * w.F * es
    return flops, bytes_, touched, rows


def down_kernel_work(w, touched, rows):
    """Algorithmic work of one down launch: FLOPs 2 * rows * F * d; bytes =
    W2 of every touched expert once + H read (rows * F) + fp32 rows written."""
    es = es_of(w)
    ew = weight_elem_bytes(w)
    flops = 2.0 * rows * w.F * w.d
    wbytes = w.F * w.d * ew + (w.d * 4.0 if w.wdtype == "fp8" else 0.0)
    return flops, touched * wbytes + rows * w.F * es + rows * w.d * 4.0


def dispatch_bytes(w, n_kept):
    """Index traffic of the dispatch: ids read; slot_row, sorted_slot and
    row_token (kept rows plus the shared expert's T rows) written; counts
    and offsets."""
    tk = w.T * w.k
    return 4.0 * (tk + tk + n_kept + n_kept + (w.T if w.n_shared else 0) + 2 * w.E + 1)


def combine_bytes(w, n_kept):
    """The combine's algorithmic traffic: every kept fp32 expert row once
    (plus the shared expert's row per token), slot_row and gates, and Y."""
    es = es_of(w)
    rows = n_kept + (w.T if w.n_shared else 0)
    return rows * w.d * 4.0 + w.T * w.k * 8.0 + w.T * w.d * es


def roof_of(flops, bytes_, ms, peak_flops):
    """Fraction of the binding roof for work (flops, bytes) done in ms."""
    t_mfma = flops / (peak_flops * 1e12)
    t_hbm = bytes_ / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        ach = flops / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": ach, "peak": peak_flops, "unit": "TFLOP/s",
                "frac": ach / peak_flops}
    ach = bytes_ / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": ach, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": ach / PEAK_HBM_GBS}


def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count()
    return model, os.cpu_count(), avail


def cpu_baseline(w, inp, target_s=15.0):
    """Time the oracle on the first S tokens of the batch (S sized for ~target_s)."""
    import numpy as np
    import torch
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([p.get("num_threads", 0) for p in threadpool_info()
                     if p.get("user_api") == "blas"] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        cores = os.cpu_count()

    def f64(t, scale=None):
        if t.dtype == torch.uint8:       # E4M3 codes: the oracle decodes them
            return O.dequantize_rows(t.cpu().numpy(), scale.cpu().numpy())
        return t.detach().to("cpu", torch.float64).numpy()
    log("cpu baseline: copying weights to host (untimed)")
    sc = inp.get("scales") or (None, None, None)
    Wg = f64(inp["Wg"]).T
    W1 = f64(inp["W1"], sc[0]).transpose(0, 2, 1)
    W3 = f64(inp["W3"], sc[1]).transpose(0, 2, 1)
    W2 = f64(inp["W2"], sc[2]).transpose(0, 2, 1)
    ss = inp.get("shared_scales") or (None, None, None)
    sh = (None if inp["shared"] is None else
          tuple(f64(t, q).T for t, q in zip(inp["shared"], ss)))
    bias = None if inp["bias"] is None else f64(inp["bias"])
    off = None if inp["offset"] is None else f64(inp["offset"])
    X = f64(inp["X"])

    def run(S):
        t0 = time.perf_counter()
        if w.routing == "expert":
            C = min(S, O.capacity(w.cf or 1.0, S, w.k, w.E))
            O.forward_expert_choice(X[:S], Wg, W1, W3, W2, C=C, score_func=w.score, offset=off,
                                    shared=sh, bf16_h=(w.dtype == "bf16"))
        else:
            cap = O.capacity(w.cf, S, w.k, w.E) if w.cf else None
            O.forward(X[:S], Wg, W1, W3, W2, k=w.k, score_func=w.score, renorm=w.renorm,
                      bias=bias, offset=off, cap=cap, shared=sh, bf16_h=(w.dtype == "bf16"))
        return time.perf_counter() - t0
    # grow the sample (doubling) until one run takes >= target_s / 4, then
    # repeat it so the timed CPU work is about target_s
    S = min(w.T, 64)
    t = run(S)
    while t < target_s / 4 and S < w.T:
        S = min(w.T, 2 * S)
        t = run(S)
    reps = max(1, int(round(target_s / max(t, 1e-3))))
    reps = min(reps, 8)
    tot = t + sum(run(S) for _ in range(reps - 1))
    model, ncpu, avail = cpu_info()
    return {"value": S * reps / tot, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": model, "nproc": ncpu, "cpus_available": avail,
            "sample": f"first {S} of {w.T} tokens of the {w.name} batch x {reps} runs, full "
                      f"resident expert weights, numpy float64 oracle (tier 1), {tot:.1f} s, "
                      f"{cores} BLAS threads"}


COPY_BYTES = 512 << 20


def copy_calibration(torch):
    """Reads COPY_BYTES and writes COPY_BYTES per launch (elementwise negation)."""
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": COPY_BYTES,
                      "copy_calibration_bytes_written": COPY_BYTES}), flush=True)


def parse_marks(marks):
    """[(phase, ms or None)] -> ({phase: mean ms}, [device ms per step])."""
    import numpy as np
    phases, steps_ms, cur = {}, [], None
    for name, ms in marks:
        if ms is None:             # a call's first mark: the previous call is complete
            if cur is not None:
                steps_ms.append(cur)
            cur = 0.0
        else:
            phases.setdefault(name, []).append(ms)
            cur = (cur or 0.0) + ms
    if cur is not None:
        steps_ms.append(cur)
    return {k: float(np.mean(v)) for k, v in phases.items()}, steps_ms


def prepare(w):
    """Inputs of workload w on the GPU, its layer, and one call with the
    optional outputs for the per-expert row counts (untimed)."""
    import torch
    import mixture_experts_layer_47_amd as moe
    from mixture_experts_layer_47_amd.workloads import make_inputs

    dev = torch.device("cuda:0")
    log(f"workload {w.name}: T={w.T} d={w.d} E={w.E}+{w.n_shared} k={w.k} F={w.F} "
        f"dtype={w.dtype} cf={w.cf}")
    inp = make_inputs(w, dev)
    layer = moe.layer_from_inputs(inp)
    # one call with the optional outputs for the per-expert row counts
    probe = moe.Forward(layer, inp["X"], aux=True)
    probe()
    torch.cuda.synchronize()
    kept = probe.aux["offsets"].diff().cpu().numpy()
    n_kept = int(probe.aux["n_kept"].item())
    balance = health = None
    if "balance" in probe.aux:        # top-k routing only
        balance = float(probe.aux["balance"].item())
        health = dict(zip(("token_entropy", "load_entropy", "load_cv", "drop_rate"),
                          (float(v) for v in probe.aux["health"].cpu().tolist())))
    del probe
    torch.cuda.empty_cache()
    return {"w": w, "inp": inp, "layer": layer, "kept": kept, "n_kept": n_kept,
            "balance": balance, "health": health}


def measure(w, steps, warmup, keep_inputs=False, ctx=None):
    """Time `steps` moe_forward calls of workload w with no instrumentation,
    then `steps` more with phase events; returns the measurement dict (and
    the inputs when asked).  ctx: the result of prepare(w), if done before."""
    import numpy as np
    import torch
    import mixture_experts_layer_47_amd as moe

    if ctx is None:
        ctx = prepare(w)
    inp, layer, kept, n_kept = ctx["inp"], ctx["layer"], ctx["kept"], ctx["n_kept"]
    balance, health = ctx["balance"], ctx["health"]
    del ctx
    fwd = moe.Forward(layer, inp["X"], aux=False)
    for _ in range(warmup):
        fwd()
    torch.cuda.synchronize()

    # timed region: plain calls, nothing recorded inside
    t0 = time.perf_counter()
    for _ in range(steps):
        fwd()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / steps

    # instrumented pass: one HIP event per phase boundary on the launch stream
    moe.timing_enable(steps * 12 + 16)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fwd()
    torch.cuda.synchronize()
    ms_step_instr = (time.perf_counter() - t0) * 1e3 / steps
    phase_ms, steps_ms = parse_marks(moe.timing_read())
    moe.timing_enable(0)

    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    up_ms = phase_ms.get("ffn_up", float("nan"))
    dn_ms = phase_ms.get("ffn_down", float("nan"))
    flops, bytes_, touched, rows = up_kernel_work(w, kept, n_kept)
    dflops, dbytes = down_kernel_work(w, touched, rows)
    roof = roof_of(flops, bytes_, up_ms, peak)
    roof.update(kernel="grouped gate/up GEMM + SwiGLU (ffn_up phase)", kernel_ms=up_ms,
                algorithmic={"flops": flops, "bytes": bytes_, "rows": rows,
                             "touched_experts": touched})
    roof_dn = roof_of(dflops, dbytes, dn_ms, peak)
    roof_dn.update(kernel="grouped down GEMM (ffn_down phase, with k_tail_sum)", kernel_ms=dn_ms,
                   algorithmic={"flops": dflops, "bytes": dbytes})

    # whole layer against its binding roof
    es = es_of(w)
    layer_flops = 2.0 * w.T * w.d * w.E + 6.0 * rows * w.d * w.F
    layer_bytes = (touched * 3.0 * w.d * w.F * weight_elem_bytes(w) + w.E * w.d * es
                   + 2.0 * w.T * w.d * es)
    mfma_frac = layer_flops / (ms_step * 1e-3) / (peak * 1e12)
    hbm_frac = layer_bytes / (ms_step * 1e-3) / (PEAK_HBM_GBS * 1e9)
    bound = "mfma" if layer_flops / (peak * 1e12) >= layer_bytes / (PEAK_HBM_GBS * 1e9) \
        else "hbm"
    disp_ms = phase_ms.get("dispatch", float("nan"))
    comb_ms = phase_ms.get("combine", float("nan"))
    dbyt = dispatch_bytes(w, n_kept)
    cbyt = combine_bytes(w, n_kept)
    out = {
        "workload": w.name, "T": w.T, "d": w.d, "E": w.E, "k": w.k, "F": w.F,
        "n_shared": w.n_shared, "capacity_factor": w.cf, "dtype": w.dtype,
        "ms_per_step": ms_step, "tokens_per_s": w.T / (ms_step * 1e-3),
        "layer": {"bound": bound, "frac": mfma_frac if bound == "mfma" else hbm_frac,
                  "flops": layer_flops, "bytes": layer_bytes, "mfma_frac": mfma_frac,
                  "hbm_frac": hbm_frac},
        "ffn_up": roof, "ffn_down": roof_dn,
        "dispatch": {"ms": disp_ms, "bytes": dbyt, "GB_per_s": dbyt / (disp_ms * 1e-3) / 1e9,
                     "hbm_frac": dbyt / (disp_ms * 1e-3) / (PEAK_HBM_GBS * 1e9)},
        "combine": {"ms": comb_ms, "bytes": cbyt, "GB_per_s": cbyt / (comb_ms * 1e-3) / 1e9,
                    "hbm_frac": cbyt / (comb_ms * 1e-3) / (PEAK_HBM_GBS * 1e9)},
        "kept_rows": n_kept, "dropped_slots": w.T * w.k - n_kept,
        "touched_experts": touched, "balance_stat": balance, "router_health": health,
        "instrumented": {"ms_per_step": ms_step_instr, "phases_ms": phase_ms,
                         "device_step_ms": ({"median": float(np.median(steps_ms)),
                                             "min": float(np.min(steps_ms)),
                                             "max": float(np.max(steps_ms)),
                                             "n": len(steps_ms)} if steps_ms else None)},
    }
    del fwd, layer
    if keep_inputs:
        return out, inp
    del inp
    torch.cuda.empty_cache()
    return out, None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="mixtral_prefill")
    ap.add_argument("--no-configs", action="store_true",
                    help="measure only --workload, not every layer shape of the suite")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-target-s", type=float, default=15.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 512 MiB device copy (negation kernel), five times, "
                         "to calibrate the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library runs on one GPU; the multi-GPU design is written up, not built).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibration:
        copy_calibration(torch)
        return
    from mixture_experts_layer_47_amd.workloads import WORKLOADS

    torch.cuda.set_device(torch.device("cuda:0"))
    w = WORKLOADS[args.workload]
    ctx = prepare(w)
    # The other layer shapes are timed first, so the headline's warm-up and
    # timed steps run on a GPU that is already under load: started from idle,
    # the first tens of steps run a few % slower while the clocks ramp up.
    configs = {}
    if not args.no_configs:
        for tag, name in SUITE:
            if name != w.name:
                configs[tag], _ = measure(WORKLOADS[name], args.steps, args.warmup)
    head, inp = measure(w, args.steps, args.warmup, keep_inputs=not args.no_cpu_baseline,
                        ctx=ctx)
    del ctx
    if configs:
        configs = {tag: (head if name == w.name else configs[tag]) for tag, name in SUITE
                   if name == w.name or tag in configs}
    roof = dict(head["ffn_up"])
    roof["traffic"] = None
    tfile = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("gemm_src_sha256_16") == kernel_hash():
            roof["traffic"] = tr.get("ffn_up_hbm_bytes")
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp, args.cpu_target_s)
        del inp
        torch.cuda.empty_cache()

    out = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded N(0,1) tokens, N(0,1/sqrt(fan_in)) "
                                  "random-init weights)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "E": w.E, "k": w.k, "F": w.F,
                   "expert_weights": "fp8 e4m3 + per-channel fp32 scales" if w.wdtype == "fp8"
                   else w.dtype,
                   "n_shared": w.n_shared, "router": w.score, "capacity_factor": w.cf,
                   "routing": "expert choice" if w.routing == "expert" else "top-k",
                   "parallelism": "single GPU"},
        "roofline": roof,
        "layer": dict(head["layer"], judged_on="layer frac against its binding roof "
                      "(target >= 0.60 of bf16 MFMA on the MFMA-bound prefill, >= 0.70 of HBM "
                      "on the HBM-bound shapes); roofline.frac is the gate/up kernel alone",
                      ffn_down=head["ffn_down"], dispatch=head["dispatch"],
                      combine=head["combine"], kept_rows=head["kept_rows"],
                      balance_stat=head["balance_stat"], router_health=head["router_health"],
                      instrumented=head["instrumented"]),
    }
    if configs:
        out["configs"] = configs
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
