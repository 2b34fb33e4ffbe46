"""Seeded synthetic workloads for the MoE layer: shapes, seeds and generators.

This module holds no arithmetic of the MoE method itself; it only draws the
layer's inputs (tokens, router and expert weights, selection bias, logit
offsets) so that the HIP library and the CPU oracle see identical data.

Storage layout of the drawn tensors (the layout the library consumes):
  X       [T, d]       tokens, row-major
  Wg      [E, d]       router: row e scores expert e   (logical W_g[d, E] = Wg.T)
  W1, W3  [E, F, d]    gate / up projections, d contiguous (logical [E, d, F])
  W2      [E, d, F]    down projection, F contiguous     (logical [E, F, d])
  shared  (W1s[F,d], W3s[F,d], W2s[d,F]) or None
  bias    [E] fp32 selection-only bias, or None
  offset  [E] fp32 additive logit offset, or None

Distributions: X ~ N(0, 1); W1, W3 ~ N(0, 1/sqrt(d)); W2 ~ N(0, 1/sqrt(F));
W_g ~ N(0, 1/sqrt(d)) unless the workload fixes another std; bias ~ N(0, std);
all drawn in fp32, then rounded to bf16 (round-to-nearest-even) for bf16
workloads.  The skewed-load workload adds o_e = -s * ln(r_e) with r a seeded
random permutation of 1..E, i.e. expert popularity proportional to r^-s.

FP8 workloads (wdtype "fp8") draw the same fp32 expert weights and store them
as FP8 E4M3 codes with one fp32 scale per output channel (storage row):
scale = max|row| / 448, code = E4M3(row / scale) rounded to nearest even
(torch's float8_e4m3fn cast); "scales" holds (W1_scale [E,F], W3_scale [E,F],
W2_scale [E,d]) and "shared_scales" the shared expert's three vectors.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d: int
    E: int
    k: int
    F: int
    dtype: str = "bf16"            # "bf16" | "f32"
    score: str = "softmax"         # "softmax" | "sigmoid"
    renorm: bool = True
    n_shared: int = 0
    cf: float | None = None        # capacity factor; None = no capacity limit
    wg_std: float | None = None    # None -> 1/sqrt(d)
    bias_std: float | None = None  # sigmoid selection bias std, None = no bias
    zipf_s: float | None = None    # per-expert logit offset exponent
    wdtype: str = "same"           # "same" | "fp8" (E4M3 expert weights, bf16 layer)
    n_group: int = 1               # group-limited routing: groups of E / n_group experts
    topk_group: int = 1            # groups a token may use
    routing: str = "token"         # "token" (top-k) | "expert" (each expert takes C tokens)
    reroute: bool = False          # capacity overflow re-routed to a backup expert
    seed: int = 0                  # seed of the weights
    x_seed: int | None = None      # seed of X (defaults to ``seed``)
    note: str = field(default="", compare=False)

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five layer shapes the measurements are quoted on.
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", T=256, d=256, E=8, k=2, F=512,
                          dtype="f32", wg_std=0.02, seed=1,
                          note="tiny fp32 layer, softmax top-2 renorm"),
    "mixtral_prefill": Workload("mixtral_prefill", T=4096, d=4096, E=8, k=2,
                                F=14336, seed=2,
                                note="Mixtral-8x7B-shaped prefill, top-2"),
    "dsv3_prefill": Workload("dsv3_prefill", T=4096, d=7168, E=256, k=8,
                             F=2048, score="sigmoid", n_shared=1,
                             bias_std=0.01, seed=3,
                             note="DeepSeek-V3-shaped prefill, 256+1 experts"),
    "dsv3_decode": Workload("dsv3_decode", T=64, d=7168, E=256, k=8, F=2048,
                            score="sigmoid", n_shared=1, bias_std=0.01,
                            seed=3, x_seed=4,
                            note="DeepSeek-V3-shaped decode step, 64 tokens"),
    "switch_capacity": Workload("switch_capacity", T=8192, d=2048, E=64, k=1,
                                F=4096, cf=1.0, zipf_s=1.2, seed=5,
                                note="Switch-style top-1, skewed, CF 1.0"),
}
WORKLOADS["switch_capacity_cf125"] = WORKLOADS["switch_capacity"].with_(
    name="switch_capacity_cf125", cf=1.25, note="Switch-style top-1, CF 1.25")
# DeepSeek-V3 routing with its group limit: 8 groups of 32 experts, 4 per token.
WORKLOADS["dsv3_prefill_grouped"] = WORKLOADS["dsv3_prefill"].with_(
    name="dsv3_prefill_grouped", n_group=8, topk_group=4,
    note="DeepSeek-V3-shaped prefill, group-limited routing (8 groups, 4 used)")
# The same layers with FP8 E4M3 expert weights (per-output-channel scales).
for _n in ("dsv3_prefill", "dsv3_decode", "switch_capacity", "mixtral_prefill"):
    WORKLOADS[_n + "_fp8"] = WORKLOADS[_n].with_(name=_n + "_fp8", wdtype="fp8",
                                                 note=WORKLOADS[_n].note + ", FP8 weights")

# Expert-choice routing on the Mixtral and DeepSeek-V3 shapes: every expert
# takes C = T*k/E tokens (1024 and 128), the same number of rows as top-k.
WORKLOADS["mixtral_prefill_ec"] = WORKLOADS["mixtral_prefill"].with_(
    name="mixtral_prefill_ec", routing="expert", renorm=False,
    note="Mixtral-8x7B-shaped prefill, expert choice, 1024 tokens per expert")
WORKLOADS["dsv3_prefill_ec"] = WORKLOADS["dsv3_prefill"].with_(
    name="dsv3_prefill_ec", routing="expert", renorm=False, bias_std=None,
    note="DeepSeek-V3-shaped prefill, expert choice (sigmoid scores), 128 tokens per expert")

# The skewed Switch layer with its overflow re-routed to each token's second choice.
WORKLOADS["switch_capacity_reroute"] = WORKLOADS["switch_capacity"].with_(
    name="switch_capacity_reroute", reroute=True,
    note="Switch-style top-1, skewed, CF 1.0, overflow re-routed to the second choice")

# Reduced versions: same routing rule and dtype, sizes the CPU oracle finishes
# in seconds, with several tiles per expert and ragged tails.
SMALL = {
    "tiny_fp32": WORKLOADS["tiny_fp32"],
    "mixtral_prefill": WORKLOADS["mixtral_prefill"].with_(
        name="mixtral_prefill_small", T=600, d=512, F=640),
    "dsv3_prefill": WORKLOADS["dsv3_prefill"].with_(
        name="dsv3_prefill_small", T=200, d=512, E=32, F=256),
    "dsv3_decode": WORKLOADS["dsv3_decode"].with_(
        name="dsv3_decode_small", T=16, d=512, E=32, F=256),
    "switch_capacity": WORKLOADS["switch_capacity"].with_(
        name="switch_capacity_small", T=700, d=256, E=16, F=512),
    "switch_capacity_cf125": WORKLOADS["switch_capacity_cf125"].with_(
        name="switch_capacity_cf125_small", T=700, d=256, E=16, F=512),
}
for _n in ("dsv3_prefill", "dsv3_decode", "switch_capacity", "mixtral_prefill"):
    SMALL[_n + "_fp8"] = SMALL[_n].with_(name=SMALL[_n].name + "_fp8", wdtype="fp8")
SMALL["dsv3_prefill_grouped"] = SMALL["dsv3_prefill"].with_(
    name="dsv3_prefill_grouped_small", n_group=8, topk_group=4)
SMALL["mixtral_prefill_ec"] = SMALL["mixtral_prefill"].with_(
    name="mixtral_prefill_ec_small", routing="expert", renorm=False)
SMALL["dsv3_prefill_ec"] = SMALL["dsv3_prefill"].with_(
    name="dsv3_prefill_ec_small", routing="expert", renorm=False, bias_std=None)
SMALL["tiny_fp32_ec"] = SMALL["tiny_fp32"].with_(
    name="tiny_fp32_ec", routing="expert", renorm=False, cf=1.25)
SMALL["switch_capacity_reroute"] = SMALL["switch_capacity"].with_(
    name="switch_capacity_reroute_small", reroute=True)
SMALL["dsv3_prefill_reroute"] = SMALL["dsv3_prefill"].with_(
    name="dsv3_prefill_reroute_small", cf=1.0, reroute=True)
SMALL["mixtral_grouped_reroute"] = SMALL["mixtral_prefill"].with_(
    name="mixtral_grouped_reroute_small", E=16, k=4, n_group=4, topk_group=2, cf=0.9,
    reroute=True)
SMALL["mixtral_grouped"] = SMALL["mixtral_prefill"].with_(
    name="mixtral_grouped_small", E=16, k=4, n_group=4, topk_group=2)


def _seed(*parts: int) -> int:
    """Mix integer parts into one 63-bit generator seed."""
    ss = np.random.SeedSequence([int(p) & 0xFFFFFFFF for p in parts])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _normal(shape, std, seed_parts, device, dtype):
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*seed_parts))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


# tensor ids inside a workload's seed stream
_X, _WG, _W1, _W3, _W2, _S1, _S3, _S2, _BIAS, _PERM = range(10)


E4M3_MAX = 448.0


def quantize_e4m3_rows(t: torch.Tensor):
    """fp32 [..., N, K] -> (uint8 E4M3 codes [..., N, K], fp32 scales [..., N])."""
    amax = t.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    codes = (t / scale.unsqueeze(-1)).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.to(torch.float32)


def make_inputs(w: Workload, device="cpu") -> dict:
    """Draw every input of workload ``w`` on ``device`` (storage layout)."""
    dt = w.torch_dtype
    dev = torch.device(device)
    fp8 = w.wdtype == "fp8"
    if fp8 and w.dtype != "bf16":
        raise ValueError("FP8 expert weights need a bf16 layer")
    xs = w.seed if w.x_seed is None else w.x_seed
    out = {"workload": w}
    out["X"] = _normal((w.T, w.d), 1.0, (xs, _X), dev, dt)
    wg_std = w.wg_std if w.wg_std is not None else 1.0 / np.sqrt(w.d)
    out["Wg"] = _normal((w.E, w.d), wg_std, (w.seed, _WG), dev, dt)
    s_in, s_out = 1.0 / np.sqrt(w.d), 1.0 / np.sqrt(w.F)
    scales = []
    for name, tid, shp, std in (("W1", _W1, (w.F, w.d), s_in),
                                ("W3", _W3, (w.F, w.d), s_in),
                                ("W2", _W2, (w.d, w.F), s_out)):
        t = torch.empty((w.E,) + shp, device=dev, dtype=torch.uint8 if fp8 else dt)
        sc = torch.empty((w.E, shp[0]), device=dev, dtype=torch.float32) if fp8 else None
        for e in range(w.E):            # one expert at a time bounds the fp32 temp
            if fp8:
                t[e], sc[e] = quantize_e4m3_rows(
                    _normal(shp, std, (w.seed, tid, e), dev, torch.float32))
            else:
                t[e] = _normal(shp, std, (w.seed, tid, e), dev, dt)
        out[name] = t
        scales.append(sc)
    out["scales"] = tuple(scales) if fp8 else None
    out["shared_scales"] = None
    if w.n_shared:
        shp3 = (((w.F, w.d), s_in, _S1), ((w.F, w.d), s_in, _S3), ((w.d, w.F), s_out, _S2))
        if fp8:
            q = [quantize_e4m3_rows(_normal(shp, std, (w.seed, tid), dev, torch.float32))
                 for shp, std, tid in shp3]
            out["shared"] = tuple(c for c, _ in q)
            out["shared_scales"] = tuple(sc for _, sc in q)
        else:
            out["shared"] = tuple(_normal(shp, std, (w.seed, tid), dev, dt)
                                  for shp, std, tid in shp3)
    else:
        out["shared"] = None
    out["bias"] = (None if w.bias_std is None else
                   _normal((w.E,), w.bias_std, (w.seed, _BIAS), dev,
                           torch.float32))
    if w.zipf_s is not None:
        rng = np.random.default_rng(_seed(w.seed, _PERM))
        ranks = rng.permutation(np.arange(1, w.E + 1)).astype(np.float64)
        out["offset"] = torch.tensor(-w.zipf_s * np.log(ranks),
                                     dtype=torch.float32, device=dev)
    else:
        out["offset"] = None
    return out


def weight_elem_bytes(w: Workload) -> int:
    """Bytes per stored expert-weight element."""
    return 1 if w.wdtype == "fp8" else (2 if w.dtype == "bf16" else 4)


def weight_bytes(w: Workload) -> int:
    """Bytes of all resident expert weights (routed + shared), scales excluded."""
    return (w.E + w.n_shared) * 3 * w.d * w.F * weight_elem_bytes(w)
