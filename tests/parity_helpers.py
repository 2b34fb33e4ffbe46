"""Helpers shared by the GPU parity tests: storage layout -> the oracle's
logical float64 arrays, and the tolerance checks (documented in the design
notes).  No arithmetic of the method lives here."""
import numpy as np
import torch

from oracle import moe_oracle as O

# Tolerances.  Element-wise relative error is ill-posed near zero, so float
# results are compared against the reference's RMS.
LOGIT_REL = 1e-5       # per row: max_e |dl| <= 1e-5 * RMS_e(l_ref)
F32_REL = 1e-4         # fp32 outputs: max |dY| <= 1e-4 * RMS(Y_ref)
BF16_REL = 2e-2        # bf16 outputs: max |dY| <= 2e-2 * RMS(Y_ref)
GATE_REL, GATE_ABS = 1e-5, 1e-7
SIGMOID_TIE = 1e-12    # keys closer than this may legitimately order either way


def np64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def e4m3_table():
    """The oracle's value of each of the 256 E4M3 codes."""
    return O.decode_e4m3(np.arange(256))


def weights64(t, scale=None):
    """Storage-layout weights as float64.  E4M3 codes (uint8) become
    O.dequantize_rows(codes, scale) = value(code) * scale of their row,
    evaluated as a lookup in the oracle's table of the 256 code values
    followed by one fp64 multiply (the same numbers; pinned against
    O.dequantize_rows in the CPU tests).  The lookup runs where the codes
    live, so full-size expert matrices decode in milliseconds."""
    if t.dtype == torch.uint8:
        lut = torch.as_tensor(e4m3_table(), dtype=torch.float64, device=t.device)
        w = lut[t.long()] * scale.detach().to(torch.float64).unsqueeze(-1)
        return w.cpu().numpy()
    return np64(t)


def logical(inp):
    """Oracle-side view of a workload's tensors (pages' logical shapes)."""
    sc = inp.get("scales") or (None, None, None)
    out = {
        "X": np64(inp["X"]),
        "Wg": np64(inp["Wg"]).T,
        "W1": weights64(inp["W1"], sc[0]).transpose(0, 2, 1),
        "W3": weights64(inp["W3"], sc[1]).transpose(0, 2, 1),
        "W2": weights64(inp["W2"], sc[2]).transpose(0, 2, 1),
        "bias": None if inp["bias"] is None else np64(inp["bias"]),
        "offset": None if inp["offset"] is None else np64(inp["offset"]),
        "shared": None,
    }
    if inp["shared"] is not None:
        s1, s3, s2 = inp["shared"]
        ss = inp.get("shared_scales") or (None, None, None)
        out["shared"] = (weights64(s1, ss[0]).T, weights64(s3, ss[1]).T, weights64(s2, ss[2]).T)
    return out


def expert_logical(inp, e):
    """One expert's logical matrices (W1 [d,F], W3 [d,F], W2 [F,d])."""
    sc = inp.get("scales") or (None, None, None)
    pick = (lambda i: None) if sc[0] is None else (lambda i: sc[i][e])
    return (weights64(inp["W1"][e], pick(0)).T, weights64(inp["W3"][e], pick(1)).T,
            weights64(inp["W2"][e], pick(2)).T)


def rel_err(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2)) if ref.size else 0.0
    if ref.size == 0:
        return 0.0
    return float(np.abs(got - ref).max() / max(rms, 1e-30))


def check_logits(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rms = np.sqrt(np.mean(ref ** 2, axis=1))
    worst = np.abs(got - ref).max(axis=1) / np.maximum(rms, 1e-30)
    assert worst.max() <= LOGIT_REL, f"logit rel err {worst.max():.3e}"


def check_ids(gpu_ids, ref_ids, keys=None):
    """Bit-exact ids; for sigmoid keys, a mismatch is accepted only when the
    swapped experts' keys are within SIGMOID_TIE (both orders correct)."""
    gpu_ids = np.asarray(gpu_ids)
    ref_ids = np.asarray(ref_ids)
    bad = np.flatnonzero((gpu_ids != ref_ids).any(axis=1))
    if bad.size and keys is not None:
        for t in bad:
            kg = keys[t, gpu_ids[t]]
            kr = keys[t, ref_ids[t]]
            assert np.abs(np.sort(kg)[::-1] - np.sort(kr)[::-1]).max() <= SIGMOID_TIE, t
        return bad.size
    assert bad.size == 0, f"{bad.size} tokens with different expert ids, first {bad[:5]}"
    return 0


def check_gates(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert (np.abs(got - ref) <= GATE_REL * np.abs(ref) + GATE_ABS).all(), \
        f"gate err {np.abs(got - ref).max():.3e}"


def active_rms(ref):
    """RMS over rows that receive any contribution.  Rows whose every path
    was dropped by the capacity limit are exactly zero on both sides; they
    would shrink RMS(Y) and turn the output's own bf16 rounding into a false
    failure.  Without drops this is RMS(Y)."""
    ref = np.asarray(ref, np.float64)
    live = np.abs(ref).max(axis=1) > 0 if ref.ndim == 2 else np.ones(ref.shape, bool)
    return float(np.sqrt(np.mean(ref[live] ** 2))) if live.any() else 0.0


def check_rows(got, ref, bf16, label="", output_rounding=False):
    """max|got - ref| / RMS(ref) <= tol.  With ``output_rounding`` the result
    is stored in its own dtype (the layer output Y), and that format's
    half-ulp (2^-9 |ref| for bf16, 2^-24 |ref| for fp32) is allowed element by
    element on top of the budget: the final store cannot be more exact."""
    tol = BF16_REL if bf16 else F32_REL
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = active_rms(ref)
    rms = rms if rms > 0 else 1.0
    d = np.abs(got - ref)
    e = float(d.max() / rms)
    if output_rounding:
        half_ulp = (2.0 ** -9 if bf16 else 2.0 ** -24) * np.abs(ref)
        e_cmp = float(np.maximum(d - half_ulp, 0.0).max() / rms)
    else:
        e_cmp = e
    if label:
        print(f"[err] {label}: max|d|/rms = {e:.3e}, beyond output rounding {e_cmp:.3e} "
              f"(tol {tol})", flush=True)
    assert e_cmp <= tol, f"{label} rel err {e_cmp:.3e} > {tol}"
    return e


EC_TIE = 1e-12         # expert-choice scores closer than this may order either way


def check_expert_choice(slot_row, gates, lg, score, C):
    """The device's expert-choice assignment against the oracle's, both on
    the device's fp32 logits.  Every expert must take exactly min(C, T)
    tokens; a column that differs from the oracle's is accepted only when
    every token it took scores within EC_TIE of every token it left (a
    near-tie, both choices correct).  Gates must be the oracle's scores on
    taken slots and exactly 0 elsewhere.  Returns (mask, near-tie columns)."""
    lg = np.asarray(lg, np.float64)
    T, E = lg.shape
    mask_ref, g_ref, p = O.expert_choice(lg, score, C)
    sr = np.asarray(slot_row).reshape(T, E)
    mask = sr >= 0
    assert (mask.sum(axis=0) == min(C, T)).all(), "an expert took the wrong number of tokens"
    bad = np.flatnonzero((mask != mask_ref).any(axis=0))
    for e in bad:
        lo = p[mask[:, e], e].min()
        hi = p[~mask[:, e], e].max()
        assert lo >= hi - EC_TIE, f"expert {e}: taken score {lo} < left score {hi}"
    g = np.asarray(gates, np.float64).reshape(T, E)
    assert (g[~mask] == 0).all()
    check_gates(g[mask], p[mask])
    return mask, int(bad.size)
