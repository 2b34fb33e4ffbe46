"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Reduced workloads (several tiles per expert, ragged tails) are compared
element by element; the full-size workloads are in test_gpu_fullsize.py.
"""
import numpy as np
import pytest
import torch

import mixture_experts_layer_47_amd as moe
from mixture_experts_layer_47_amd.workloads import SMALL, Workload, make_inputs, quantize_e4m3_rows
from oracle import moe_oracle as O
from tests import parity_helpers as H

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _announce(msg):
    print(f"[case] {msg}", flush=True)


def _oracle_forward(inp, lg_gpu):
    w = inp["workload"]
    L = H.logical(inp)
    cap = O.capacity(w.cf, w.T, w.k, w.E) if w.cf else None
    return O.forward(L["X"], L["Wg"], L["W1"], L["W3"], L["W2"], k=w.k, score_func=w.score,
                     renorm=w.renorm, bias=L["bias"], offset=L["offset"], cap=cap,
                     shared=L["shared"], bf16_h=(w.dtype == "bf16"), logits=lg_gpu,
                     n_group=w.n_group, topk_group=w.topk_group, reroute=w.reroute), cap


def _full_check(inp):
    w = inp["workload"]
    layer = moe.layer_from_inputs(inp)
    Y, aux = moe.forward(layer, inp["X"], aux=True)
    torch.cuda.synchronize()
    lg = H.np64(aux["logits"])
    ref, cap = _oracle_forward(inp, lg)
    bf16 = w.dtype == "bf16"
    # R1: logits against the oracle's own fp64 logits
    H.check_logits(lg, ref["logits"])
    # R2: ids exact (oracle top-k on the device's fp32 logits), gates within tolerance
    _, keys = O.select_topk(lg, w.k, w.score, H.logical(inp)["bias"], w.n_group, w.topk_group)
    ties = H.check_ids(H.np64(aux["topk_ids"]).astype(np.int64), ref["ids"],
                       keys if w.score == "sigmoid" else None)
    assert ties == 0, "near-tie reordering in a small workload"
    H.check_gates(H.np64(aux["topk_w"]), ref["gates"])
    # D1: dispatch bit-exact (with the backup round when the layer re-routes)
    d = ref["dispatch"]
    R = d["n_kept"]
    if w.reroute:
        print(f"[info] {w.name}: re-routed {d['n_rerouted']} of "
              f"{w.T * w.k - O.dispatch(ref['ids'], w.E, cap)['n_kept']} dropped slots",
              flush=True)
    assert int(aux["n_kept"].item()) == R
    assert aux["counts"].cpu().numpy().tolist() == d["counts"].tolist()
    assert aux["offsets"].cpu().numpy().tolist() == d["offsets"].tolist()
    assert aux["slot_row"].cpu().numpy().tolist() == d["slot_row"].tolist()
    assert aux["sorted_slot"].cpu().numpy()[:R].tolist() == d["sorted_slot"].tolist()
    # G1/G2: expert rows; S: shared rows
    rows = H.np64(aux["Yrows"])
    if R:
        H.check_rows(rows[:R], ref["rows"], bf16, f"{w.name} expert rows")
    if ref["shared"] is not None:
        H.check_rows(rows[R:R + w.T], ref["shared"], bf16, f"{w.name} shared rows")
    # C: layer output
    H.check_rows(H.np64(Y), ref["Y"], bf16, f"{w.name} Y", output_rounding=True)
    # dropped-everything tokens are exactly zero
    dead = (np.asarray(d["slot_row"]).reshape(w.T, w.k) < 0).all(axis=1) if w.T else \
        np.zeros(0, bool)
    if ref["shared"] is None and dead.any():
        assert (H.np64(Y)[dead] == 0).all()
    # B: prob_sum and the balance statistic
    ps_ref = ref["probs"].sum(axis=0)
    ps = H.np64(aux["prob_sum"])
    assert np.abs(ps - ps_ref).max() <= 1e-5 * max(1.0, np.abs(ps_ref).max())
    bal_ref = O.balance_stat(d["counts"], ps_ref, w.T, w.k)
    assert abs(aux["balance"].item() - bal_ref) <= 1e-5 * max(1.0, abs(bal_ref))
    # router health: entropies, load CV, drop rate
    hr = O.router_health(lg, w.score, d["counts"], R, w.T, w.k)
    hg = aux["health"].cpu().numpy()
    assert abs(hg[0] - hr["token_entropy"]) <= 1e-4 * max(1.0, hr["token_entropy"])
    assert abs(hg[1] - hr["load_entropy"]) <= 1e-12 * max(1.0, hr["load_entropy"])
    assert abs(hg[2] - hr["load_cv"]) <= 1e-12 * max(1.0, hr["load_cv"])
    assert abs(hg[3] - hr["drop_rate"]) <= 1e-15
    return Y, aux


def _ec_capacity(w):
    return min(w.T, O.capacity(w.cf or 1.0, w.T, w.k, w.E)) if w.T else 0


def _full_check_ec(inp):
    """Expert-choice forward: every step against the oracle on the device's
    logits; the device's assignment is validated first (near-ties aside it
    must be the oracle's), then the rows, layout and output use it."""
    w = inp["workload"]
    layer = moe.layer_from_inputs(inp)
    Y, aux = moe.forward(layer, inp["X"], aux=True)
    torch.cuda.synchronize()
    L = H.logical(inp)
    lg = H.np64(aux["logits"])
    H.check_logits(lg, O.router_logits(L["X"], L["Wg"], L["offset"]))
    Ce = _ec_capacity(w)
    mask, ties = H.check_expert_choice(H.np64(aux["slot_row"]).astype(np.int64),
                                       H.np64(aux["topk_w"]), lg, w.score, Ce)
    assert ties == 0, "near-tie reordering in a small workload"
    bf16 = w.dtype == "bf16"
    ref = O.forward_expert_choice(L["X"], L["Wg"], L["W1"], L["W3"], L["W2"], C=Ce,
                                  score_func=w.score, offset=L["offset"], shared=L["shared"],
                                  bf16_h=bf16, logits=lg, mask=mask)
    d = ref["dispatch"]
    R = d["n_kept"]
    assert R == w.E * Ce and int(aux["n_kept"].item()) == R
    assert aux["counts"].cpu().tolist() == [Ce] * w.E
    assert aux["offsets"].cpu().tolist() == d["offsets"].tolist()
    assert aux["slot_row"].cpu().reshape(-1).tolist() == d["slot_row"].tolist()
    assert aux["sorted_slot"].cpu()[:R].tolist() == d["sorted_slot"].tolist()
    rows = H.np64(aux["Yrows"])
    if R:
        H.check_rows(rows[:R], ref["rows"], bf16, f"{w.name} expert rows")
    if ref["shared"] is not None:
        H.check_rows(rows[R:R + w.T], ref["shared"], bf16, f"{w.name} shared rows")
    H.check_rows(H.np64(Y), ref["Y"], bf16, f"{w.name} Y", output_rounding=True)
    untaken = ~mask.any(axis=1)
    print(f"[info] {w.name}: C={Ce}, tokens taken by no expert {int(untaken.sum())}, "
          f"most experts on one token {int(mask.sum(axis=1).max()) if w.T else 0}", flush=True)
    if ref["shared"] is None and untaken.any():
        assert (H.np64(Y)[untaken] == 0).all()
    return Y, aux, mask


def _random_layer(seed):
    """A seeded random layer inside the library's limits: d and F multiples
    of 128, k <= min(8, E), one shared expert or none, FP8 weights only on a
    bf16 layer, expert choice without renorm, bias or groups, re-route only
    with a capacity factor, groups only where they divide E and can hold k."""
    r = np.random.default_rng(1000 + seed)
    E = int(r.choice([2, 4, 8, 12, 16, 32, 64, 96, 256]))
    k = int(r.integers(1, min(8, E) + 1))
    dtype = "f32" if r.random() < 0.2 else "bf16"
    score = str(r.choice(["softmax", "sigmoid"]))
    kw = dict(name=f"random{seed}", T=int(r.choice([1, 3, 17, 64, 129, 300, 513, 700])),
              d=int(r.choice([128, 256, 384, 512])), E=E, k=k,
              F=int(r.choice([128, 256, 384, 640])), dtype=dtype, score=score,
              n_shared=int(r.random() < 0.4), seed=5000 + seed)
    if dtype == "bf16" and r.random() < 0.3:
        kw["wdtype"] = "fp8"
    if r.random() < 0.3:
        kw["zipf_s"] = 1.1
    if r.random() < 0.2:
        kw.update(routing="expert", renorm=False)
        if r.random() < 0.5:
            kw["cf"] = float(r.choice([0.5, 1.0, 1.5]))
        return Workload(**kw)
    kw["renorm"] = bool(r.random() < 0.6)
    if score == "sigmoid" and r.random() < 0.6:
        kw["bias_std"] = 0.01
    if r.random() < 0.5:
        kw["cf"] = float(r.choice([0.5, 1.0, 1.25, 2.0]))
        kw["reroute"] = bool(r.random() < 0.5)
    divs = [g for g in (2, 4, 8) if E % g == 0]
    if divs and r.random() < 0.3:
        ng = int(r.choice(divs))
        tg = int(r.integers(1, ng + 1))
        if k <= tg * (E // ng):
            kw.update(n_group=ng, topk_group=tg)
    return Workload(**kw)


@pytest.mark.parametrize("seed", range(64))
def test_forward_random_layers(seed):
    """Seeded random layer configurations (shapes, router, renorm, capacity,
    re-route, groups, shared expert, expert choice, fp32 / bf16 / FP8), each
    checked step by step against the oracle like the named workloads."""
    w = _random_layer(seed)
    _announce(f"random layer {seed}: {w}")
    inp = make_inputs(w, DEV)
    if w.routing == "expert":
        _full_check_ec(inp)
    else:
        _full_check(inp)


@pytest.mark.parametrize("name", list(SMALL))
def test_forward_small_workloads(name):
    w = SMALL[name]
    _announce(f"forward {w.name} T={w.T} d={w.d} E={w.E} k={w.k} F={w.F} routing={w.routing}")
    inp = make_inputs(w, DEV)
    if w.routing == "expert":
        _full_check_ec(inp)
    else:
        _full_check(inp)


EC_EDGE = {
    "T1": Workload("ec_T1", T=1, d=256, E=8, k=2, F=256, routing="expert", renorm=False,
                   seed=31),
    "E1_ties": Workload("ec_E1", T=70, d=128, E=1, k=1, F=128, routing="expert",
                        renorm=False, cf=0.5, seed=32),
    "dense_cap": Workload("ec_dense", T=40, d=256, E=4, k=2, F=256, dtype="f32",
                          routing="expert", renorm=False, cf=8.0, seed=33),
    "decode_sigmoid_shared": Workload("ec_decode", T=16, d=512, E=32, k=8, F=256,
                                      score="sigmoid", n_shared=1, routing="expert",
                                      renorm=False, seed=34),
    "many_chunks": Workload("ec_chunks", T=2500, d=128, E=8, k=2, F=128, routing="expert",
                            renorm=False, cf=0.75, seed=35),
    "E256_fp8": Workload("ec_E256_fp8", T=96, d=256, E=256, k=8, F=128, score="sigmoid",
                         routing="expert", renorm=False, wdtype="fp8", seed=36),
}


@pytest.mark.parametrize("name", list(EC_EDGE))
def test_forward_expert_choice_edge_cases(name):
    w = EC_EDGE[name]
    _announce(f"expert-choice edge {name}")
    inp = make_inputs(w, DEV)
    Y, aux, mask = _full_check_ec(inp)
    if name == "E1_ties":
        # every softmax score is 1: the tie rule takes the first C tokens
        assert np.flatnonzero(mask[:, 0]).tolist() == list(range(_ec_capacity(w)))
    if name == "dense_cap":
        assert mask.all()          # C >= T: every expert takes every token


def test_expert_choice_empty_batch():
    w = Workload("ec_empty", T=0, d=256, E=8, k=2, F=256, routing="expert", renorm=False,
                 seed=37)
    _announce("expert-choice empty batch")
    inp = make_inputs(w, DEV)
    Y, aux = moe.forward(moe.layer_from_inputs(inp), inp["X"], aux=True)
    torch.cuda.synchronize()
    assert Y.shape == (0, 256)
    assert aux["counts"].cpu().tolist() == [0] * 8
    assert int(aux["n_kept"].item()) == 0


EDGE = {
    "T1": Workload("T1", T=1, d=256, E=8, k=2, F=256, seed=11),
    "k_eq_E": Workload("k_eq_E", T=37, d=256, E=4, k=4, F=256, seed=12),
    "E1_k1": Workload("E1_k1", T=70, d=128, E=1, k=1, F=128, seed=13),
    "ragged_tk": Workload("ragged_tk", T=45, d=384, E=6, k=3, F=384, seed=14),
    "cap_c1": Workload("cap_c1", T=50, d=256, E=8, k=2, F=256, cf=0.08, seed=15),
    "cap_large": Workload("cap_large", T=50, d=256, E=8, k=2, F=256, cf=64.0, seed=16),
    "sigmoid_norenorm": Workload("sigmoid_norenorm", T=64, d=256, E=16, k=4, F=256,
                                 score="sigmoid", renorm=False, bias_std=0.01, seed=17),
    "softmax_norenorm_f32": Workload("softmax_norenorm_f32", T=40, d=256, E=8, k=2, F=256,
                                     dtype="f32", renorm=False, seed=18),
    "shared_f32": Workload("shared_f32", T=33, d=256, E=8, k=2, F=256, dtype="f32",
                           n_shared=1, seed=19),
    "E256_k16": Workload("E256_k16", T=20, d=256, E=256, k=16, F=128, score="sigmoid",
                         bias_std=0.01, seed=20),
    # many tokens through a narrow layer: 131072 slots (128 dispatch chunks),
    # 65536 combine blocks, thousands of row tiles
    "T65536": Workload("T65536", T=65536, d=128, E=8, k=2, F=128, cf=1.1, seed=24),
}


@pytest.mark.parametrize("name", list(EDGE))
def test_forward_edge_cases(name):
    w = EDGE[name]
    _announce(f"edge {name}")
    inp = make_inputs(w, DEV)
    if name == "E1_k1":
        # a single expert: the layer reduces to one dense SwiGLU FFN
        Y = moe.forward(moe.layer_from_inputs(inp), inp["X"])
        L = H.logical(inp)
        dense = O.expert_ffn(L["X"], L["W1"][0], L["W3"][0], L["W2"][0], bf16_h=True)
        H.check_rows(H.np64(Y), dense, True, "E1 dense", output_rounding=True)
    _full_check(inp)


def test_collapse_all_tokens_to_one_expert():
    """Router collapse: every token's top choice is expert 5; capacity keeps
    only the first C of its slots and drops the rest."""
    w = Workload("collapse", T=300, d=256, E=8, k=2, F=256, cf=1.0, seed=21)
    _announce("collapse")
    inp = make_inputs(w, DEV)
    inp["Wg"].zero_()
    off = torch.zeros(8, device=DEV)
    off[5] = 10.0
    off[2] = 5.0
    inp["offset"] = off
    Y, aux = _full_check(inp)
    C = O.capacity(1.0, 300, 2, 8)
    counts = aux["counts"].cpu().tolist()
    assert counts[5] == 300 and counts[2] == 300
    assert int(aux["n_kept"].item()) == 2 * C


def test_empty_batch():
    w = Workload("empty", T=0, d=256, E=8, k=2, F=256, seed=22)
    _announce("empty batch")
    inp = make_inputs(w, DEV)
    Y, aux = moe.forward(moe.layer_from_inputs(inp), inp["X"], aux=True)
    torch.cuda.synchronize()
    assert Y.shape == (0, 256)
    assert aux["counts"].cpu().tolist() == [0] * 8
    assert int(aux["n_kept"].item()) == 0


@pytest.mark.parametrize("name", ["dsv3_prefill", "mixtral_prefill_ec", "switch_capacity_reroute",
                                  "mixtral_prefill"])
def test_deterministic_bitwise(name):
    """Every output is bit-identical run to run (no floating-point atomics;
    top-k, expert-choice selection, re-route and the K-split down path)."""
    w = SMALL[name]
    _announce(f"determinism {w.name}")
    inp = make_inputs(w, DEV)
    f = moe.Forward(moe.layer_from_inputs(inp), inp["X"], aux=True)
    Y1 = f().clone()
    a1 = {k: v.clone() for k, v in f.aux.items()}
    for _ in range(3):
        Y2 = f()
        torch.cuda.synchronize()
        assert torch.equal(Y1, Y2)
        for k in a1:
            assert torch.equal(a1[k], f.aux[k]), k


@pytest.mark.parametrize("name", ["mixtral_prefill", "dsv3_prefill", "dsv3_prefill_fp8",
                                  "mixtral_prefill_ec", "switch_capacity_reroute"])
def test_forward_graph_replay(name):
    """moe_forward launches kernels only (no allocation, no host
    synchronisation, no memset nodes), so a HIP graph can record it. Every
    replay, with eager work on the stream between replays, matches the eager
    call bit for bit, also after new tokens are copied into the captured
    input (routing, counts and tile lists are rebuilt on the device)."""
    import dataclasses
    w = SMALL[name]
    _announce(f"graph replay {w.name}")
    inp = make_inputs(w, DEV)
    layer = moe.layer_from_inputs(inp)
    X2 = make_inputs(dataclasses.replace(w, x_seed=w.seed + 101), DEV)["X"]
    want = []
    for X in (inp["X"], X2):
        e = moe.Forward(layer, X.clone(), aux=True)
        for t in e.aux.values():
            t.fill_(-7)  # rows the layer leaves unwritten (dropped slots) hold -7 on both sides
        want.append((e().clone(), {k: v.clone() for k, v in e.aux.items()}))
    f = moe.Forward(layer, inp["X"].clone(), aux=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        f()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        f()
    torch.cuda.synchronize()
    for rep, which in enumerate((0, 1, 0, 1)):
        f.X.copy_(inp["X"] if which == 0 else X2)
        f.Y.fill_(float("nan"))
        for t in f.aux.values():
            t.fill_(-7)
        junk = torch.randn(4096, 256, device=DEV) @ torch.randn(256, 256, device=DEV)
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk).all()
        Y_ref, aux_ref = want[which]
        assert torch.equal(f.Y, Y_ref), f"replay {rep}"
        for k in aux_ref:
            assert torch.equal(f.aux[k], aux_ref[k]), (rep, k)


# ---------------------------------------------------------- entry points --
@pytest.mark.parametrize("score,ng,tg", [("sigmoid", 1, 1), ("sigmoid", 8, 4), ("sigmoid", 4, 1),
                                         ("softmax", 8, 2), ("softmax", 32, 32)])
def test_route_entry_point(score, ng, tg):
    w = SMALL["dsv3_prefill"].with_(T=333, score=score,
                                    bias_std=0.01 if score == "sigmoid" else None)
    _announce(f"moe_route {score} n_group={ng} topk_group={tg}")
    inp = make_inputs(w, DEV)
    r = moe.route(inp["X"], inp["Wg"], w.k, w.score, w.renorm, bias=inp["bias"], n_group=ng,
                  topk_group=tg)
    torch.cuda.synchronize()
    L = H.logical(inp)
    lg = H.np64(r["logits"])
    H.check_logits(lg, O.router_logits(L["X"], L["Wg"]))
    ids, g, p = O.route(lg, w.k, w.score, w.renorm, L["bias"], ng, tg)
    _, keys = O.select_topk(lg, w.k, w.score, L["bias"], ng, tg)
    H.check_ids(H.np64(r["ids"]).astype(np.int64), ids, keys)
    H.check_gates(H.np64(r["w"]), g)
    assert np.allclose(H.np64(r["prob_sum"]), p.sum(axis=0), rtol=1e-5, atol=1e-5)
    # backups: the next choices in the same key order
    rb = moe.route(inp["X"], inp["Wg"], w.k, w.score, w.renorm, bias=inp["bias"], n_group=ng,
                   topk_group=tg, n_backup=min(w.k, w.E - w.k))
    torch.cuda.synchronize()
    assert torch.equal(rb["ids"], r["ids"]) and torch.equal(rb["w"], r["w"])
    bk_ref = O.backup_experts(lg, w.k, w.score, L["bias"], ng, tg)
    bk = H.np64(rb["backup"]).astype(np.int64)
    if w.score == "softmax":
        assert np.array_equal(bk, bk_ref)
    else:   # near-ties aside; the device's picks must hold keys equal to the oracle's
        diff = np.flatnonzero((bk != bk_ref).any(axis=1))
        for t in diff:
            kg = np.where(bk[t] >= 0, keys[t, np.maximum(bk[t], 0)], -np.inf)
            kr = np.where(bk_ref[t] >= 0, keys[t, np.maximum(bk_ref[t], 0)], -np.inf)
            assert np.allclose(kg, kr, atol=H.SIGMOID_TIE, rtol=0), t


@pytest.mark.parametrize("score,E,ng,tg,dtype", [("softmax", 8, 1, 1, "bf16"),
                                                  ("softmax", 32, 1, 1, "bf16"),
                                                  ("sigmoid", 32, 8, 4, "bf16"),
                                                  ("sigmoid", 20, 1, 1, "bf16"),
                                                  ("softmax", 64, 1, 1, "bf16"),
                                                  ("softmax", 16, 4, 2, "f32"),
                                                  ("sigmoid", 24, 1, 1, "f32")])
def test_route_many_tokens_entry_point(score, E, ng, tg, dtype):
    """moe_route with 2000+ tokens (up to 32 experts: logits and selection
    in one fused launch; 64: the split-K path): logits, ids, gates,
    backups and the probability sums against the oracle."""
    T, k = 2345, min(4, E // 2)
    w = Workload("route_many", T=T, d=512, E=E, k=k, F=128, score=score, dtype=dtype,
                 bias_std=0.01 if score == "sigmoid" else None, zipf_s=1.2, seed=E + T)
    _announce(f"moe_route T={T} E={E} {score} n_group={ng} topk_group={tg} {dtype}")
    inp = make_inputs(w, DEV)
    nb = min(k, E - k)
    r = moe.route(inp["X"], inp["Wg"], k, score, True, bias=inp["bias"], offset=inp["offset"],
                  n_group=ng, topk_group=tg, n_backup=nb)
    torch.cuda.synchronize()
    L = H.logical(inp)
    lg = H.np64(r["logits"])
    H.check_logits(lg, O.router_logits(L["X"], L["Wg"], L["offset"]))
    ids, g, p = O.route(lg, k, score, True, L["bias"], ng, tg)
    _, keys = O.select_topk(lg, k, score, L["bias"], ng, tg)
    H.check_ids(H.np64(r["ids"]).astype(np.int64), ids, keys if score == "sigmoid" else None)
    H.check_gates(H.np64(r["w"]), O.gates(lg, H.np64(r["ids"]).astype(np.int64), score, True))
    assert np.allclose(H.np64(r["prob_sum"]), p.sum(axis=0), rtol=1e-5, atol=1e-4)
    bk_ref = O.backup_experts(lg, k, score, L["bias"], ng, tg)
    bk = H.np64(r["backup"]).astype(np.int64)
    bad = np.flatnonzero((bk != bk_ref).any(axis=1))
    for t in bad:        # only near-ties may order differently
        kg = np.where(bk[t] >= 0, keys[t, np.maximum(bk[t], 0)], -np.inf)
        kr = np.where(bk_ref[t] >= 0, keys[t, np.maximum(bk_ref[t], 0)], -np.inf)
        assert np.allclose(kg, kr, atol=H.SIGMOID_TIE, rtol=0), t
    if score == "softmax":
        assert bad.size == 0


@pytest.mark.parametrize("score,E,k,cf,reroute", [("softmax", 16, 2, 1.25, True),
                                                   ("sigmoid", 32, 6, None, False)])
def test_forward_many_tokens(score, E, k, cf, reroute):
    """A whole layer with 2100 tokens and at most 32 experts, so the router
    runs its fused launch: every step, the balance statistic and the router
    health against the oracle."""
    w = Workload("fwd_many", T=2100, d=256, E=E, k=k, F=256, score=score, cf=cf,
                 reroute=reroute, bias_std=0.01 if score == "sigmoid" else None,
                 n_shared=1 if score == "sigmoid" else 0, zipf_s=1.2 if cf else None, seed=E)
    _announce(f"forward many tokens {score} E={E} k={k} cf={cf} reroute={reroute}")
    _full_check(make_inputs(w, DEV))


@pytest.mark.parametrize("score,T,E,C", [("softmax", 333, 32, 40), ("sigmoid", 333, 32, 40),
                                         ("softmax", 100, 8, 100), ("softmax", 100, 8, 150),
                                         ("sigmoid", 50, 256, 3), ("softmax", 1, 4, 1),
                                         ("softmax", 64, 8, 0), ("softmax", 2500, 8, 700),
                                         ("sigmoid", 3000, 64, 47)])
def test_route_expert_choice_entry_point(score, T, E, C):
    _announce(f"moe_route_expert_choice {score} T={T} E={E} C={C}")
    w = Workload("ec_route", T=T, d=256, E=E, k=1, F=128, score=score, seed=T + E)
    inp = make_inputs(w, DEV)
    X = inp["X"]
    if T >= 8:
        # duplicated tokens: equal logits rows give exact score ties
        X[1:8:2] = X[0:8:2]
    r = moe.route_expert_choice(X, inp["Wg"], C, score)
    torch.cuda.synchronize()
    L = H.logical(inp)
    lg = H.np64(r["logits"])
    H.check_logits(lg, O.router_logits(H.np64(X), L["Wg"]))
    mask, ties = H.check_expert_choice(H.np64(r["slot_row"]).astype(np.int64),
                                       H.np64(r["gates"]), lg, score, C)
    print(f"[info] near-tie experts {ties}", flush=True)
    d = O.expert_choice_dispatch(mask)
    assert r["offsets"].cpu().tolist() == d["offsets"].tolist()
    assert r["sorted_slot"].cpu().tolist() == d["sorted_slot"].tolist()
    assert r["slot_row"].cpu().reshape(-1).tolist() == d["slot_row"].tolist()
    for i in range(0, min(T, 8) - 1, 2):
        if (lg[i] == lg[i + 1]).all():
            # bit-equal scores: a token is never taken while its earlier twin is left
            assert not (mask[i + 1] & ~mask[i]).any()


@pytest.mark.parametrize("T,k,E,C", [(1, 1, 1, 0), (100, 2, 8, 0), (1000, 8, 256, 0),
                                     (1000, 8, 256, 20), (3000, 1, 64, 40), (777, 3, 5, 1),
                                     (5000, 4, 17, 900),
                                     # the one-block path ends at 8192 slots
                                     (8192, 1, 8, 0), (8193, 1, 8, 0), (1024, 8, 256, 40),
                                     (2049, 4, 256, 30)])
@pytest.mark.parametrize("reroute", [False, True])
def test_dispatch_entry_point(T, k, E, C, reroute):
    _announce(f"moe_dispatch T={T} k={k} E={E} C={C} reroute={reroute}")
    _check_dispatch(T, k, E, C, reroute, T * 31 + E, 2.0)


@pytest.mark.parametrize("seed", range(32))
def test_dispatch_random(seed):
    """Seeded random (T, k, E, capacity, re-route, skew): slot counts on
    both sides of the one-block limit (8192), capacities from 1 to none;
    integer outputs bit-exact against the oracle."""
    r = np.random.default_rng(3000 + seed)
    E = int(r.choice([1, 2, 7, 16, 64, 100, 256]))
    k = int(r.integers(1, min(8, E) + 1))
    T = int(r.choice([0, 1, 5, 100, 1000, 1023, 1025, 3000, 8192 // k, 8192 // k + 1, 20000]))
    C = int(r.choice([0, 0, 1, max(1, T * k // E), max(1, (5 * T * k) // (4 * E)), 10 ** 6]))
    reroute = bool(k < E and C > 0 and r.random() < 0.5)
    skew = float(r.choice([0.0, 2.0, 20.0]))
    _announce(f"moe_dispatch random {seed}: T={T} k={k} E={E} C={C} reroute={reroute} "
              f"skew={skew}")
    _check_dispatch(T, k, E, C, reroute, 9000 + seed, skew)


def _check_dispatch(T, k, E, C, reroute, seed, skew):
    g = torch.Generator().manual_seed(seed)
    # skewed distinct ids per token; the next choices are the backups
    pri = torch.rand((T, E), generator=g) * torch.linspace(1.0, 1.0 + skew, E)
    nb = min(k, E - k) if reroute else 0
    order = torch.topk(pri, k + nb, dim=1).indices.to(torch.int32)
    ids = order[:, :k].contiguous()
    bk = order[:, k:].contiguous() if nb else None
    if nb:
        bk[::7, -1] = -1                   # some tokens without a last backup
    X = torch.randn((T, 128), generator=g).to(torch.bfloat16)
    out = moe.dispatch(ids.to(DEV), E, C, X=X.to(DEV),
                       backup=None if bk is None else bk.to(DEV))
    torch.cuda.synchronize()
    ref = O.dispatch(ids.numpy(), E, C if C > 0 else None,
                     None if bk is None else bk.numpy())
    R = ref["n_kept"]
    assert int(out["n_kept"].item()) == R
    assert out["counts"].cpu().tolist() == ref["counts"].tolist()
    assert out["offsets"].cpu().tolist() == ref["offsets"].tolist()
    assert out["slot_row"].cpu().tolist() == ref["slot_row"].tolist()
    assert out["sorted_slot"].cpu()[:R].tolist() == ref["sorted_slot"].tolist()
    # D2: the gather is an exact copy of the chosen token rows
    tok = torch.as_tensor(ref["sorted_slot"] // k)
    assert torch.equal(out["X_sorted"][:R].cpu(), X[tok])


FFN_SHAPES = {
    # medium tiles: empty, single-row, multi-tile and ragged groups
    "medium": (256, 384, [0, 1, 300, 31, 64, 129, 7], 5),
    # large tiles, down projection with d % 256 != 0
    "large_d384": (384, 256, [300, 257, 520], 5),
    # large tiles, one empty group
    "large_d512": (512, 512, [600, 0], 5),
    # decode-sized groups (a few rows each)
    "decode": (512, 256, [2, 0, 1, 3, 2, 2, 0, 1, 4, 2, 1, 2, 3, 1, 2, 2], 0),
    # large tiles with a long reduction, fewer tiles than CUs: every down
    # tile is split along K in four parts (K / 4 = 1024)
    "large_ksplit": (768, 4096, [300, 260, 280, 290], 0),
    # three down tiles, each split along K in eight parts of 1024
    "large_split8": (256, 8192, [300, 200], 0),
    # medium tiles 256 rows tall: every count of 32-row blocks from 1 to 8
    "tall_tiles": (512, 512, [1, 33, 65, 97, 129, 161, 193, 225, 256, 250, 70], 3),
    # large tiles, nine groups (one short): 264 down tiles, more than one
    # dispatch round
    "large_tail": (2048, 256, [1024, 1000, 900, 800, 1024, 1024, 1024, 1024, 100], 0),
    # large tiles, groups just above a multiple of 256 rows: their M-tiles are
    # of equal height (1045 rows: five tiles of 224 rows, the last 149)
    "large_uneven": (512, 512, [1045, 1069, 513, 289, 257, 33], 2),
    # large tiles, groups of 1, 16, 17 and 48 rows beside full ones: the two
    # wave groups split a tile's rows in 16-row blocks, so the second group
    # has no row (1, 16), one partial block (17) or one full block (48)
    "large_small_groups": (512, 512, [1000, 1, 16, 17, 48, 513], 2),
    # medium tiles with a long reduction (bf16 on the ping-pong kernel):
    # gate/up with K = d = 4096, then the down projection with K = F = 4096
    "medium_long_d": (4096, 256, [0, 1, 150, 31, 64, 129, 7, 250], 3),
    "medium_long_f": (256, 4096, [0, 1, 150, 31, 64, 129, 7, 250], 3),
}


@pytest.mark.parametrize("dtype", ["bf16", "f32", "fp8"])
@pytest.mark.parametrize("use_row_token", [False, True])
@pytest.mark.parametrize("shape", list(FFN_SHAPES))
def test_grouped_ffn_entry_point(dtype, use_row_token, shape):
    """bf16 / fp32 layers, and bf16 activations with E4M3 weights ("fp8")."""
    _announce(f"moe_grouped_ffn {shape} {dtype} row_token={use_row_token}")
    d, F, counts, slack = FFN_SHAPES[shape]
    _check_grouped_ffn(dtype, use_row_token, d, F, counts, slack, 5)


@pytest.mark.parametrize("seed", range(24))
def test_grouped_ffn_random(seed):
    """Seeded random groups: empty, decode-sized, medium and above-256-row
    counts, so the tile plan (large, medium or decode tiles) changes across
    the draws; random d, F, dtype, row gathering and slack rows."""
    r = np.random.default_rng(2000 + seed)
    G = int(r.integers(1, 13))
    kind = r.choice(["decode", "medium", "large", "mixed"])
    lo, hi = {"decode": (0, 6), "medium": (20, 200), "large": (180, 700), "mixed": (0, 700)}[kind]
    counts = [int(c) for c in r.integers(lo, hi + 1, G)]
    if r.random() < 0.3:
        counts[int(r.integers(0, G))] = 0
    d = int(r.choice([128, 256, 384, 512, 768, 1024]))
    F = int(r.choice([128, 256, 384, 512, 1024, 4096 if kind == "decode" else 640]))
    dtype = str(r.choice(["bf16", "bf16", "f32", "fp8"]))
    use_row_token = bool(r.random() < 0.5)
    slack = int(r.choice([0, 0, 3, 64]))
    _announce(f"moe_grouped_ffn random {seed}: d={d} F={F} {dtype} row_token={use_row_token} "
              f"counts={counts} slack={slack}")
    _check_grouped_ffn(dtype, use_row_token, d, F, counts, slack, 7000 + seed)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_down_tail_split_after_full_rounds(dtype):
    """272 large down tiles (d 2048: 8 N-tiles; 8 experts of 1024 rows and
    one of 512): on 256 CUs one full dispatch round runs whole tiles and the
    last 16 (the 512-row expert's) are split along K in four parts of 1024.
    Every row of that expert and sampled rows of the others against the
    oracle, and the bits of two runs."""
    _announce(f"moe_grouped_ffn tail split after full rounds {dtype}")
    d, F = 2048, 4096
    counts = [1024] * 8 + [512]
    G = len(counts)
    g = torch.Generator().manual_seed(41)
    T = 1024
    X = torch.randn((T, d), generator=g).to(torch.bfloat16)
    Ws = [torch.randn((G, F, d), generator=g) / d ** 0.5,
          torch.randn((G, F, d), generator=g) / d ** 0.5,
          torch.randn((G, d, F), generator=g) / F ** 0.5]
    if dtype == "fp8":
        q = [quantize_e4m3_rows(w) for w in Ws]
        dev_w = [c.to(DEV) for c, _ in q]
        scales = tuple(sc.to(DEV) for _, sc in q)
        ref_w = [(c, sc) for c, sc in q]
    else:
        Ws = [w.to(torch.bfloat16) for w in Ws]
        dev_w = [w.to(DEV) for w in Ws]
        scales = None
    R = sum(counts)
    offs = torch.tensor([0] + np.cumsum(counts).tolist(), dtype=torch.int32)
    tok = torch.randint(0, T, (R,), generator=g, dtype=torch.int32)
    A = X[tok.long()].to(DEV)

    def run():
        return moe.grouped_ffn(A, offs.to(DEV), *dev_w, R, scales=scales)
    Y = run()
    torch.cuda.synchronize()
    assert torch.equal(run(), Y)
    Yh = H.np64(Y)
    Xr = X[tok.long()].double().numpy()
    for e in range(G):
        a, b = int(offs[e]), int(offs[e + 1])
        if e == G - 1:
            rows = np.arange(a, b)
        else:
            rows = np.unique(np.concatenate([[a, b - 1], np.random.default_rng(e).integers(a, b, 16)]))
        if dtype == "fp8":
            w1, w3, w2 = (O.dequantize_rows(c[e].numpy(), sc[e].numpy()) for c, sc in ref_w)
        else:
            w1, w3, w2 = (w[e].double().numpy() for w in Ws)
        ref = O.expert_ffn(Xr[rows], w1.T, w3.T, w2.T, bf16_h=True)
        H.check_rows(Yh[rows], ref, True)


def _check_grouped_ffn(dtype, use_row_token, d, F, counts, slack, seed):
    G = len(counts)
    g = torch.Generator().manual_seed(seed)
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    T = 400
    X = torch.randn((T, d), generator=g).to(tdt)
    Ws = [torch.randn((G, F, d), generator=g) / d ** 0.5,
          torch.randn((G, F, d), generator=g) / d ** 0.5,
          torch.randn((G, d, F), generator=g) / F ** 0.5]
    if dtype == "fp8":
        q = [quantize_e4m3_rows(w) for w in Ws]
        dev_w = [c.to(DEV) for c, _ in q]
        scales = tuple(sc.to(DEV) for _, sc in q)
        ref_w = [O.dequantize_rows(c.numpy(), sc.numpy()) for c, sc in q]
    else:
        Ws = [w.to(tdt) for w in Ws]
        dev_w = [w.to(DEV) for w in Ws]
        scales = None
        ref_w = [w.double().numpy() for w in Ws]
    R = sum(counts)
    offs = torch.tensor([0] + np.cumsum(counts).tolist(), dtype=torch.int32)
    tok = torch.randint(0, T, (R,), generator=g, dtype=torch.int32)
    A = X if use_row_token else X[tok.long()]
    def run():
        return moe.grouped_ffn(A.to(DEV), offs.to(DEV), *dev_w, R + slack,
                               row_token=tok.to(DEV) if use_row_token else None, scales=scales)
    Y = run()
    torch.cuda.synchronize()
    if F >= 2048 and dtype != "f32":
        # down tiles split along K are summed in part order by whichever part
        # finishes last: the bits must not depend on that order
        assert torch.equal(run()[:R], Y[:R])
    Xr = X[tok.long()].double().numpy()
    bf16 = dtype != "f32"
    for e in range(G):
        a, b = int(offs[e]), int(offs[e + 1])
        if b == a:
            continue
        ref = O.expert_ffn(Xr[a:b], ref_w[0][e].T, ref_w[1][e].T, ref_w[2][e].T, bf16_h=bf16)
        H.check_rows(H.np64(Y[a:b]), ref, bf16)


def test_forward_ksplit_paths_agree():
    """A shape whose down tiles are all split along K (fewer tiles than CUs,
    four parts each): the plain forward and the one with every optional output must give
    the same bits, and both must match the oracle."""
    w = Workload("ksplit", T=600, d=768, E=4, k=2, F=4096, seed=23)
    _announce("forward K-split")
    inp = make_inputs(w, DEV)
    layer = moe.layer_from_inputs(inp)
    Y_plain = moe.forward(layer, inp["X"]).clone()
    Y_aux, aux = _full_check(inp)
    torch.cuda.synchronize()
    assert torch.equal(Y_plain, Y_aux)


@pytest.mark.parametrize("T,k,d,keep", [(257, 3, 384, 0.5), (64, 256, 256, 0.05),
                                        (40, 64, 128, 0.3), (9, 16, 128, 0.0),
                                        # all kept: rows summed in groups of 4, then 2, then 1
                                        (33, 7, 256, 1.0), (20, 5, 128, 1.0), (16, 8, 1024, 1.0)])
def test_combine_entry_point(T, k, d, keep):
    _announce(f"moe_combine T={T} k={k} d={d}")
    g = torch.Generator().manual_seed(9)
    R = 600
    rows = torch.randn((R, d), generator=g)
    sr = torch.randint(0, R, (T * k,), generator=g, dtype=torch.int32)
    sr[torch.rand((T * k,), generator=g) >= keep] = -1
    w = torch.rand((T, k), generator=g)
    sh = torch.randn((T, d), generator=g)
    for dt in (torch.float32, torch.bfloat16):
        Y = moe.combine(rows.to(DEV), sr.to(DEV), w.to(DEV), dt, shared=sh.to(DEV))
        torch.cuda.synchronize()
        ref = O.combine(rows.double().numpy(), sr.numpy(), w.double().numpy(),
                        sh.double().numpy())
        H.check_rows(H.np64(Y), ref, dt == torch.bfloat16, f"combine {dt}",
                     output_rounding=True)
        if dt == torch.float32:
            assert H.rel_err(H.np64(Y), ref) <= 1e-6


def test_bias_update_entry_point():
    """The load rule on the capacity example's loads [5, 3, 2, 2] and on a
    random 256-expert step, against the oracle (one fp32 addition each)."""
    _announce("moe_bias_update")
    b = torch.tensor([0.5, -0.25, 0.0, 1.0], device=DEV)
    moe.bias_update(torch.tensor([5, 3, 2, 2], dtype=torch.int32, device=DEV), 6, 2, 0.001, b)
    ref = O.bias_update([0.5, -0.25, 0.0, 1.0], [5, 3, 2, 2], 6, 2, 0.001)
    assert np.allclose(H.np64(b), ref, rtol=0, atol=2 ** -23)
    assert b[1].item() == -0.25                      # load at the mean: unchanged
    g = torch.Generator().manual_seed(3)
    counts = torch.randint(0, 260, (256,), generator=g, dtype=torch.int32)
    counts[:4] = 128                                 # 4096 * 8 / 256 = 128: the mean
    b0 = torch.randn(256, generator=g) * 0.01
    b = b0.to(DEV)
    moe.bias_update(counts.to(DEV), 4096, 8, 0.001, b)
    ref = O.bias_update(b0.double().numpy(), counts.numpy(), 4096, 8, 0.001)
    assert np.abs(H.np64(b) - ref).max() <= 2 ** -24 * 0.05 + 1e-9
    assert torch.equal(b[:4].cpu(), b0[:4])


def test_balance_entry_point_page_example():
    """The balance statistic kernel on the page's example values:
    f = [.7,.1,.1,.1], P = [.4,.2,.2,.2] -> 1.36 (T = 10, top-1)."""
    _announce("moe_balance")
    counts = torch.tensor([7, 1, 1, 1], dtype=torch.int32, device=DEV)
    ps = torch.tensor([4.0, 2.0, 2.0, 2.0], device=DEV)
    out = moe.balance(counts, ps, 10, 1)
    assert abs(out.item() - 1.36) < 1e-12


# ------------------------------------------------ composition of entry points --
def test_entry_points_compose_to_forward():
    """moe_route -> moe_dispatch (with the gather) -> moe_grouped_ffn ->
    moe_combine gives moe_forward's output bit for bit (same kernels, same
    summation order), for top-k routing with a capacity limit."""
    w = SMALL["mixtral_prefill"].with_(cf=1.0)
    _announce("entry points compose (top-k)")
    inp = make_inputs(w, DEV)
    Y_fused = moe.forward(moe.layer_from_inputs(inp), inp["X"])
    r = moe.route(inp["X"], inp["Wg"], w.k, w.score, w.renorm)
    C = moe.capacity(w.cf, w.T, w.k, w.E)
    dsp = moe.dispatch(r["ids"], w.E, C, X=inp["X"])
    rows = moe.grouped_ffn(dsp["X_sorted"], dsp["offsets"], inp["W1"], inp["W3"], inp["W2"],
                           w.T * w.k)
    Y = moe.combine(rows, dsp["slot_row"], r["w"], inp["X"].dtype)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y_fused)


def test_expert_choice_entry_points_compose_to_forward():
    """moe_route_expert_choice -> moe_grouped_ffn (row -> token through
    sorted_slot / E) -> moe_combine with k = E gives moe_forward's output bit
    for bit."""
    w = SMALL["mixtral_prefill_ec"]
    _announce("entry points compose (expert choice)")
    inp = make_inputs(w, DEV)
    layer = moe.layer_from_inputs(inp)
    Y_fused = moe.forward(layer, inp["X"])
    C = layer.expert_capacity(w.T)
    r = moe.route_expert_choice(inp["X"], inp["Wg"], C, w.score)
    row_token = (r["sorted_slot"] // w.E).to(torch.int32)
    rows = moe.grouped_ffn(inp["X"], r["offsets"], inp["W1"], inp["W3"], inp["W2"], w.E * C,
                           row_token=row_token)
    Y = moe.combine(rows, r["slot_row"].reshape(-1), r["gates"], inp["X"].dtype)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y_fused)
