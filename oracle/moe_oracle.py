"""Plain CPU oracle of one Mixture-of-Experts layer's forward pass (numpy float64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or run
this module: only the test-suite, the package-level ``smoke()`` entry and the
CPU-baseline leg of the benchmark use it.  It shares no code, constants or
helpers with the HIP library; both sides only receive the same seeded inputs.

Every function follows a passage of the source pages; citations name the page
and its section:

* [Book 14.2.1]  LLM Internals, section 14.2 "Mixture-of-Experts models", 14.2.1
  "One MoE forward pass: six steps and shapes" (steps 1-6).
* [Book 14.2.2]  same page, 14.2.2 "How active parameters are counted" (one
  SwiGLU expert is three [7168, 2048] matrices).
* [Book 14.2.3]  same page, 14.2.3 "Routing and load balancing": the balance
  loss alpha*N*sum f_i p_i and its worked example; the bias-for-selection rule
  (DeepSeek-V3 report eq. 16); capacity factor and token dropping.
* [Book 14.2.4]  same page, 14.2.4 "Fine-grained MoE and shared experts".
* [KMap router]  AI Knowledge Map, "Mixture of Experts (MoE)", the four router
  steps: score W_r x, softmax, top-k hard selection, renormalise inside the
  chosen set S and combine y = sum_{e in S} g^_e E_e(x).
* [KMap capacity] same page, the capacity formula C = ceil(c*N*k/E) and its
  6-token / 4-expert / top-2 worked example, overflow handling by drop.
* [Study case 1] estelledc study note "Mixture of Experts (MoE)", practice
  case 1: the minimal top-k routing pseudo-code (router -> top-k -> softmax
  over the k kept scores -> weighted sum of the chosen experts).
* [Study pitfalls] same note, "pitfalls": the router softmax runs in fp32.
* [Blog frontier] oscine.io "MoE 03: efficiency frontiers", the section on
  the further frontier: expert-choice routing, each expert picks the C tokens
  it suits best.
* [Explainer routing] smallfiredragon.com "Mixture of Experts (MoE) in depth"
  (Chinese), the routing-mechanism list: expert-choice routing lets every
  expert pick its tokens, so the number of experts per token varies.

Readings where the pages are silent or ambiguous (each one also listed in the
design notes of the repository):

R1  SwiGLU expert: h = silu(x W1) * (x W3), y = h W2; W1 is the gate, W3 the up
    projection, silu(z) = z / (1 + exp(-z)).  The pages give only "three
    [d, F] matrices".
R2  Logical weight shapes (the pages' notation): W_g[d, E], W1/W3[E, d, F],
    W2[E, F, d].  The oracle works on these logical shapes.
R3  Top-k order: key descending, ties to the lower expert id.
R4  Softmax routers select on the logit (same set as selecting on p, free of
    exp-rounding ties); sigmoid routers select on s + b (eq. 16).
R5  Renormalisation happens over S before any capacity drop; kept gates are not
    renormalised again after a drop.
R6  Overflow priority: slot s = t*k + j; an expert keeps the first C slots in
    increasing slot order (lowest token index first).
R7  Capacity C = ceil(c*N*k/E) in exact rational arithmetic, c taken as the
    decimal number its shortest repr spells.
R8  f_e = pre-drop count_e / (T*k);  P_e = mean over tokens of the full-row
    score (softmax p, or sigmoid s); statistic = E * sum_e f_e P_e (alpha
    omitted).
R9  bf16 mode: the activation h is rounded to bf16 (round-to-nearest-even)
    before the down projection, mirroring a bf16 matrix-core input; all other
    intermediates stay exact.
R10 Shared expert: same width F, weight 1, added to every token's output.
R11 Optional per-expert logit offset o_e is added to the logits before scoring.
R12 FP8 expert weights (the format the DeepSeek-V3 weights are stored in,
    [Book 14.2.5]): OCP FP8 E4M3 codes with one fp32 scale per output channel,
    W = value(code) * scale.  The format itself is not spelled out on the
    pages; its public definition is restated in decode_e4m3.
R13 Group-limited routing (node-limited routing of [Book 14.2.3], M = 4 for
    DeepSeek-V3; on one GPU the E experts are split into n_group equal,
    contiguous groups standing in for nodes): a group's score is the sum of
    its k // topk_group highest affinities (at least 1) - the full-row softmax
    probability or the raw sigmoid s, without the bias - summed largest first;
    the topk_group best groups (ties to the lower group id) stay eligible and
    top-k then runs over their experts only.
R14 Router health ([Book 14.2.3]'s three signals plus the load CV of
    [KMap]): mean per-token routing entropy of the full-row distribution
    (sigmoid scores normalised to sum 1), entropy of the pre-drop load
    fractions, population-std CV of the per-expert counts, and the drop rate.

R20 Expert-choice routing ([Book 14.2.3] "two selection paradigms", [Blog
    frontier], [Explainer routing]): the scores are the token-choice router's
    (full-row softmax over experts, or the sigmoid affinity); expert e takes
    the min(C, T) tokens with the highest score in its column, ties to the
    lower token index, with C the capacity formula's value for the layer's
    mean experts per token k (c = 1 when no factor is given).  A token's gate
    for an expert that took it is its score, with no renormalisation (the
    number of experts per token is not fixed); a token no expert took gets
    only the shared expert.  Rows are grouped by expert, tokens ascending
    inside; slot s = t*E + e.
R21 Overflow re-route ([KMap capacity], the second/backup option: the
    overflowing requests go to other experts that still have room, so the
    token keeps its full set of paths): one backup round after the capacity
    drop.  Token t's backups are its next choices after the top-k, in the
    same key order.  The m-th dropped slot of token t (j ascending) proposes
    the token's m-th backup; experts accept proposals in slot order while
    they have room (C minus the slots kept in the first pass); a proposal
    that finds no room, or a slot without a backup, stays dropped.  A
    re-routed slot keeps its gate.  An expert's rows are its first-pass slots
    in slot order followed by its accepted proposals in slot order.
R22 Bias update (the load rule of DeepSeek-V3's auxiliary-loss-free
    balancing, [Book 14.2.3]): after a step, expert e's selection bias moves
    by -gamma when its load (pre-drop count) is above the mean T*k/E, by
    +gamma when below, and stays when equal.
(R15-R19 concern the device comparison and the inputs, not this module.)

Parity status: every function here is pinned by the CPU tests (worked examples
printed on the pages, closed forms, brute force and cross-tier agreement).  The
bf16 rounding of h (R9) is a reading, pinned only by its own RNE unit test; the
E4M3 decode (R12) is pinned by closed-form codes and by a library decoder, and
the per-output-channel scale of dequantize_rows by a round trip through the
library encoder (error within half an E4M3 ulp times the row's scale).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

__all__ = [
    "capacity", "router_logits", "scores", "select_topk", "gates", "route",
    "dispatch", "silu", "round_bf16", "expert_ffn", "combine", "forward",
    "forward_token_loop", "forward_dense_masked", "balance_value",
    "balance_stat", "expert_weight_shapes", "decode_e4m3", "dequantize_rows", "group_mask",
    "router_health", "expert_choice", "expert_choice_dispatch", "forward_expert_choice",
    "forward_expert_choice_loop", "bias_update", "backup_experts",
]


# ---------------------------------------------------------------- capacity --
def capacity(cf: float, n_tokens: int, k: int, n_experts: int) -> int:
    """C = ceil(c * N * k / E)  [KMap capacity]; GShard form [Book 14.2.3].

    c is read as the exact decimal that its shortest repr spells (reading R7),
    so 1.25 * 8192 * 2 / 64 is exactly 320 and 1.1 * 10 is exactly 11.
    """
    if not (cf > 0) or n_tokens < 0 or k < 1 or n_experts < 1:
        raise ValueError("capacity needs cf > 0, N >= 0, k >= 1, E >= 1")
    c = Fraction(repr(float(cf)))
    return math.ceil(c * n_tokens * k / n_experts)


# ----------------------------------------------------------------- routing --
def router_logits(X, Wg, offset=None):
    """Step 2 [Book 14.2.1]: s = X[T,d] x W_g[d,E]; [KMap router] step 1.

    ``offset`` (length E) is an optional per-expert additive logit term (R11).
    """
    X = np.asarray(X, dtype=np.float64)
    Wg = np.asarray(Wg, dtype=np.float64)
    lg = X @ Wg
    if offset is not None:
        lg = lg + np.asarray(offset, dtype=np.float64)[None, :]
    return lg


def scores(logits, score_func: str):
    """Per-row softmax over all E experts [KMap router] step 2, or the
    per-cell sigmoid affinity of DeepSeek-V3 [Book 14.2.1] step 2."""
    lg = np.asarray(logits, dtype=np.float64)
    if score_func == "softmax":
        m = lg.max(axis=1, keepdims=True)
        ex = np.exp(lg - m)
        return ex / ex.sum(axis=1, keepdims=True)
    if score_func == "sigmoid":
        return 1.0 / (1.0 + np.exp(-lg))
    raise ValueError(score_func)


def group_mask(logits, k: int, score_func: str, n_group: int, topk_group: int):
    """Eligible experts under group-limited routing (R13), bool [T,E]."""
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    if n_group < 1 or E % n_group or not 1 <= topk_group <= n_group:
        raise ValueError("need E % n_group == 0 and 1 <= topk_group <= n_group")
    gs = E // n_group
    gk = min(max(1, k // topk_group), gs)
    aff = scores(lg, score_func)
    ok = np.zeros((T, E), dtype=bool)
    for t in range(T):
        gscore = np.empty(n_group)
        for g in range(n_group):
            top = np.sort(aff[t, g * gs:(g + 1) * gs])[::-1][:gk]
            acc = 0.0
            for v in top:                 # largest first
                acc += v
            gscore[g] = acc
        for g in np.argsort(-gscore, kind="stable")[:topk_group]:
            ok[t, g * gs:(g + 1) * gs] = True
    return ok


def select_topk(logits, k: int, score_func: str, bias=None, n_group: int = 1,
                topk_group: int = 1):
    """Top-k hard selection [Book 14.2.1] step 3, [KMap router] step 3.

    Key: the logit for a softmax router (R4); s + b for a sigmoid router with a
    selection-only bias (eq. 16, [Book 14.2.3]).  With n_group > 1 only the
    experts of the chosen groups are eligible (R13).  Returns ids [T,k] ordered
    by key descending, ties to the lower id (R3), and the keys themselves.
    """
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    if score_func == "softmax":
        key = lg.copy()
    else:
        key = scores(lg, "sigmoid")
        if bias is not None:
            key = key + np.asarray(bias, dtype=np.float64)[None, :]
    if n_group > 1:
        if k > topk_group * (E // n_group):
            raise ValueError("the chosen groups hold fewer than k experts")
        key = np.where(group_mask(lg, k, score_func, n_group, topk_group), key, -np.inf)
    ids = np.empty((T, k), dtype=np.int64)
    for t in range(T):
        # a stable sort of -key keeps equal keys in ascending id order
        order = np.argsort(-key[t], kind="stable")
        ids[t] = order[:k]
    return ids, key


def gates(logits, ids, score_func: str, renorm: bool):
    """Gate weights of the chosen experts.

    renorm: g^_e = g_e / sum_{e' in S} g_e' ([KMap router] step 4, eqs. 13-14 in
    [Book 14.2.1] step 3); for a sigmoid router g is the raw affinity s, never
    s + b (eq. 16, [Book 14.2.3]).  Without renorm the raw score is the gate.
    """
    p = scores(logits, score_func)
    g = np.take_along_axis(p, np.asarray(ids), axis=1)
    if renorm:
        g = g / g.sum(axis=1, keepdims=True)
    return g


def route(logits, k, score_func, renorm, bias=None, n_group=1, topk_group=1):
    """Steps 2-3 on given logits: ids [T,k], gates [T,k], full scores [T,E]."""
    ids, _ = select_topk(logits, k, score_func, bias, n_group, topk_group)
    g = gates(logits, ids, score_func, renorm)
    return ids, g, scores(logits, score_func)


# ---------------------------------------------------------------- dispatch --
def dispatch(ids, n_experts: int, cap=None, backups=None):
    """Step 4 [Book 14.2.1] with the capacity drop of [KMap capacity].

    Slot s = t*k + j.  Its rank is the number of earlier slots that chose the
    same expert (R6); it is kept iff rank < C.  With ``backups`` [T, B] (the
    tokens' next choices after their top-k, -1 for none) the dropped slots
    get one backup round (R21).  Returns a dict with
      counts[E]      pre-drop requests per expert (top-k choices)
      kept[E]        rows per expert (min(counts, C), plus accepted backups)
      offsets[E+1]   exclusive scan of kept
      sorted_slot[R] kept slots grouped by expert, first-pass slots then
                     re-routed ones, increasing slot order inside each part
      slot_row[T*k]  row of slot s in the sorted buffer, -1 if dropped
      expert[T*k]    expert that computes slot s, -1 if dropped
      n_kept         R
      n_rerouted     slots placed by the backup round
    Written as plain first-come loops over slots.
    """
    ids = np.asarray(ids, dtype=np.int64)
    flat = ids.reshape(-1)
    k = ids.shape[1] if ids.ndim == 2 else 1
    E = int(n_experts)
    counts = [0] * E
    rank = [0] * flat.size
    for s, e in enumerate(flat.tolist()):
        if not 0 <= e < E:
            raise ValueError("expert id out of range")
        rank[s] = counts[e]
        counts[e] += 1
    C = None if cap is None or cap <= 0 else int(cap)
    members = [[] for _ in range(E)]          # slots of each expert, in row order
    expert = [-1] * flat.size
    for s, e in enumerate(flat.tolist()):
        if C is None or rank[s] < C:
            members[e].append(s)
            expert[s] = e
    n_rerouted = 0
    if backups is not None and C is not None:
        bk = (np.asarray(backups, dtype=np.int64).reshape(flat.size // k, -1).tolist()
              if flat.size else [])
        room = [C - len(members[e]) for e in range(E)]
        for t in range(flat.size // k):
            m = 0                                  # dropped slots of token t so far
            for j in range(k):
                s = t * k + j
                if expert[s] >= 0:
                    continue
                m += 1
                if m > len(bk[t]) or bk[t][m - 1] < 0:
                    continue
                e = bk[t][m - 1]
                if room[e] > 0:                    # accepted in slot order
                    room[e] -= 1
                    members[e].append(s)
                    expert[s] = e
                    n_rerouted += 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + len(members[e]))
    sorted_slot = [s for e in range(E) for s in members[e]]
    slot_row = [-1] * flat.size
    for row, s in enumerate(sorted_slot):
        slot_row[s] = row
    return {
        "counts": np.array(counts, dtype=np.int64),
        "kept": np.array([len(m) for m in members], dtype=np.int64),
        "offsets": np.array(offsets, dtype=np.int64),
        "sorted_slot": np.array(sorted_slot, dtype=np.int64),
        "slot_row": np.array(slot_row, dtype=np.int64),
        "expert": np.array(expert, dtype=np.int64),
        "n_kept": int(len(sorted_slot)),
        "n_rerouted": n_rerouted,
    }


def backup_experts(logits, k: int, score_func: str, bias=None, n_group: int = 1,
                   topk_group: int = 1):
    """Each token's next B = min(k, E - k) choices after its top-k, in the
    selection's own key order (R21); -1 where the key is -inf (an expert
    outside the chosen groups)."""
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    B = min(k, E - k)
    _, key = select_topk(lg, k, score_func, bias, n_group, topk_group)
    bk = np.full((T, B), -1, dtype=np.int64)
    for t in range(T):
        order = np.argsort(-key[t], kind="stable")      # the top-k's own order
        for m, e in enumerate(order[k:k + B].tolist()):
            if key[t, e] > -np.inf:
                bk[t, m] = e
    return bk


# ------------------------------------------------------------- expert FFN --
def silu(z):
    """silu(z) = z * sigmoid(z) (R1)."""
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 (8 significant bits),
    ties to even (R9).  Written from the format definition: keep 8 bits of
    significand, round-half-even via np.rint."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)              # x = m * 2**e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def decode_e4m3(codes):
    """Values of FP8 E4M3 codes (R12): bit 7 sign, bits 6-3 exponent with bias
    7, bits 2-0 mantissa.  Exponent field 0 is subnormal, (m/8) * 2^-6; fields
    1..15 are normal, (1 + m/8) * 2^(e-7), except S.1111.111, which is NaN.
    There are no infinities; the largest finite magnitude is 448."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def dequantize_rows(codes, scale):
    """W[..., n, :] = value(codes[..., n, :]) * scale[..., n] (R12): one scale
    per output channel, i.e. per row of the reduction-contiguous storage."""
    return decode_e4m3(codes) * np.asarray(scale, dtype=np.float64)[..., None]


def expert_weight_shapes(d: int, F: int):
    """Shapes of one SwiGLU expert's three matrices [Book 14.2.2] (R1, R2)."""
    return {"W1": (d, F), "W3": (d, F), "W2": (F, d)}


def expert_ffn(x, W1, W3, W2, bf16_h: bool = False):
    """One SwiGLU expert on rows x[m,d]: (silu(x W1) * (x W3)) W2  (R1, R9).

    Step 5 of [Book 14.2.1]: [m_i, d] x W_i[d, F] -> [m_i, F], projected back to d.
    """
    x = np.asarray(x, dtype=np.float64)
    h = silu(x @ np.asarray(W1, np.float64)) * (x @ np.asarray(W3, np.float64))
    if bf16_h:
        h = round_bf16(h)
    return h @ np.asarray(W2, np.float64)


# ----------------------------------------------------------------- forward --
def forward(X, Wg, W1, W3, W2, *, k, score_func="softmax", renorm=True,
            bias=None, offset=None, cap=None, shared=None, bf16_h=False,
            logits=None, n_group=1, topk_group=1, reroute=False):
    """Tier 1: the six steps of [Book 14.2.1] with per-expert matmuls.

    X[T,d]; Wg[d,E]; W1,W3[E,d,F]; W2[E,F,d]; shared = (W1s[d,F], W3s[d,F],
    W2s[F,d]) or None.  ``logits`` (e.g. the device's fp32 logits) replaces
    the oracle's own scoring for the routing decision when given.
    Returns a dict with every intermediate.
    """
    X = np.asarray(X, dtype=np.float64)
    T, d = X.shape
    E = np.asarray(Wg).shape[1]
    own = router_logits(X, Wg, offset)
    lg = own if logits is None else np.asarray(logits, dtype=np.float64)
    ids, g, p = route(lg, k, score_func, renorm, bias, n_group, topk_group)
    bk = backup_experts(lg, k, score_func, bias, n_group, topk_group) if reroute else None
    disp = dispatch(ids, E, cap, bk)
    rows = np.zeros((disp["n_kept"], d))
    for e in range(E):
        a, b = disp["offsets"][e], disp["offsets"][e + 1]
        if b > a:
            tok = disp["sorted_slot"][a:b] // k
            rows[a:b] = expert_ffn(X[tok], W1[e], W3[e], W2[e], bf16_h)
    sh = None
    if shared is not None:
        sh = expert_ffn(X, shared[0], shared[1], shared[2], bf16_h)
    Y = combine(rows, disp["slot_row"], g, sh)
    return {"logits": own, "route_logits": lg, "ids": ids, "gates": g, "backups": bk,
            "probs": p, "dispatch": disp, "rows": rows, "shared": sh, "Y": Y}


def combine(rows, slot_row, gates, shared_rows=None):
    """Step 6 [Book 14.2.1]: Y[t] = sum_j g[t,j] * rows[slot_row[t*k+j]] over
    kept slots (dropped slots, row -1, add nothing: [KMap capacity]), plus the
    shared expert's output with weight 1 (R10)."""
    g = np.asarray(gates, dtype=np.float64)
    T, k = g.shape
    rows = np.asarray(rows, dtype=np.float64)
    sr = np.asarray(slot_row).reshape(T, k)
    d = rows.shape[1] if rows.ndim == 2 else 0
    if shared_rows is not None:
        d = np.asarray(shared_rows).shape[1]
    Y = np.zeros((T, d))
    for j in range(k):
        r = sr[:, j]
        ok = r >= 0
        Y[ok] += g[ok, j][:, None] * rows[r[ok]]
    if shared_rows is not None:
        Y = Y + np.asarray(shared_rows, dtype=np.float64)
    return Y


def forward_token_loop(X, Wg, W1, W3, W2, *, k, score_func="softmax",
                       renorm=True, bias=None, offset=None, cap=None,
                       shared=None, bf16_h=False):
    """Tier 0: a literal per-token loop in plain Python arithmetic.

    Follows [Study case 1] (score -> keep top-k -> weights -> accumulate
    w * expert(token)) with the renormalisation of [KMap router] step 4, the
    sigmoid + bias rule of eq. 16, and capacity handled first-come per expert
    as the tokens arrive (R6).  Only for tiny shapes.
    """
    X = np.asarray(X, dtype=np.float64)
    Wg = np.asarray(Wg, dtype=np.float64)
    T, d = X.shape
    E = Wg.shape[1]
    F = np.asarray(W1).shape[2]
    C = None if cap is None or cap <= 0 else int(cap)
    load = [0] * E

    def run_expert(x, w1, w3, w2):
        h = []
        for f in range(F):
            a = sum(x[i] * w1[i][f] for i in range(d))
            u = sum(x[i] * w3[i][f] for i in range(d))
            hv = a / (1.0 + math.exp(-a)) * u
            if bf16_h:
                hv = float(round_bf16(hv))
            h.append(hv)
        return [sum(h[f] * w2[f][j] for f in range(F)) for j in range(d)]

    w1l, w3l, w2l = (np.asarray(W, np.float64).tolist() for W in (W1, W3, W2))
    Y = []
    for t in range(T):
        x = X[t].tolist()
        sc = [sum(x[i] * Wg[i][e] for i in range(d)) for e in range(E)]
        if offset is not None:
            sc = [sc[e] + float(offset[e]) for e in range(E)]
        if score_func == "softmax":
            mx = max(sc)
            ex = [math.exp(v - mx) for v in sc]
            z = sum(ex)
            prob = [v / z for v in ex]
            key = sc
        else:
            prob = [1.0 / (1.0 + math.exp(-v)) for v in sc]
            key = [prob[e] + (0.0 if bias is None else float(bias[e]))
                   for e in range(E)]
        chosen = sorted(range(E), key=lambda e: (-key[e], e))[:k]
        w = [prob[e] for e in chosen]
        if renorm:
            tot = sum(w)
            w = [v / tot for v in w]
        out = [0.0] * d
        for wi, e in zip(w, chosen):
            if C is not None and load[e] >= C:
                load[e] += 1
                continue                       # overflow: this path is dropped
            load[e] += 1
            y = run_expert(x, w1l[e], w3l[e], w2l[e])
            out = [o + wi * v for o, v in zip(out, y)]
        if shared is not None:
            s1, s3, s2 = (np.asarray(W, np.float64).tolist() for W in shared)
            y = run_expert(x, s1, s3, s2)
            out = [o + v for o, v in zip(out, y)]
        Y.append(out)
    return np.array(Y, dtype=np.float64)


def forward_dense_masked(X, Wg, W1, W3, W2, *, k, score_func="softmax",
                         renorm=True, bias=None, offset=None, cap=None,
                         shared=None, bf16_h=False):
    """Tier B: run every expert on every token, then keep only the top-k (and
    capacity-kept) contributions: y = sum_{i in TopK} g_i Expert_i(x)
    ([Book 14.2.1] opening formula) evaluated densely."""
    X = np.asarray(X, dtype=np.float64)
    T, d = X.shape
    E = np.asarray(Wg).shape[1]
    lg = router_logits(X, Wg, offset)
    ids, g, _ = route(lg, k, score_func, renorm, bias)
    allout = np.stack([expert_ffn(X, W1[e], W3[e], W2[e], bf16_h)
                       for e in range(E)])                 # [E, T, d]
    keep = np.ones((T, k), dtype=bool)
    if cap is not None and cap > 0:
        seen = np.zeros(E, dtype=np.int64)
        for t in range(T):
            for j in range(k):
                e = ids[t, j]
                keep[t, j] = seen[e] < cap
                seen[e] += 1
    mask = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            if keep[t, j]:
                mask[t, ids[t, j]] = g[t, j]
    Y = np.einsum("te,etd->td", mask, allout)
    if shared is not None:
        Y = Y + expert_ffn(X, shared[0], shared[1], shared[2], bf16_h)
    return Y


# ----------------------------------------------------------- expert choice --
def expert_choice(logits, score_func: str, C: int):
    """Expert-choice selection (R20): each expert takes a fixed number of
    tokens from the batch [Book 14.2.3], the C it scores highest [Blog
    frontier].

    The score matrix is the token-choice router's (softmax across the E
    experts of each token, or the sigmoid affinity).  Column e is ranked by
    score, highest first, ties to the lower token index; the first min(C, T)
    tokens are taken.  Returns (mask [T,E] bool, gates [T,E] = score where
    taken, else 0, scores [T,E]).
    """
    p = scores(logits, score_func)
    T, E = p.shape
    if C < 0:
        raise ValueError("C must be >= 0")
    take = min(int(C), T)
    mask = np.zeros((T, E), dtype=bool)
    for e in range(E):
        # a stable sort of -score keeps equal scores in ascending token order
        order = np.argsort(-p[:, e], kind="stable")
        mask[order[:take], e] = True
    return mask, np.where(mask, p, 0.0), p


def expert_choice_dispatch(mask):
    """Row layout of an expert-choice assignment (R20): slot s = t*E + e;
    the taken slots grouped by expert, ascending token index inside (the
    same grouping as ``dispatch``).  Returns counts[E] (tokens per expert),
    offsets[E+1], sorted_slot[R], slot_row[T*E] (-1 where not taken), n_kept.
    """
    mask = np.asarray(mask, dtype=bool)
    T, E = mask.shape
    offsets = [0]
    sorted_slot = []
    slot_row = np.full(T * E, -1, dtype=np.int64)
    for e in range(E):
        for t in np.flatnonzero(mask[:, e]).tolist():
            slot_row[t * E + e] = len(sorted_slot)
            sorted_slot.append(t * E + e)
        offsets.append(len(sorted_slot))
    counts = np.diff(np.array(offsets, dtype=np.int64))
    return {"counts": counts, "kept": counts.copy(),
            "offsets": np.array(offsets, dtype=np.int64),
            "sorted_slot": np.array(sorted_slot, dtype=np.int64),
            "slot_row": slot_row, "n_kept": len(sorted_slot)}


def forward_expert_choice(X, Wg, W1, W3, W2, *, C, score_func="softmax", offset=None,
                          shared=None, bf16_h=False, logits=None, mask=None):
    """Tier 1 of an expert-choice layer (R20): score, let every expert take
    its C tokens, run each expert on its rows, then combine with the scores
    as gates plus the shared expert (R10).  ``logits`` replaces the oracle's
    own scoring and ``mask`` the selection (e.g. the device's, once checked).
    """
    X = np.asarray(X, dtype=np.float64)
    T, d = X.shape
    E = np.asarray(Wg).shape[1]
    own = router_logits(X, Wg, offset)
    lg = own if logits is None else np.asarray(logits, dtype=np.float64)
    m, g, p = expert_choice(lg, score_func, C)
    if mask is not None:
        m = np.asarray(mask, dtype=bool)
        g = np.where(m, p, 0.0)
    disp = expert_choice_dispatch(m)
    rows = np.zeros((disp["n_kept"], d))
    for e in range(E):
        a, b = disp["offsets"][e], disp["offsets"][e + 1]
        if b > a:
            tok = disp["sorted_slot"][a:b] // E
            rows[a:b] = expert_ffn(X[tok], W1[e], W3[e], W2[e], bf16_h)
    sh = None
    if shared is not None:
        sh = expert_ffn(X, shared[0], shared[1], shared[2], bf16_h)
    Y = combine(rows, disp["slot_row"], g, sh)
    return {"logits": own, "route_logits": lg, "mask": m, "gates": g, "probs": p,
            "dispatch": disp, "rows": rows, "shared": sh, "Y": Y}


def forward_expert_choice_loop(X, Wg, W1, W3, W2, *, C, score_func="softmax",
                               offset=None, shared=None):
    """Tier 0 of an expert-choice layer: plain Python loops over experts and
    tokens (R20).  Only for tiny shapes."""
    X = np.asarray(X, dtype=np.float64).tolist()
    Wg = np.asarray(Wg, dtype=np.float64).tolist()
    T, d, E = len(X), len(X[0]), len(Wg[0])
    prob = []
    for t in range(T):
        sc = [sum(X[t][i] * Wg[i][e] for i in range(d)) for e in range(E)]
        if offset is not None:
            sc = [sc[e] + float(offset[e]) for e in range(E)]
        if score_func == "softmax":
            mx = max(sc)
            ex = [math.exp(v - mx) for v in sc]
            prob.append([v / sum(ex) for v in ex])
        else:
            prob.append([1.0 / (1.0 + math.exp(-v)) for v in sc])

    def swiglu(x, w1, w3, w2):
        F = len(w1[0])
        h = []
        for f in range(F):
            a = sum(x[i] * w1[i][f] for i in range(d))
            u = sum(x[i] * w3[i][f] for i in range(d))
            h.append(a / (1.0 + math.exp(-a)) * u)
        return [sum(h[f] * w2[f][j] for f in range(F)) for j in range(d)]

    Y = [[0.0] * d for _ in range(T)]
    for e in range(E):
        ranked = sorted(range(T), key=lambda t: (-prob[t][e], t))
        w1, w3, w2 = (np.asarray(W[e], np.float64).tolist() for W in (W1, W3, W2))
        for t in ranked[:min(C, T)]:
            y = swiglu(X[t], w1, w3, w2)
            Y[t] = [a + prob[t][e] * b for a, b in zip(Y[t], y)]
    if shared is not None:
        s1, s3, s2 = (np.asarray(W, np.float64).tolist() for W in shared)
        for t in range(T):
            Y[t] = [a + b for a, b in zip(Y[t], swiglu(X[t], s1, s3, s2))]
    return np.array(Y, dtype=np.float64)


# ----------------------------------------------------------- router health --
def router_health(logits, score_func: str, counts, n_kept: int, n_tokens: int, k: int):
    """The three router signals [Book 14.2.3] names - routing entropy, the
    per-expert token distribution, the token drop rate - and the expert-load
    CV of [KMap] (std / mean of the per-expert loads), as four numbers (R14):

      token_entropy  mean over tokens of -sum_e q ln q, q the full-row softmax
                     p, or s / sum(s) for a sigmoid router (nats)
      load_entropy   -sum_e f ln f of f_e = counts_e / (T*k), pre-drop (nats)
      load_cv        population std of counts_e over their mean T*k / E
      drop_rate      1 - R / (T*k)
    """
    q = scores(logits, score_func)
    if score_func == "sigmoid":
        q = q / q.sum(axis=1, keepdims=True)
    with np.errstate(divide="ignore", invalid="ignore"):
        h = -np.where(q > 0, q * np.log(q), 0.0).sum(axis=1)
    c = np.asarray(counts, dtype=np.float64)
    tk = float(n_tokens * k)
    f = c / tk if tk > 0 else np.zeros_like(c)
    with np.errstate(divide="ignore", invalid="ignore"):
        h_load = float(-np.where(f > 0, f * np.log(f), 0.0).sum())
    mean = tk / c.size
    cv = float(np.sqrt(np.mean((c - mean) ** 2)) / mean) if mean > 0 else 0.0
    return {"token_entropy": float(h.mean()) if n_tokens else 0.0, "load_entropy": h_load,
            "load_cv": cv, "drop_rate": 1.0 - n_kept / tk if tk > 0 else 0.0}


# ------------------------------------------------------------ bias update --
def bias_update(bias, counts, n_tokens: int, k: int, gamma: float):
    """One step of the selection-bias rule [Book 14.2.3] (R22): overloaded
    experts (count above the mean load T*k/E) lose gamma, underloaded ones
    gain gamma.  The comparison count > T*k/E is made as count*E > T*k in
    integers, so a load equal to the mean is recognised exactly."""
    b = np.asarray(bias, dtype=np.float64).copy()
    c = [int(v) for v in np.asarray(counts).tolist()]
    E = len(c)
    tk = int(n_tokens) * int(k)
    for e in range(E):
        if c[e] * E > tk:
            b[e] -= gamma
        elif c[e] * E < tk:
            b[e] += gamma
    return b


# ----------------------------------------------------------------- balance --
def balance_value(f, p):
    """N * sum_i f_i p_i, the balance loss of [Book 14.2.3] without alpha."""
    f = np.asarray(f, dtype=np.float64)
    p = np.asarray(p, dtype=np.float64)
    return float(f.size * np.sum(f * p))


def balance_stat(counts, prob_sum, n_tokens: int, k: int):
    """f_e = counts_e / (T*k) (pre-drop top-k counts), P_e = prob_sum_e / T
    (R8); returns E * sum f_e P_e  [Book 14.2.3]."""
    counts = np.asarray(counts, dtype=np.float64)
    f = counts / float(n_tokens * k)
    P = np.asarray(prob_sum, dtype=np.float64) / float(n_tokens)
    return balance_value(f, P)
