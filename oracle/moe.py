"""Float64 CPU oracle for the forward pass of a top-k routed MoE FFN layer.

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
baseline may import this module. The GPU library never calls it and shares no
code with it; the only thing both sides share is the seeded input generator.

Everything here is the plain definition of each stage, in float64, written
from the pages (cited by page title and section):

* [CME295] "Week 2 Day 2: Mixture of Experts" course notes (semidirectx.com),
  §1.3 formalism, §3.2 balance loss, §3.3 capacity, §3.4 z-loss, §4.2
  selection bias, §A.2 implementation pitfalls.
* [FANDEX] "Mixture-of-Experts models" (fanquanpp.github.io), "Step 1: the
  router" code.
* [CS336] "Stanford CS336 Lecture 04: MoE architecture" (devpress.csdn.net),
  §2.1.2 top-K routing, §2.3.3 balancing loss.
* [15-779] "Lecture 21: Mixture-of-Experts" notes for CMU 15-779
  (semidirectx.com), §2.1 gating, §2.5 top-1 pitfall, §3.2 four steps,
  §3.3 permutation by prefix sum, §3.5 capacity, §10 exercises.
* [W11] "W11: MoE routing and parallel cost" (botof.cn), §2 toy MoE, §3
  capacity factor, §5 balance metrics.

Readings where the pages are silent or disagree:
* SwiGLU expert: f(x) = W2 (silu(W1 x) * (W3 x)), silu(u) = u / (1 + e^-u),
  no biases ([CME295] §2.1 counts 3·d·d_ff weights, no bias).
* The selection bias is added to the logits z ([CME295] §4.2, [FANDEX]
  step 1), not to the softmax probabilities ([CS336] §2.3.3 c).
* Ties in top-k go to the lower expert index (a stable descending sort, as in
  [FANDEX] step 1; [CME295] §A.2 warns that an unstable top-k is not
  reproducible).
* Capacity C = ceil(cf·T·k/E) ([15-779] §3.5, [W11] §3); within one expert all
  first choices are served before any second choice, tokens in order (the
  GShard rule described in [15-779] §3.5). A dropped assignment contributes 0
  and the surviving gates are not renormalised ([CME295] §3.3: the token only
  takes the residual path).
* f_i counts the router's choices before any drop, all k of them
  ([CME295] §3.2 and §A.2).
"""
from __future__ import annotations

import math
from typing import Callable, Optional, Sequence, Tuple

import numpy as np

GATE_SELECTED = "selected"
GATE_ALL = "all"
NEAR_TIE = 1e-3


# ------------------------------------------------------------------ routing

def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """z = W_r^T x for every token ([CME295] §1.3; [15-779] §2.1).

    ``w_router`` is stored [E, d]: row e is expert e's score vector ([FANDEX]
    step 1 writes one d-vector ``W_router[e]`` per expert), i.e. the columns of
    the pages' W_r in R^{d x E}.  Returns z[T, E].
    """
    return np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T


def select_topk(s: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray]:
    """Greedy top-k of each row of s, highest first, ties to the lower index
    ([CME295] §1.3 TopK; [FANDEX] step 1's stable ``sorted``).

    Returns (idx[T, k] int64 in rank order, margin[T]) where the margin is the
    k-th minus the (k+1)-th largest score (inf when k == E): tokens with a small
    margin have a selection that rounding can flip.
    """
    s = np.asarray(s, np.float64)
    T, E = s.shape
    order = np.argsort(-s, axis=1, kind="stable")
    idx = order[:, :k]
    if k < E:
        kth = np.take_along_axis(s, order[:, k - 1:k], 1)[:, 0]
        nxt = np.take_along_axis(s, order[:, k:k + 1], 1)[:, 0]
        margin = kth - nxt
    else:
        margin = np.full(T, np.inf)
    return idx, margin


def softmax(z: np.ndarray) -> np.ndarray:
    """Row softmax p = e^z / sum e^z, shifted by the row max."""
    z = np.asarray(z, np.float64)
    m = z.max(axis=1, keepdims=True)
    e = np.exp(z - m)
    return e / e.sum(axis=1, keepdims=True)


def gates_selected(z: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """g_i = e^{z_i} / sum_{j in T} e^{z_j} over the selected set
    ([CME295] §1.3; [FANDEX] step 1 shifts by the max of the chosen raw scores)."""
    zs = np.take_along_axis(np.asarray(z, np.float64), idx, 1)
    e = np.exp(zs - zs.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def gates_all(z: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """g_i = softmax(z)_i of the chosen experts, not renormalised
    (Switch top-1, [CME295] §1.3 and [15-779] §2.5; [CS336] §2.1.2)."""
    return np.take_along_axis(softmax(z), idx, 1)


def route(x, w_router, k: int, gate: str = GATE_SELECTED, bias=None):
    """Router scores, selection on z + b, gates on the unbiased z
    ([CME295] §4.2: the bias only changes which experts are chosen).

    Returns dict(z, s, idx, margin, gates, probs); s = z + b is the score the
    selection ranks."""
    z = router_logits(x, w_router)
    s = z if bias is None else z + np.asarray(bias, np.float64)[None, :]
    idx, margin = select_topk(s, k)
    g = gates_selected(z, idx) if gate == GATE_SELECTED else gates_all(z, idx)
    return dict(z=z, s=s, idx=idx, margin=margin, gates=g, probs=softmax(z))


# ------------------------------------------------------------------ stats

def load_fractions(idx: np.ndarray, E: int) -> np.ndarray:
    """f_i = (1/T) #{(t, j): token t chose i}, all k choices counted
    ([CME295] §3.2 and §A.2)."""
    T = idx.shape[0]
    return np.bincount(np.asarray(idx).ravel(), minlength=E).astype(np.float64) / T


def mean_probs(probs: np.ndarray) -> np.ndarray:
    """P_i = (1/T) sum_t p_{t,i} ([CME295] §3.2)."""
    return np.asarray(probs, np.float64).mean(axis=0)


def aux_loss(f: np.ndarray, P: np.ndarray, alpha: float) -> float:
    """L_aux = alpha · E · sum_i f_i P_i ([CME295] §3.2; [CS336] §2.3.3 a;
    [15-779] §2.4)."""
    f = np.asarray(f, np.float64)
    return float(alpha * f.shape[0] * np.dot(f, np.asarray(P, np.float64)))


def logsumexp_rows(z: np.ndarray) -> np.ndarray:
    """log sum_i e^{z_{t,i}} per token, with the row maximum factored out."""
    z = np.asarray(z, np.float64)
    m = z.max(axis=1)
    return m + np.log(np.exp(z - m[:, None]).sum(axis=1))


def z_loss(z: np.ndarray) -> float:
    """Router z-loss L_z = (1/T) sum_t (log sum_i e^{z_{t,i}})^2 on the
    unbiased logits ([CME295] §3.4, the ST-MoE penalty on the logits' scale)."""
    return float(np.mean(logsumexp_rows(z) ** 2))


def router_entropy(z: np.ndarray) -> float:
    """Mean over tokens of the Shannon entropy (natural log) of the full
    softmax p_t = softmax(z_t). [W11] §5 lists router entropy as a quantity to
    monitor without a formula; this is its plainest reading."""
    p = softmax(z)
    with np.errstate(divide="ignore", invalid="ignore"):
        h = -np.where(p > 0, p * np.log(p), 0.0).sum(axis=1)
    return float(np.mean(h))


def mean_max_prob(z: np.ndarray) -> float:
    """Mean over tokens of max_i p_{t,i} ([CME295] §3.4 reports it beside the
    z-loss)."""
    return float(np.mean(softmax(z).max(axis=1)))


def top_gap(z: np.ndarray) -> float:
    """Mean over tokens of p_{t,(1)} - p_{t,(2)}, the two largest entries of the
    full softmax of the unbiased logits (p_{(2)} = 0 when E = 1). [W11] §5 lists
    the top-1/top-2 gap without a formula; this is its plainest reading."""
    p = np.sort(softmax(z), axis=1)[:, ::-1]
    second = p[:, 1] if p.shape[1] > 1 else np.zeros(p.shape[0])
    return float(np.mean(p[:, 0] - second))


def bias_update(bias: np.ndarray, counts: np.ndarray, T: int, k: int, gamma: float) -> np.ndarray:
    """Auxiliary-loss-free balancing step ([CME295] §4.2; [15-779] §2.4): after a
    step, every expert loaded above the mean T·k/E has its selection bias lowered
    by gamma, every expert below it raised by gamma, one exactly at the mean
    left alone. The bias only enters the top-k selection, never the gates."""
    b = np.asarray(bias, np.float64)
    c = np.asarray(counts, np.int64)
    E = b.shape[0]
    # c_e > T k / E compared as integers: c_e·E vs T·k
    direction = np.sign(c * E - T * k).astype(np.float64)
    return b - gamma * direction


def coverage_fraction(k: int, E: int, B: int) -> float:
    """Expected fraction of experts chosen by at least one of B tokens that
    each pick a uniformly random k-subset: 1 - (1 - k/E)^B ([CME295] §2.3;
    [15-779] §3.1)."""
    return 1.0 - (1.0 - k / E) ** B


def touched_experts(idx: np.ndarray, E: int) -> int:
    """Number of distinct experts chosen by a batch."""
    return int(np.count_nonzero(np.bincount(np.asarray(idx).ravel(), minlength=E)))


def max_over_mean_load(counts: np.ndarray, T: int, k: int) -> float:
    """The busiest expert's load over the mean load T·k/E ([CME295] §3.3 and
    §4.2; [15-779] §3.4); counts[e] are expert e's assignments before drops."""
    counts = np.asarray(counts)
    return float(np.max(counts)) / (T * k / counts.size)


# ------------------------------------------------------------------ permutation

def capacity(cf: float, T: int, k: int, E: int) -> Optional[int]:
    """C = ceil(k·T/E · cf) ([15-779] §3.5; [W11] §3); None when cf <= 0."""
    if cf is None or cf <= 0:
        return None
    return int(math.ceil(k * T / E * cf))


def assign_rows(idx: np.ndarray, E: int, cf: float = 0.0):
    """Histogram, capacity and permutation of the (token, slot) assignments.

    Without capacity every assignment gets a row: rows are grouped by expert
    (expert-major) and ordered by token inside a group, which is the row that
    the prefix sum over the transposed 0/1 selection mask gives
    ([15-779] §3.3, worked examples there and in §10 exercise 2). The group
    boundaries are the CSR indptr ("offsets", length E+1).

    With capacity C, assignment (t, j) to expert e has priority position
    (#first..(j-1)-th choices of e over all tokens) + (#tokens t' < t whose j-th
    choice is e); it is kept iff that position < C ([15-779] §3.5 GShard rule).
    Kept assignments are then laid out as above; dropped ones get dest = -1.

    Returns dict(counts[E], kept[E], offsets[E+1], dest[T,k], src[R], n_dropped, C).
    """
    idx = np.asarray(idx, np.int64)
    T, k = idx.shape
    counts = np.bincount(idx.ravel(), minlength=E)
    C = capacity(cf, T, k, E)
    keep = np.ones((T, k), bool)
    if C is not None:
        used = np.zeros(E, np.int64)        # positions handed out so far per expert
        for j in range(k):                   # all j-th choices before any (j+1)-th
            for t in range(T):
                e = idx[t, j]
                keep[t, j] = used[e] < C
                used[e] += 1
    kept = np.zeros(E, np.int64)
    for t in range(T):
        for j in range(k):
            if keep[t, j]:
                kept[idx[t, j]] += 1
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(kept)
    dest = np.full((T, k), -1, np.int64)
    src = np.zeros(int(offsets[E]), np.int64)
    nxt = offsets[:E].copy()
    for t in range(T):                       # token order inside each expert's group
        for j in range(k):
            if keep[t, j]:
                e = idx[t, j]
                dest[t, j] = nxt[e]
                src[nxt[e]] = t
                nxt[e] += 1
    return dict(counts=counts, kept=kept, offsets=offsets, dest=dest, src=src,
                n_dropped=int(T * k - offsets[E]), C=C)


def permutation_by_prefix_sum(idx: np.ndarray, E: int):
    """The prefix-sum formulation of [15-779] §3.3, kept separate from
    ``assign_rows`` so the two can be checked against each other: flatten the
    transposed (T x E) 0/1 mask expert-major, take the inclusive cumulative sum,
    read it back at the mask's ones and subtract 1; indptr is 0 followed by the
    running total at the end of each expert's column."""
    idx = np.asarray(idx, np.int64)
    T, k = idx.shape
    mask = np.zeros((T, E), np.int64)
    for t in range(T):
        mask[t, idx[t]] = 1
    cs = np.cumsum(mask.T.reshape(-1)).reshape(E, T).T     # [T, E]
    dest = np.take_along_axis(cs, idx, 1) - 1
    indptr = np.concatenate([[0], cs[T - 1, :]]) if T > 0 else np.zeros(E + 1, np.int64)
    return dest, indptr, cs


# ------------------------------------------------------------------ experts

# ---------------------------------------------------------------- expert parallelism, simulated

def ep_group_ids(idx: np.ndarray, E: int, n: int) -> np.ndarray:
    """Expert parallelism over n ranks ([15-779] §5.1; [CME295] §5): rank r holds
    experts [r·E/n, (r+1)·E/n) and tokens [r·T/n, (r+1)·T/n). An assignment (t, e)
    travels from source rank s = t // (T/n) to destination rank r = e // (E/n).
    Its group is (r, s, local expert) numbered destination-major, so the rows a
    source sends to a destination, and everything a destination receives, are
    contiguous: group = (r·n + s)·(E/n) + e mod (E/n)."""
    idx = np.asarray(idx, np.int64)
    T = idx.shape[0]
    El, Tl = E // n, T // n
    t = np.repeat(np.arange(T)[:, None], idx.shape[1], axis=1)
    return ((idx // El) * n + t // Tl) * El + idx % El


def ep_permutation(idx: np.ndarray, E: int, n: int):
    """Rows grouped by (destination rank, source rank, local expert), token order
    inside a group: the permutation by prefix sum ([15-779] §3.3) over the n·E
    groups. Returns offsets[n·E + 1], dest[T, k], src[R]."""
    a = assign_rows(ep_group_ids(idx, E, n), n * E)
    return a["offsets"], a["dest"], a["src"]


def ep_group_expert(g: np.ndarray, E: int, n: int) -> np.ndarray:
    """Expert whose weights group g multiplies."""
    El = E // n
    g = np.asarray(g, np.int64)
    return (g // (n * El)) * El + g % El


def ep_send_rows(offsets: np.ndarray, E: int, n: int) -> np.ndarray:
    """rows[s, r]: rows source rank s sends to destination rank r in the dispatch
    all-to-all (s == r stays local); the combine all-to-all returns the same rows."""
    El = E // n
    o = np.asarray(offsets, np.int64)
    rows = np.zeros((n, n), np.int64)
    for r in range(n):
        for s in range(n):
            g0 = (r * n + s) * El
            rows[s, r] = o[g0 + El] - o[g0]
    return rows


def ep_dispatch_bytes(tokens_per_rank: int, k: int, n: int, d: int, elt: int) -> float:
    """Bytes one rank sends in one all-to-all under uniform routing:
    N·k·(1 - 1/n)·d·bytes ([15-779] §5.1 and §10 exercise 6), independent of E."""
    return tokens_per_rank * k * (1.0 - 1.0 / n) * d * elt


def silu(u: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return u / (1.0 + np.exp(-u))


def swiglu_hidden(X, w1, w3) -> np.ndarray:
    """The SwiGLU hidden activation a = silu(X W1^T) * (X W3^T) on rows X[n, d],
    with W1, W3 stored [d_ff, d]: silu on the W1 ("gate") branch."""
    X = np.asarray(X, np.float64)
    return silu(X @ np.asarray(w1, np.float64).T) * (X @ np.asarray(w3, np.float64).T)


def swiglu(X: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """One SwiGLU expert on rows X[n, d]: swiglu_hidden(X) W2^T, with W2 stored
    [d, d_ff]."""
    return swiglu_hidden(X, w1, w3) @ np.asarray(w2, np.float64).T


ExpertFn = Callable[[int], Tuple[np.ndarray, np.ndarray, np.ndarray]]


def expert_ffn(rows: np.ndarray, offsets: np.ndarray, experts: ExpertFn) -> np.ndarray:
    """Z = GroupGemm(data, indptr, weights) of [15-779] §3.3: rows
    [offsets[e], offsets[e+1]) go through expert e. ``experts(e)`` returns that
    expert's (W1, W3, W2); it is called once per non-empty group so large
    layers can be streamed one expert at a time."""
    rows = np.asarray(rows, np.float64)
    out = np.zeros((rows.shape[0], rows.shape[1]), np.float64)
    E = len(offsets) - 1
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            w1, w3, w2 = experts(e)
            out[lo:hi] = swiglu(rows[lo:hi], w1, w3, w2)
    return out


def combine(yp: np.ndarray, dest: np.ndarray, gates: np.ndarray, d: int,
            shared: Optional[np.ndarray] = None) -> np.ndarray:
    """Unpermute and mix: y_t = sum_{j kept} g_{t,j} yp[dest[t,j]] (+ shared_t)
    ([CME295] §1.3 y = sum g_i f_i(x); [15-779] §3.2 step 4)."""
    T, k = dest.shape
    y = np.zeros((T, d), np.float64)
    for j in range(k):
        ok = dest[:, j] >= 0
        y[ok] += gates[ok, j][:, None] * yp[dest[ok, j]]
    if shared is not None:
        y += shared
    return y


def forward(x, w_router, experts: ExpertFn, k: int, gate: str = GATE_SELECTED,
            bias=None, cf: float = 0.0, shared=None, alpha: float = 0.0,
            idx_override: Optional[np.ndarray] = None, ep: int = 1):
    """The whole layer: route -> permute -> grouped experts -> combine
    ([15-779] §3.2). ``shared`` is (W1, W3, W2) of an always-on expert whose
    output is added with weight 1 ([CME295] §4.1). ``idx_override`` replaces
    the selection (gates are recomputed from z for it), which lets a caller
    evaluate the layer under another implementation's routing. ``ep`` > 1 lays
    the rows out as ``ep`` simulated expert-parallel ranks (``ep_permutation``;
    no capacity).

    Returns a dict with every intermediate and the stats."""
    x = np.asarray(x, np.float64)
    T, d = x.shape
    r = route(x, w_router, k, gate, bias)
    idx = r["idx"] if idx_override is None else np.asarray(idx_override, np.int64)
    if idx_override is not None:
        r["gates"] = (gates_selected(r["z"], idx) if gate == GATE_SELECTED
                      else gates_all(r["z"], idx))
    E = np.asarray(w_router).shape[0]
    if ep > 1:
        if cf > 0:
            raise ValueError("capacity is not modelled with simulated expert parallelism")
        offsets, dest, src = ep_permutation(idx, E, ep)
        counts = np.bincount(idx.ravel(), minlength=E)
        p = dict(counts=counts, kept=counts.copy(), offsets=offsets, dest=dest, src=src,
                 n_dropped=0, C=None)
        xp = x[src]
        yp = expert_ffn(xp, offsets, lambda g: experts(int(ep_group_expert(g, E, ep))))
    else:
        p = assign_rows(idx, E, cf)
        xp = x[p["src"]]
        yp = expert_ffn(xp, p["offsets"], experts)
    sh = swiglu(x, *shared) if shared is not None else None
    y = combine(yp, p["dest"], r["gates"], d, sh)
    f = load_fractions(idx, E)
    P = mean_probs(r["probs"])
    return dict(y=y, idx=idx, gates=r["gates"], z=r["z"], margin=r["margin"],
                probs=r["probs"], f=f, P=P, aux=aux_loss(f, P, alpha),
                yp=yp, shared_out=sh, **p)


# ---------------------------------------------------------------- backward

def silu_grad(u: np.ndarray) -> np.ndarray:
    """d silu(u)/du = sigma(u) (1 + u (1 - sigma(u)))."""
    u = np.asarray(u, np.float64)
    s = 1.0 / (1.0 + np.exp(-u))
    return s * (1.0 + u * (1.0 - s))


def swiglu_backward(X, w1, w3, w2, dY):
    """Gradients of sum <dY, W2 (silu(X W1^T) * (X W3^T))> for one expert's rows:
    returns (dX, dW1, dW3, dW2) ([15-779] §7: dW2 = H^T dY and the other
    transposed products of the two expert matmuls)."""
    X = np.asarray(X, np.float64)
    dY = np.asarray(dY, np.float64)
    h1, h3 = X @ np.asarray(w1, np.float64).T, X @ np.asarray(w3, np.float64).T
    a = silu(h1) * h3
    dW2 = dY.T @ a
    da = dY @ np.asarray(w2, np.float64)
    dh3 = da * silu(h1)
    dh1 = da * h3 * silu_grad(h1)
    dW1, dW3 = dh1.T @ X, dh3.T @ X
    dX = dh1 @ np.asarray(w1, np.float64) + dh3 @ np.asarray(w3, np.float64)
    return dX, dW1, dW3, dW2


def aux_loss_logit_grad(probs: np.ndarray, f: np.ndarray, alpha: float) -> np.ndarray:
    """dL_aux/dz_{t,i} = (alpha E / T) p_{t,i} (f_i - sum_j p_{t,j} f_j), the
    closed form of [CME295] §3.2 (f held constant: it is a count)."""
    p = np.asarray(probs, np.float64)
    T, E = p.shape
    f = np.asarray(f, np.float64)
    return alpha * E / T * p * (f[None, :] - (p @ f)[:, None])


def backward(x, w_router, experts: ExpertFn, k: int, dy, gate: str = GATE_SELECTED,
             bias=None, cf: float = 0.0, shared=None, alpha: float = 0.0,
             idx_override: Optional[np.ndarray] = None):
    """Gradients of L = sum_t <dy_t, y_t> + L_aux (L_aux only when alpha > 0) with
    respect to x, W_r and every expert's (and the shared expert's) weights.

    The top-k selection and the capacity drops are discrete and pass no gradient
    ([CME295] §1.3: the router learns through the gates of the selected experts).
    Gates: SELECTED mode g = softmax of the selected logits, so
    dz_sel = g (dg - sum g dg) on the selected entries (dropped slots keep their
    gate, with dg = 0); ALL mode g_j = p_{idx_j}, dz = p (dp - sum p dp) with dp
    the dg summed per expert ([15-779] §2.5 contrasts the two for k = 1). The
    selection bias enters neither gates nor gradients ([CME295] §4.2).

    ``idx_override`` evaluates everything under another implementation's
    selection (as in ``forward``).

    Returns dict(dx, dw_router, dw1[E], dw3[E], dw2[E], dws1, dws3, dws2, dz, dg, fwd)."""
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    wr = np.asarray(w_router, np.float64)
    T, d = x.shape
    E = wr.shape[0]
    fwd = forward(x, wr, experts, k, gate, bias, cf, shared, alpha, idx_override=idx_override)
    idx, gates, dest, src, offsets = fwd["idx"], fwd["gates"], fwd["dest"], fwd["src"], fwd["offsets"]
    yp = fwd["yp"]
    # combine backward
    dg = np.zeros((T, k))
    dyp = np.zeros_like(yp)
    for t in range(T):
        for j in range(k):
            r = dest[t, j]
            if r >= 0:
                dg[t, j] = float(dy[t] @ yp[r])
                dyp[r] = gates[t, j] * dy[t]
    # experts
    dx = np.zeros_like(x)
    dw1, dw3, dw2 = [None] * E, [None] * E, [None] * E
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        w1, w3, w2 = (np.asarray(w, np.float64) for w in experts(e))
        if hi > lo:
            rows_t = src[lo:hi]
            dX, dw1[e], dw3[e], dw2[e] = swiglu_backward(x[rows_t], w1, w3, w2, dyp[lo:hi])
            np.add.at(dx, rows_t, dX)
        else:
            dw1[e], dw3[e], dw2[e] = np.zeros_like(w1), np.zeros_like(w3), np.zeros_like(w2)
    dws1 = dws3 = dws2 = None
    if shared is not None:
        dXs, dws1, dws3, dws2 = swiglu_backward(x, *shared, dy)
        dx += dXs
    # gates -> logits
    z = fwd["z"]
    dz = np.zeros((T, E))
    if gate == GATE_SELECTED:
        s = (gates * dg).sum(axis=1, keepdims=True)
        dsel = gates * (dg - s)
        for j in range(k):
            np.add.at(dz, (np.arange(T), idx[:, j]), dsel[:, j])
    else:
        p = fwd["probs"]
        dp = np.zeros((T, E))
        for j in range(k):
            np.add.at(dp, (np.arange(T), idx[:, j]), dg[:, j])
        dz = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    if alpha > 0:
        dz = dz + aux_loss_logit_grad(fwd["probs"], fwd["f"], alpha)
    dw_router = dz.T @ x
    dx += dz @ wr
    return dict(dx=dx, dw_router=dw_router, dw1=dw1, dw3=dw3, dw2=dw2, dws1=dws1,
                dws3=dws3, dws2=dws2, dz=dz, dg=dg, fwd=fwd)


def token_input_grad(x_t, dy_t, z_t, idx_t, gates_t, experts: ExpertFn, w_router,
                     gate: str = GATE_SELECTED, keep_t=None, shared=None, alpha: float = 0.0,
                     f=None, T: int = 1) -> np.ndarray:
    """dx for one token, from its own slots only (the same quantity as ``backward``'s
    dx row, without the other tokens' products).

    Per kept slot j (expert e, gate g): h1 = W1 x, h3 = W3 x, da = g W2^T dy,
    dx += W1^T (da h3 silu'(h1)) + W3^T (da silu(h1)) ([15-779] §7), and the gate's
    gradient dg_j = <dy, f_e(x)> (0 for a dropped slot). The logits' gradient dz
    follows from dg as in ``backward`` (selected or full softmax), plus, when
    alpha > 0, the balance-loss term (alpha E / T) p (f - p.f) with the layer's load
    fractions f over all T tokens ([CME295] §3.2); dx += dz W_r. A shared expert adds
    its own input gradient with gate 1."""
    x = np.asarray(x_t, np.float64)
    dy = np.asarray(dy_t, np.float64)
    wr = np.asarray(w_router, np.float64)
    E = wr.shape[0]
    k = len(idx_t)

    def expert_dx(w1, w3, w2, g):
        w1, w3, w2 = (np.asarray(w, np.float64) for w in (w1, w3, w2))
        h1, h3 = w1 @ x, w3 @ x
        u = w2.T @ dy
        da = g * u
        dx_e = w1.T @ (da * h3 * silu_grad(h1)) + w3.T @ (da * silu(h1))
        return dx_e, float(u @ (silu(h1) * h3))      # <dy, W2 act> = <W2^T dy, act>

    dx = np.zeros_like(x)
    dg = np.zeros(k)
    for j in range(k):
        if keep_t is not None and not keep_t[j]:
            continue
        dx_e, dg[j] = expert_dx(*experts(int(idx_t[j])), float(gates_t[j]))
        dx += dx_e
    if shared is not None:
        dx += expert_dx(*shared, 1.0)[0]
    g = np.asarray(gates_t, np.float64)
    dz = np.zeros(E)
    p = softmax(np.asarray(z_t, np.float64)[None, :])[0]
    if gate == GATE_SELECTED:
        sgd = float(g @ dg)
        for j in range(k):
            dz[int(idx_t[j])] += g[j] * (dg[j] - sgd)
    else:
        dp = np.zeros(E)
        for j in range(k):
            dp[int(idx_t[j])] += dg[j]
        dz = p * (dp - p @ dp)
    if alpha > 0:
        fv = np.asarray(f, np.float64)
        dz = dz + alpha * E / T * p * (fv - p @ fv)
    return dx + dz @ wr


def expert_unit_grads(X_rows, dY_rows, g_rows, w1, w3, w2, units):
    """Weight gradients of one expert for the hidden units ``units`` only: rows
    dW1[units, :], dW3[units, :] and columns dW2[:, units], summed over the expert's
    rows (token x_r, upstream gradient g_r dy_r), from the per-unit chain rule
    h1 = x W1[f], h3 = x W3[f], a = silu(h1) h3, da = g_r dy_r W2[:, f]:
    dW2[:, f] = sum_r g_r dy_r a_r, dW1[f] = sum_r da_r h3_r silu'(h1_r) x_r,
    dW3[f] = sum_r da_r silu(h1_r) x_r ([15-779] §7). Equal to those entries of
    ``swiglu_backward`` on the same rows. Returns (dW1u [n, d], dW3u [n, d], dW2u [d, n])."""
    X = np.asarray(X_rows, np.float64)
    dY = np.asarray(dY_rows, np.float64) * np.asarray(g_rows, np.float64)[:, None]
    units = np.asarray(units)
    w1u = np.asarray(w1, np.float64)[units]
    w3u = np.asarray(w3, np.float64)[units]
    w2u = np.asarray(w2, np.float64)[:, units]
    h1, h3 = X @ w1u.T, X @ w3u.T
    a = silu(h1) * h3
    da = dY @ w2u
    dW2u = dY.T @ a
    dW1u = (da * h3 * silu_grad(h1)).T @ X
    dW3u = (da * silu(h1)).T @ X
    return dW1u, dW3u, dW2u


def dense_all_experts(x, experts: ExpertFn, G: np.ndarray) -> np.ndarray:
    """Every expert on every token, weighted by a dense [T, E] gate matrix:
    y = sum_e G[:, e] f_e(x) ([15-779] §3.4 formulation 0; with G zero outside
    the selected set it equals the top-k layer, [15-779] §2.1 demo)."""
    x = np.asarray(x, np.float64)
    y = np.zeros_like(x)
    for e in range(G.shape[1]):
        if np.any(G[:, e] != 0):
            y += G[:, e:e + 1] * swiglu(x, *experts(e))
    return y


def scatter_gates(idx: np.ndarray, gates: np.ndarray, E: int) -> np.ndarray:
    """Dense [T, E] gate matrix with zeros outside each token's selection."""
    T = idx.shape[0]
    G = np.zeros((T, E), np.float64)
    np.put_along_axis(G, np.asarray(idx, np.int64), np.asarray(gates, np.float64), 1)
    return G


def token_output(x_t: np.ndarray, idx_t: Sequence[int], gates_t: Sequence[float],
                 experts: ExpertFn, keep_t: Optional[Sequence[bool]] = None,
                 shared=None) -> np.ndarray:
    """y for one token, straight from y = sum_i g_i f_i(x) (+ shared): the
    one-token-at-a-time form used to sample outputs of full-size runs."""
    x_t = np.asarray(x_t, np.float64)[None, :]
    y = np.zeros(x_t.shape[1])
    for j, e in enumerate(idx_t):
        if keep_t is None or keep_t[j]:
            y += gates_t[j] * swiglu(x_t, *experts(int(e)))[0]
    if shared is not None:
        y += swiglu(x_t, *shared)[0]
    return y
