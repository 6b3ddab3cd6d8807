"""Plain, slow CPU oracle of one shared + routed MoE FFN layer forward (fp64).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use this module.  It shares no code
with the HIP path.

What it computes (the pages' definition, written out):

    out_t = sum over shared experts s of FFN_s(u_t)
          + sum over routed experts e of  g_{t,e} * FFN_e(u_t)
    FFN(x) = W2 (SiLU(W1 x) * W3 x),  SiLU(z) = z * sigmoid(z)
    g_{t,e} = p_{t,e} if e is among the top-k logits of token t, else 0
    p_t     = softmax over *all* routed experts of l_t,  l_{t,e} = u_t . c_e (+ b_e)

Sources: "Shared Expert" page on DeepSeek-V3 (How it works: eq. 12 and the
SwiGLU definition; Official code: shared + routed returned without residual,
fused shared width N_s * f; Watch-outs: shared coefficient exactly 1);
"What is an 'expert', really?" (glossary: softmax gives blend weights that add
to 1, the router keeps the top-k; panel 2: a linear router scores the experts
and the kept experts' outputs are blended by its weights); "Shared and
fine-grained experts" (Researcher level: the layer sums g_i E_i(x) over the
selected set, plus the always-on shared experts).

Readings taken where the pages are silent (each is listed with its reason in
the design notes):
* the kept gates are the full-softmax probabilities, not renormalised over the
  top-k;
* the ranking key is the exact real value of u . c_e + b_e computed from the
  stored inputs; exact ties go to the lower expert index; the k slots are in
  descending key order;
* the shared output is added with coefficient 1 and no residual is added;
* every token goes to all of its k experts unless a capacity (seats per
  expert) is given; then each expert keeps the first seats of its pairs in
  token order and the dropped slots contribute nothing.

Inputs are numpy arrays holding the exact stored values (fp32 or bf16 widened
to fp64, which is exact).  Expert weight stacks may be any object whose
``[e]`` returns expert e's matrix, so that large workloads can be widened to
fp64 one expert at a time.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Optional, Sequence

import numpy as np

_U = 2.0 ** -53  # unit roundoff of fp64


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------- router
def router_logits(u, w_router, bias=None):
    """Router logits l = u . c_e (+ b_e) in fp64, with a rigorous error bound.

    The router is a bias-free linear layer whose rows are the experts'
    centroids ("What is an 'expert', really?", panel 2; "Shared Expert", How it
    works: the N_r centroids).  The optional bias is the workload's router
    bias, added before the softmax.

    Returns (l, beta): |l - exact| <= beta elementwise, whatever order or FMA
    use the BLAS picks.  For an n-term dot product |fl - exact| <= gamma_n *
    sum|x_i y_i| with gamma_n = n u / (1 - n u); beta doubles that as margin
    and uses the computed |u| . |c|^T (itself within gamma_n).
    """
    u = _f64(u)
    w = _f64(w_router)
    l = u @ w.T
    a = np.abs(u) @ np.abs(w).T
    n = u.shape[1]
    if bias is not None:
        b = _f64(bias)
        l = l + b[None, :]
        a = a + np.abs(b)[None, :]
        n += 1
    beta = 2.0 * (n + 2) * _U * a
    return l, beta


def exact_logit(u_row, w_row, b=None) -> Fraction:
    """Exact rational value of u . w (+ b) from the stored floating-point inputs."""
    num = 0
    den_exp = 0  # common denominator 2**den_exp
    terms = []
    for x, y in zip(_f64(u_row).tolist(), _f64(w_row).tolist()):
        if x == 0.0 or y == 0.0:
            continue
        nx, dx = x.as_integer_ratio()
        ny, dy = y.as_integer_ratio()
        terms.append((nx * ny, (dx * dy).bit_length() - 1))
    if b is not None and float(b) != 0.0:
        nb, db = float(b).as_integer_ratio()
        terms.append((nb, db.bit_length() - 1))
    for _, e in terms:
        den_exp = max(den_exp, e)
    for t_num, e in terms:
        num += t_num << (den_exp - e)
    return Fraction(num, 1 << den_exp)


def softmax(l) -> np.ndarray:
    """Softmax over the last axis, max-subtracted, fp64 ("What is an 'expert',
    really?", glossary: raw scores become fractions that add to 1)."""
    l = _f64(l)
    z = np.exp(l - l.max(axis=-1, keepdims=True))
    return z / z.sum(axis=-1, keepdims=True)


def _kept_groups(l_t, lo_t, hi_t, n_group: int, topk_group: int, exact_of):
    """The topk_group groups with the largest best-expert logit (ties to the lower
    group index), as a sorted list.  Experts are split into n_group contiguous
    groups of N_r / n_group.  Returns (groups, settled_exactly)."""
    G = l_t.shape[0] // n_group
    gl, glo, ghi = (a.reshape(n_group, G).max(axis=1) for a in (l_t, lo_t, hi_t))
    order = np.lexsort((np.arange(n_group), -gl))
    kept = order[:topk_group]
    if topk_group == n_group or glo[kept].min() > ghi[order[topk_group:]].max():
        return sorted(int(g) for g in kept), False
    # A group whose upper bound is below the topk_group-th largest lower bound has
    # that many groups certainly above it; inside a group, only experts whose upper
    # bound reaches the group's largest lower bound can be its best expert.
    cut = np.sort(glo)[::-1][topk_group - 1]
    best = {}
    for g in range(n_group):
        if ghi[g] >= cut:
            es = [g * G + i for i in range(G) if hi_t[g * G + i] >= glo[g]]
            best[g] = max(exact_of(e) for e in es)
    ranked = sorted(best, key=lambda g: (-best[g], g))
    return sorted(ranked[:topk_group]), True


def route(u, w_router, k: int, bias=None, n_group: Optional[int] = None, topk_group: Optional[int] = None):
    """Per-token top-k selection and gates.

    Returns (topk_idx [T,k] int32, topk_w [T,k] fp64, logits [T,N_r] fp64,
    n_exact) where n_exact counts tokens whose order had to be settled with
    exact arithmetic.

    Selection is on the logits (softmax is strictly increasing, so this is the
    top-k of the probabilities too).  A token's fp64 order is accepted when
    every comparison that decides the ordered top-k is separated by more than
    the two error bounds; otherwise the candidates that may belong to the
    top-k are re-ranked by their exact rational logits.

    Group-limited routing (n_group, topk_group): "Shared and fine-grained
    experts" names DeepSeek-V3's node-limited routing (Developer level, 'Why not
    go finer still': it caps the machines a token's experts live on; Researcher
    level, Systems limits: n_group 8, topk_group 4); the rule for scoring a
    group is not on the pages.  Reading: the
    experts form n_group contiguous groups, a group's score is its best expert's
    logit, the token keeps the topk_group best groups (ties to the lower group
    index) and its top-k is taken among their experts only.  The gates stay the
    full-softmax probabilities.
    """
    u = _f64(u)
    w = _f64(w_router)
    T, E = u.shape[0], w.shape[0]
    if not (1 <= k <= E):
        raise ValueError("top_k must be in [1, n_routed]")
    grouped = n_group is not None and n_group > 1 and topk_group is not None and topk_group < n_group
    if grouped and (E % n_group or not 1 <= topk_group or topk_group * (E // n_group) < k):
        raise ValueError("need N_r divisible by n_group and topk_group * N_r / n_group >= k")
    l, beta = router_logits(u, w, bias)
    lo, hi = l - beta, l + beta
    idx = np.empty((T, k), dtype=np.int32)
    n_exact = 0
    experts = np.arange(E)
    b = None if bias is None else _f64(bias)
    for t in range(T):
        exact_of = lambda e: exact_logit(u[t], w[e], None if b is None else b[e])
        lt, lot, hit = l[t], lo[t], hi[t]
        settled_exactly = False
        if grouped:
            kept, settled_exactly = _kept_groups(lt, lot, hit, n_group, topk_group, exact_of)
            out = np.ones(E, dtype=bool)
            G = E // n_group
            for g in kept:
                out[g * G:(g + 1) * G] = False
            lt, lot, hit = (np.where(out, -np.inf, a) for a in (lt, lot, hit))
        order = np.lexsort((experts, -lt))  # descending logit, ties -> lower index
        top = order[:k]
        ok = all(lot[top[j]] > hit[top[j + 1]] for j in range(k - 1))
        if ok and k < E:
            ok = lot[top[k - 1]] > hit[order[k:]].max()
        if not ok:
            settled_exactly = True
            # Any expert whose upper bound is below the k-th largest lower bound
            # has at least k experts certainly above it: it cannot be selected.
            kth_lo = np.sort(lot)[::-1][k - 1]
            cand = [int(e) for e in experts if hit[e] >= kth_lo]
            keys = {e: exact_of(e) for e in cand}
            top = sorted(cand, key=lambda e: (-keys[e], e))[:k]
        n_exact += settled_exactly
        idx[t] = top
    p = softmax(l)
    gates = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    return idx, gates, l, n_exact


# ---------------------------------------------------------------------- permutation
def permute(topk_idx, n_routed: int, capacity: Optional[int] = None):
    """Group the T*k (token, slot) pairs by expert, tokens ascending inside a group.

    Returns counts [N_r], offsets [N_r+1] (exclusive prefix of counts),
    row_token [offsets[N_r]] (row r of an expert group -> its token) and
    token_row [T,k] (token t's slot j -> its row, or -1 when the pair was
    dropped).  This is the expert-to-token grouping that feeds the scatter-sum
    of routed expert outputs ("Shared Expert", How it works).

    capacity: seats per expert ("What is an 'expert', really?", glossary:
    capacity factor / token dropping -- each expert takes at most a fixed
    number of tokens per batch and the overflow is skipped).  Reading: an
    expert keeps the first ``capacity`` of its pairs in token order, i.e. a
    prefix of its group in the stable grouping; the rest are dropped and
    contribute nothing.  None = no limit (every pair kept).
    """
    idx = np.asarray(topk_idx, dtype=np.int64)
    T, k = idx.shape
    flat = idx.ravel()
    raw = np.bincount(flat, minlength=n_routed)
    order = np.argsort(flat, kind="stable")  # pairs grouped by expert, token order inside
    start = np.zeros(n_routed + 1, dtype=np.int64)
    np.cumsum(raw, out=start[1:])
    rank = np.empty(T * k, dtype=np.int64)  # position of each pair inside its expert's group
    rank[order] = np.arange(T * k) - start[flat[order]]
    seats = raw if capacity is None else np.minimum(raw, capacity)
    keep = np.ones(T * k, dtype=bool) if capacity is None else rank < capacity
    offsets = np.zeros(n_routed + 1, dtype=np.int64)
    np.cumsum(seats, out=offsets[1:])
    token_row = np.full(T * k, -1, dtype=np.int64)
    token_row[keep] = offsets[flat[keep]] + rank[keep]
    row_token = np.empty(int(offsets[-1]), dtype=np.int64)
    row_token[token_row[keep]] = np.nonzero(keep)[0] // k
    return (seats.astype(np.int32), offsets.astype(np.int32), row_token.astype(np.int32),
            token_row.reshape(T, k).astype(np.int32))


def capacity_seats(capacity_factor, T: int, k: int, n_routed: int) -> int:
    """Seats per expert for a capacity factor: ceil(cf * T * k / N_r), exactly.

    The glossary of "What is an 'expert', really?" gives each expert a seat
    limit per batch; the usual way to size it from a capacity factor is cf
    times the balanced load T*k/N_r, rounded up.  cf is taken as the exact
    rational value of the given number (a float is its binary value)."""
    q = Fraction(capacity_factor) * T * k / n_routed
    return int(-((-q.numerator) // q.denominator))


# -------------------------------------------------------------------------- experts
def silu(z):
    """SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu(x, w1, w3, w2):
    """One SwiGLU expert on the rows of x: W2 (SiLU(W1 x) * W3 x).

    "Shared Expert", How it works: the expert MLP; W1 is the gate (SiLU)
    branch, W3 the up branch, W2 the down projection; weights in [out, in]
    layout: W1, W3 are [f, d] and W2 is [d, f]."""
    x = _f64(x)
    g = x @ _f64(w1).T
    v = x @ _f64(w3).T
    return (silu(g) * v) @ _f64(w2).T


def expert_ffn(u, w1, w3, w2, counts, offsets, row_token, w1s=None, w3s=None, w2s=None):
    """Every routed expert on its grouped rows, plus the shared MLP on all tokens.

    Returns y_rows [T*k, d] (row r = expert of group r applied to token
    row_token[r]) and y_shared [T, d] or None.  The N_s shared experts are one
    MLP of width N_s * f applied to the full token batch ("Shared Expert",
    Official code)."""
    u = _f64(u)
    R = int(offsets[-1])
    y_rows = np.zeros((R, u.shape[1]), dtype=np.float64)
    for e in range(len(counts)):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            y_rows[a:b] = swiglu(u[row_token[a:b]], w1[e], w3[e], w2[e])
    y_shared = None if w1s is None else swiglu(u, w1s, w3s, w2s)
    return y_rows, y_shared


def combine(y_rows, y_shared, topk_w, token_row):
    """out_t = shared_t + sum_j g_{t,j} * y_rows[token_row[t, j]], slots in order.

    The shared term enters with coefficient exactly 1, is not scaled by any
    gate nor by 1/N_s ("Shared Expert", Overview and Watch-outs), and no
    residual is added (MoE.forward returns shared + routed only).  A slot whose
    pair was dropped for capacity (token_row -1) contributes nothing."""
    y_rows = _f64(y_rows)
    g = _f64(topk_w)
    T, k = g.shape
    d = y_rows.shape[1] if y_shared is None else np.shape(y_shared)[1]
    out = np.zeros((T, d), dtype=np.float64) if y_shared is None else _f64(y_shared).copy()
    tr = np.asarray(token_row)
    for j in range(k):
        kept = tr[:, j] >= 0
        out[kept] += g[kept, j, None] * y_rows[tr[kept, j]]
    return out


def forward(u, w_router, w1, w3, w2, k: int, bias=None, w1s=None, w3s=None, w2s=None,
            capacity: Optional[int] = None, n_group: Optional[int] = None, topk_group: Optional[int] = None):
    """The whole layer: route, group, run experts, combine.  Returns a dict.
    capacity: seats per expert (see ``permute``); None = no limit.
    n_group, topk_group: group-limited routing (see ``route``); None = none."""
    E = _f64(w_router).shape[0]
    idx, gates, l, n_exact = route(u, w_router, k, bias, n_group, topk_group)
    counts, offsets, row_token, token_row = permute(idx, E, capacity)
    y_rows, y_shared = expert_ffn(u, w1, w3, w2, counts, offsets, row_token, w1s, w3s, w2s)
    out = combine(y_rows, y_shared, gates, token_row)
    routed = combine(y_rows, None, gates, token_row)
    return {"topk_idx": idx, "topk_w": gates, "logits": l, "n_exact": n_exact,
            "counts": counts, "offsets": offsets, "row_token": row_token, "token_row": token_row,
            "y_rows": y_rows, "y_shared": y_shared, "out": out, "routed": routed}


def forward_dense(u, w_router, w1, w3, w2, k: int, bias=None, w1s=None, w3s=None,
                  w2s=None, experts: Optional[Sequence[int]] = None):
    """Brute force for tiny shapes: every expert on every token, masked gates.

    The selected set of each token is found from exact rational logits of all
    N_r experts (ties to the lower index), independently of ``route``; the
    layer output is the dense masked mixture sum_e ghat_{t,e} FFN_e(u_t) plus
    the shared MLP, which the sparse path must reach exactly up to rounding
    ("Shared and fine-grained experts", Researcher level)."""
    u = _f64(u)
    wr = _f64(w_router)
    T, E = u.shape[0], wr.shape[0]
    b = None if bias is None else _f64(bias)
    l = u @ wr.T + (0.0 if b is None else b[None, :])
    p = softmax(l)
    ghat = np.zeros((T, E))
    sel = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        keys = [exact_logit(u[t], wr[e], None if b is None else b[e]) for e in range(E)]
        top = sorted(range(E), key=lambda e: (-keys[e], e))[:k]
        sel[t] = top
        ghat[t, top] = p[t, top]
    out = np.zeros_like(u) if w1s is None else swiglu(u, w1s, w3s, w2s)
    for e in (range(E) if experts is None else experts):
        out = out + ghat[:, e, None] * swiglu(u, w1[e], w3[e], w2[e])
    return {"topk_idx": sel, "ghat": ghat, "out": out}
