"""fp64 CPU oracle for the batched verify step of speculative decoding.

TEST INFRASTRUCTURE ONLY.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import this module.  The
product path (the HIP library and its Python binding) never calls it, and
this module imports nothing from the product path.

What it computes, and where the pages fix it
--------------------------------------------
* Temperature softmax of every verify row: page "Speculative Decoding in
  Custom LLM Servicing: Implementing Draft Models in Rust", section "The
  Verification Algorithm" (target rows) and section "Orchestrating the
  Inference Loop" (draft rows are tempered the same way).
* Per-row temperature / top-k / top-p: page "FreeToken PR #836", section
  "Design", rejection bullet (each verify row samples with its request's
  temperature, top-k, top-p and greedy flag).
* Acceptance of draft x_i with probability min(1, p(x_i)/q(x_i)), position
  by position, stopping at the first rejection: page "Speculative Decoding:
  Draft Model Sampling, Rejection Sampling & On-Device Acceleration", Key
  Topic 2 and Section 2; the Rust page, section "The Memory Bandwidth Wall
  and Speculative Math".
* Residual max(0, p - q) / sum max(0, p - q) at the first rejection: same
  passages; the catalog page "Adding Speculative Decoding", section
  "Verification and sampling", item 2.
* Bonus token from the last target row when every draft is accepted: the
  Rust page, section "The Verification Algorithm" (snippet 2, tail).
* Greedy verify (accept while draft == argmax, commit the argmax at the
  first mismatch), the degenerate case of the above with a one-hot target:
  catalog page, sections "The existing base" and "Verification and
  sampling" item 2.
* Prefix-match verify of argmax drafts (draft kind MATCH): every verify row
  is sampled the way decode samples it, and the drafts are accepted while
  each equals its row's sample; the sample at the first mismatch (or of the
  last row) is committed.  Page "FreeToken PR #836", section "Design",
  rejection row and the bullet on argmax drafts (the PR's own verify, equal
  in law to rejection sampling with one-hot drafts).
* Presence and frequency penalties per verify row, the drafts before a row
  counted as already generated: page "FreeToken PR #836", section "Design",
  the bullet on argmax drafts, and its test list (``test_rejection``).

Readings where the pages are silent or disagree (each one is listed in
the design doc as well):
* Acceptance compares ``u < min(1, p/q)`` with a strict ``<`` and no epsilon
  guard; q = 0 gives threshold 1 when p > 0 and 0 when p = 0.
* The uniform -> token map of every draw is the inverse CDF in ascending
  token id with a strict ``>``: t = min{t : C_t > u * W}, C accumulated
  sequentially in token order.
* The residual falls back to p only when its total mass W is exactly 0.
* Filters apply in the order temperature -> top-k -> top-p; top-k keeps every
  value >= the K-th largest (ties kept); top-p keeps the shortest prefix of
  whole tie groups whose mass reaches P, measured on the tempered top-k
  distribution, then renormalises.  A top-p cut whose group mass lies
  within 1e-6 of P is flagged as a near tie.
* Draft probability rows (kind PROBS) are used exactly as supplied; draft
  logit rows (kind LOGITS) get the request's temperature and filters; a
  one-hot draft (kind ONEHOT) has q = e_x.
* A request whose temperature is not a normal positive float (T <= 0, NaN,
  subnormal) is greedy; greedy ignores filters, draft rows and uniforms.
  Argmax ties go to the lowest index; -0 equals +0.
* Status codes, first match wins: BAD_K, BAD_PARAM, BAD_TOKEN, NONFINITE,
  EMPTY (see ``verify``).
* Penalties (the pages name them, not their formula): the usual additive
  form.  Row j of request b sees the count c(t) = h_b(t) + #{i < j : x_i = t}
  (h_b: the request's generated-token counts; the drafts x_0..x_{j-1} before
  the row), and every token with c(t) > 0 gets
  l'(t) = l(t) - (frequency_b * c(t) + presence_b), evaluated in fp64 and
  rounded to fp32, then to the logits' storage type (bf16 rows stay bf16
  values: the logits are processed in their own dtype).  Penalties apply to
  the target rows of every request, greedy ones included, before the
  temperature and the filters; draft rows are used as supplied (they are the
  drafter's distribution).  Non-finite penalties make the request
  BAD_PARAM.  History entries with a token outside [0, V) or a negative
  count are ignored, and a request whose history offsets are out of order or
  out of range has no history.

Parity status of each function
------------------------------
Every function here is pinned by the ``-m "not gpu"`` tests against
library routines, closed forms, the pages' worked examples, brute force or
exact enumeration of the lossless law.  Two conventions are *parity
unpinned by the pages* and pinned only against brute force of their own
definition: the tie semantics of top-k/top-p and the pointwise
uniform -> token map (the pages fix only its law).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# dtype codes of the boundary
F32, BF16 = 0, 1
# draft kinds
ONEHOT, LOGITS, PROBS, MATCH = 0, 1, 2, 3
# per-request status codes
ROW_OK, ROW_NONFINITE, ROW_EMPTY, ROW_BAD_K, ROW_BAD_TOKEN = 0, 1, 2, 3, 4
ROW_INTERNAL = 6

NEAR_TIE = 1e-6


# --------------------------------------------------------------------------
# input widening
# --------------------------------------------------------------------------
def widen(a, dtype: int) -> np.ndarray:
    """Widen stored values exactly to float64.

    bf16 values arrive as their raw 16-bit patterns (uint16); a bf16 number
    is the float32 whose upper half is those 16 bits.
    """
    a = np.asarray(a)
    if dtype == BF16:
        bits = a.astype(np.uint32) << np.uint32(16)
        return bits.view(np.float32).astype(np.float64)
    if dtype == F32:
        return a.astype(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype code {dtype}")


# --------------------------------------------------------------------------
# distribution of one verify row
# --------------------------------------------------------------------------
@dataclass
class Dist:
    p: np.ndarray          # float64 [V], sums to 1 over the kept set
    near_tie: bool = False  # top-p cut within 1e-6 of P


def process(z_raw: np.ndarray, T: float, top_k: int = 0, top_p: float = 1.0) -> Dist:
    """Tempered, filtered softmax of one row of raw logits (float64).

    Follows the Rust page's "The Verification Algorithm" (softmax of logits
    divided by the temperature) and the FreeToken PR's per-row
    temperature/top-k/top-p.  Masked tokens are the ones at -inf.
    """
    z = np.asarray(z_raw, dtype=np.float64) / float(T)
    V = z.shape[0]
    kept = z > -np.inf
    n_kept = int(kept.sum())
    if n_kept == 0:
        raise ValueError("row has no finite logit")

    # top-k: keep every token whose value is >= the K-th largest kept value
    if 0 < top_k < n_kept:
        ordered = np.sort(z[kept])[::-1]
        tau = ordered[top_k - 1]
        kept = kept & (z >= tau)

    # softmax over the kept set, normalised by the sum in token order
    m = np.max(z[kept])
    e = np.zeros(V, dtype=np.float64)
    e[kept] = np.exp(z[kept] - m)
    p = e / np.sum(e)

    near = False
    # top-p: shortest prefix of whole tie groups (descending value) with mass >= P
    if 0.0 < top_p < 1.0:
        values, group = np.unique(z[kept], return_inverse=True)   # ascending
        group_mass = np.bincount(group, weights=p[kept], minlength=values.shape[0])
        values, group_mass = values[::-1], group_mass[::-1]       # descending
        G = np.cumsum(group_mass)
        reach = np.nonzero(G >= top_p)[0]
        J = int(reach[0]) if reach.size else len(values) - 1
        if abs(G[J] - top_p) < NEAR_TIE or (J > 0 and abs(G[J - 1] - top_p) < NEAR_TIE):
            near = True
        kept = kept & (z >= values[J])
        p = np.where(kept, p, 0.0)
        p = p / np.sum(p)
    return Dist(p=p, near_tie=near)


# --------------------------------------------------------------------------
# greedy verify
# --------------------------------------------------------------------------
def round_to_dtype(v: np.ndarray, dtype: int) -> np.ndarray:
    """fp64 values rounded to fp32 (nearest, ties to even), then, for bf16,
    to bf16 (nearest, ties to even, written out on the fp32 bit pattern);
    returned as fp64."""
    with np.errstate(over="ignore"):   # beyond the fp32 range rounds to +-inf
        f = np.asarray(v, dtype=np.float64).astype(np.float32)
    if dtype == F32:
        return f.astype(np.float64)
    bits = f.view(np.uint32).astype(np.uint64)
    keep = bits >> np.uint64(16)
    rest = bits & np.uint64(0xFFFF)
    up = (rest > 0x8000) | ((rest == 0x8000) & ((keep & np.uint64(1)) == 1))
    rounded = (keep + up.astype(np.uint64)).astype(np.uint32)
    nan = np.isnan(f)
    rounded[nan] = 0x7FC0
    out = (rounded << np.uint32(16)).view(np.float32).astype(np.float64)
    return out


def penalize(row: np.ndarray, dtype: int, hist_tokens, hist_counts, drafts_before,
             presence: float, frequency: float) -> np.ndarray:
    """One verify row's logits after presence / frequency penalties.

    row: the stored values widened to fp64; hist_tokens / hist_counts: the
    request's generated-token counts; drafts_before: x_0..x_{j-1}.  FreeToken
    PR #836, section "Design" (the drafts before a row count as generated).
    """
    V = row.shape[0]
    counts: dict[int, int] = {}
    for t, h in zip(np.asarray(hist_tokens, dtype=np.int64).tolist(),
                    np.asarray(hist_counts, dtype=np.int64).tolist()):
        if 0 <= t < V and h >= 0:
            counts[t] = counts.get(t, 0) + h
    for x in np.asarray(drafts_before, dtype=np.int64).tolist():
        counts[x] = counts.get(x, 0) + 1
    out = row.copy()
    for t, c in counts.items():
        if c > 0:
            d = float(row[t]) - (float(np.float32(frequency)) * c + float(np.float32(presence)))
            out[t] = round_to_dtype(np.array([d]), dtype)[0]
    return out


def argmax_lowest(row: np.ndarray) -> int:
    """min{y : l_y = max l} on raw values (-0 == +0 under float compare)."""
    m = np.max(row)
    return int(np.nonzero(row == m)[0][0])


def greedy_request(rows: np.ndarray, drafts: np.ndarray):
    """Accept while x_i equals the row's argmax; commit the argmax at the
    first mismatch (or the last row's argmax if all k drafts match)."""
    k = drafts.shape[0]
    g = [argmax_lowest(rows[j]) for j in range(k + 1)]
    a = k
    for i in range(k):
        if int(drafts[i]) != g[i]:
            a = i
            break
    tokens = [int(drafts[i]) for i in range(a)] + [g[a]]
    return a, tokens, g


# --------------------------------------------------------------------------
# sampled verify: acceptance scan, final distribution, inverse CDF
# --------------------------------------------------------------------------
def accept_threshold(p_x: float, q_x: float) -> float:
    """min(1, p/q); q = 0 gives 1 if p > 0 else 0 (no epsilon guard)."""
    if q_x > 0.0:
        return min(1.0, p_x / q_x)
    return 1.0 if p_x > 0.0 else 0.0


def accept_scan(p_x, q_x, u):
    """Walk the k drafts in order; accept x_i while u_i < min(1, p/q).

    Returns (a, theta, margins): a = index of the first rejection (k if none),
    the thresholds of every position and |u_i - theta_i| of the positions
    that were examined (0..a, or 0..k-1).
    """
    k = len(p_x)
    theta = [accept_threshold(float(p_x[i]), float(q_x[i])) for i in range(k)]
    margins = []
    for i in range(k):
        margins.append(abs(float(u[i]) - theta[i]))
        if not (float(u[i]) < theta[i]):
            return i, theta, margins
    return k, theta, margins


def final_weights(p_a: np.ndarray, q_a, rejected: bool):
    """Residual max(0, p - q) after a rejection (p itself if its total mass
    is exactly 0), or p of the last row for the bonus draw.

    Returns (w, fallback_used)."""
    if not rejected:
        return p_a, False
    w = np.maximum(0.0, p_a - q_a)
    if np.sum(w) == 0.0:
        return p_a, True
    return w, False


def inverse_cdf(w: np.ndarray, u: float):
    """t = min{t : C_t > u*W}, C summed sequentially in token order.

    Returns (t, C, W).  If rounding leaves no such t, the last token with
    positive mass is taken.
    """
    C = np.cumsum(w)          # numpy accumulates sequentially, in token order
    W = float(C[-1])
    hit = np.nonzero(C > u * W)[0]
    if hit.size:
        t = int(hit[0])
    else:
        t = int(np.nonzero(w > 0)[0][-1])
    return t, C, W


@dataclass
class SampledRecord:
    a: int
    tokens: list
    p_x: list                 # p_i(x_i), i < k
    q_x: list                 # q_i(x_i), i < k
    theta: list               # acceptance thresholds, i < k
    margins: list             # |u_i - theta_i| for the examined positions
    t: int
    final_w: np.ndarray = field(repr=False, default=None)
    final_C: np.ndarray = field(repr=False, default=None)
    final_W: float = 0.0
    final_u: float = 0.0
    margin_final: float = 0.0
    near_tie: bool = False
    residual_fallback: bool = False


def final_draw(p_a, q_a, rejected: bool, u_final: float):
    """Token of the last committed position: inverse CDF of the residual
    (after a rejection) or of p_k (bonus)."""
    w, fb = final_weights(p_a, q_a, rejected)
    t, C, W = inverse_cdf(w, u_final)
    lo = (C[t - 1] if t > 0 else 0.0) / W
    hi = C[t] / W
    return t, w, C, W, min(u_final - lo, hi - u_final), fb


def match_request(p_rows, drafts, u) -> SampledRecord:
    """Prefix-match verify of argmax drafts: y_j = inverse_cdf(p_j, u_j) for
    every row j (each row's own uniform), a = the first j < k with y_j != x_j
    (k if none), committed tokens x_0..x_{a-1}, y_a.

    The record uses the fields of a sampled record: margins[j] is the distance
    of u_j from the nearest end of x_j's interval [C_{x-1}/W, C_x/W) (the
    boundary that decides the match), the final fields describe row a's draw.
    p_x are p_j(x_j); q_x are 1 (a one-hot draft)."""
    k = len(drafts)
    xs = [int(d) for d in drafts]
    margins = []
    a = k
    for j in range(k):
        y, C, W = inverse_cdf(p_rows[j], float(u[j]))     # the row's own sample
        lo = (C[xs[j] - 1] if xs[j] > 0 else 0.0) / W
        hi = C[xs[j]] / W
        uj = float(u[j])
        margins.append(min(abs(uj - lo), abs(hi - uj)))
        if y != xs[j]:
            a = j
            break
    t, C, W = inverse_cdf(p_rows[a], float(u[a]))
    lo = (C[t - 1] if t > 0 else 0.0) / W
    hi = C[t] / W
    p_x = [float(p_rows[i][xs[i]]) for i in range(k)]
    return SampledRecord(a=a, tokens=xs[:a] + [t], p_x=p_x, q_x=[1.0] * k,
                         theta=p_x, margins=margins, t=t, final_w=p_rows[a], final_C=C,
                         final_W=W, final_u=float(u[a]),
                         margin_final=min(float(u[a]) - lo, hi - float(u[a])))


def sampled_request(p_rows, q_rows, drafts, u) -> SampledRecord:
    """One sampled request given its processed target rows p_0..p_k, draft
    rows q_0..q_{k-1} (float64 arrays or lazy row accessors), drafts
    x_0..x_{k-1} and uniforms u_0..u_k (u_k is the final draw)."""
    k = len(drafts)
    xs = [int(d) for d in drafts]
    p_x = [float(p_rows[i][xs[i]]) for i in range(k)]
    q_x = [float(q_rows[i][xs[i]]) for i in range(k)]
    a, theta, margins = accept_scan(p_x, q_x, u)
    rejected = a < k
    t, w, C, W, mf, fb = final_draw(p_rows[a], q_rows[a] if rejected else None, rejected,
                                    float(u[k]))
    return SampledRecord(a=a, tokens=xs[:a] + [t], p_x=p_x, q_x=q_x, theta=theta,
                         margins=margins, t=t, final_w=w, final_C=C, final_W=W,
                         final_u=float(u[k]), margin_final=mf, residual_fallback=fb)


# --------------------------------------------------------------------------
# batch driver with the boundary's packing and status conventions
# --------------------------------------------------------------------------
ROW_BAD_PARAM = 5
FLT_MIN = float(np.finfo(np.float32).tiny)


def is_greedy_temperature(T: float) -> bool:
    """A request is greedy unless its temperature is a normal positive float
    (T <= 0, NaN and subnormal temperatures are greedy)."""
    return not (T >= FLT_MIN)


def _nonfinite(row: np.ndarray) -> bool:
    return bool(np.any(np.isnan(row)) or np.any(row == np.inf))


def _bad_prob(v) -> bool:
    v = np.asarray(v, dtype=np.float64)
    return bool(np.any(~np.isfinite(v)) or np.any(v < 0))


@dataclass
class BatchResult:
    status: np.ndarray
    accepted: np.ndarray
    out_tokens: np.ndarray
    p_at_draft: np.ndarray
    q_at_draft: np.ndarray
    records: list            # per request: SampledRecord, ("greedy", g) or None


def request_bounds(cu, b: int, batch: int, total_rows: int, max_k: int):
    """(k, valid) of request b from the cu_seqlens offsets: the request owns
    target rows cu[b]..cu[b+1]-1 and draft rows cu[b]-b .. cu[b+1]-b-2.

    Offsets must be non-decreasing: a request is invalid when its first target
    row cu[b] is below an earlier request's, or its first draft row cu[b]-b is
    below an earlier request's cu[e]-e (after a request with no rows, or with
    offsets that go back, the draft rows that follow would reach back into an
    earlier request's).  So neither the target rows nor the draft rows of
    valid requests overlap."""
    c0, c1 = int(cu[b]), int(cu[b + 1])
    k = c1 - c0 - 1
    ok = (c0 >= 0 and c1 <= total_rows and 0 <= k <= max_k
          and c0 - b >= 0 and c0 - b + k <= total_rows - batch
          and all(c0 >= int(cu[e]) for e in range(b))
          and all(c0 - b >= int(cu[e]) - e for e in range(b)))
    return k, ok


class _OneHotRows:
    """q_i = e_{x_i} for a one-hot (argmax) draft."""

    def __init__(self, xs, V):
        self.xs, self.V = xs, V

    def __getitem__(self, i):
        q = np.zeros(self.V, dtype=np.float64)
        q[int(self.xs[i])] = 1.0
        return q


class _ProbRows:
    """Supplied draft probability rows, widened on access, used as they are."""

    def __init__(self, draft, d0, V, dtype):
        self.draft, self.d0, self.V, self.dtype = draft, d0, V, dtype

    def __getitem__(self, i):
        return widen(self.draft[self.d0 + i, :self.V], self.dtype)


def _history(hist_offsets, hist_tokens, hist_counts, b: int):
    """Request b's (tokens, counts) from the CSR history, empty when its
    offsets are out of order or out of range."""
    if hist_offsets is None:
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    off = np.asarray(hist_offsets, dtype=np.int64)
    nnz = int(np.asarray(hist_tokens).shape[0])
    h0, h1 = int(off[b]), int(off[b + 1])
    if not (0 <= h0 <= h1 <= nnz):
        return np.zeros(0, np.int64), np.zeros(0, np.int64)
    return (np.asarray(hist_tokens, dtype=np.int64)[h0:h1],
            np.asarray(hist_counts, dtype=np.int64)[h0:h1])


def verify(target, target_dtype, cu_seqlens, draft_tokens, uniforms=None, temperature=None,
           draft=None, draft_dtype=F32, draft_kind=None, top_k=None, top_p=None,
           vocab=None, max_k=63, greedy_entry=False, keep_cdf=True, presence=None,
           frequency=None, hist_offsets=None, hist_tokens=None,
           hist_counts=None) -> BatchResult:
    """Whole-batch verify with the boundary's packing.

    target:  [total_rows, ld] stored values (uint16 bf16 bits or float32)
    draft:   [total_rows - batch, ld] or None
    Request b owns target rows cu[b]..cu[b]+k_b, draft rows and draft tokens
    cu[b]-b .. cu[b]-b+k_b-1, and uniforms u[cu[b]+i] (i < k_b: acceptance
    draws; i = k_b: the final draw).

    presence, frequency ([batch] or None) and the CSR history
    (hist_offsets [batch + 1], hist_tokens / hist_counts [nnz]) give the
    penalties of ``penalize``; a request with both penalties 0 is left alone.

    Status per request, first match wins: BAD_K (offsets out of range or
    k_b > max_k), BAD_PARAM (unknown draft kind, a kind that needs draft rows
    with no draft buffer, an infinite temperature, or a non-finite penalty),
    BAD_TOKEN (a draft id
    outside [0, V)), NONFINITE (NaN or +inf in a needed logit row; NaN, inf
    or a negative value in a needed probability), EMPTY (a needed logit row
    with no finite value).  A request with a non-OK status gets accepted = -1,
    out_tokens = -1 and NaN probabilities; BAD_K requests leave out_tokens
    untouched.
    """
    target = np.asarray(target)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    batch = cu.shape[0] - 1
    total_rows = int(target.shape[0])
    V = int(vocab if vocab is not None else target.shape[1])
    n_draft = total_rows - batch
    status = np.zeros(batch, dtype=np.int32)
    accepted = np.full(batch, -1, dtype=np.int32)
    out_tokens = np.full(total_rows, -1, dtype=np.int32)
    p_at = np.full(max(n_draft, 0), np.nan, dtype=np.float32)
    q_at = np.full(max(n_draft, 0), np.nan, dtype=np.float32)
    records = [None] * batch
    dt = np.asarray(draft_tokens)

    for b in range(batch):
        k, ok = request_bounds(cu, b, batch, total_rows, max_k)
        if not ok:
            status[b] = ROW_BAD_K
            continue
        c0 = int(cu[b])
        d0 = c0 - b
        T = 0.0 if greedy_entry else float(np.float32(temperature[b]))
        greedy = greedy_entry or is_greedy_temperature(T)
        kind = None if greedy else int(draft_kind[b])

        a_p = float(np.float32(presence[b])) if presence is not None else 0.0
        a_f = float(np.float32(frequency[b])) if frequency is not None else 0.0
        pen = a_p != 0.0 or a_f != 0.0
        if pen and not (np.isfinite(a_p) and np.isfinite(a_f)):
            status[b] = ROW_BAD_PARAM
            continue
        if not greedy and (T == np.inf or kind not in (ONEHOT, LOGITS, PROBS, MATCH)
                           or (kind in (LOGITS, PROBS) and draft is None)):
            status[b] = ROW_BAD_PARAM
            continue
        xs = dt[d0:d0 + k].astype(np.int64)
        if np.any((xs < 0) | (xs >= V)):
            status[b] = ROW_BAD_TOKEN
            continue

        rows = [widen(target[c0 + j, :V], target_dtype) for j in range(k + 1)]
        if pen:
            ht, hc = _history(hist_offsets, hist_tokens, hist_counts, b)
            rows = [penalize(rows[j], target_dtype, ht, hc, xs[:j], a_p, a_f)
                    for j in range(k + 1)]
        drows = None
        if kind == LOGITS:
            drows = [widen(np.asarray(draft)[d0 + j, :V], draft_dtype) for j in range(k)]
        need = rows + (drows if drows is not None else [])
        if any(_nonfinite(r) for r in need):
            status[b] = ROW_NONFINITE
            continue
        if kind == PROBS and k > 0:
            gathered = [widen(np.asarray(draft)[d0 + i, int(xs[i]):int(xs[i]) + 1],
                              draft_dtype)[0] for i in range(k)]
            if _bad_prob(gathered):
                status[b] = ROW_NONFINITE
                continue
        if any(not np.any(r > -np.inf) for r in need):
            status[b] = ROW_EMPTY
            continue

        if greedy:
            a, tokens, g = greedy_request(np.stack(rows), xs)
            records[b] = ("greedy", g)
            accepted[b] = a
            out_tokens[c0:c0 + a + 1] = tokens
            for i in range(k):
                p_at[d0 + i] = 1.0 if int(xs[i]) == g[i] else 0.0
                q_at[d0 + i] = 1.0
            continue

        K = int(top_k[b]) if top_k is not None else 0
        P = float(np.float32(top_p[b])) if top_p is not None else 1.0
        pd = [process(r, T, K, P) for r in rows]
        p_rows = [d.p for d in pd]
        near = any(d.near_tie for d in pd)
        if kind == LOGITS:
            qd = [process(r, T, K, P) for r in drows]
            q_rows = [d.p for d in qd]
            near = near or any(d.near_tie for d in qd)
        elif kind == PROBS:
            q_rows = _ProbRows(np.asarray(draft), d0, V, draft_dtype)
        else:
            q_rows = _OneHotRows(xs, V)

        u = np.asarray(uniforms, dtype=np.float32)[c0:c0 + k + 1].astype(np.float64)
        if kind == MATCH:
            rec = match_request(p_rows, xs, u)
            rec.near_tie = near
            if not keep_cdf:
                rec.final_w = rec.final_C = None
            records[b] = rec
            accepted[b] = rec.a
            out_tokens[c0:c0 + rec.a + 1] = rec.tokens
            for i in range(k):
                p_at[d0 + i] = np.float32(rec.p_x[i])
                q_at[d0 + i] = np.float32(1.0)
            continue
        p_x = [float(p_rows[i][int(xs[i])]) for i in range(k)]
        q_x = [float(q_rows[i][int(xs[i])]) for i in range(k)]
        a, theta, margins = accept_scan(p_x, q_x, u)
        rejected = a < k
        q_a = q_rows[a] if rejected else None
        if kind == PROBS and rejected and _bad_prob(q_a):
            status[b] = ROW_NONFINITE
            continue
        t, w, C, W, mf, fb = final_draw(p_rows[a], q_a, rejected, float(u[k]))
        rec = SampledRecord(a=a, tokens=[int(x) for x in xs[:a]] + [t], p_x=p_x, q_x=q_x,
                            theta=theta, margins=margins, t=t,
                            final_w=w if keep_cdf else None, final_C=C if keep_cdf else None,
                            final_W=W, final_u=float(u[k]), margin_final=mf, near_tie=near,
                            residual_fallback=fb)
        records[b] = rec
        accepted[b] = a
        out_tokens[c0:c0 + a + 1] = rec.tokens
        for i in range(k):
            p_at[d0 + i] = np.float32(p_x[i])
            q_at[d0 + i] = np.float32(q_x[i])

    for b in range(batch):
        if status[b] not in (ROW_OK, ROW_BAD_K):
            k, _ = request_bounds(cu, b, batch, total_rows, max_k)
            out_tokens[int(cu[b]):int(cu[b]) + k + 1] = -1
    return BatchResult(status, accepted, out_tokens, p_at, q_at, records)


# --------------------------------------------------------------------------
# after the verify: drain (commit) and acceptance accounting
# --------------------------------------------------------------------------
def drain(cu_seqlens, accepted, status, out_tokens, max_k=63):
    """Commit the verified tokens of a batch and give back the unused slots.

    Page "FreeToken PR #836", section "Design", drain row: commit
    n = accepted + 1 tokens and roll back the unused slots of the k+1 verify
    rows; the catalog page "Adding Speculative Decoding", "The four high-risk
    coupling points" item 1 (accept all / some / none).

    Per request b with k_b = cu[b+1] - cu[b] - 1 and a_b = accepted[b]:
      n_b = a_b + 1 when status[b] is OK and 0 <= a_b <= k_b, else 0;
      rollback_b = k_b + 1 - n_b, or 0 for a request whose offsets the verify
      rejected (BAD_K: its slots are not known) or whose rows do not lie inside
      the token buffer (the verify never reports such a request OK);
      offsets = exclusive running sum of n; committed[offsets[b] + i] =
      out_tokens[cu[b] + i] for i < n_b.
    Returns (committed [offsets[-1]], offsets [B+1], rollback [B]), int32."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    B = cu.shape[0] - 1
    acc = np.asarray(accepted, dtype=np.int64)
    st = np.asarray(status, dtype=np.int64)
    toks = np.asarray(out_tokens, dtype=np.int64)
    n = np.zeros(B, dtype=np.int64)
    rollback = np.zeros(B, dtype=np.int64)
    for b in range(B):
        if st[b] == ROW_BAD_K or not (0 <= cu[b] < cu[b + 1] <= toks.shape[0]):
            continue
        k = int(cu[b + 1] - cu[b] - 1)
        if st[b] == ROW_OK and 0 <= acc[b] <= k:
            n[b] = acc[b] + 1
        rollback[b] = k + 1 - n[b]
    offsets = np.zeros(B + 1, dtype=np.int64)
    for b in range(B):
        offsets[b + 1] = offsets[b] + n[b]
    committed = np.zeros(int(offsets[-1]), dtype=np.int64)
    for b in range(B):
        for i in range(int(n[b])):
            committed[offsets[b] + i] = toks[cu[b] + i]
    return committed.astype(np.int32), offsets.astype(np.int32), rollback.astype(np.int32)


def accounting(cu_seqlens, accepted, status, ema, beta, threshold, k_low, k_high, counters):
    """Acceptance accounting of one verify step and the next lookahead.

    Counters (the Rust page, section "Production Pitfalls & Mitigation
    Strategies", its metrics snippet): over the requests with status OK,
    tokens generated += a_b + 1, tokens drafted += k_b, tokens accepted +=
    a_b, and requests += 1 (so mean tokens per step = generated / requests,
    acceptance rate = accepted / drafted; the catalog page, Acceptance bars
    item 2).

    Per request, the moving average of the acceptance rate and the adaptive
    lookahead (same Rust page section, item 3: below a threshold such as
    40 %, K drops from 5 to 2, and goes back up when the rate recovers):
      r = a_b / k_b in float32; ema' = ema + beta * (r - ema), float32, in
      that order (requests with k_b = 0 or a status other than OK keep ema);
      k_next = k_low if ema' < threshold else k_high.
    The moving average is float32 state, so it is computed in float32 here,
    the precision in which the lookahead decision is taken.
    Returns (ema' float32 [B], k_next int32 [B], counters int64 [4])."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    B = cu.shape[0] - 1
    acc = np.asarray(accepted, dtype=np.int64)
    st = np.asarray(status, dtype=np.int64)
    ema_out = np.asarray(ema, dtype=np.float32).copy()
    k_next = np.zeros(B, dtype=np.int32)
    cnt = np.asarray(counters, dtype=np.int64).copy()
    f32 = np.float32
    for b in range(B):
        k = int(cu[b + 1] - cu[b] - 1)
        ok = st[b] == ROW_OK and 0 <= acc[b] <= k
        if ok:
            cnt[0] += acc[b] + 1
            cnt[1] += k
            cnt[2] += acc[b]
            cnt[3] += 1
            if k > 0:
                r = f32(f32(acc[b]) / f32(k))
                ema_out[b] = f32(ema_out[b] + f32(f32(beta) * f32(r - ema_out[b])))
        k_next[b] = k_low if ema_out[b] < f32(threshold) else k_high
    return ema_out, k_next, cnt


# --------------------------------------------------------------------------
# closed forms used as pins, and the comparison rule
# --------------------------------------------------------------------------
def expected_tokens_per_step(alpha: float, gamma: int) -> float:
    """E[tokens] = (1 - alpha^(gamma+1)) / (1 - alpha) for i.i.d. acceptance
    (the Draft-Model-Sampling page, Key Topic 4)."""
    if alpha == 1.0:
        return float(gamma + 1)
    return (1.0 - alpha ** (gamma + 1)) / (1.0 - alpha)


def acceptance_rate(p: np.ndarray, q: np.ndarray) -> float:
    """alpha = sum_y min(p_y, q_y), the probability that a draft x ~ q is
    accepted."""
    return float(np.sum(np.minimum(p, q)))


def excusal(rec: SampledRecord, gpu_a: int, gpu_t: int, window: float = NEAR_TIE) -> str:
    """Classify a GPU result against the oracle record: 'match', 'excused'
    or 'fail'.

    A differing accept decision at position i is excused iff
    |u_i - theta_i| < window; a differing final token t' is excused iff u
    lies in the oracle's interval of t' widened by the window and t' has
    positive mass.  A request whose filters hit a top-p near tie is excused
    whenever it differs.  An accepted count outside [0, k] or a token outside
    the vocabulary always fails.
    """
    k = len(rec.p_x)
    if not (0 <= gpu_a <= k) or gpu_t < 0 or (rec.final_w is not None
                                               and gpu_t >= len(rec.final_w)):
        return "fail"          # outside the outputs any correct verify can give
    if gpu_a == rec.a and gpu_t == rec.t:
        return "match"
    if rec.near_tie:
        return "excused"
    if gpu_a != rec.a:
        i = min(gpu_a, rec.a)
        if 0 <= i < len(rec.margins) and rec.margins[i] < window:
            return "excused"
        return "fail"
    w, C, W, u = rec.final_w, rec.final_C, rec.final_W, rec.final_u
    if w is None or gpu_t < 0 or gpu_t >= len(w) or not (w[gpu_t] > 0):
        return "fail"
    lo = (C[gpu_t - 1] if gpu_t > 0 else 0.0) / W
    hi = C[gpu_t] / W
    if lo - window <= u < hi + window:
        return "excused"
    return "fail"


__all__ = [
    "F32", "BF16", "ONEHOT", "LOGITS", "PROBS", "MATCH", "match_request",
    "ROW_OK", "ROW_NONFINITE", "ROW_EMPTY", "ROW_BAD_K", "ROW_BAD_TOKEN", "ROW_BAD_PARAM",
    "ROW_INTERNAL",
    "widen", "process", "Dist", "argmax_lowest", "greedy_request", "accept_threshold",
    "accept_scan", "final_weights", "inverse_cdf", "final_draw", "sampled_request",
    "SampledRecord", "verify", "BatchResult", "request_bounds", "is_greedy_temperature",
    "expected_tokens_per_step", "acceptance_rate", "excusal", "drain", "accounting",
    "penalize", "round_to_dtype",
]
