"""Seeded synthetic verify workloads.

Shared by the tests, the smoke check and the benchmark.  It holds no step of
the verify method itself (no tempered softmax of a verify row, no acceptance
test, no residual, no inverse CDF): it only makes inputs.  Draft tokens are
drawn with the Gumbel-max trick, which samples from a tempered softmax
without computing it; the cached probability rows of the PROBS draft kind are
the drafter's own output and are normalised here as input data.

Recipe (all streams are numpy PCG64 keyed by SeedSequence(entropy, spawn_key=
(config, stream)); the draft-side streams use entropy = seed ^ (1 << 30)):

* target logits  L = 3 N(0,1) - 1.1 ln(1 + rank(y)), rank = one seeded vocab
  permutation per (config, seed), computed in float64 and rounded to the
  storage dtype (bf16 round-to-nearest-even via float32);
* draft logits   D = L_stored + sigma N(0,1), rounded to storage;
* draft tokens   LOGITS: Gumbel-max over D/T restricted to the request's
  top-k set (temperature and top-k; the drafter does not apply top-p);
  PROBS: Gumbel-max over log q; greedy, ONEHOT and MATCH: lowest-index argmax
  of L_stored + sigma N (a noisy copy that is not handed to the verifier);
* uniforms       randint(0, 2^24) * 2^-24 as float32, k_b + 1 per request.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

F32, BF16 = 0, 1
ONEHOT, LOGITS, PROBS, MATCH = 0, 1, 2, 3
DRAFT_SALT = 1 << 30

# stream ids
S_PERM, S_TARGET, S_PARAMS, S_UNIF = 0, 1, 2, 3
S_DNOISE, S_DDRAW, S_GNOISE = 0, 1, 2


def _rng(seed: int, config: int, stream: int, draft: bool = False) -> np.random.Generator:
    entropy = (seed ^ DRAFT_SALT) if draft else seed
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(entropy=entropy, spawn_key=(config, stream))))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64/float32 values to bf16 (nearest, ties to even) and
    return the 16-bit patterns as uint16."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = (bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    out = rounded.astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def store(x: np.ndarray, dtype: int) -> np.ndarray:
    return to_bf16_bits(x) if dtype == BF16 else np.asarray(x, dtype=np.float32)


def stored_f64(a: np.ndarray, dtype: int) -> np.ndarray:
    return bf16_bits_to_f64(a) if dtype == BF16 else np.asarray(a, dtype=np.float64)


@dataclass
class Workload:
    name: str
    config: int
    seed: int
    vocab: int
    target: np.ndarray            # [total_rows, vocab] uint16 (bf16) or float32
    target_dtype: int
    cu_seqlens: np.ndarray        # int32 [B+1]
    draft_tokens: np.ndarray      # int32 [total_rows - B]
    uniforms: np.ndarray          # float32 [total_rows]
    temperature: np.ndarray       # float32 [B]
    draft_kind: np.ndarray        # int32 [B]
    draft: np.ndarray | None = None   # [total_rows - B, vocab]
    draft_dtype: int = F32
    top_k: np.ndarray | None = None   # int32 [B]
    top_p: np.ndarray | None = None   # float32 [B]
    max_k: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def total_rows(self) -> int:
        return int(self.cu_seqlens[-1])

    def greedy_mask(self) -> np.ndarray:
        return ~(self.temperature >= np.finfo(np.float32).tiny)


# ----------------------------------------------------------------------------
# building blocks
# ----------------------------------------------------------------------------
def _target_rows(rng_t: np.random.Generator, log_rank: np.ndarray, n: int) -> np.ndarray:
    """n rows of 3 N(0,1) - 1.1 ln(1 + rank), float64."""
    return 3.0 * rng_t.standard_normal((n, log_rank.shape[0])) - 1.1 * log_rank


def _gumbel_argmax(rng: np.random.Generator, scores: np.ndarray) -> int:
    """Index of max(scores + Gumbel noise): a draw from softmax(scores)."""
    g = rng.gumbel(size=scores.shape[0])
    return int(np.argmax(scores + g))


def _topk_restrict(scores: np.ndarray, K: int) -> np.ndarray:
    """Scores with everything below the K-th largest set to -inf (drafter's
    top-k; ties at the K-th value are kept)."""
    if K <= 0 or K >= scores.shape[0]:
        return scores
    kth = np.partition(scores, scores.shape[0] - K)[scores.shape[0] - K]
    return np.where(scores >= kth, scores, -np.inf)


def _uniforms(rng: np.random.Generator, n: int) -> np.ndarray:
    return (rng.integers(0, 1 << 24, size=n).astype(np.float64) * 2.0 ** -24).astype(np.float32)


def build(config: int, *, seed: int = 0, batch: int, vocab: int, ks, target_dtype: int,
          draft_dtype: int, kinds, temps, sigma, top_k=None, top_p=None, name: str = "",
          replicate_rows: bool = False, probs_sigma: float = 0.8, max_k: int | None = None,
          ld: int | None = None) -> Workload:
    """Assemble a workload from per-request arrays (ks, kinds, temps, sigma)."""
    ks = np.asarray(ks, dtype=np.int64)
    kinds = np.asarray(kinds, dtype=np.int32)
    temps = np.asarray(temps, dtype=np.float32)
    sig = np.broadcast_to(np.asarray(sigma, dtype=np.float64), (batch,))
    cu = np.zeros(batch + 1, dtype=np.int32)
    cu[1:] = np.cumsum(ks + 1)
    total = int(cu[-1])
    n_draft = total - batch
    ld = vocab if ld is None else ld

    perm = _rng(seed, config, S_PERM).permutation(vocab)
    log_rank = np.log1p(perm.astype(np.float64))
    rng_t = _rng(seed, config, S_TARGET)
    rng_u = _rng(seed, config, S_UNIF)
    rng_dn = _rng(seed, config, S_DNOISE, draft=True)
    rng_dd = _rng(seed, config, S_DDRAW, draft=True)
    rng_gn = _rng(seed, config, S_GNOISE, draft=True)

    tdt = np.uint16 if target_dtype == BF16 else np.float32
    target = np.zeros((total, ld), dtype=tdt)
    greedy = ~(temps >= np.finfo(np.float32).tiny)
    need_draft = bool(np.any((kinds == LOGITS) & ~greedy) or np.any((kinds == PROBS) & ~greedy))
    ddt = np.uint16 if draft_dtype == BF16 else np.float32
    draft = np.zeros((max(n_draft, 0), ld), dtype=ddt) if need_draft else None
    draft_tokens = np.zeros(max(n_draft, 0), dtype=np.int32)

    shared_rows = None
    shared_draft = None
    if replicate_rows:
        k0 = int(ks[0])
        shared_rows = store(_target_rows(rng_t, log_rank, k0 + 1), target_dtype)
        if kinds[0] == LOGITS:
            base = stored_f64(shared_rows[:k0], target_dtype)
            shared_draft = store(base + sig[0] * rng_dn.standard_normal(base.shape), draft_dtype)

    for b in range(batch):
        c0, k = int(cu[b]), int(ks[b])
        d0 = c0 - b
        if replicate_rows:
            rows = shared_rows
        else:
            rows = store(_target_rows(rng_t, log_rank, k + 1), target_dtype)
        target[c0:c0 + k + 1, :vocab] = rows
        L = stored_f64(rows, target_dtype)
        T = float(temps[b])
        if greedy[b] or kinds[b] in (ONEHOT, MATCH):
            for i in range(k):
                noisy = L[i] + sig[b] * rng_gn.standard_normal(vocab)
                draft_tokens[d0 + i] = int(np.argmax(noisy))
        elif kinds[b] == LOGITS:
            if replicate_rows:
                D_st = shared_draft
            else:
                D_st = store(L[:k] + sig[b] * rng_dn.standard_normal((k, vocab)), draft_dtype)
            draft[d0:d0 + k, :vocab] = D_st
            D = stored_f64(D_st, draft_dtype)
            K = int(top_k[b]) if top_k is not None else 0
            for i in range(k):
                scores = _topk_restrict(D[i] / T, K)
                draft_tokens[d0 + i] = _gumbel_argmax(rng_dd, scores)
        elif kinds[b] == PROBS:
            for i in range(k):
                d = L[i] + probs_sigma * rng_dn.standard_normal(vocab)
                e = np.exp(d - d.max())
                q = (e / e.sum()).astype(np.float32)
                draft[d0 + i, :vocab] = q if draft_dtype == F32 else to_bf16_bits(q)
                with np.errstate(divide="ignore"):
                    lq = np.log(stored_f64(draft[d0 + i, :vocab], draft_dtype))
                draft_tokens[d0 + i] = _gumbel_argmax(rng_dd, lq)
    uniforms = _uniforms(rng_u, total)
    return Workload(name=name or f"config{config}", config=config, seed=seed, vocab=vocab,
                    target=target, target_dtype=target_dtype, cu_seqlens=cu,
                    draft_tokens=draft_tokens, uniforms=uniforms, temperature=temps,
                    draft_kind=kinds, draft=draft, draft_dtype=draft_dtype,
                    top_k=None if top_k is None else np.asarray(top_k, dtype=np.int32),
                    top_p=None if top_p is None else np.asarray(top_p, dtype=np.float32),
                    max_k=int(ks.max()) if max_k is None else max_k,
                    meta={"sigma": sig.tolist() if batch <= 8 else float(sig.mean())})


# ----------------------------------------------------------------------------
# the five workload families
# ----------------------------------------------------------------------------
def config0(seed: int = 0, trials: int = 1000) -> Workload:
    """Tiny CPU-checkable verify: k=4, V=1024, fp32 logits, LOGITS drafts with
    sigma 0.5, T=1, no filters.  One request's logits replicated over
    `trials` requests, each with fresh draft draws and uniforms."""
    B = trials
    return build(0, seed=seed, batch=B, vocab=1024, ks=np.full(B, 4), target_dtype=F32,
                 draft_dtype=F32, kinds=np.full(B, LOGITS), temps=np.ones(B), sigma=0.5,
                 replicate_rows=True, name=f"B={B}x(k=4) V=1024 f32 LOGITS")


def config1(seed: int = 0, batch: int = 32, vocab: int = 32000) -> Workload:
    """B=32, k=5, V=32000, fp32 target and draft logits, sigma 0.7, T=0.8."""
    B = batch
    return build(1, seed=seed, batch=B, vocab=vocab, ks=np.full(B, 5), target_dtype=F32,
                 draft_dtype=F32, kinds=np.full(B, LOGITS), temps=np.full(B, 0.8), sigma=0.7,
                 name=f"B={B} k=5 V={vocab} f32 LOGITS T=0.8")


def config2(seed: int = 0, batch: int = 64, vocab: int = 128256) -> Workload:
    """B=64, k=6, V=128256, bf16.  A seeded shuffle makes half the requests
    greedy (T=0) and the rest sampled at T ~ U[0.5, 1.2]; half the sampled
    ones use one-hot argmax drafts and half draft logits with sigma 0.5."""
    B = batch
    rng = _rng(seed, 2, S_PARAMS)
    roles = np.array([0] * (B // 2) + [1] * (B // 4) + [2] * (B - B // 2 - B // 4))
    rng.shuffle(roles)
    temps = np.where(roles == 0, 0.0, rng.uniform(0.5, 1.2, size=B)).astype(np.float32)
    kinds = np.where(roles == 2, LOGITS, ONEHOT).astype(np.int32)
    return build(2, seed=seed, batch=B, vocab=vocab, ks=np.full(B, 6), target_dtype=BF16,
                 draft_dtype=BF16, kinds=kinds, temps=temps, sigma=0.5,
                 name=f"B={B} k=6 V={vocab} bf16 mixed greedy/onehot/logits")


def config3(seed: int = 0, batch: int = 256, vocab: int = 128256) -> Workload:
    """Varlen: k_b ~ U{1..8} packed by cu_seqlens, V=128256 bf16, per-request
    top-k in {0, 20, 50}, top-p in {1.0, 0.9, 0.95}, T ~ U[0.3, 1.2],
    LOGITS drafts with sigma 0.6."""
    B = batch
    rng = _rng(seed, 3, S_PARAMS)
    ks = rng.integers(1, 9, size=B)
    top_k = rng.choice(np.array([0, 20, 50]), size=B).astype(np.int32)
    top_p = rng.choice(np.array([1.0, 0.9, 0.95]), size=B).astype(np.float32)
    temps = rng.uniform(0.3, 1.2, size=B).astype(np.float32)
    return build(3, seed=seed, batch=B, vocab=vocab, ks=ks, target_dtype=BF16,
                 draft_dtype=BF16, kinds=np.full(B, LOGITS), temps=temps, sigma=0.6,
                 top_k=top_k, top_p=top_p, max_k=8,
                 name=f"B={B} varlen k in 1..8 V={vocab} bf16 top-k/top-p")


def config4(seed: int = 0, batch: int = 512, vocab: int = 152064) -> Workload:
    """B=512, k=5, V=152064: bf16 target, cached fp32 draft probabilities
    (softmax of target + 0.8 N), all sampled at T=1, bonus drawn when every
    draft is accepted."""
    B = batch
    return build(4, seed=seed, batch=B, vocab=vocab, ks=np.full(B, 5), target_dtype=BF16,
                 draft_dtype=F32, kinds=np.full(B, PROBS), temps=np.ones(B), sigma=0.8,
                 probs_sigma=0.8, name=f"B={B} k=5 V={vocab} bf16 target, f32 PROBS")


CONFIGS = {0: config0, 1: config1, 2: config2, 3: config3, 4: config4}


def make(config: int, seed: int = 0, **kw) -> Workload:
    return CONFIGS[config](seed=seed, **kw)


def algorithmic_bytes(w: Workload, accepted: np.ndarray | None = None) -> int:
    """First-touch bytes one verify call must move.

    Target: every row, V elements.  Draft: LOGITS rows in full; PROBS one
    gathered value per draft plus the whole row at the rejection position
    (needs `accepted`); ONEHOT and greedy nothing.  Small arrays: per row the
    draft id, the uniform and the output token (4 B each), per request
    cu_seqlens, kind, temperature, filters, accepted and status (~24 B).
    """
    tsz = 2 if w.target_dtype == BF16 else 4
    dsz = 2 if w.draft_dtype == BF16 else 4
    total = 0
    greedy = w.greedy_mask()
    cu = w.cu_seqlens
    for b in range(w.batch):
        k = int(cu[b + 1] - cu[b] - 1)
        total += (k + 1) * w.vocab * tsz
        if greedy[b]:
            continue
        if w.draft_kind[b] == LOGITS:
            total += k * w.vocab * dsz
        elif w.draft_kind[b] == PROBS:
            total += k * dsz
            if accepted is not None and 0 <= accepted[b] < k:
                total += w.vocab * dsz
    total += 12 * w.total_rows + 24 * w.batch
    return int(total)


@dataclass
class PenaltyInputs:
    """Presence / frequency penalties of a batch and its generated-token
    counts (CSR: request b owns entries offsets[b]..offsets[b+1])."""
    presence: np.ndarray      # float32 [batch]
    frequency: np.ndarray     # float32 [batch]
    offsets: np.ndarray       # int32 [batch + 1]
    tokens: np.ndarray        # int32 [nnz], unique within a request
    counts: np.ndarray        # int32 [nnz]


def penalties(w: Workload, seed: int = 0, share: float = 0.75, hist_len=(0, 200),
              max_count: int = 5, from_drafts: float = 0.3) -> PenaltyInputs:
    """Seeded penalty inputs for workload w: a `share` of the requests get
    nonzero penalties (multiples of 1/16 in [-0.5, 2], exact in bf16 and fp32);
    each request's history holds a random number of distinct tokens in
    `hist_len`, some of them (`from_drafts`) taken from its own drafts, with
    counts in [0, max_count]."""
    rng = np.random.default_rng([seed, w.config, 77])
    B, V = w.batch, w.vocab
    on = rng.random(B) < share
    grid = np.arange(-8, 33) / 16.0
    presence = np.where(on, rng.choice(grid, size=B), 0.0).astype(np.float32)
    frequency = np.where(on, rng.choice(grid, size=B), 0.0).astype(np.float32)
    cu = w.cu_seqlens
    offsets = np.zeros(B + 1, dtype=np.int32)
    toks, cnts = [], []
    for b in range(B):
        n = int(rng.integers(hist_len[0], hist_len[1] + 1))
        d0, k = int(cu[b]) - b, int(cu[b + 1] - cu[b] - 1)
        own = np.asarray(w.draft_tokens[d0:d0 + k], dtype=np.int64)
        pick = own[rng.random(own.shape[0]) < from_drafts] if own.size else own
        rest = rng.choice(V, size=min(n, V), replace=False)
        t = np.unique(np.concatenate([pick, rest]).astype(np.int64))[:max(n, pick.size)]
        t = rng.permutation(t)
        toks.append(t)
        cnts.append(rng.integers(0, max_count + 1, size=t.size))
        offsets[b + 1] = offsets[b] + t.size
    return PenaltyInputs(presence, frequency, offsets,
                         np.concatenate(toks).astype(np.int32) if toks else np.zeros(0, np.int32),
                         np.concatenate(cnts).astype(np.int32) if cnts else np.zeros(0, np.int32))
