"""GPU-vs-oracle comparison under the acceptance bar of the verify:

* greedy requests: accepted counts and tokens identical, bit for bit;
* sampled requests: identical, except a differing accept decision whose
  uniform lies within 1e-6 of its threshold, a differing final token whose
  uniform lies within 1e-6 of the oracle's CDF interval of that token, or a
  request whose top-p cut is a near tie (all counted as excused);
* status codes identical; p(x), q(x) within 1e-5 relative (+1e-30 absolute).
"""

from __future__ import annotations

import numpy as np

import oracle

REL = 1e-5
ABS = 1e-30

# comparison counts of every GPU check in this session, printed at its end
SESSION_COUNTS: list = []


def record_counts(label: str, counts: dict) -> None:
    SESSION_COUNTS.append((label, dict(counts)))


def run_oracle(w, greedy_entry=False, keep_cdf=True):
    return oracle.verify(w.target, w.target_dtype, w.cu_seqlens, w.draft_tokens,
                         uniforms=w.uniforms, temperature=w.temperature, draft=w.draft,
                         draft_dtype=w.draft_dtype, draft_kind=w.draft_kind, top_k=w.top_k,
                         top_p=w.top_p, vocab=w.vocab, max_k=w.max_k,
                         greedy_entry=greedy_entry, keep_cdf=keep_cdf)


def compare(w, gpu: dict, ora, requests=None, greedy_entry=False, check_probs=True) -> dict:
    """gpu: numpy arrays accepted, out_tokens, status (+ p_at, q_at).
    `ora` may be computed on a sub-batch: `requests` then lists the original
    request ids of its requests, in order.  Raises AssertionError on failure."""
    cu = np.asarray(w.cu_seqlens, dtype=np.int64)
    B = cu.shape[0] - 1
    reqs = list(range(B)) if requests is None else list(requests)
    counts = {"match": 0, "excused_accept": 0, "excused_final": 0, "excused_near_tie": 0,
              "greedy": 0, "status": 0}
    fails = []
    total_rows = int(np.asarray(w.target).shape[0])
    for ob, b in enumerate(reqs):
        # offsets of request b in the oracle's (sub-)batch
        k, ok = oracle.request_bounds(cu, b, B, total_rows, w.max_k)
        if requests is None:
            oc0 = int(cu[b]) if ok else 0
        else:
            oc0 = int(sum(int(cu[r + 1] - cu[r]) for r in reqs[:ob]))
        st_o = int(ora.status[ob])
        st_g = int(gpu["status"][b])
        if st_o != st_g:
            fails.append((b, "status", st_o, st_g))
            continue
        if st_o != oracle.ROW_OK:
            counts["status"] += 1
            if gpu["accepted"][b] != -1:
                fails.append((b, "accepted on fault", int(gpu["accepted"][b])))
            if st_o != oracle.ROW_BAD_K:
                seg = gpu["out_tokens"][cu[b]:cu[b] + k + 1]
                if np.any(seg != -1):
                    fails.append((b, "tokens on fault", seg.tolist()))
            continue
        c0 = int(cu[b])
        d0 = c0 - b
        od0 = oc0 - ob
        ga = int(gpu["accepted"][b])
        gseg = np.asarray(gpu["out_tokens"][c0:c0 + k + 1])
        oseg = np.asarray(ora.out_tokens[oc0:oc0 + k + 1])
        rec = ora.records[ob]
        if isinstance(rec, tuple):            # greedy
            counts["greedy"] += 1
            if ga != int(ora.accepted[ob]) or not np.array_equal(gseg, oseg):
                fails.append((b, "greedy", int(ora.accepted[ob]), ga, oseg.tolist(), gseg.tolist()))
        else:
            if not (0 <= ga <= k):
                fails.append((b, "accepted range", ga))
                continue
            gt = int(gseg[ga])
            verdict = oracle.excusal(rec, ga, gt)
            drafts = np.asarray(w.draft_tokens[d0:d0 + k])
            valid = (np.array_equal(gseg[:ga], drafts[:ga]) and np.all(gseg[ga + 1:] == -1)
                     and 0 <= gt < w.vocab)
            if not valid:
                fails.append((b, "layout", gseg.tolist()))
            elif verdict == "match":
                counts["match"] += 1
                if not np.array_equal(gseg, oseg):
                    fails.append((b, "tokens", oseg.tolist(), gseg.tolist()))
            elif verdict == "excused":
                if rec.near_tie:
                    counts["excused_near_tie"] += 1
                elif ga != rec.a:
                    counts["excused_accept"] += 1
                else:
                    counts["excused_final"] += 1
            else:
                fails.append((b, "sampled", (rec.a, rec.t), (ga, gt),
                              rec.margins, rec.margin_final))
        if check_probs and gpu.get("p_at") is not None and k > 0:
            gp = np.asarray(gpu["p_at"][d0:d0 + k], dtype=np.float64)
            gq = np.asarray(gpu["q_at"][d0:d0 + k], dtype=np.float64)
            if isinstance(rec, tuple):
                rp = np.asarray(ora.p_at_draft[od0:od0 + k], dtype=np.float64)
                rq = np.asarray(ora.q_at_draft[od0:od0 + k], dtype=np.float64)
            else:
                rp = np.asarray(rec.p_x)
                rq = np.asarray(rec.q_x)
            for name, g, r in (("p", gp, rp), ("q", gq, rq)):
                if not np.all(np.abs(g - r) <= REL * np.abs(r) + ABS):
                    fails.append((b, f"{name}_at_draft", r.tolist(), g.tolist()))
    if fails:
        msg = "\n".join(repr(f) for f in fails[:20])
        raise AssertionError(f"{len(fails)} parity failures (counts {counts}):\n{msg}")
    return counts


def to_numpy(res) -> dict:
    accepted, tokens, status = res[0], res[1], res[2]
    out = {"accepted": accepted.cpu().numpy(), "out_tokens": tokens.cpu().numpy(),
           "status": status.cpu().numpy()}
    if len(res) > 3 and res[3] is not None:
        out["p_at"] = res[3].cpu().numpy()
        out["q_at"] = res[4].cpu().numpy()
    return out


def sub_workload(w, reqs):
    """The requests `reqs` of w as a workload of their own (same order)."""
    import copy
    cu = np.asarray(w.cu_seqlens, dtype=np.int64)
    rows, drows, ks = [], [], []
    for b in reqs:
        c0, c1 = int(cu[b]), int(cu[b + 1])
        rows.extend(range(c0, c1))
        drows.extend(range(c0 - b, c1 - b - 1))
        ks.append(c1 - c0 - 1)
    s = copy.copy(w)
    s.target = w.target[rows]
    s.draft = None if w.draft is None else w.draft[drows]
    s.draft_tokens = w.draft_tokens[drows]
    s.uniforms = w.uniforms[rows]
    s.temperature = w.temperature[reqs]
    s.draft_kind = w.draft_kind[reqs]
    s.top_k = None if w.top_k is None else w.top_k[reqs]
    s.top_p = None if w.top_p is None else w.top_p[reqs]
    s.cu_seqlens = np.concatenate([[0], np.cumsum(np.array(ks) + 1)]).astype(np.int32)
    return s
