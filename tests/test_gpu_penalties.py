"""GPU parity of the penalized verify (spec_verify_sampled_penalized) with the
oracle: presence and frequency penalties per verify row, the drafts before a
row counted as already generated (FreeToken PR #836, section "Design").  Same
bar as the other parity tests (parity_util): greedy requests bit-exact,
sampled ones identical except near a boundary, p(x) / q(x) within 1e-5."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from lossless_rejection_sampling_spec_amd import binding, synth  # noqa: E402
from parity_util import compare, record_counts, to_numpy  # noqa: E402
from test_gpu_parity import say  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    binding.lib()
    yield


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=DEV, dtype=dtype)


def gpu_penalized(w, pen, plain=False):
    t = binding.workload_tensors(w, DEV)
    kw = {}
    if not plain:
        kw = dict(presence=_dev(pen.presence, torch.float32),
                  frequency=_dev(pen.frequency, torch.float32),
                  history=(_dev(pen.offsets, torch.int32), _dev(pen.tokens, torch.int32),
                           _dev(pen.counts, torch.int32)) if pen.tokens.size else None)
    res = binding.verify_sampled(t["target"], t["draft"], t["draft_kind"], t["cu_seqlens"],
                                 t["draft_tokens"], t["uniforms"], t["temperature"],
                                 t["top_k"], t["top_p"], max_k=w.max_k, vocab=w.vocab,
                                 want_probs=True, **kw)
    torch.cuda.synchronize()
    return to_numpy(res)


def oracle_penalized(w, pen):
    return oracle.verify(w.target, w.target_dtype, w.cu_seqlens, w.draft_tokens,
                         uniforms=w.uniforms, temperature=w.temperature, draft=w.draft,
                         draft_dtype=w.draft_dtype, draft_kind=w.draft_kind, top_k=w.top_k,
                         top_p=w.top_p, vocab=w.vocab, max_k=w.max_k, presence=pen.presence,
                         frequency=pen.frequency, hist_offsets=pen.offsets,
                         hist_tokens=pen.tokens, hist_counts=pen.counts)


def check(w, pen, label):
    say(f"penalties {label}: B={w.batch} V={w.vocab} max_k={w.max_k} "
        f"penalized={int(np.sum((pen.presence != 0) | (pen.frequency != 0)))} "
        f"history={pen.tokens.size}")
    gpu = gpu_penalized(w, pen)
    counts = compare(w, gpu, oracle_penalized(w, pen))
    say(f"  {counts}")
    record_counts(f"penalties {label}", counts)
    return gpu


@pytest.mark.parametrize("cfg,dtype", [(2, synth.BF16), (3, synth.BF16), (1, synth.F32)])
def test_penalized_batches(cfg, dtype):
    """Greedy, one-hot, draft-logit and probability requests (configs 1-3
    reduced to a few chunks and a ragged tail), three quarters of them with
    penalties and histories that share tokens with their drafts."""
    for seed in (0, 1):
        w = synth.make(cfg, seed=seed, batch=24, vocab=9000 + 37 * seed)
        assert w.target_dtype == dtype
        check(w, synth.penalties(w, seed=seed), f"config {cfg} seed {seed}")


def test_penalized_prefix_match_and_probability_drafts():
    w = synth.make(4, seed=3, batch=16, vocab=12000)
    check(w, synth.penalties(w, seed=3, hist_len=(50, 400)), "config 4 reduced")
    w = synth.make(2, seed=5, batch=24, vocab=9000)
    w.draft_kind[:] = np.where(w.draft_kind == synth.ONEHOT, synth.MATCH, w.draft_kind)
    check(w, synth.penalties(w, seed=5), "config 2 with prefix-match drafts")


def test_penalized_full_size_headline_workload():
    w = synth.make(2, seed=0)
    check(w, synth.penalties(w, seed=9, hist_len=(100, 1000)), "config 2 full size")


def test_zero_penalties_equal_the_plain_entry_bitwise():
    w = synth.make(3, seed=2, batch=24, vocab=20000)
    pen = synth.penalties(w, seed=2, share=0.0)
    a = gpu_penalized(w, pen)
    b = gpu_penalized(w, pen, plain=True)
    for key in ("accepted", "out_tokens", "status", "p_at", "q_at"):
        np.testing.assert_array_equal(a[key], b[key])


def test_penalized_is_deterministic():
    w = synth.make(2, seed=4, batch=32, vocab=30000)
    pen = synth.penalties(w, seed=4)
    a = gpu_penalized(w, pen)
    b = gpu_penalized(w, pen)
    for key in ("accepted", "out_tokens", "status", "p_at", "q_at"):
        np.testing.assert_array_equal(a[key], b[key])


def test_penalty_edges():
    """Repeated drafts, drafts in the history, greedy requests on penalized
    argmax ties, non-finite penalties, and history offsets out of order."""
    rng = np.random.default_rng(21)
    V, B, k = 3000, 6, 4
    for dtype in (synth.BF16, synth.F32):
        w = synth.build(6, seed=21, batch=B, vocab=V, ks=np.full(B, k), target_dtype=dtype,
                        draft_dtype=dtype, kinds=np.array([0, 1, 3, 0, 1, 0]),
                        temps=np.array([0.9, 1.1, 0.8, 0.0, 0.0, 0.7]), sigma=0.4)
        # every request drafts the same token four times
        w.draft_tokens[:] = np.repeat(rng.integers(0, V, size=B), k)
        pres = np.array([1.0, 0.5, 2.0, 1.5, np.nan, 0.25], np.float32)
        freq = np.array([0.5, 1.0, 0.0, 0.25, 0.0, np.inf], np.float32)
        toks, offs = [], [0]
        for b in range(B):
            t = np.unique(np.concatenate([[w.draft_tokens[b * k]], rng.choice(V, 20)]))
            toks.append(t)
            offs.append(offs[-1] + t.size)
        tokens = np.concatenate(toks).astype(np.int32)
        pen = synth.PenaltyInputs(pres, freq, np.array(offs, np.int32), tokens,
                                  rng.integers(0, 4, size=tokens.size).astype(np.int32))
        gpu = check(w, pen, f"edges dtype={dtype}")
        assert gpu["status"][4] == oracle.ROW_BAD_PARAM and gpu["status"][5] == oracle.ROW_BAD_PARAM
        # offsets out of order: those requests get no history
        bad = synth.PenaltyInputs(pres, freq, np.array([0, 30, 10, 60, 70, 80, 200], np.int32),
                                  tokens, pen.counts)
        check(w, bad, f"edges, bad offsets, dtype={dtype}")
