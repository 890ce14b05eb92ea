"""GPU parity of the prefix-match verify of argmax drafts (draft kind MATCH,
FreeToken PR #836, Design: sample every row as decode does, accept the prefix
that matches): mixed batches, the full-size mixed workload with its one-hot
requests switched to MATCH, planted drafts that realise every accept count,
filters, k = 0, and drafts in the first and the ragged last chunk."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from lossless_rejection_sampling_spec_amd import binding, synth  # noqa: E402
from test_gpu_parity import _workspace_left_clean, check, say  # noqa: E402,F401

pytestmark = pytest.mark.gpu
F32, BF16 = synth.F32, synth.BF16
ONEHOT, LOGITS, PROBS, MATCH = synth.ONEHOT, synth.LOGITS, synth.PROBS, synth.MATCH


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    binding.lib()
    yield


@pytest.mark.parametrize("tdt", [BF16, F32])
def test_match_in_mixed_batches(tdt):
    rng = np.random.default_rng(40 + tdt)
    B = 40
    ks = rng.integers(0, 8, size=B)
    kinds = rng.choice(np.array([MATCH, MATCH, ONEHOT, LOGITS]), size=B).astype(np.int32)
    temps = rng.uniform(0.4, 1.3, size=B).astype(np.float32)
    temps[rng.random(B) < 0.2] = 0.0
    top_k = rng.choice(np.array([0, 0, 7, 300]), size=B).astype(np.int32)
    top_p = rng.choice(np.array([1.0, 1.0, 0.8]), size=B).astype(np.float32)
    w = synth.build(30, seed=tdt, batch=B, vocab=20011, ks=ks, target_dtype=tdt, draft_dtype=tdt,
                    kinds=kinds, temps=temps, sigma=0.4, top_k=top_k, top_p=top_p,
                    name=f"MATCH mix dtype {tdt}")
    _, c = check(w)
    assert c["match"] + c["excused_accept"] + c["excused_final"] + c["excused_near_tie"] >= 25


def test_match_full_size_mixed_workload():
    """B=64, k=6, V=128256 bf16: the benchmark's mix with its 16 one-hot-draft
    requests verified by prefix match instead."""
    w = synth.make(2)
    w.draft_kind = np.where(w.draft_kind == ONEHOT, MATCH, w.draft_kind).astype(np.int32)
    w.name = "B=64 k=6 V=128256 bf16 with MATCH requests"
    check(w)


def test_match_planted_every_accept_count():
    """Drafts set to each row's own sample (the oracle's inverse CDF of the
    row at its uniform), then one planted mismatch per request at position
    b % (k+1): every a in 0..k occurs, and the committed token at a is row a's
    sample."""
    k, V = 6, 17000
    B = 3 * (k + 1)
    w = synth.build(31, seed=2, batch=B, vocab=V, ks=np.full(B, k), target_dtype=BF16,
                    draft_dtype=BF16, kinds=np.full(B, MATCH), temps=np.full(B, 0.7),
                    sigma=0.0, name="MATCH planted")
    L = synth.stored_f64(w.target, BF16)
    cu = w.cu_seqlens
    for b in range(B):
        plant = b % (k + 1)
        for i in range(k):
            p = oracle.process(L[cu[b] + i], np.float32(0.7)).p
            y, _, _ = oracle.inverse_cdf(p, float(w.uniforms[cu[b] + i]))
            w.draft_tokens[cu[b] - b + i] = y if i != plant else (y + 1 + (b % 5)) % V
    gpu, c = check(w)
    assert sorted(set(gpu["accepted"].tolist())) == list(range(k + 1))


def test_match_edges():
    """k = 0 (one plain sample of row 0), drafts in chunk 0 and in the ragged
    last chunk, masked draft tokens (p(x) = 0 never matches), and rows whose
    temperature makes them nearly one-hot."""
    V, k = 8193 + 8192, 3
    rng = np.random.default_rng(7)
    rows = rng.normal(0, 2, size=(k + 1, V))
    rows[:, 100] = -np.inf
    for xs in ([0, 5, V - 1], [V - 1, V - 2, 8192], [100, 2, 3]):
        for T in (1.0, 0.05):
            u = (rng.integers(0, 1 << 24, size=k + 1) * 2.0 ** -24).tolist()
            w = synth.Workload(name="MATCH edge", config=32, seed=0, vocab=V,
                               target=synth.store(rows, BF16), target_dtype=BF16,
                               cu_seqlens=np.array([0, k + 1], np.int32),
                               draft_tokens=np.asarray(xs, np.int32),
                               uniforms=np.asarray(u, np.float32),
                               temperature=np.array([T], np.float32),
                               draft_kind=np.array([MATCH], np.int32), max_k=k)
            check(w)
    w = synth.Workload(name="MATCH k=0", config=32, seed=0, vocab=V,
                       target=synth.store(rows[:1], F32), target_dtype=F32,
                       cu_seqlens=np.array([0, 1], np.int32), draft_tokens=np.zeros(0, np.int32),
                       uniforms=np.array([0.4], np.float32), temperature=np.array([0.9], np.float32),
                       draft_kind=np.array([MATCH], np.int32), max_k=0)
    check(w)
