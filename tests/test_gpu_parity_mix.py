"""GPU parity on the paths the configuration workloads leave out: every pair
of target and draft element types with each draft kind, batches that mix all
kinds with greedy requests and k_b = 0, k = 63 at the largest vocabulary the
finalizer's LDS stage admits, and the largest batch one call takes."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from lossless_rejection_sampling_spec_amd import binding, synth  # noqa: E402
from test_gpu_parity import _workspace_left_clean, check, say  # noqa: E402,F401

pytestmark = pytest.mark.gpu
F32, BF16 = synth.F32, synth.BF16
ONEHOT, LOGITS, PROBS = synth.ONEHOT, synth.LOGITS, synth.PROBS


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    binding.lib()
    yield


def _mixed(config, seed, B, V, tdt, ddt, kinds_from, ks=None, greedy_frac=0.25,
           filters=False):
    rng = np.random.default_rng(1000 + seed)
    ks = rng.integers(1, 7, size=B) if ks is None else np.asarray(ks)
    kinds = rng.choice(np.array(kinds_from), size=B).astype(np.int32)
    temps = rng.uniform(0.5, 1.3, size=B).astype(np.float32)
    temps[rng.random(B) < greedy_frac] = 0.0
    top_k = top_p = None
    if filters:
        top_k = rng.choice(np.array([0, 3, 40, 1000]), size=B).astype(np.int32)
        top_p = rng.choice(np.array([1.0, 0.5, 0.9]), size=B).astype(np.float32)
    return synth.build(config, seed=seed, batch=B, vocab=V, ks=ks, target_dtype=tdt,
                       draft_dtype=ddt, kinds=kinds, temps=temps, sigma=0.6, top_k=top_k,
                       top_p=top_p, name=f"mix B={B} V={V} t{tdt}/d{ddt} kinds={kinds_from}")


@pytest.mark.parametrize("tdt,ddt", [(F32, BF16), (BF16, F32), (F32, F32), (BF16, BF16)])
@pytest.mark.parametrize("kind", [LOGITS, PROBS])
def test_element_type_pairs(tdt, ddt, kind):
    """Each draft kind with every pair of element types (fp32 target with bf16
    draft rows, bf16 probability rows, ...), a ragged last chunk, greedy and
    one-hot requests in the same batch."""
    w = _mixed(20, seed=tdt * 2 + ddt, B=12, V=20011, tdt=tdt, ddt=ddt,
               kinds_from=[kind, kind, ONEHOT])
    _, c = check(w)
    assert c["greedy"] + c["match"] + c["excused_accept"] + c["excused_final"] >= 10


@pytest.mark.parametrize("ddt", [F32, BF16])
def test_varlen_with_empty_requests_and_all_kinds(ddt):
    """k_b in 0..8 with several k_b = 0 requests among longer ones, every draft
    kind, greedy requests, and per-request top-k / top-p."""
    rng = np.random.default_rng(3)
    B = 40
    ks = rng.integers(0, 9, size=B)
    ks[rng.choice(B, size=8, replace=False)] = 0
    w = _mixed(21, seed=7 + ddt, B=B, V=9001, tdt=BF16, ddt=ddt,
               kinds_from=[ONEHOT, LOGITS, PROBS], ks=ks, filters=True)
    gpu, c = check(w)
    assert int(np.sum(ks == 0)) >= 8
    cu = w.cu_seqlens
    for b in np.nonzero(ks == 0)[0]:
        assert int(gpu["accepted"][b]) == 0
        assert 0 <= int(gpu["out_tokens"][cu[b]]) < w.vocab


def test_k63_at_the_stage_limit():
    """k = 63 (the ballot's last lane is the bonus position) with 48 chunks per
    row, the largest count for which (2k+1) chunk words per row fit the
    finalizer's stage: a draft-logit request whose draft rows equal its target
    rows (every draft accepted, bonus drawn from row 63), a draft-logit request
    that rejects, and greedy requests accepting 62 and 63 drafts."""
    k, V = 63, 47 * 8192 + 1000                  # 48 chunks, the last one ragged
    B = 4
    w = synth.build(22, seed=1, batch=B, vocab=V, ks=np.full(B, k), target_dtype=BF16,
                    draft_dtype=BF16, kinds=np.array([LOGITS, LOGITS, ONEHOT, ONEHOT]),
                    temps=np.array([0.9, 0.9, 0.0, 0.0]), sigma=np.array([0.0, 0.5, 0.0, 0.0]),
                    name="k=63 V=384216 bf16")
    L = synth.stored_f64(w.target, BF16)
    cu = w.cu_seqlens
    for b in (2, 3):
        for i in range(k):
            g = int(np.argmax(L[cu[b] + i]))
            w.draft_tokens[cu[b] - b + i] = g if (b == 3 or i != 62) else (g + 1) % V
    gpu, c = check(w)
    acc = [int(v) for v in gpu["accepted"]]
    say(f"  accepted {acc}")
    assert acc[0] == 63 and acc[2] == 62 and acc[3] == 63
    assert 0 <= acc[1] < 63


def test_largest_batch():
    """1,024 requests (the most one call takes), k_b in 0..2, tiny vocabulary:
    every workgroup finds its request among 16 per lane."""
    rng = np.random.default_rng(4)
    B = 1024
    w = _mixed(23, seed=2, B=B, V=300, tdt=F32, ddt=F32, kinds_from=[ONEHOT, LOGITS, PROBS],
               ks=rng.integers(0, 3, size=B))
    _, c = check(w)
    assert c["status"] == 0
