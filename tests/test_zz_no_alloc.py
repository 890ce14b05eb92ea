"""The allocation-free entry point (spec_verify_sampled_noalloc, static
scratch array) against the workspace entry point (spec_verify_sampled): the
same kernels must give identical outputs, on two calls in a row, the second
with a smaller input."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from lossless_rejection_sampling_spec_amd import binding, synth  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _outs(w):
    B, R = w.batch, w.total_rows
    n = max(R - B, 1)
    return (torch.full((B,), -7, dtype=torch.int32, device=DEV),
            torch.full((R,), -7, dtype=torch.int32, device=DEV),
            torch.full((B,), -7, dtype=torch.int32, device=DEV),
            torch.full((n,), -7.0, dtype=torch.float32, device=DEV),
            torch.full((n,), -7.0, dtype=torch.float32, device=DEV))


def _both(w):
    t = binding.workload_tensors(w, DEV)
    args = (t["target"], t["draft"], t["draft_kind"], t["cu_seqlens"], t["draft_tokens"],
            t["uniforms"], t["temperature"], t["top_k"], t["top_p"])
    ref = binding.verify_sampled(*args, max_k=w.max_k, vocab=w.vocab, want_probs=True,
                                 out=_outs(w))
    got = binding.verify_sampled_noalloc(*args, max_k=w.max_k, vocab=w.vocab, out=_outs(w))
    torch.cuda.synchronize()
    return [r.cpu().numpy() for r in ref], [g.cpu().numpy() for g in got]


def test_noalloc_matches_the_workspace_entry_point_on_two_calls():
    assert torch.cuda.is_available()
    first = synth.make(3, seed=12, batch=24, vocab=30011)          # varlen, filters
    second = synth.make(4, seed=13, batch=6, vocab=9001)           # smaller, probabilities
    for w in (first, second):
        ref, got = _both(w)
        names = ("accepted", "out_tokens", "status", "p_at", "q_at")
        for name, r, g in zip(names, ref, got):
            assert np.array_equal(r, g, equal_nan=True), (w.name, name)
        assert np.all(ref[2] == 0), ref[2]


def test_noalloc_rejects_calls_beyond_its_scratch():
    L = binding.lib()
    fake = 0x1000
    # B=1024, 8192 rows, V=1,000,000: the workspace would need far more than 8 MiB
    rc = L.spec_verify_sampled_noalloc(fake, 1, 1000000, None, 0, 0, fake, fake, fake, fake, fake,
                                       None, None, 1024, 8192, 7, 1000000, fake, fake, None, None,
                                       fake, None)
    assert rc == 6, rc
    assert "scratch" in binding.status_string(rc)
