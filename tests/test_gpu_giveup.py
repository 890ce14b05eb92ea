"""The give-up path of the waits between workgroups, on a test-only build
whose every wait gives up after one poll (every kernel still exits
normally): requests end OK or SV_ROW_INTERNAL, INTERNAL requests report
accepted = -1, the OK ones match the oracle, the workspace is poisoned so the
next call reports INTERNAL everywhere, and after spec_verify_workspace_init a
normal call on the same workspace is parity-green with no hand-off word left
in flight."""

import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from lossless_rejection_sampling_spec_amd import binding, build, synth  # noqa: E402
from parity_util import compare, record_counts, run_oracle, sub_workload, to_numpy  # noqa: E402
from test_gpu_parity import say  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    yield


def _call(w, ws):
    t = binding.workload_tensors(w, DEV)
    res = binding.verify_sampled(t["target"], t["draft"], t["draft_kind"], t["cu_seqlens"],
                                 t["draft_tokens"], t["uniforms"], t["temperature"],
                                 t["top_k"], t["top_p"], max_k=w.max_k, vocab=w.vocab,
                                 want_probs=True, workspace=ws)
    torch.cuda.synchronize()
    return to_numpy(res)


@pytest.fixture
def one_poll(monkeypatch):
    if not os.path.exists(build.LIB_ONE_POLL):
        pytest.fail("the one-poll test build is missing: run build()")
    monkeypatch.setattr(binding, "_lib", binding.load_library(build.LIB_ONE_POLL))
    yield
    monkeypatch.setattr(binding, "_lib", None)


@pytest.mark.parametrize("cfg", [2, 4])
def test_waits_that_give_up(cfg, one_poll):
    w = synth.make(cfg, seed=31, batch=24, vocab=40000)
    need = binding.workspace_bytes(w.batch, w.total_rows, w.vocab, w.max_k)
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    say(f"one-poll build, config {cfg} B={w.batch} V={w.vocab}")
    gpu = _call(w, ws)
    st = gpu["status"]
    assert set(np.unique(st).tolist()) <= {binding.ROW_OK, binding.ROW_INTERNAL}, st
    internal = st == binding.ROW_INTERNAL
    assert np.all(gpu["accepted"][internal] == -1)
    say(f"  {int(internal.sum())} of {w.batch} requests gave up")
    ok = [int(b) for b in np.nonzero(~internal)[0]]
    if ok:
        counts = compare(w, gpu, run_oracle(sub_workload(w, ok)), requests=ok)
        record_counts(f"one-poll config {cfg}: requests that finished", counts)
    if internal.any():
        again = _call(w, ws)
        assert np.all(again["status"] == binding.ROW_INTERNAL), again["status"]
        assert np.all(again["accepted"] == -1)
    # clear the mark and the words left in flight, then a normal build on the
    # same workspace must give the oracle's results
    binding.reset_workspace(ws)
    torch.cuda.synchronize()
    binding._lib = None
    gpu = _call(w, ws)
    counts = compare(w, gpu, run_oracle(w))
    record_counts(f"config {cfg} after reset", counts)
    words = ws[: ws.numel() // 8 * 8].view(torch.int64)
    assert int((words < 0).sum().item()) == 0, "hand-off word left in flight"
