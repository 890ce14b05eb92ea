"""GPU drain and acceptance accounting against the oracle, bit for bit: on
the outputs of real verify calls (greedy, one-hot, prefix-match, draft-logit
and probability requests, varlen), on hand-built batches with every status
and with counts that must not be trusted, and over several accounting steps
that keep their moving averages and counters on the device."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from lossless_rejection_sampling_spec_amd import binding, synth  # noqa: E402
from test_gpu_parity import _workspace_left_clean, gpu_sampled, say  # noqa: E402,F401

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    binding.lib()
    yield


def _t(a, dtype=torch.int32):
    return torch.from_numpy(np.ascontiguousarray(a)).to(device=DEV, dtype=dtype)


def check_drain(cu, acc, st, toks):
    c, o, r = binding.drain(_t(cu), _t(acc), _t(st), _t(toks))
    torch.cuda.synchronize()
    rc, ro, rr = oracle.drain(cu, acc, st, toks)
    o = o.cpu().numpy()
    assert np.array_equal(o, ro), (o, ro)
    assert np.array_equal(r.cpu().numpy(), rr)
    total = int(ro[-1])
    assert np.array_equal(c.cpu().numpy()[:total], rc)
    return ro, rr


def check_accounting(cu, acc, st, ema, beta, thr, k_low, k_high, counters):
    e = _t(ema, torch.float32)
    cnt = _t(counters, torch.int64)
    kn = binding.accounting(_t(cu), _t(acc), _t(st), e, cnt, beta=beta, threshold=thr,
                            k_low=k_low, k_high=k_high)
    torch.cuda.synchronize()
    re, rk, rc = oracle.accounting(cu, acc, st, ema, beta, thr, k_low, k_high, counters)
    assert np.array_equal(e.cpu().numpy().view(np.uint32), re.view(np.uint32))
    assert np.array_equal(kn.cpu().numpy(), rk)
    assert np.array_equal(cnt.cpu().numpy(), rc)
    return re, rc


@pytest.mark.parametrize("cfg,kw", [(2, dict(batch=24, vocab=20000)), (3, dict(batch=40, vocab=9000)),
                                    (4, dict(batch=16, vocab=9000))])
def test_drain_and_accounting_of_real_verify_outputs(cfg, kw):
    w = synth.make(cfg, seed=5, **kw)
    if cfg == 2:
        kinds = w.draft_kind.copy()
        kinds[::3] = synth.MATCH * (w.temperature[::3] > 0) + kinds[::3] * (w.temperature[::3] <= 0)
        w.draft_kind = kinds.astype(np.int32)
    gpu = gpu_sampled(w, want_probs=False)
    cu = w.cu_seqlens
    offsets, rollback = check_drain(cu, gpu["accepted"], gpu["status"], gpu["out_tokens"])
    say(f"config {cfg}: {int(offsets[-1])} tokens committed, {int(rollback.sum())} slots given back")
    B = w.batch
    rng = np.random.default_rng(cfg)
    ema = rng.random(B).astype(np.float32)
    check_accounting(cu, gpu["accepted"], gpu["status"], ema, 0.25, 0.4, 2, 5,
                     np.array([7, 11, 3, 2], np.int64))


def test_hand_built_batches_with_every_status():
    rng = np.random.default_rng(8)
    for B in (1, 37, 1024):
        ks = rng.integers(0, 9, size=B)
        cu = np.concatenate([[0], np.cumsum(ks + 1)]).astype(np.int32)
        acc = np.array([int(rng.integers(-1, k + 3)) for k in ks], np.int32)
        st = rng.choice(np.array([0, 0, 0, 1, 2, 3, 4, 5, 6]), size=B).astype(np.int32)
        toks = rng.integers(0, 50000, size=int(cu[-1])).astype(np.int32)
        if B > 1:
            cu2 = cu.copy()
            cu2[B // 2] = cu2[-1] + 5          # one request's rows run past the buffer
            check_drain(cu2, acc, st, toks)
        check_drain(cu, acc, st, toks)
        ema = rng.random(B).astype(np.float32)
        check_accounting(cu, acc, st, ema, 0.1, 0.4, 0, 5, np.zeros(4, np.int64))


def test_accounting_state_stays_on_the_device_over_steps():
    """Ten verify steps of one batch: the moving averages and counters live in
    device tensors updated in place; after every step they equal the oracle's
    chain of the same steps (the last five steps draw uniforms next to 1, so
    the rates fall)."""
    w = synth.make(1, seed=2, batch=16, vocab=8000)
    B = w.batch
    ema_d = torch.full((B,), 0.8, dtype=torch.float32, device=DEV)
    cnt_d = torch.zeros(4, dtype=torch.int64, device=DEV)
    ema_h = np.full(B, 0.8, np.float32)
    cnt_h = np.zeros(4, np.int64)
    rng = np.random.default_rng(3)
    for step in range(10):
        w.uniforms = (rng.integers(0, 1 << 24, size=w.total_rows) * 2.0 ** -24).astype(np.float32)
        if step >= 5:
            w.uniforms[:] = np.float32(1 - 2 ** -24)       # accept only where p(x) >= q(x)
        gpu = gpu_sampled(w, want_probs=False)
        kn = binding.accounting(_t(w.cu_seqlens), _t(gpu["accepted"]), _t(gpu["status"]), ema_d,
                                cnt_d, beta=0.3, threshold=0.4, k_low=2, k_high=5)
        torch.cuda.synchronize()
        ema_h, kn_h, cnt_h = oracle.accounting(w.cu_seqlens, gpu["accepted"], gpu["status"],
                                               ema_h, 0.3, 0.4, 2, 5, cnt_h)
        assert np.array_equal(ema_d.cpu().numpy().view(np.uint32), ema_h.view(np.uint32))
        assert np.array_equal(kn.cpu().numpy(), kn_h)
        assert np.array_equal(cnt_d.cpu().numpy(), cnt_h)
    say(f"after 10 steps: counters {cnt_h.tolist()}, mean tokens/step {cnt_h[0] / cnt_h[3]:.3f}")
