"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects bad arguments on the host before anything is launched
(each call here fails validation, so no GPU is touched)."""

import os
import re

import pytest

from lossless_rejection_sampling_spec_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_verify_\w+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("spec_verify_greedy", "spec_verify_sampled", "spec_verify_workspace_bytes",
              "spec_verify_workspace_init", "spec_verify_abi_version",
              "spec_verify_status_string", "spec_verify_sampled_penalized",
              "spec_verify_sampled_noalloc", "spec_verify_drain", "spec_verify_accounting"):
        assert n in names


def test_library_exports_every_declared_symbol():
    from lossless_rejection_sampling_spec_amd import build
    for L in (binding.lib(), binding.load_library(build.LIB_ONE_POLL)):
        for n in _declared():
            assert hasattr(L, n), n


def test_abi_version_and_strings():
    assert binding.abi_version() == 1
    for code in range(7):
        assert binding.status_string(code)
    for code in range(6):
        assert binding.status_string(100 + code).startswith("row")
    assert binding.status_string(999) == "unknown code"


def test_workspace_bytes():
    assert binding.workspace_bytes(0, 1, 10, 1) == 0
    assert binding.workspace_bytes(2, 1, 10, 1) == 0
    assert binding.workspace_bytes(1, 1, 10, 64) == 0
    assert binding.workspace_bytes(1, 1, 0, 0) == 0
    assert binding.workspace_bytes(1, 1, 8192 * 512 + 1, 0) == 0
    a = binding.workspace_bytes(64, 448, 128256, 6)
    b = binding.workspace_bytes(64, 448, 8192 * 16 + 1, 6)
    assert 0 < a < b
    assert a % 256 == 0


FAKE = 0x1000     # a non-NULL pointer value that validation never dereferences


def _sampled(**kw):
    args = dict(target=FAKE, tdt=0, ldt=100, draft=None, ddt=0, ldd=0, kind=FAKE, cu=FAKE,
                drafts=FAKE, u=FAKE, temp=FAKE, top_k=None, top_p=None, batch=2, rows=6,
                max_k=3, vocab=100, acc=FAKE, out=FAKE, p=None, q=None, status=FAKE, ws=FAKE,
                wsb=1 << 40, stream=None)
    args.update(kw)
    return binding.lib().spec_verify_sampled(*args.values())


def _greedy(**kw):
    args = dict(target=FAKE, tdt=1, ldt=100, cu=FAKE, drafts=FAKE, batch=2, rows=6, max_k=3,
                vocab=100, acc=FAKE, out=FAKE, status=FAKE, ws=FAKE, wsb=1 << 40, stream=None)
    args.update(kw)
    return binding.lib().spec_verify_greedy(*args.values())


@pytest.mark.parametrize("field", ["target", "kind", "cu", "u", "temp", "acc", "out", "status",
                                   "ws", "drafts"])
def test_sampled_null_pointers(field):
    assert _sampled(**{field: None}) == 1


def test_sampled_shapes_and_dtypes():
    assert _sampled(batch=0) == 2
    assert _sampled(rows=1) == 2
    assert _sampled(max_k=64) == 2
    assert _sampled(max_k=-1) == 2
    assert _sampled(vocab=0) == 2
    assert _sampled(ldt=99) == 2
    assert _sampled(draft=FAKE, ldd=50) == 2
    assert _sampled(tdt=2) == 3
    assert _sampled(draft=FAKE, ldd=100, ddt=7) == 3
    assert _sampled(wsb=10) == 4
    assert _sampled(batch=1 << 20, rows=1 << 20, max_k=63, vocab=8192 * 100) == 2
    assert _sampled(batch=1025, rows=3000) == 2      # more requests than a launch schedules
    assert _greedy(batch=1025, rows=3000) == 2


def test_greedy_validation():
    assert _greedy(target=None) == 1
    assert _greedy(drafts=None) == 1
    assert _greedy(tdt=9) == 3
    assert _greedy(ldt=5) == 2
    assert _greedy(wsb=0) == 4


def test_noalloc_rejects_before_any_device_call():
    fake = FAKE
    L = binding.lib()
    # a workspace far beyond the static scratch array: rejected on the host
    assert L.spec_verify_sampled_noalloc(fake, 1, 1000000, None, 0, 0, fake, fake, fake, fake,
                                         fake, None, None, 1024, 8192, 7, 1000000, fake, fake,
                                         None, None, fake, None) == 6
    assert L.spec_verify_sampled_noalloc(None, 1, 100, None, 0, 0, fake, fake, fake, fake, fake,
                                         None, None, 2, 6, 3, 100, fake, fake, None, None, fake,
                                         None) == 1


def test_penalized_validation():
    """The penalized entry point checks its extra pointers and sizes on the host."""
    L = binding.lib()
    f = FAKE

    def call(pres=f, freq=f, off=None, tok=None, cnt=None, nnz=0, pen=f, ws=f):
        return L.spec_verify_sampled_penalized(
            f, 1, 100, None, 0, 0, f, f, f, f, f, None, None, pres, freq, off, tok, cnt, nnz,
            pen, 2, 6, 3, 100, f, f, None, None, f, ws, 1 << 20, None)

    assert call(pres=None) == 1
    assert call(freq=None) == 1
    assert call(pen=None) == 1
    assert call(ws=None) == 1
    assert call(nnz=5) == 1               # history arrays missing
    assert call(nnz=-1) == 2
    assert call(off=f, tok=f, cnt=f, nnz=1 << 31) == 2


def test_drain_and_accounting_validation():
    L = binding.lib()
    f = FAKE
    assert L.spec_verify_drain(None, f, f, f, 2, 6, f, f, f, None) == 1
    assert L.spec_verify_drain(f, f, f, f, 0, 6, f, f, f, None) == 2
    assert L.spec_verify_drain(f, f, f, f, 1025, 2000, f, f, f, None) == 2
    assert L.spec_verify_drain(f, f, f, f, 4, 3, f, f, f, None) == 2
    assert L.spec_verify_accounting(f, f, f, 2, f, f, 0.1, 0.4, 2, 5, f, None, None) == 1
    assert L.spec_verify_accounting(f, f, f, 2, f, f, 1.5, 0.4, 2, 5, f, f, None) == 2
    assert L.spec_verify_accounting(f, f, f, 2, f, f, 0.1, float("nan"), 2, 5, f, f, None) == 2
    assert L.spec_verify_accounting(f, f, f, 2, f, f, 0.1, 0.4, -1, 5, f, f, None) == 2
    assert L.spec_verify_accounting(f, f, f, 2, f, f, 0.1, 0.4, 2, 64, f, f, None) == 2


def test_workspace_init_null():
    assert binding.lib().spec_verify_workspace_init(None, 100, None) == 1


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(binding.SpecVerifyError):
        binding.lib()


def test_ctypes_signatures_match_header_arity():
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    for name in ("spec_verify_greedy", "spec_verify_sampled", "spec_verify_sampled_noalloc",
                 "spec_verify_sampled_penalized", "spec_verify_drain", "spec_verify_accounting"):
        m = re.search(name + r"\s*\(([^;]*)\);", src, flags=re.S)
        n_args = len([a for a in m.group(1).split(",") if a.strip()])
        assert len(getattr(binding.lib(), name).argtypes) == n_args, name

