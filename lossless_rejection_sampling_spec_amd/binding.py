"""Thin Python binding of libspecverify.so (argument marshalling only).

Every step of the verify runs in the library's HIP kernels; this module only
turns torch tensors into device pointers, allocates outputs and the workspace
with torch on the tensors' device, and passes torch's current stream.  It
raises when the library is missing: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SV_F32, SV_BF16 = 0, 1
ONEHOT, LOGITS, PROBS, MATCH = 0, 1, 2, 3
ROW_OK, ROW_NONFINITE, ROW_EMPTY, ROW_BAD_K, ROW_BAD_TOKEN, ROW_BAD_PARAM, ROW_INTERNAL = range(7)
MAX_K = 63

_lib = None
_lock = threading.Lock()
_ws_cache: dict = {}

_vp = ctypes.c_void_p
_i32 = ctypes.c_int
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t


class SpecVerifyError(RuntimeError):
    pass


def load_library(path: str) -> ctypes.CDLL:
    """Open a build of the library at `path` with the C ABI's signatures."""
    if not os.path.exists(path):
        raise SpecVerifyError(
            f"{path} is missing; build it with `python -m lossless_rejection_sampling_spec_amd.build`")
    L = ctypes.CDLL(path)
    L.spec_verify_abi_version.restype = _i32
    L.spec_verify_abi_version.argtypes = []
    L.spec_verify_status_string.restype = ctypes.c_char_p
    L.spec_verify_status_string.argtypes = [_i32]
    L.spec_verify_workspace_bytes.restype = _sz
    L.spec_verify_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32]
    L.spec_verify_workspace_init.restype = _i32
    L.spec_verify_workspace_init.argtypes = [_vp, _sz, _vp]
    L.spec_verify_greedy.restype = _i32
    L.spec_verify_greedy.argtypes = [
        _vp, _i32, _i64, _vp, _vp, _i32, _i32, _i32, _i32,
        _vp, _vp, _vp, _vp, _sz, _vp]
    L.spec_verify_sampled.restype = _i32
    L.spec_verify_sampled.argtypes = [
        _vp, _i32, _i64, _vp, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
        _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    L.spec_verify_drain.restype = _i32
    L.spec_verify_drain.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp]
    L.spec_verify_accounting.restype = _i32
    L.spec_verify_accounting.argtypes = [_vp, _vp, _vp, _i32, _vp, _vp, ctypes.c_float,
                                         ctypes.c_float, _i32, _i32, _vp, _vp, _vp]
    L.spec_verify_sampled_penalized.restype = _i32
    L.spec_verify_sampled_penalized.argtypes = [
        _vp, _i32, _i64, _vp, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
        _vp, _vp, _vp, _vp, _vp, _i64, _vp,
        _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
    L.spec_verify_sampled_noalloc.restype = _i32
    L.spec_verify_sampled_noalloc.argtypes = [
        _vp, _i32, _i64, _vp, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
        _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]
    return L


def lib() -> ctypes.CDLL:
    """Load libspecverify.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                _lib = load_library(LIB_PATH)
    return _lib


def abi_version() -> int:
    return int(lib().spec_verify_abi_version())


def status_string(code: int) -> str:
    return lib().spec_verify_status_string(int(code)).decode()


def workspace_bytes(batch: int, total_rows: int, vocab: int, max_k: int) -> int:
    return int(lib().spec_verify_workspace_bytes(batch, total_rows, vocab, max_k))


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype == torch.bfloat16:
        return SV_BF16
    raise ValueError(f"unsupported logit dtype {t.dtype} (float32 or bfloat16)")


def _check_rows(t: torch.Tensor, name: str) -> None:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be 2-D with unit stride along the vocabulary")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _check_vec(t: torch.Tensor | None, name: str, dtype, n: int | None = None) -> None:
    if t is None:
        return
    if t.dtype != dtype or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} device tensor")
    if n is not None and t.numel() < n:
        raise ValueError(f"{name} needs at least {n} elements")


def get_workspace(device: torch.device, nbytes: int) -> torch.Tensor:
    """A zero-initialised workspace cached per (device, current stream).

    The library leaves a workspace ready after every call, so it is reused
    without clearing.  Calls that may run concurrently must not share one, so
    each stream gets its own: calls on one stream are ordered by the stream."""
    device = torch.device(device)
    stream = torch.cuda.current_stream(device)
    key = (device.type, device.index, stream.cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def reset_workspace(workspace: torch.Tensor | None = None, device=None) -> None:
    """Zero-fill a workspace on the current stream (spec_verify_workspace_init).

    Call it after any request reports ROW_INTERNAL (a wait between the
    library's workgroups ran out): such a call can leave hand-off words in
    flight that the next call would take as fresh.  With no argument, every
    workspace cached for `device` (default: the current device) is cleared,
    each on the stream it belongs to."""
    if workspace is not None:
        targets = [(workspace, torch.cuda.current_stream(workspace.device).cuda_stream)]
    else:
        dev = torch.device(device) if device is not None else torch.device(
            "cuda", torch.cuda.current_device())
        targets = [(ws, key[2]) for key, ws in _ws_cache.items()
                   if key[0] == dev.type and key[1] == dev.index]
    for ws, stream in targets:
        _raise(lib().spec_verify_workspace_init(_ptr(ws), ws.numel(), stream))


def _raise(rc: int) -> None:
    if rc != 0:
        raise ValueError(f"spec_verify: {status_string(rc)} (code {rc})")


def verify_greedy(target: torch.Tensor, cu_seqlens: torch.Tensor, draft_tokens: torch.Tensor,
                  *, max_k: int, vocab: int | None = None, workspace: torch.Tensor | None = None,
                  out: tuple | None = None):
    """Greedy prefix-match verify.  Returns (accepted[B], out_tokens[R], status[B])."""
    _check_rows(target, "target")
    dev = target.device
    batch = cu_seqlens.numel() - 1
    total_rows = target.shape[0]
    V = target.shape[1] if vocab is None else int(vocab)
    _check_vec(cu_seqlens, "cu_seqlens", torch.int32, batch + 1)
    _check_vec(draft_tokens, "draft_tokens", torch.int32)
    if out is None:
        accepted = torch.empty(batch, dtype=torch.int32, device=dev)
        tokens = torch.empty(total_rows, dtype=torch.int32, device=dev)
        status = torch.empty(batch, dtype=torch.int32, device=dev)
    else:
        accepted, tokens, status = out
    need = workspace_bytes(batch, total_rows, V, max_k)
    if need == 0:
        raise ValueError("invalid sizes for spec_verify_greedy")
    ws = get_workspace(dev, need) if workspace is None else workspace
    rc = lib().spec_verify_greedy(
        _ptr(target), _dtype_code(target), target.stride(0), _ptr(cu_seqlens),
        _ptr(draft_tokens) if draft_tokens.numel() else None, batch, total_rows, max_k, V,
        _ptr(accepted), _ptr(tokens), _ptr(status), _ptr(ws), ws.numel(), _stream(dev))
    _raise(rc)
    return accepted, tokens, status


def verify_sampled(target: torch.Tensor, draft: torch.Tensor | None, draft_kind: torch.Tensor,
                   cu_seqlens: torch.Tensor, draft_tokens: torch.Tensor, uniforms: torch.Tensor,
                   temperature: torch.Tensor, top_k: torch.Tensor | None = None,
                   top_p: torch.Tensor | None = None, *, max_k: int, vocab: int | None = None,
                   want_probs: bool = False, workspace: torch.Tensor | None = None,
                   out: tuple | None = None, presence: torch.Tensor | None = None,
                   frequency: torch.Tensor | None = None, history: tuple | None = None,
                   penalized: torch.Tensor | None = None):
    """Sampled verify by rejection sampling (greedy requests mixed in).

    With presence and frequency (float32 [B]) the call goes to
    spec_verify_sampled_penalized: history = (offsets int32 [B+1], tokens
    int32 [nnz], counts int32 [nnz]) or None, and `penalized` the scratch of
    the penalized rows (allocated like `target` when None).

    Returns (accepted[B], out_tokens[R], status[B], p_at_draft, q_at_draft);
    the last two are None unless want_probs."""
    _check_rows(target, "target")
    dev = target.device
    batch = cu_seqlens.numel() - 1
    total_rows = target.shape[0]
    V = target.shape[1] if vocab is None else int(vocab)
    n_draft = total_rows - batch
    if draft is not None:
        _check_rows(draft, "draft")
    _check_vec(cu_seqlens, "cu_seqlens", torch.int32, batch + 1)
    _check_vec(draft_kind, "draft_kind", torch.int32, batch)
    _check_vec(draft_tokens, "draft_tokens", torch.int32, n_draft)
    _check_vec(uniforms, "uniforms", torch.float32, total_rows)
    _check_vec(temperature, "temperature", torch.float32, batch)
    _check_vec(top_k, "top_k", torch.int32, batch)
    _check_vec(top_p, "top_p", torch.float32, batch)
    if out is None:
        accepted = torch.empty(batch, dtype=torch.int32, device=dev)
        tokens = torch.empty(total_rows, dtype=torch.int32, device=dev)
        status = torch.empty(batch, dtype=torch.int32, device=dev)
        p_at = torch.empty(max(n_draft, 1), dtype=torch.float32, device=dev) if want_probs else None
        q_at = torch.empty(max(n_draft, 1), dtype=torch.float32, device=dev) if want_probs else None
    else:
        accepted, tokens, status, p_at, q_at = out
    need = workspace_bytes(batch, total_rows, V, max_k)
    if need == 0:
        raise ValueError("invalid sizes for spec_verify_sampled")
    ws = get_workspace(dev, need) if workspace is None else workspace
    if presence is None and frequency is None:
        rc = lib().spec_verify_sampled(
            _ptr(target), _dtype_code(target), target.stride(0),
            _ptr(draft), _dtype_code(draft) if draft is not None else SV_F32,
            draft.stride(0) if draft is not None else 0,
            _ptr(draft_kind), _ptr(cu_seqlens), _ptr(draft_tokens) if n_draft else None,
            _ptr(uniforms), _ptr(temperature), _ptr(top_k), _ptr(top_p),
            batch, total_rows, max_k, V, _ptr(accepted), _ptr(tokens), _ptr(p_at), _ptr(q_at),
            _ptr(status), _ptr(ws), ws.numel(), _stream(dev))
    else:
        _check_vec(presence, "presence", torch.float32, batch)
        _check_vec(frequency, "frequency", torch.float32, batch)
        h_off = h_tok = h_cnt = None
        nnz = 0
        if history is not None:
            h_off, h_tok, h_cnt = history
            nnz = h_tok.numel()
            _check_vec(h_off, "history offsets", torch.int32, batch + 1)
            _check_vec(h_tok, "history tokens", torch.int32, nnz)
            _check_vec(h_cnt, "history counts", torch.int32, nnz)
        if penalized is None:
            penalized = torch.empty_strided(target.shape, target.stride(), dtype=target.dtype,
                                            device=dev)
        if (penalized.dtype != target.dtype or penalized.stride() != target.stride()
                or penalized.shape != target.shape or penalized.device != dev):
            raise ValueError("penalized must match target's shape, strides, dtype and device")
        rc = lib().spec_verify_sampled_penalized(
            _ptr(target), _dtype_code(target), target.stride(0),
            _ptr(draft), _dtype_code(draft) if draft is not None else SV_F32,
            draft.stride(0) if draft is not None else 0,
            _ptr(draft_kind), _ptr(cu_seqlens), _ptr(draft_tokens) if n_draft else None,
            _ptr(uniforms), _ptr(temperature), _ptr(top_k), _ptr(top_p),
            _ptr(presence), _ptr(frequency), _ptr(h_off) if nnz else None,
            _ptr(h_tok) if nnz else None, _ptr(h_cnt) if nnz else None, nnz, _ptr(penalized),
            batch, total_rows, max_k, V, _ptr(accepted), _ptr(tokens), _ptr(p_at), _ptr(q_at),
            _ptr(status), _ptr(ws), ws.numel(), _stream(dev))
    _raise(rc)
    return accepted, tokens, status, p_at, q_at


def verify_sampled_noalloc(target: torch.Tensor, draft: torch.Tensor | None,
                           draft_kind: torch.Tensor, cu_seqlens: torch.Tensor,
                           draft_tokens: torch.Tensor, uniforms: torch.Tensor,
                           temperature: torch.Tensor, top_k: torch.Tensor | None = None,
                           top_p: torch.Tensor | None = None, *, max_k: int, vocab: int,
                           out: tuple):
    """spec_verify_sampled_noalloc: the sampled verify with the library's
    static scratch array instead of a workspace.  `out` = (accepted, tokens,
    status, p_at or None, q_at or None), preallocated by the caller, so this
    call allocates nothing."""
    batch = cu_seqlens.numel() - 1
    total_rows = target.shape[0]
    accepted, tokens, status, p_at, q_at = out
    rc = lib().spec_verify_sampled_noalloc(
        _ptr(target), _dtype_code(target), target.stride(0),
        _ptr(draft), _dtype_code(draft) if draft is not None else SV_F32,
        draft.stride(0) if draft is not None else 0,
        _ptr(draft_kind), _ptr(cu_seqlens),
        _ptr(draft_tokens) if total_rows > batch else None,
        _ptr(uniforms), _ptr(temperature), _ptr(top_k), _ptr(top_p),
        batch, total_rows, max_k, int(vocab), _ptr(accepted), _ptr(tokens), _ptr(p_at),
        _ptr(q_at), _ptr(status), _stream(target.device))
    _raise(rc)
    return accepted, tokens, status, p_at, q_at


def drain(cu_seqlens: torch.Tensor, accepted: torch.Tensor, status: torch.Tensor,
          out_tokens: torch.Tensor):
    """spec_verify_drain: (committed [total_rows], commit_offsets [B+1],
    rollback [B]); only committed[:commit_offsets[B]] is written."""
    dev = out_tokens.device
    batch = cu_seqlens.numel() - 1
    total_rows = out_tokens.numel()
    for t, n in ((cu_seqlens, batch + 1), (accepted, batch), (status, batch), (out_tokens, total_rows)):
        _check_vec(t, "drain input", torch.int32, n)
    committed = torch.empty(total_rows, dtype=torch.int32, device=dev)
    offsets = torch.empty(batch + 1, dtype=torch.int32, device=dev)
    rollback = torch.empty(batch, dtype=torch.int32, device=dev)
    _raise(lib().spec_verify_drain(_ptr(cu_seqlens), _ptr(accepted), _ptr(status), _ptr(out_tokens),
                                   batch, total_rows, _ptr(committed), _ptr(offsets),
                                   _ptr(rollback), _stream(dev)))
    return committed, offsets, rollback


def accounting(cu_seqlens: torch.Tensor, accepted: torch.Tensor, status: torch.Tensor,
               ema: torch.Tensor, counters: torch.Tensor, *, beta: float = 0.1,
               threshold: float = 0.4, k_low: int = 2, k_high: int = 5):
    """spec_verify_accounting: updates `ema` (float32 [B]) and `counters`
    (int64 [4]: generated, drafted, accepted, requests) in place and returns
    k_next (int32 [B])."""
    dev = ema.device
    batch = cu_seqlens.numel() - 1
    _check_vec(cu_seqlens, "cu_seqlens", torch.int32, batch + 1)
    _check_vec(accepted, "accepted", torch.int32, batch)
    _check_vec(status, "status", torch.int32, batch)
    _check_vec(ema, "ema", torch.float32, batch)
    _check_vec(counters, "counters", torch.int64, 4)
    k_next = torch.empty(batch, dtype=torch.int32, device=dev)
    _raise(lib().spec_verify_accounting(_ptr(cu_seqlens), _ptr(accepted), _ptr(status), batch,
                                        _ptr(ema), _ptr(ema), float(beta), float(threshold),
                                        int(k_low), int(k_high), _ptr(k_next), _ptr(counters),
                                        _stream(dev)))
    return k_next


def workload_tensors(w, device) -> dict:
    """Device tensors of a synthetic workload (see synth.Workload)."""
    def rows(a, dt):
        if a is None:
            return None
        if dt == SV_BF16:
            return torch.from_numpy(a.view("int16")).to(device).view(torch.bfloat16)
        return torch.from_numpy(a).to(device)

    def vec(a, dtype):
        return None if a is None else torch.from_numpy(a).to(device=device, dtype=dtype)

    return dict(
        target=rows(w.target, w.target_dtype),
        draft=rows(w.draft, w.draft_dtype),
        draft_kind=vec(w.draft_kind, torch.int32),
        cu_seqlens=vec(w.cu_seqlens, torch.int32),
        draft_tokens=vec(w.draft_tokens, torch.int32),
        uniforms=vec(w.uniforms, torch.float32),
        temperature=vec(w.temperature, torch.float32),
        top_k=vec(w.top_k, torch.int32),
        top_p=vec(w.top_p, torch.float32),
    )
