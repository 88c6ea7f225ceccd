"""Thin Python binding of ``libdspark.so`` (argument marshalling only).

Every step of the hot path runs in the library's HIP kernels; this module only
checks tensor shapes / dtypes / devices, allocates outputs and workspace with
torch when the caller passes none, and forwards raw device pointers and the
current HIP stream through ctypes.  Importing it does not need a GPU; calling a
compute entry point without the built library raises ``DsparkError``.
"""
from __future__ import annotations

import ctypes
import os
import re

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdspark.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "dspark.h")

DSPARK_OK = 0
DSPARK_ERR_INVALID_ARG = 1
DSPARK_ERR_UNSUPPORTED_DTYPE = 2
DSPARK_ERR_WORKSPACE_TOO_SMALL = 3
DSPARK_ERR_HIP = 4

DSPARK_F32 = 0
DSPARK_BF16 = 1

# dspark_kernel ids (bit positions of the profiling mask)
KERNELS = ("draft_strip", "draft_combine", "verify_rows", "verify_resolve", "residual_strip",
           "residual_combine", "schedule")
_DT = {torch.float32: DSPARK_F32, torch.bfloat16: DSPARK_BF16}


class DsparkError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"dspark status {status}: {msg}")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64
_SZ = ctypes.c_size_t


def lib():
    """Load the built library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise DsparkError(DSPARK_ERR_HIP, f"{LIB_PATH} is missing: build it with "
                              "`python -m draft_sampling_verification_04_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.dspark_version.restype = ctypes.c_char_p
        L.dspark_version.argtypes = []
        L.dspark_last_error.restype = ctypes.c_char_p
        L.dspark_last_error.argtypes = []
        L.dspark_draft_workspace_bytes.restype = _SZ
        L.dspark_draft_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32]
        L.dspark_draft_sample.restype = ctypes.c_int
        L.dspark_draft_sample.argtypes = [_P, ctypes.c_int, _P, _P, ctypes.c_int, _P, _P, _U64,
                                          _I32, _I32, _I32, _I32, _P, _P, _P, _P, _SZ, _P]
        L.dspark_draft_sample_noalloc.restype = ctypes.c_int
        L.dspark_draft_sample_noalloc.argtypes = [_P, ctypes.c_int, _P, _P, ctypes.c_int, _P, _P,
                                                  _U64, _I32, _I32, _I32, _I32, _P, _P, _P, _P]
        L.dspark_schedule_workspace_bytes.restype = _SZ
        L.dspark_schedule_workspace_bytes.argtypes = [_I32, _I32]
        L.dspark_schedule.restype = ctypes.c_int
        L.dspark_schedule.argtypes = [_P, _I32, _I32, _I64, _P, _P, _I32, _P, _P, _P, _P, _SZ, _P]
        L.dspark_verify_workspace_bytes.restype = _SZ
        L.dspark_verify_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32]
        L.dspark_verify.restype = ctypes.c_int
        L.dspark_verify.argtypes = [_P, _P, _P, _P, _P, ctypes.c_int, _P, _P, ctypes.c_int, _P,
                                    _I64, _P, _P, _P, _U64, _I32, _I32, _I32, _I32, _P, _P, _P,
                                    _P, _P, _SZ, _P]
        L.dspark_profile_begin.restype = ctypes.c_int
        L.dspark_profile_begin.argtypes = [ctypes.c_uint32, _I32]
        L.dspark_profile_end.restype = ctypes.c_int
        L.dspark_profile_end.argtypes = [_P, _P, _P]
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/dspark.h declares."""
    with open(HEADER) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_\w+)\s*\(", text)))


def _check(status: int):
    if status != DSPARK_OK:
        raise DsparkError(status, lib().dspark_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, name):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise DsparkError(DSPARK_ERR_INVALID_ARG, f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise DsparkError(DSPARK_ERR_INVALID_ARG, f"{name} must be contiguous")
    return t


def _dtype(t, name):
    if t.dtype not in _DT:
        raise DsparkError(DSPARK_ERR_UNSUPPORTED_DTYPE, f"{name}: dtype {t.dtype}")
    return _DT[t.dtype]


def _workspace(ws, nbytes, device):
    if ws is None:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    return ws


def dspark_version() -> str:
    return lib().dspark_version().decode()


def dspark_draft_workspace_bytes(B, K, V, r) -> int:
    return int(lib().dspark_draft_workspace_bytes(B, K, V, r))


def dspark_schedule_workspace_bytes(B, K) -> int:
    return int(lib().dspark_schedule_workspace_bytes(B, K))


def dspark_verify_workspace_bytes(B, K, V, r) -> int:
    return int(lib().dspark_verify_workspace_bytes(B, K, V, r))


def _draft_marshal(base_logits, A, W, prev_token, temperature, draft_tokens, draft_logp,
                   draft_lse):
    _dev(base_logits, "base_logits")
    _dev(prev_token, "prev_token")
    _dev(temperature, "temperature")
    B, K, V = base_logits.shape
    if A is None and W is None:
        r, fdt = 1, _dtype(base_logits, "base_logits")
    else:
        _dev(A, "A")
        _dev(W, "W")
        r = A.shape[1]
        if A.shape != (V, r) or W.shape != (r, V) or A.dtype != W.dtype:
            raise DsparkError(DSPARK_ERR_INVALID_ARG, "A must be [V, r] and W [r, V], same dtype")
        fdt = _dtype(A, "A")
    if prev_token.dtype != torch.int32 or temperature.dtype != torch.float32:
        raise DsparkError(DSPARK_ERR_INVALID_ARG, "prev_token int32, temperature float32")
    dev = base_logits.device
    if draft_tokens is None:
        draft_tokens = torch.empty((B, K), dtype=torch.int32, device=dev)
    if draft_logp is None:
        draft_logp = torch.empty((B, K), dtype=torch.float32, device=dev)
    if draft_lse is None:
        draft_lse = torch.empty((B, K), dtype=torch.float32, device=dev)
    return (B, K, V, r, fdt, draft_tokens, draft_logp, draft_lse)


def dspark_draft_sample(base_logits, A, W, prev_token, temperature, seed, *, draft_tokens=None,
                        draft_logp=None, draft_lse=None, workspace=None, stream=None):
    """Markov-head draft of K tokens per request; returns (tokens, logp, lse).
    A = W = None drafts without the Markov head (every position from its own
    base logits, all in one pass)."""
    B, K, V, r, fdt, draft_tokens, draft_logp, draft_lse = _draft_marshal(
        base_logits, A, W, prev_token, temperature, draft_tokens, draft_logp, draft_lse)
    dev = base_logits.device
    nbytes = dspark_draft_workspace_bytes(B, K, V, r)
    workspace = _workspace(workspace, nbytes, dev)
    _check(lib().dspark_draft_sample(
        _ptr(base_logits), _dtype(base_logits, "base_logits"), _ptr(A), _ptr(W), fdt,
        _ptr(prev_token), _ptr(temperature), int(seed) & (2**64 - 1), B, K, V, r,
        _ptr(draft_tokens), _ptr(draft_logp), _ptr(draft_lse), _ptr(workspace),
        workspace.numel(), _stream(stream, dev)))
    return draft_tokens, draft_logp, draft_lse


def dspark_draft_sample_noalloc(base_logits, A, W, prev_token, temperature, seed, *,
                                draft_tokens=None, draft_logp=None, draft_lse=None, stream=None):
    """dspark_draft_sample on the library's fixed per-device scratch (no
    workspace; the library allocates nothing).  Pass the output tensors to
    allocate nothing on this side either."""
    B, K, V, r, fdt, draft_tokens, draft_logp, draft_lse = _draft_marshal(
        base_logits, A, W, prev_token, temperature, draft_tokens, draft_logp, draft_lse)
    dev = base_logits.device
    _check(lib().dspark_draft_sample_noalloc(
        _ptr(base_logits), _dtype(base_logits, "base_logits"), _ptr(A), _ptr(W), fdt,
        _ptr(prev_token), _ptr(temperature), int(seed) & (2**64 - 1), B, K, V, r,
        _ptr(draft_tokens), _ptr(draft_logp), _ptr(draft_lse), _stream(stream, dev)))
    return draft_tokens, draft_logp, draft_lse


def dspark_schedule(conf, budget_tokens, curve_n=None, curve_latency=None, *, lengths=None,
                    row_offsets=None, survival=None, workspace=None, stream=None):
    """Confidence-scheduled lengths; returns (lengths [B], row_offsets [B+1], survival)."""
    _dev(conf, "conf")
    if conf.dtype != torch.float32:
        raise DsparkError(DSPARK_ERR_INVALID_ARG, "conf must be float32")
    B, K = conf.shape
    dev = conf.device
    if lengths is None:
        lengths = torch.empty(B, dtype=torch.int32, device=dev)
    if row_offsets is None:
        row_offsets = torch.empty(B + 1, dtype=torch.int64, device=dev)
    if survival is None:
        survival = torch.empty((B, K), dtype=torch.float32, device=dev)
    if curve_n is None:
        cn = ct = None
        npts = 0
    else:
        cn = (ctypes.c_float * len(curve_n))(*[float(x) for x in curve_n])
        ct = (ctypes.c_float * len(curve_latency))(*[float(x) for x in curve_latency])
        npts = len(curve_n)
    workspace = _workspace(workspace, dspark_schedule_workspace_bytes(B, K), dev)
    _check(lib().dspark_schedule(
        _ptr(conf), B, K, int(budget_tokens), cn, ct, npts, _ptr(lengths), _ptr(row_offsets),
        _ptr(survival), _ptr(workspace), workspace.numel(), _stream(stream, dev)))
    return lengths, row_offsets, survival


def dspark_verify(draft_tokens, prev_token, draft_logp, draft_lse, base_logits, A, W,
                  target_logits, target_row_offsets, temperature, seed, lengths=None, *,
                  accepted=None, next_token=None, row_lse_t=None, row_logratio=None,
                  row_outputs=True, workspace=None, stream=None):
    """Rejection-sampling verification; returns (accepted, next_token, row_lse_t, row_logratio).

    target_logits is [rows, V] (or [B, K+1, V], viewed as rows); request b's
    rows start at target_row_offsets[b] (int64, [B] or more entries).
    row_outputs=False passes no per-row outputs (both returned as None): the
    library then reads only the target rows that can decide the result.
    A = W = None verifies tokens drafted without the Markov head (zero bias)."""
    for t, n in ((draft_tokens, "draft_tokens"), (prev_token, "prev_token"),
                 (draft_logp, "draft_logp"), (draft_lse, "draft_lse"),
                 (base_logits, "base_logits"),
                 (target_logits, "target_logits"), (target_row_offsets, "target_row_offsets"),
                 (temperature, "temperature")):
        _dev(t, n)
    B, K, V = base_logits.shape
    if A is None and W is None:
        r, fdt = 1, _dtype(base_logits, "base_logits")
    else:
        _dev(A, "A")
        _dev(W, "W")
        r, fdt = A.shape[1], _dtype(A, "A")
    if target_logits.dtype != base_logits.dtype:
        raise DsparkError(DSPARK_ERR_INVALID_ARG, "target and base logits must share a dtype")
    if target_row_offsets.dtype != torch.int64 or target_row_offsets.numel() < B:
        raise DsparkError(DSPARK_ERR_INVALID_ARG, "target_row_offsets: int64 with >= B entries")
    n_rows = target_logits.numel() // V
    dev = base_logits.device
    if lengths is not None:
        _dev(lengths, "lengths")
    if accepted is None:
        accepted = torch.empty(B, dtype=torch.int32, device=dev)
    if next_token is None:
        next_token = torch.empty(B, dtype=torch.int32, device=dev)
    if not row_outputs:
        if row_lse_t is not None or row_logratio is not None:
            raise DsparkError(DSPARK_ERR_INVALID_ARG, "row outputs given with row_outputs=False")
    else:
        if row_lse_t is None:
            row_lse_t = torch.full((n_rows,), float("nan"), dtype=torch.float32, device=dev)
        if row_logratio is None:
            row_logratio = torch.full((n_rows,), float("nan"), dtype=torch.float32, device=dev)
    workspace = _workspace(workspace, dspark_verify_workspace_bytes(B, K, V, r), dev)
    _check(lib().dspark_verify(
        _ptr(draft_tokens), _ptr(prev_token), _ptr(draft_logp), _ptr(draft_lse),
        _ptr(base_logits), _dtype(base_logits, "base_logits"), _ptr(A), _ptr(W),
        fdt, _ptr(target_logits), n_rows, _ptr(target_row_offsets), _ptr(lengths),
        _ptr(temperature), int(seed) & (2**64 - 1), B, K, V, r, _ptr(accepted),
        _ptr(next_token), _ptr(row_lse_t), _ptr(row_logratio), _ptr(workspace),
        workspace.numel(), _stream(stream, dev)))
    return accepted, next_token, row_lse_t, row_logratio


def dspark_profile_begin(kernels=KERNELS, max_launches=4096):
    """Open a per-kernel event-timing session for the named kernels."""
    mask = 0
    for k in kernels:
        mask |= 1 << KERNELS.index(k)
    _check(lib().dspark_profile_begin(mask, max_launches))


def dspark_profile_end():
    """Close the session; returns {kernel: (total_ms, launches, timed_launches)}."""
    n = len(KERNELS)
    ms = (ctypes.c_double * n)()
    launches = (ctypes.c_int64 * n)()
    timed = (ctypes.c_int64 * n)()
    _check(lib().dspark_profile_end(ctypes.cast(ms, _P), ctypes.cast(launches, _P),
                                    ctypes.cast(timed, _P)))
    return {k: (ms[i], launches[i], timed[i]) for i, k in enumerate(KERNELS)}
