"""Python binding of ``libspecverify.so`` (the C ABI in ``include/spec_verify.h``).

Argument marshalling only: every step of the verification runs in the library's HIP
kernels.  Functions carry the C names and take torch tensors on the GPU; torch supplies
device memory and the current stream, nothing else.  If the library has not been built the
import still succeeds, but every call raises: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
from pathlib import Path
from typing import Optional

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libspecverify.so"

SPEC_F32, SPEC_BF16 = 0, 1
SPEC_MAX_GAMMA = 64
SPEC_NGRAM_MAX_N = 64
SPEC_OK = 0
SPEC_PATH_AUTO, SPEC_PATH_TWO, SPEC_PATH_ONE = 0, 1, 2
SPEC_ERR_TOO_LARGE = -6
# the static scratch of spec_verify_sample_static (per device, for the life of the process)
SPEC_STATIC_SCRATCH_BYTES = 16 << 20
# the workspace's leading counter region (2 x 2048 counters, one per 128-byte line), which
# must be zero before a workspace's first use and which every call leaves at zero
COUNTER_BYTES = 2 * 2048 * 128

_lib = None


class SpecVerifyError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__(f"{where}: {spec_verify_strerror(code)} (code {code})")
        self.code = code


class _Probe(ctypes.Structure):
    _fields_ = [("p_x", ctypes.c_void_p), ("q_x", ctypes.c_void_p),
                ("row_max_t", ctypes.c_void_p), ("row_sum_t", ctypes.c_void_p),
                ("row_max_d", ctypes.c_void_p), ("row_sum_d", ctypes.c_void_p),
                ("resid_mass", ctypes.c_void_p), ("events", ctypes.c_void_p * 8),
                ("path", ctypes.c_int), ("spin_limit", ctypes.c_uint)]


def lib():
    """Load the HIP library; raises if it is missing (build it with ``build.build()``)."""
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(
                f"{LIB_PATH} is missing: build the HIP library first "
                "(python -m speculative_sampling_verification_spec_amd.build)")
        L = ctypes.CDLL(str(LIB_PATH))
        P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.spec_verify_sample.restype = ctypes.c_int
        L.spec_verify_sample.argtypes = [P, P, ctypes.c_int, P, P, P, i32, i32, P, i64, P, P,
                                         P, sz, P, P]
        L.spec_verify_sample_static.restype = ctypes.c_int
        L.spec_verify_sample_static.argtypes = [P, P, ctypes.c_int, P, P, P, i32, i32, P, i64,
                                                P, P, P, P]
        L.spec_verify_greedy.restype = ctypes.c_int
        L.spec_verify_greedy.argtypes = [P, ctypes.c_int, P, i32, i32, P, i64, P, P, P, sz, P,
                                         P]
        L.spec_verify_commit.restype = ctypes.c_int
        L.spec_verify_commit.argtypes = [P, P, P, i32, i32, P, i64, P, P, P, P]
        L.spec_ngram_propose.restype = ctypes.c_int
        L.spec_ngram_propose.argtypes = [P, i64, P, i32, i32, i32, i32, P, P, P, P, P]
        L.spec_verify_workspace_size.restype = sz
        L.spec_verify_workspace_size.argtypes = [i32, i32, i64, ctypes.c_int]
        L.spec_verify_strerror.restype = ctypes.c_char_p
        L.spec_verify_strerror.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def spec_verify_strerror(code: int) -> str:
    return lib().spec_verify_strerror(int(code)).decode()


def spec_verify_workspace_size(B: int, gamma: int, V: int, dtype: int) -> int:
    return int(lib().spec_verify_workspace_size(int(B), int(gamma), int(V), int(dtype)))


# ----------------------------------------------------------------------------- torch glue

def _torch():
    import torch
    return torch


def dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return SPEC_F32
    if t.dtype == torch.bfloat16:
        return SPEC_BF16
    raise ValueError(f"logits must be float32 or bfloat16, got {t.dtype}")


def _dev(t, name, dtype=None, numel=None):
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{name} has {t.numel()} elements, needs {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def make_probe(p_x=None, q_x=None, row_max_t=None, row_sum_t=None, row_max_d=None,
               row_sum_d=None, resid_mass=None, events=None, path=SPEC_PATH_AUTO,
               spin_limit=0) -> _Probe:
    """Diagnostics and launch-control struct; tensors (device) or None, ``events`` a list of
    up to 8 raw hipEvent_t handles (ints) or None, ``path`` one of SPEC_PATH_*,
    ``spin_limit`` the one-launch path's polling bound (0: the library's default)."""
    pr = _Probe()
    torch = _torch()
    for name, t, dt in (("p_x", p_x, torch.float64), ("q_x", q_x, torch.float64),
                        ("row_max_t", row_max_t, torch.float32),
                        ("row_sum_t", row_sum_t, torch.float64),
                        ("row_max_d", row_max_d, torch.float32),
                        ("row_sum_d", row_sum_d, torch.float64),
                        ("resid_mass", resid_mass, torch.float64)):
        p = _dev(t, name, dt)
        setattr(pr, name, p.value if p is not None else None)
    for i, e in enumerate(events or []):
        pr.events[i] = e
    pr.path = int(path)
    pr.spin_limit = int(spin_limit)
    return pr


def _check(rc: int, where: str):
    if rc != SPEC_OK:
        raise SpecVerifyError(rc, where)


def _sample_args(target_logits, draft_logits, draft_tokens, uniforms, temperatures, gamma,
                 out_tokens, out_num_accepted, workspace, cu_draft, probe, stream):
    torch = _torch()
    B = temperatures.numel()
    V = target_logits.shape[-1]
    dt = dtype_code(target_logits)
    if draft_logits.dtype != target_logits.dtype:
        raise ValueError("target and draft logits must share a dtype")
    return (
        _dev(target_logits, "target_logits"), _dev(draft_logits, "draft_logits"), dt,
        _dev(draft_tokens, "draft_tokens", torch.int32),
        _dev(uniforms, "uniforms", torch.float32),
        _dev(temperatures, "temperatures", torch.float32), B, int(gamma),
        _dev(cu_draft, "cu_draft", torch.int32, B + 1), V,
        _dev(out_tokens, "out_tokens", torch.int32),
        _dev(out_num_accepted, "out_num_accepted", torch.int32, B),
        _dev(workspace, "workspace"),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        None if probe is None else ctypes.byref(probe), _stream(stream))


def _greedy_args(target_logits, draft_tokens, gamma, out_tokens, out_num_accepted, workspace,
                 cu_draft, probe, stream):
    torch = _torch()
    B = out_num_accepted.numel()
    V = target_logits.shape[-1]
    return (
        _dev(target_logits, "target_logits"), dtype_code(target_logits),
        _dev(draft_tokens, "draft_tokens", torch.int32), B, int(gamma),
        _dev(cu_draft, "cu_draft", torch.int32, B + 1), V,
        _dev(out_tokens, "out_tokens", torch.int32),
        _dev(out_num_accepted, "out_num_accepted", torch.int32, B),
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        None if probe is None else ctypes.byref(probe), _stream(stream))


def spec_verify_sample(target_logits, draft_logits, draft_tokens, uniforms, temperatures,
                       gamma: int, out_tokens, out_num_accepted, workspace,
                       cu_draft=None, probe: Optional[_Probe] = None, stream=None) -> None:
    """Asynchronous on the current (or given) stream.  ``target_logits [R_t, V]`` and
    ``draft_logits [R_d, V]`` share one dtype (float32 / bfloat16); ``B`` is
    ``temperatures.numel()``; ``workspace`` is a uint8 tensor of at least
    ``spec_verify_workspace_size`` bytes."""
    args = _sample_args(target_logits, draft_logits, draft_tokens, uniforms, temperatures,
                        gamma, out_tokens, out_num_accepted, workspace, cu_draft, probe, stream)
    _check(lib().spec_verify_sample(*args), "spec_verify_sample")


def spec_verify_sample_static(target_logits, draft_logits, draft_tokens, uniforms,
                              temperatures, gamma: int, out_tokens, out_num_accepted,
                              cu_draft=None, probe: Optional[_Probe] = None,
                              stream=None) -> None:
    """``spec_verify_sample`` with no workspace argument and no allocation: the library's
    static per-device scratch (SPEC_STATIC_SCRATCH_BYTES) is used.  Calls that overlap on one
    device race; calls ordered on one stream are safe."""
    a = _sample_args(target_logits, draft_logits, draft_tokens, uniforms, temperatures, gamma,
                     out_tokens, out_num_accepted, None, cu_draft, probe, stream)
    _check(lib().spec_verify_sample_static(*a[:12], a[14], a[15]),
           "spec_verify_sample_static")


def spec_verify_greedy(target_logits, draft_tokens, gamma: int, out_tokens,
                       out_num_accepted, workspace, cu_draft=None,
                       probe: Optional[_Probe] = None, stream=None) -> None:
    """Temperature-zero verification; ``B`` is ``out_num_accepted.numel()``."""
    args = _greedy_args(target_logits, draft_tokens, gamma, out_tokens, out_num_accepted,
                        workspace, cu_draft, probe, stream)
    _check(lib().spec_verify_greedy(*args), "spec_verify_greedy")


def spec_verify_commit(out_tokens, out_num_accepted, gamma: int, seq_tokens, seq_len,
                       cu_draft=None, stats=None, accept_hist=None, stream=None) -> None:
    """Append a verification step's emitted tokens to the histories ``seq_tokens [B, cap]``
    (int32) at ``seq_len [B]`` (int32, updated), on the device; ``stats`` (int64 tensor of 5,
    read as uint64) and ``accept_hist`` (int64 tensor of gamma + 1) accumulate the step's
    counters.  ``B`` is ``out_num_accepted.numel()``."""
    torch = _torch()
    B = out_num_accepted.numel()
    if seq_tokens.dim() != 2 or seq_tokens.shape[0] < B:
        raise ValueError("seq_tokens must be [B, capacity]")
    rc = lib().spec_verify_commit(
        _dev(out_tokens, "out_tokens", torch.int32),
        _dev(out_num_accepted, "out_num_accepted", torch.int32, B),
        _dev(cu_draft, "cu_draft", torch.int32, B + 1), B, int(gamma),
        _dev(seq_tokens, "seq_tokens", torch.int32), seq_tokens.shape[1],
        _dev(seq_len, "seq_len", torch.int32, B),
        _dev(stats, "stats", torch.int64, 5),
        _dev(accept_hist, "accept_hist", torch.int64, int(gamma) + 1), _stream(stream))
    _check(rc, "spec_verify_commit")


def spec_ngram_propose(seq_tokens, seq_len, n_min: int, n_max: int, gamma: int, out_counts,
                       out_dense, out_cu=None, out_packed=None, stream=None) -> None:
    """Prompt-lookup drafts for the contexts ``seq_tokens [B, capacity]`` (int32) of lengths
    ``seq_len [B]``: ``out_counts [B]``, ``out_dense [B, gamma]`` and, optionally, the CSR pair
    ``out_cu [B + 1]`` / ``out_packed [B * gamma]`` that spec_verify_* take as cu_draft /
    draft_tokens.  ``B`` is ``seq_len.numel()``."""
    torch = _torch()
    B = seq_len.numel()
    if seq_tokens.dim() != 2 or seq_tokens.shape[0] < B:
        raise ValueError("seq_tokens must be [B, capacity]")
    rc = lib().spec_ngram_propose(
        _dev(seq_tokens, "seq_tokens", torch.int32), seq_tokens.shape[1],
        _dev(seq_len, "seq_len", torch.int32, B), B, int(n_min), int(n_max), int(gamma),
        _dev(out_counts, "out_counts", torch.int32, B),
        _dev(out_dense, "out_dense", torch.int32, B * int(gamma)),
        _dev(out_cu, "out_cu", torch.int32, B + 1),
        _dev(out_packed, "out_packed", torch.int32, B * int(gamma)), _stream(stream))
    _check(rc, "spec_ngram_propose")


class PreparedCall:
    """One entry-point call with its arguments checked and marshalled once.  Calling it runs
    the entry point again on the same buffers and stream; the caller keeps the tensors (and
    the probe) alive and refills the inputs in place between calls."""

    def __init__(self, fn, args, where, keep):
        self._fn, self._args, self._where, self._keep = fn, args, where, keep

    def __call__(self) -> None:
        _check(self._fn(*self._args), self._where)


def prepare_sample(target_logits, draft_logits, draft_tokens, uniforms, temperatures,
                   gamma: int, out_tokens, out_num_accepted, workspace, cu_draft=None,
                   probe: Optional[_Probe] = None, stream=None) -> PreparedCall:
    """``spec_verify_sample`` with the same arguments, marshalled once for repeated calls."""
    args = _sample_args(target_logits, draft_logits, draft_tokens, uniforms, temperatures,
                        gamma, out_tokens, out_num_accepted, workspace, cu_draft, probe, stream)
    return PreparedCall(lib().spec_verify_sample, args, "spec_verify_sample", probe)


def prepare_greedy(target_logits, draft_tokens, gamma: int, out_tokens, out_num_accepted,
                   workspace, cu_draft=None, probe: Optional[_Probe] = None,
                   stream=None) -> PreparedCall:
    """``spec_verify_greedy`` with the same arguments, marshalled once for repeated calls."""
    args = _greedy_args(target_logits, draft_tokens, gamma, out_tokens, out_num_accepted,
                        workspace, cu_draft, probe, stream)
    return PreparedCall(lib().spec_verify_greedy, args, "spec_verify_greedy", probe)


def alloc_workspace(B: int, gamma: int, V: int, dtype: int, device="cuda"):
    """Zero-filled uint8 device tensor of the size the library asks for (torch's allocations
    are 256-byte aligned); calls leave it ready for the next call of any shape."""
    torch = _torch()
    n = spec_verify_workspace_size(B, gamma, V, dtype)
    if n == 0:
        raise ValueError("invalid sizes for spec_verify")
    return torch.zeros(n, dtype=torch.uint8, device=device)
