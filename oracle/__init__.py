"""fp64 CPU oracle of the speculative-sampling verification step (ctypes binding).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this package.  The HIP library never calls it and shares no code
with it: the oracle is written from the method's definition in plain C (``spec_oracle.c``,
which states every passage and reading it follows) and compiled with gcc, no fast-math and no
FMA contraction.

Parity status: every function here is pinned by the CPU tests in ``tests/test_oracle_pins.py``
against closed forms, library routines, invariants and the worked example of the pages; no
function is left "parity unpinned" except the specific token ids of the seeded workloads,
which the pages cannot fix (the oracle is their only reference).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path
from typing import Optional, Sequence

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "spec_oracle.c"
_LIB_PATH = _HERE / "liboracle.so"
_lib = None

GCC_FLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-shared", "-fPIC",
             "-std=c11", "-Wall"]


def build() -> Path:
    """Compile the oracle to ``oracle/liboracle.so`` (always recompiles)."""
    tmp = _LIB_PATH.with_suffix(".so.tmp")
    cmd = ["gcc", *GCC_FLAGS, str(_SRC), "-o", str(tmp), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not _LIB_PATH.exists():
            build()
        lib = ctypes.CDLL(str(_LIB_PATH))
        P = ctypes.c_void_p
        lib.oracle_verify.restype = ctypes.c_int
        lib.oracle_verify.argtypes = [P, P, ctypes.c_int, P, P, P, ctypes.c_int32,
                                      ctypes.c_int32, P, ctypes.c_int64, P, ctypes.c_int32,
                                      P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int]
        lib.oracle_commit.restype = ctypes.c_int
        lib.oracle_commit.argtypes = [P, P, P, ctypes.c_int32, ctypes.c_int32, P,
                                      ctypes.c_int64, P, P, P]
        lib.oracle_ngram.restype = ctypes.c_int
        lib.oracle_ngram.argtypes = [P, ctypes.c_int64, P, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P]
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def verify(w, requests: Optional[Sequence[int]] = None, greedy: bool = False,
           threads: int = 0) -> dict:
    """Run the oracle on workload ``w`` (a ``workloads.Workload``).

    ``requests``: subset of request ids to compute (default all); slots of other requests
    stay at their fill values (tokens -2, diagnostics NaN).  ``greedy=True`` gives the
    greedy entry point's semantics: temperatures ignored, draft logits never read.
    """
    lib = _load()
    dt = {"f32": 0, "bf16": 1}[w.dtype]
    tgt = np.ascontiguousarray(w.target)
    dft = np.ascontiguousarray(w.draft)
    toks = np.ascontiguousarray(w.draft_tokens, dtype=np.int32)
    unif = np.ascontiguousarray(w.uniforms, dtype=np.float32)
    temps = None if greedy else np.ascontiguousarray(w.temperatures, dtype=np.float32)
    cu = None if w.cu_draft is None else np.ascontiguousarray(w.cu_draft, dtype=np.int32)
    req = None if requests is None else np.ascontiguousarray(requests, dtype=np.int32)
    R_t, R_d, B = w.R_t, w.R_d, w.B
    out = dict(
        out_tokens=np.full(R_t, -2, dtype=np.int32),
        num_accepted=np.full(B, -2, dtype=np.int32),
        p_x=np.full(R_d, np.nan), q_x=np.full(R_d, np.nan), margin=np.full(R_d, np.nan),
        row_max_t=np.full(R_t, np.nan), row_sum_t=np.full(R_t, np.nan),
        row_max_d=np.full(R_d, np.nan), row_sum_d=np.full(R_d, np.nan),
        resid_mass=np.full(B, np.nan), cdf_gap=np.full(B, np.nan),
        fallback=np.zeros(B, dtype=np.int32),
    )
    rc = lib.oracle_verify(
        _ptr(tgt), _ptr(dft), dt, _ptr(toks), _ptr(unif), _ptr(temps), B, w.gamma, _ptr(cu),
        w.V, _ptr(req), 0 if req is None else len(req), _ptr(out["out_tokens"]),
        _ptr(out["num_accepted"]), _ptr(out["p_x"]), _ptr(out["q_x"]), _ptr(out["margin"]),
        _ptr(out["row_max_t"]), _ptr(out["row_sum_t"]), _ptr(out["row_max_d"]),
        _ptr(out["row_sum_d"]), _ptr(out["resid_mass"]), _ptr(out["cdf_gap"]),
        _ptr(out["fallback"]), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_verify rejected its arguments (rc={rc})")
    return out


def commit(out_tokens: np.ndarray, num_accepted: np.ndarray, gamma: int, seq_tokens: np.ndarray,
           seq_len: np.ndarray, cu_draft: Optional[np.ndarray] = None,
           stats: Optional[np.ndarray] = None, hist: Optional[np.ndarray] = None) -> None:
    """Commit one step's emitted tokens into the histories ``seq_tokens [B, capacity]``
    (int32, updated in place with ``seq_len [B]``) and accumulate ``stats`` (uint64[5]:
    proposed, accepted, emitted, requests, truncated) and ``hist`` (uint64[gamma + 1])."""
    lib = _load()
    B = len(num_accepted)
    for a, dt in ((seq_tokens, np.int32), (seq_len, np.int32)):
        assert a.dtype == dt and a.flags.c_contiguous
    for a in (stats, hist):
        assert a is None or (a.dtype == np.uint64 and a.flags.c_contiguous)
    if hist is not None:
        assert len(hist) >= gamma + 1
    toks = np.ascontiguousarray(out_tokens, dtype=np.int32)
    nacc = np.ascontiguousarray(num_accepted, dtype=np.int32)
    cu = None if cu_draft is None else np.ascontiguousarray(cu_draft, dtype=np.int32)
    rc = lib.oracle_commit(_ptr(toks), _ptr(nacc), _ptr(cu), B, int(gamma), _ptr(seq_tokens),
                           seq_tokens.shape[1], _ptr(seq_len), _ptr(stats), _ptr(hist))
    if rc != 0:
        raise ValueError(f"oracle_commit rejected its arguments (rc={rc})")


def ngram(seq_tokens: np.ndarray, seq_len: np.ndarray, n_min: int, n_max: int,
          gamma: int) -> dict:
    """Prompt-lookup proposals for every request's context ``seq_tokens[b, :seq_len[b]]``:
    counts, dense [B, gamma] (-1 padded), cu [B + 1], packed [sum counts], match_j, match_n."""
    lib = _load()
    seq = np.ascontiguousarray(seq_tokens, dtype=np.int32)
    ln = np.ascontiguousarray(seq_len, dtype=np.int32)
    B, cap = seq.shape
    out = dict(counts=np.full(B, -2, dtype=np.int32),
               dense=np.full((B, gamma), -2, dtype=np.int32),
               cu=np.full(B + 1, -2, dtype=np.int32),
               packed=np.full(max(B * gamma, 1), -2, dtype=np.int32),
               match_j=np.full(B, -2, dtype=np.int32), match_n=np.full(B, -2, dtype=np.int32))
    rc = lib.oracle_ngram(_ptr(seq), cap, _ptr(ln), B, int(n_min), int(n_max), int(gamma),
                          _ptr(out["counts"]), _ptr(out["dense"]), _ptr(out["cu"]),
                          _ptr(out["packed"]), _ptr(out["match_j"]), _ptr(out["match_n"]))
    if rc != 0:
        raise ValueError(f"oracle_ngram rejected its arguments (rc={rc})")
    out["packed"] = out["packed"][: int(out["cu"][-1])]
    return out


def tokens_by_request(w, out_tokens: np.ndarray) -> list:
    """Split the flat output slots into one array of gamma_b + 1 slots per request."""
    tb = w.target_base
    return [out_tokens[tb[b]: tb[b] + g + 1] for b, g in enumerate(w.gammas)]
