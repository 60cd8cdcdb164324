"""Run a seeded workload through the HIP library (C ABI via the binding) on cuda:0."""
from __future__ import annotations

import numpy as np

import speculative_sampling_verification_spec_amd as sv
import workloads


def to_device(w, device="cuda"):
    return workloads.to_torch(w, device)


def launches(w, *, greedy: bool = False, path: int = sv.SPEC_PATH_AUTO) -> int:
    """Kernel launches one call makes on workload ``w``, read from the probe's event slots
    (the library records events 2k / 2k+1 around its k-th launch)."""
    import ctypes
    import torch
    hip = ctypes.CDLL("libamdhip64.so")
    evs = []
    for _ in range(8):
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    d = to_device(w)
    code = sv.SPEC_F32 if w.dtype == "f32" else sv.SPEC_BF16
    ws = sv.alloc_workspace(w.B, w.gamma, w.V, code)
    out = torch.empty(w.R_t, dtype=torch.int32, device="cuda")
    nacc = torch.empty(w.B, dtype=torch.int32, device="cuda")
    pr = sv.make_probe(events=evs, path=path)
    if greedy:
        sv.spec_verify_greedy(d["target"], d["tokens"], w.gamma, out, nacc, ws,
                              cu_draft=d["cu"], probe=pr)
    else:
        sv.spec_verify_sample(d["target"], d["draft"], d["tokens"], d["uniforms"], d["temps"],
                              w.gamma, out, nacc, ws, cu_draft=d["cu"], probe=pr)
    torch.cuda.synchronize()
    n = 0
    ms = ctypes.c_float()
    for k in range(4):
        if hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(evs[2 * k]),
                                   ctypes.c_void_p(evs[2 * k + 1])) != 0:
            hip.hipGetLastError()  # events never recorded: clear the error the query left
            break
        n += 1
    for e in evs:
        hip.hipEventDestroy(ctypes.c_void_p(e))
    return n


def run(w, *, greedy: bool = False, probe: bool = True, dev=None, workspace=None,
        sync: bool = True, path: int = sv.SPEC_PATH_AUTO) -> dict:
    """Verify workload ``w`` on the GPU; returns numpy outputs (and probe arrays).  ``path``
    selects the launch path (one of sv.SPEC_PATH_*; the library's choice by default)."""
    import torch
    d = to_device(w) if dev is None else dev
    code = sv.SPEC_F32 if w.dtype == "f32" else sv.SPEC_BF16
    ws = sv.alloc_workspace(w.B, w.gamma, w.V, code) if workspace is None else workspace
    out = torch.full((w.R_t,), -7, dtype=torch.int32, device="cuda")
    nacc = torch.full((w.B,), -7, dtype=torch.int32, device="cuda")
    pr = None
    tensors = {}
    if probe:
        f64 = dict(dtype=torch.float64, device="cuda")
        f32 = dict(dtype=torch.float32, device="cuda")
        tensors = dict(p_x=torch.full((w.R_d,), np.nan, **f64),
                       q_x=torch.full((w.R_d,), np.nan, **f64),
                       row_max_t=torch.full((w.R_t,), np.nan, **f32),
                       row_sum_t=torch.full((w.R_t,), np.nan, **f64),
                       row_max_d=torch.full((w.R_d,), np.nan, **f32),
                       row_sum_d=torch.full((w.R_d,), np.nan, **f64),
                       resid_mass=torch.full((w.B,), np.nan, **f64))
        pr = sv.make_probe(**tensors, path=path)
    elif path != sv.SPEC_PATH_AUTO:
        pr = sv.make_probe(path=path)
    if greedy:
        sv.spec_verify_greedy(d["target"], d["tokens"], w.gamma, out, nacc, ws,
                              cu_draft=d["cu"], probe=pr)
    else:
        sv.spec_verify_sample(d["target"], d["draft"], d["tokens"], d["uniforms"], d["temps"],
                              w.gamma, out, nacc, ws, cu_draft=d["cu"], probe=pr)
    if not sync:
        return dict(out=out, nacc=nacc, **tensors)
    torch.cuda.synchronize()
    res = dict(out_tokens=out.cpu().numpy(), num_accepted=nacc.cpu().numpy())
    for k, t in tensors.items():
        res[k] = t.cpu().numpy()
    return res
