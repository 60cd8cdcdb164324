"""The C-ABI library on the host: it loads, exports every symbol the header declares, and
rejects bad arguments before touching the GPU.  No kernel is launched here."""
import ctypes
import re
from pathlib import Path

import pytest

import speculative_sampling_verification_spec_amd as sv

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "spec_verify.h"

P = ctypes.c_void_p
FAKE = P(4096)   # never dereferenced: every call below fails validation first


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(spec_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert names == ["spec_ngram_propose", "spec_verify_commit", "spec_verify_greedy",
                     "spec_verify_sample", "spec_verify_sample_static", "spec_verify_strerror",
                     "spec_verify_workspace_size"]
    lib = sv.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_workspace_size_and_strerror():
    assert sv.spec_verify_workspace_size(64, 4, 128256, sv.SPEC_BF16) > 0
    assert sv.spec_verify_workspace_size(1, 0, 1, sv.SPEC_F32) > 0
    assert sv.spec_verify_workspace_size(1, 65, 100, sv.SPEC_F32) == 0
    assert sv.spec_verify_workspace_size(1, 4, 0, sv.SPEC_F32) == 0
    assert sv.spec_verify_workspace_size(1, 4, 100, 7) == 0
    assert sv.spec_verify_workspace_size(-1, 4, 100, 0) == 0
    for code in (0, -1, -2, -3, -4, -5, -6, -99):
        assert isinstance(sv.spec_verify_strerror(code), str)
    assert "NULL" in sv.spec_verify_strerror(-1)


def _sample(**kw):
    a = dict(t=FAKE, d=FAKE, dtype=0, tok=FAKE, u=FAKE, temp=FAKE, B=2, gamma=3, cu=None,
             V=1000, out=FAKE, n=FAKE, ws=P(4096), wsb=1 << 20, probe=None, stream=None)
    a.update(kw)
    return sv.lib().spec_verify_sample(a["t"], a["d"], a["dtype"], a["tok"], a["u"], a["temp"],
                                       a["B"], a["gamma"], a["cu"], a["V"], a["out"], a["n"],
                                       a["ws"], a["wsb"], a["probe"], a["stream"])


def _greedy(**kw):
    a = dict(t=FAKE, dtype=1, tok=FAKE, B=2, gamma=3, cu=None, V=1000, out=FAKE, n=FAKE,
             ws=P(4096), wsb=1 << 20, probe=None, stream=None)
    a.update(kw)
    return sv.lib().spec_verify_greedy(a["t"], a["dtype"], a["tok"], a["B"], a["gamma"], a["cu"],
                                       a["V"], a["out"], a["n"], a["ws"], a["wsb"], a["probe"],
                                       a["stream"])


@pytest.mark.parametrize("field", ["t", "d", "tok", "u", "temp", "out", "n", "ws"])
def test_sample_rejects_null_pointers(field):
    assert _sample(**{field: None}) == -1


@pytest.mark.parametrize("field", ["t", "tok", "out", "n", "ws"])
def test_greedy_rejects_null_pointers(field):
    assert _greedy(**{field: None}) == -1


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=2), -3), (dict(dtype=-1), -3),
    (dict(B=-1), -2), (dict(gamma=-1), -2), (dict(gamma=65), -2), (dict(V=0), -2),
    (dict(V=1 << 31), -2), (dict(V=(1 << 24) + 1), -2),
    (dict(wsb=16), -4), (dict(ws=P(4096 + 8)), -4),
])
def test_bad_arguments_return_codes(kw, code):
    assert _sample(**kw) == code
    kw = {k: v for k, v in kw.items()}
    assert _greedy(**kw) == code


def test_largest_vocabulary_is_accepted():
    # V = 2^24 is the largest vocabulary; its workspace is sized, and only the workspace
    # (too small here) stops the call before anything is enqueued
    assert sv.spec_verify_workspace_size(2, 2, 1 << 24, sv.SPEC_BF16) > 0
    assert _sample(V=1 << 24, wsb=4096) == -4
    assert _greedy(V=1 << 24, wsb=4096) == -4


def test_empty_batch_is_a_no_op():
    assert _sample(B=0, t=None, d=None, tok=None, u=None, temp=None, out=None, n=None,
                   ws=None, wsb=0) == 0
    assert _greedy(B=0, t=None, tok=None, out=None, n=None, ws=None, wsb=0) == 0


def test_workspace_one_byte_short_is_refused():
    need = sv.spec_verify_workspace_size(2, 3, 1000, 0)
    assert _sample(wsb=need - 1) == -4


def _commit(**kw):
    a = dict(out=FAKE, n=FAKE, cu=None, B=2, gamma=3, seq=FAKE, cap=16, seq_len=FAKE,
             stats=None, hist=None, stream=None)
    a.update(kw)
    return sv.lib().spec_verify_commit(a["out"], a["n"], a["cu"], a["B"], a["gamma"], a["seq"],
                                       a["cap"], a["seq_len"], a["stats"], a["hist"],
                                       a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), -2), (dict(gamma=65), -2), (dict(gamma=-1), -2), (dict(cap=-1), -2),
    (dict(out=None), -1), (dict(n=None), -1), (dict(seq=None), -1), (dict(seq_len=None), -1),
])
def test_commit_rejects_bad_arguments_before_launching(kw, code):
    assert _commit(**kw) == code


def test_commit_with_no_requests_is_a_no_op():
    assert _commit(B=0, out=None, n=None, seq=None, seq_len=None) == 0


def _ngram(**kw):
    a = dict(seq=FAKE, cap=32, ln=FAKE, B=2, n_min=1, n_max=3, gamma=4, counts=FAKE, dense=FAKE,
             cu=None, packed=None, stream=None)
    a.update(kw)
    return sv.lib().spec_ngram_propose(a["seq"], a["cap"], a["ln"], a["B"], a["n_min"],
                                       a["n_max"], a["gamma"], a["counts"], a["dense"], a["cu"],
                                       a["packed"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), -2), (dict(n_min=0), -2), (dict(n_min=4, n_max=3), -2), (dict(n_max=65), -2),
    (dict(gamma=65), -2), (dict(cap=-1), -2), (dict(cap=1 << 31), -2),
    (dict(B=1 << 30, gamma=64), -2),
    (dict(seq=None), -1), (dict(ln=None), -1), (dict(counts=None), -1), (dict(dense=None), -1),
    (dict(cu=FAKE), -1), (dict(packed=FAKE), -1),
])
def test_ngram_rejects_bad_arguments_before_launching(kw, code):
    assert _ngram(**kw) == code


def test_ngram_outputs_may_be_null_when_nothing_is_proposed():
    # gamma == 0: out_dense and out_packed are never written; the call proceeds to launch,
    # so only the argument check is exercised here (B == 0 keeps it off the GPU)
    assert _ngram(B=0, gamma=0, dense=None, cu=FAKE, packed=None) == 0


def test_ngram_with_no_requests_is_a_no_op():
    assert _ngram(B=0, seq=None, ln=None, counts=None, dense=None) == 0


@pytest.mark.parametrize("path", [-1, 3, 7])
def test_unknown_launch_path_is_a_shape_error(path):
    # the probe's launch-path field is checked on the host, before anything is enqueued
    pr = sv.make_probe(path=path)
    assert _sample(probe=ctypes.byref(pr)) == -2
    assert _greedy(probe=ctypes.byref(pr)) == -2


def test_workspace_keeps_a_fixed_counter_region():
    # the one-launch counters (2 x 2048, one per 128-byte line) come first in every workspace,
    # so sizes grow by that much at least and any shape finds them at offset 0
    assert sv.spec_verify_workspace_size(1, 0, 1, sv.SPEC_F32) >= sv.COUNTER_BYTES
    assert sv.spec_verify_workspace_size(1, 0, 1, sv.SPEC_F32) < sv.COUNTER_BYTES + 4096


def test_probe_struct_matches_the_header(tmp_path):
    # the binding's ctypes mirror of spec_probe against the C compiler's layout of the header
    import subprocess
    fields = [f for f, _ in sv._Probe._fields_]
    src = tmp_path / "layout.c"
    src.write_text('#include <stdio.h>\n#include "spec_verify.h"\nint main(void) {\n'
                   '  printf("%zu\\n", sizeof(spec_probe));\n' +
                   "".join(f'  printf("%zu\\n", offsetof(spec_probe, {f}));\n' for f in fields) +
                   "  return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-I", str(ROOT / "include"), str(src), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], check=True, capture_output=True,
                                          text=True).stdout.split()]
    assert got[0] == ctypes.sizeof(sv._Probe)
    assert got[1:] == [getattr(sv._Probe, f).offset for f in fields]


def _static(**kw):
    a = dict(t=FAKE, d=FAKE, dtype=1, tok=FAKE, u=FAKE, temp=FAKE, B=2, gamma=3, cu=None,
             V=1000, out=FAKE, n=FAKE, probe=None, stream=None)
    a.update(kw)
    return sv.lib().spec_verify_sample_static(a["t"], a["d"], a["dtype"], a["tok"], a["u"],
                                              a["temp"], a["B"], a["gamma"], a["cu"], a["V"],
                                              a["out"], a["n"], a["probe"], a["stream"])


@pytest.mark.parametrize("field", ["t", "d", "tok", "u", "temp", "out", "n"])
def test_static_entry_point_rejects_null_pointers(field):
    assert _static(**{field: None}) == -1


def test_static_entry_point_refuses_calls_beyond_its_scratch():
    # the size check comes before anything touches the device
    assert sv.spec_verify_workspace_size(512, 8, 128256, sv.SPEC_BF16) \
        <= sv.SPEC_STATIC_SCRATCH_BYTES
    big = dict(B=4096, gamma=8, V=128256)
    assert sv.spec_verify_workspace_size(4096, 8, 128256, sv.SPEC_BF16) \
        > sv.SPEC_STATIC_SCRATCH_BYTES
    assert _static(**big) == sv.SPEC_ERR_TOO_LARGE
    assert "SPEC_STATIC_SCRATCH_BYTES" in sv.spec_verify_strerror(sv.SPEC_ERR_TOO_LARGE)
    assert _static(B=2, gamma=65) == -2 and _static(dtype=9) == -3
    assert _static(B=0, t=None) == 0
