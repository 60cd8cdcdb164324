"""The entry points inside a captured HIP graph (torch.cuda.CUDAGraph), and on concurrent
streams.

The library neither allocates, synchronises nor records memset nodes during a call, so a
serving loop can capture a whole step once and replay it.  Each test replays its graph
several times with fresh inputs copied in eagerly between replays (and a synchronisation
after each), and checks every replay: the sampling call against the same call made eagerly
(bit-identical), the decode loop against the oracle's chain step by step.
"""
import numpy as np
import pytest

import oracle
import speculative_sampling_verification_spec_amd as sv
import workloads

pytestmark = pytest.mark.gpu

AUTO, TWO, ONE = sv.SPEC_PATH_AUTO, sv.SPEC_PATH_TWO, sv.SPEC_PATH_ONE


def _say(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.mark.parametrize("path", [TWO, ONE], ids=["two", "one"])
def test_sampling_call_replays_in_a_graph(path):
    import torch
    B, gamma, V = 24, 4, 32000
    mixed = np.where(np.arange(B) % 4 == 0, 0.0, 0.9)  # greedy requests in a sampling call
    ws_list = [workloads.generate(name=f"graph{s}", B=B, V=V, dtype="bf16", gammas=[gamma] * B,
                                  dense=True, target_sigma=3.0, draft_sigma=1.0,
                                  temperatures=0.7 if s != 1 else mixed, seed=300 + s)
               for s in range(3)]
    _say(f"graph sampling B={B} gamma={gamma} V={V} path={path}")
    host = [workloads.to_torch(w, "cpu") for w in ws_list]
    dev = {k: v.cuda() for k, v in host[0].items() if v is not None}
    assert host[0].get("cu") is None  # dense layout: the graph's buffers keep one shape
    out = torch.empty(ws_list[0].R_t, dtype=torch.int32, device="cuda")
    nacc = torch.empty(B, dtype=torch.int32, device="cuda")
    ws = sv.alloc_workspace(B, gamma, V, sv.SPEC_BF16)
    probe = sv.make_probe(path=path)

    def load(i):
        for k, v in host[i].items():
            if v is not None:
                dev[k].copy_(v)
        out.fill_(-7)
        nacc.fill_(-7)
        torch.cuda.synchronize()

    def call():
        sv.spec_verify_sample(dev["target"], dev["draft"], dev["tokens"], dev["uniforms"],
                              dev["temps"], gamma, out, nacc, ws, probe=probe)

    eager = []
    for i in range(3):
        load(i)
        call()
        torch.cuda.synchronize()
        eager.append((out.cpu().numpy().copy(), nacc.cpu().numpy().copy()))
    # the eager results themselves follow the oracle (also covered by the parity tests)
    o = oracle.verify(ws_list[0])
    assert (eager[0][1] == o["num_accepted"]).mean() > 0.9

    g = torch.cuda.CUDAGraph()
    load(0)
    with torch.cuda.graph(g):  # the eager calls above loaded the code objects
        call()
    torch.cuda.synchronize()
    for rnd, i in enumerate([0, 1, 2, 2, 0, 1]):
        load(i)
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy(), eager[i][0], err_msg=f"replay {rnd}")
        np.testing.assert_array_equal(nacc.cpu().numpy(), eager[i][1], err_msg=f"replay {rnd}")
        # eager work on the same workspace between replays
        if rnd == 2:
            load(1)
            call()
            torch.cuda.synchronize()
            np.testing.assert_array_equal(nacc.cpu().numpy(), eager[1][1])
    _say("graph sampling: every replay matched the eager call")


def _step_targets(o_ngram, seq, length, B, gamma, V, rng):
    """Target logits for one decode step, laid out by the proposals' CSR (row i of request b
    peaks at the token the target "wants" there), chosen so that the loop keeps drafting: a
    quarter of the requests reject a seeded proposal (a random token there); the others accept
    every proposal and emit the token that followed the matched window in the context, and a
    request without proposals emits a token that recreates a 2-token match."""
    counts = o_ngram["counts"]
    R_t = int(counts.sum()) + B
    target = rng.normal(0.0, 1.0, size=(B * (gamma + 1), V))
    t = 0
    for b in range(B):
        k, L, h = int(counts[b]), int(length[b]), seq[b]
        wants = [int(x) for x in o_ngram["dense"][b, :k]]
        if k and rng.random() < 0.25:
            brk = int(rng.integers(0, k))
            wants = wants[:brk] + [int((wants[brk] + 1 + rng.integers(0, V - 1)) % V)]
        elif k:
            nxt = int(o_ngram["match_j"][b]) + int(o_ngram["match_n"][b]) + k
            wants.append(int(h[nxt]) if nxt < L else int(rng.integers(0, V)))
        else:
            q = [x for x in range(L - 1) if h[x] == h[L - 1]]
            wants.append(int(h[q[-1] + 1]) if q else int(rng.integers(0, V)))
        for i, want in enumerate(wants):
            target[t + i, want] += 10.0
        t += k + 1
    return workloads.encode(target, "f32"), R_t


def test_decode_loop_replays_in_a_graph():
    # prompt lookup -> greedy verification -> commit, captured once and replayed as a decode
    # loop: each replay drafts from the histories the previous replay committed.
    import torch
    B, cap, gamma, V, n_min, n_max, steps = 64, 1024, 5, 2048, 2, 4, 8
    seq, length = workloads.token_contexts(B, cap, seed=41, alphabet=V, min_fill=0.4)
    length = np.minimum(length, cap - steps * (gamma + 1)).astype(np.int32)
    _say(f"graph decode loop B={B} gamma={gamma} V={V} steps={steps}")
    d = dict(seq=torch.from_numpy(seq).cuda(), len=torch.from_numpy(length).cuda(),
             counts=torch.zeros(B, dtype=torch.int32, device="cuda"),
             dense=torch.zeros(B * gamma, dtype=torch.int32, device="cuda"),
             cu=torch.zeros(B + 1, dtype=torch.int32, device="cuda"),
             packed=torch.zeros(B * gamma, dtype=torch.int32, device="cuda"),
             target=torch.zeros((B * (gamma + 1), V), dtype=torch.float32, device="cuda"),
             out=torch.zeros(B * (gamma + 1), dtype=torch.int32, device="cuda"),
             nacc=torch.zeros(B, dtype=torch.int32, device="cuda"),
             stats=torch.zeros(5, dtype=torch.int64, device="cuda"),
             hist=torch.zeros(gamma + 1, dtype=torch.int64, device="cuda"))
    ws = sv.alloc_workspace(B, gamma, V, sv.SPEC_F32)

    def step():
        sv.spec_ngram_propose(d["seq"], d["len"], n_min, n_max, gamma, d["counts"], d["dense"],
                              d["cu"], d["packed"])
        sv.spec_verify_greedy(d["target"], d["packed"], gamma, d["out"], d["nacc"], ws,
                              cu_draft=d["cu"])
        sv.spec_verify_commit(d["out"], d["nacc"], gamma, d["seq"], d["len"], cu_draft=d["cu"],
                              stats=d["stats"], accept_hist=d["hist"])

    # One eager step first (code objects load outside the capture), then the capture; the
    # state is restored afterwards.
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    d["seq"].copy_(torch.from_numpy(seq))
    d["len"].copy_(torch.from_numpy(length))
    d["stats"].zero_()
    d["hist"].zero_()
    torch.cuda.synchronize()

    rng = np.random.default_rng(43)
    seq_o, len_o = seq.copy(), length.copy()
    stats_o = np.zeros(5, dtype=np.uint64)
    hist_o = np.zeros(gamma + 1, dtype=np.uint64)
    accepted = 0
    for s in range(steps):
        o = oracle.ngram(seq_o, len_o, n_min, n_max, gamma)
        tgt, R_t = _step_targets(o, seq_o, len_o, B, gamma, V, rng)
        d["target"].copy_(torch.from_numpy(tgt))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        # the oracle's chain for the same step
        w = workloads.Workload(f"loop{s}", "f32", B, gamma, V, tgt[:R_t],
                               np.zeros((max(int(o["counts"].sum()), 1), V), dtype=np.float32),
                               o["packed"].astype(np.int32), np.zeros((R_t, 2), dtype=np.float32),
                               np.zeros(B, dtype=np.float32), o["cu"].astype(np.int32))
        ov = oracle.verify(w, greedy=True)
        oracle.commit(ov["out_tokens"], ov["num_accepted"], gamma, seq_o, len_o,
                      cu_draft=w.cu_draft, stats=stats_o, hist=hist_o)
        np.testing.assert_array_equal(d["counts"].cpu().numpy(), o["counts"], err_msg=f"step {s}")
        np.testing.assert_array_equal(d["nacc"].cpu().numpy(), ov["num_accepted"],
                                      err_msg=f"step {s}")
        np.testing.assert_array_equal(d["len"].cpu().numpy(), len_o, err_msg=f"step {s}")
        np.testing.assert_array_equal(d["seq"].cpu().numpy(), seq_o, err_msg=f"step {s}")
        accepted += int(ov["num_accepted"].sum())
        _say(f"  step {s}: proposed {int(o['counts'].sum())}, accepted "
             f"{int(ov['num_accepted'].sum())}")
    np.testing.assert_array_equal(d["stats"].cpu().numpy().astype(np.uint64), stats_o)
    np.testing.assert_array_equal(d["hist"].cpu().numpy().astype(np.uint64), hist_o)
    assert accepted > steps * B  # the loop keeps drafting and accepting


@pytest.mark.parametrize("path", [TWO, AUTO], ids=["two", "auto"])
def test_concurrent_calls_on_two_streams(path):
    # The library keeps no state between calls: two callers on two streams (default
    # priority), each with its own workspace and outputs, interleave their calls; every result
    # equals the same call made alone.  (The calls here are far below the one-launch path's
    # resident bound, which AUTO takes for them, so both can be resident together.)
    import torch
    ws_list = [workloads.small(B=16, gamma=4, V=32000, dtype="bf16", seed=400 + i,
                               ragged=i == 1, temperatures=np.where(np.arange(16) % 5 == 0,
                                                                    0.0, 0.8))
               for i in range(2)]
    _say(f"two streams, path={path}")
    dev = [workloads.to_torch(w) for w in ws_list]
    wsp = [sv.alloc_workspace(w.B, w.gamma, w.V, sv.SPEC_BF16) for w in ws_list]
    outs = [[torch.full((w.R_t,), -7, dtype=torch.int32, device="cuda") for _ in range(6)]
            for w in ws_list]
    naccs = [[torch.full((w.B,), -7, dtype=torch.int32, device="cuda") for _ in range(6)]
             for w in ws_list]
    probe = sv.make_probe(path=path)

    def call(i, k):
        w, d = ws_list[i], dev[i]
        sv.spec_verify_sample(d["target"], d["draft"], d["tokens"], d["uniforms"], d["temps"],
                              w.gamma, outs[i][k], naccs[i][k], wsp[i], cu_draft=d["cu"],
                              probe=probe)

    for i in range(2):  # alone
        call(i, 0)
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for k in range(1, 6):
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                call(i, k)
    torch.cuda.synchronize()
    for i in range(2):
        for k in range(1, 6):
            np.testing.assert_array_equal(outs[i][k].cpu().numpy(), outs[i][0].cpu().numpy())
            np.testing.assert_array_equal(naccs[i][k].cpu().numpy(), naccs[i][0].cpu().numpy())
        o = oracle.verify(ws_list[i])
        assert (naccs[i][0].cpu().numpy() == o["num_accepted"]).mean() > 0.9
