"""HIP path vs the fp64 oracle on the same seeded inputs, through the C ABI.

Small shapes and the five workloads at full size (in the launch configuration the benchmark
times) run the oracle on every request.  Calls small enough for the one-launch path run on
both launch paths.
"""
import numpy as np
import pytest

import oracle
import speculative_sampling_verification_spec_amd as sv
import workloads
from tests import parity
from tests.gpu_run import launches, run, to_device

pytestmark = pytest.mark.gpu

AUTO, TWO, ONE = sv.SPEC_PATH_AUTO, sv.SPEC_PATH_TWO, sv.SPEC_PATH_ONE
PATHS = pytest.mark.parametrize("path", [TWO, ONE], ids=["two", "one"])


def _both(w, greedy=False, requests=None, path=AUTO):
    print(f"[gpu] {w.name} B={w.B} gamma={w.gamma} V={w.V} {w.dtype} greedy={greedy} "
          f"path={path}", flush=True)
    g = run(w, greedy=greedy, path=path)
    o = oracle.verify(w, requests=requests, greedy=greedy)
    rep = parity.compare(w, g, o, requests=requests, greedy_call=greedy)
    print(f"[gpu]   {rep}", flush=True)
    return g, o, rep


# ----------------------------------------------------------------------- small shapes

SMALL = [
    # (B, gamma, V, dtype, ragged, temps)      V spans: odd (element loads), one tile,
    (3, 4, 37, "f32", False, 1.0),           # several tiles with a ragged tail
    (5, 3, 1000, "bf16", True, 0.7),
    (4, 6, 4099, "f32", True, "mixed"),
    (6, 5, 16392, "bf16", False, "mixed"),
    (7, 8, 50000, "f32", True, "mixed"),
    (9, 4, 33001, "bf16", True, "mixed"),
    (2, 2, 131072 + 8, "bf16", False, 1.3),
    (3, 7, 100003, "f32", False, 0.9),
]


@PATHS
@pytest.mark.parametrize("B,gamma,V,dtype,ragged,temps", SMALL)
def test_small_shapes_match_oracle(B, gamma, V, dtype, ragged, temps, path):
    if temps == "mixed":
        temps = np.where(np.arange(B) % 3 == 0, 0.0, np.linspace(0.2, 1.5, B))
    w = workloads.small(B=B, gamma=gamma, V=V, dtype=dtype, seed=B * 1000 + V, ragged=ragged,
                        temperatures=temps, draft_sigma=0.8)
    _both(w, path=path)


@PATHS
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("V", [64, 5000, 40000])
def test_greedy_entry_point_matches_oracle(dtype, V, path):
    w = workloads.small(B=11, gamma=6, V=V, dtype=dtype, seed=V, ragged=True,
                        temperatures=0.0, draft_sigma=0.3)
    _both(w, greedy=True, path=path)
    _both(w.as_greedy(), greedy=False, path=path)   # T = 0 rows inside the sampling entry point


@PATHS
def test_many_requests_peaked_rows(path):
    w = workloads.small(B=96, gamma=4, V=8192, dtype="bf16", seed=77, temperatures=0.7,
                        target_sigma=3.0, draft_sigma=1.0, peaks=5)
    _, _, rep = _both(w, path=path)
    assert rep["ambiguous"] <= 0.1 * rep["sampled"]


def test_long_rows_with_multi_tile_slices():
    # rows long enough that one slice holds several row-statistics tiles (bf16, > 64 tiles)
    # and several residual tiles (fp32, > 64 residual tiles), with ragged tails
    w = workloads.small(B=2, gamma=2, V=1_100_003 - 3, dtype="bf16", seed=31,
                        temperatures=np.array([0.9, 0.0]), draft_sigma=0.6)
    _both(w)
    w = workloads.small(B=2, gamma=3, V=600_000, dtype="f32", seed=32,
                        temperatures=np.array([1.1, 0.5]), draft_sigma=0.6)
    _both(w)


@pytest.mark.parametrize("B,gamma,V,dtype", [
    (300, 2, 4096, "bf16"),      # many requests, short rows: one slice per request
    (5, 3, 16, "f32"),           # a single chunk
    (2, 3, 300_000, "bf16"),     # few requests, long rows: many slices per request
    (3, 2, 250_001, "f32"),      # ... on the element path
    (1, 1, 65_536, "f32"),       # one request: its slices alone make the grid
])
def test_sliced_finish(B, gamma, V, dtype):
    # two launches: row statistics, then k_finish over (slice, request), whose last slice per
    # request draws; the number of slices follows B and V
    temps = np.where(np.arange(B) % 4 == 1, 0.0, np.linspace(0.4, 1.4, B))
    w = workloads.small(B=B, gamma=gamma, V=V, dtype=dtype, seed=B * 7 + V, ragged=True,
                        temperatures=temps, draft_sigma=0.9)
    assert launches(w, path=TWO) == 2
    _both(w, path=TWO)
    assert launches(w, greedy=True, path=TWO) == 2
    _both(w, greedy=True, path=TWO)


@pytest.mark.parametrize("B,gamma,V,dtype", [
    (150, 2, 4096, "bf16"),      # many requests of one tile per row
    (5, 3, 16, "f32"),           # a single chunk
    (1, 1, 65_536, "f32"),       # one request: four tiles per row
    (300, 1, 512, "bf16"),       # three hundred one-tile requests
    (3, 2, 100_001, "f32"),      # the element path, seven tiles per row
])
def test_one_launch_tiles(B, gamma, V, dtype):
    # one launch: a workgroup per (row, tile); the workgroups of a request meet on its arrival
    # counter, split its stop row(s) between them, and the last one to finish its chunk sums
    # draws
    temps = np.where(np.arange(B) % 4 == 1, 0.0, np.linspace(0.4, 1.4, B))
    w = workloads.small(B=B, gamma=gamma, V=V, dtype=dtype, seed=B * 11 + V, ragged=True,
                        temperatures=temps, draft_sigma=0.9)
    assert launches(w, path=ONE) == 1
    _both(w, path=ONE)
    assert launches(w, greedy=True, path=ONE) == 1
    _both(w, greedy=True, path=ONE)


def test_one_launch_greedy_at_the_counter_limit():
    # 2048 greedy requests (the last counter of the one-launch region) and one more, which
    # the one-launch path refuses and the library's own choice sends to two launches
    w = workloads.small(B=2048, gamma=2, V=300, dtype="bf16", seed=41, temperatures=0.0,
                        draft_sigma=0.2)
    assert launches(w, greedy=True, path=ONE) == 1
    _both(w, greedy=True, path=ONE)
    w = workloads.small(B=2049, gamma=2, V=300, dtype="bf16", seed=42, temperatures=0.0,
                        draft_sigma=0.2)
    with pytest.raises(sv.SpecVerifyError):
        run(w, greedy=True, path=ONE)
    assert launches(w, greedy=True) == 2
    _both(w, greedy=True)


def test_one_launch_refuses_calls_it_cannot_take():
    # a sampling call whose workgroups cannot all be resident at once (64 x 17 rows x 8
    # tiles): asking for one launch is a shape error, nothing runs
    w = workloads.small(B=64, gamma=8, V=128256, dtype="bf16", seed=5, temperatures=0.8)
    assert _one_launch_tiles(w) > 4 * ONE_FITS
    with pytest.raises(sv.SpecVerifyError) as e:
        run(w, path=ONE)
    assert e.value.code == -2
    assert launches(w) == 2     # the library's own choice takes two


@pytest.mark.parametrize("spin", [1, 3])
def test_one_launch_wait_bound_never_changes_results(spin):
    # The one-launch path's bounded wait, forced short from the host: a workgroup that does
    # not find all of its request's tiles in within `spin` polls leaves, and the last arrival
    # claims the spans it would have summed.  Every request must still come back complete and
    # equal to the oracle, the counter region must be back at zero, and the next calls on the
    # same workspace (the default bound, then a smaller shape with the short bound again) must
    # match as well, with no zero-fill in between.
    import torch
    ws = None
    for i, (B, gamma, V, spin_limit) in enumerate([(16, 4, 65536, spin), (16, 4, 65536, 0),
                                                   (7, 2, 30000, spin)]):
        temps = np.where(np.arange(B) % 4 == 1, 0.0, 0.8)
        w = workloads.small(B=B, gamma=gamma, V=V, dtype="bf16", seed=77 + i,
                            temperatures=temps, draft_sigma=0.9)
        print(f"[gpu] one-launch bounded wait: call {i} B={B} gamma={gamma} V={V} "
              f"spin_limit={spin_limit}", flush=True)
        if ws is None:
            ws = sv.alloc_workspace(B, gamma, V, sv.SPEC_BF16)
        d = to_device(w)
        out = torch.full((w.R_t,), -7, dtype=torch.int32, device="cuda")
        nacc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        sv.spec_verify_sample(d["target"], d["draft"], d["tokens"], d["uniforms"], d["temps"],
                              gamma, out, nacc, ws,
                              probe=sv.make_probe(path=ONE, spin_limit=spin_limit))
        torch.cuda.synchronize()
        g = dict(out_tokens=out.cpu().numpy(), num_accepted=nacc.cpu().numpy())
        parity.compare(w, g, oracle.verify(w), probes=False)
        assert int(ws[:sv.COUNTER_BYTES].count_nonzero()) == 0


@pytest.mark.parametrize("B", [8, 32])
@PATHS
def test_single_draft_small_batch(B, path):
    # one draft per request (the single-token MTP case of the Perplexity page, "Planification
    # MTP pour un jeton unique"), small decode batches at the full Llama-3 vocabulary: both
    # launch paths, the one-launch path being the latency-bound case's
    temps = np.where(np.arange(B) % 5 == 0, 0.0, np.linspace(0.5, 1.1, B))
    w = workloads.small(B=B, gamma=1, V=128256, dtype="bf16", seed=60 + B, temperatures=temps,
                        target_sigma=3.0, draft_sigma=1.0)
    assert launches(w, path=path) == (1 if path == ONE else 2)
    _both(w, path=path)


def test_single_draft_decode_batch():
    # the same with 256 requests (too many workgroups for one launch: two)
    temps = np.where(np.arange(256) % 5 == 0, 0.0, np.linspace(0.5, 1.1, 256))
    w = workloads.small(B=256, gamma=1, V=128256, dtype="bf16", seed=61, temperatures=temps,
                        target_sigma=3.0, draft_sigma=1.0)
    _both(w)


def _random_case(i):
    """Seeded random call: B, gamma, V, dtype, dense or ragged, a mix of greedy and sampled
    requests, target/draft closeness and temperatures over a wide range; from case 24 on,
    also vocabulary masks (-inf) and some extreme temperatures."""
    rng = np.random.default_rng(7000 + i)
    dtype = "bf16" if rng.random() < 0.6 else "f32"
    B = int(rng.integers(1, 48))
    gamma = int(rng.integers(1, 11))
    V = int(rng.choice([rng.integers(1, 600), rng.integers(600, 20000), rng.integers(20000, 130000)]))
    temps = np.where(rng.random(B) < 0.25, 0.0, rng.uniform(0.05, 2.0, B))
    kw = dict(B=B, gamma=gamma, V=V, dtype=dtype, seed=7000 + i, ragged=bool(rng.random() < 0.6),
              temperatures=temps, target_sigma=float(rng.uniform(0.5, 4.0)),
              draft_sigma=float(rng.uniform(0.05, 1.5)))
    if i >= 24:
        r2 = np.random.default_rng(9000 + i)
        kw["mask_frac"] = float(r2.choice([0.0, 0.3, 0.7]))
        kw["mask_span"] = int(r2.choice([0, V // 3, V // 2]))
        extreme = r2.random(B)
        kw["temperatures"] = np.where(extreme < 0.1, 1e-3, np.where(extreme > 0.9, 12.0, temps))
    return kw


def _one_launch_tiles(w, greedy=False):
    """Workgroups of the one-launch kernel for workload w: (row slots) x (16K-element tiles)."""
    spr = w.gamma + 1 if greedy else 2 * w.gamma + 1
    return w.B * spr * -(-w.V // 16384)


# sampling calls of at most this many one-launch workgroups fit the device at once with room
# to spare (three quarters of 1280 resident workgroups are 960)
ONE_FITS = 900


@pytest.mark.parametrize("i", range(48))
def test_random_calls_on_both_paths(i):
    # the same seeded call on both launch paths (one launch where its workgroups fit): each
    # matches the oracle under the parity rules, and the two agree on every request the oracle
    # does not mark ambiguous
    kw = _random_case(i)
    w = workloads.small(**kw)
    o = oracle.verify(w)
    res = {}
    for path in ((TWO, ONE) if _one_launch_tiles(w) <= ONE_FITS else (TWO,)):
        print(f"[gpu] random call {i}: B={w.B} gamma={w.gamma} V={w.V} {w.dtype} path={path}",
              flush=True)
        g = run(w, path=path)
        parity.compare(w, g, o)
        res[path] = g
    if ONE not in res:
        return
    sure = ~parity.ambiguous_requests(w, o)
    for b in np.flatnonzero(sure):
        tb, gb = w.target_base[b], w.gammas[b]
        np.testing.assert_array_equal(res[TWO]["out_tokens"][tb: tb + gb + 1],
                                      res[ONE]["out_tokens"][tb: tb + gb + 1])
    np.testing.assert_array_equal(res[TWO]["num_accepted"][sure], res[ONE]["num_accepted"][sure])


@PATHS
def test_a_request_range_verifies_as_the_batch_slice(path):
    # One GPU's share of a batch split by requests: the call over requests [lo, hi) alone
    # matches the oracle, and on every request the oracle does not mark ambiguous it emits
    # exactly what the whole batch's call emitted there (no state crosses requests; the
    # row tiling may differ with the call's size, which only moves last-bit roundings)
    temps = np.where(np.arange(24) % 4 == 0, 0.0, np.linspace(0.3, 1.2, 24))
    w = workloads.small(B=24, gamma=6, V=20000, dtype="bf16", seed=314, ragged=True,
                        temperatures=temps, draft_sigma=0.9)
    o = oracle.verify(w)
    full = run(w, path=path)
    parity.compare(w, full, o)
    for lo, hi in [(0, 7), (7, 8), (8, 24)]:
        s = w.requests(lo, hi)
        print(f"[gpu] requests {lo}..{hi - 1} of B={w.B} path={path}", flush=True)
        g = run(s, path=path)
        so = oracle.verify(s)
        parity.compare(s, g, so)
        sure = ~parity.ambiguous_requests(s, so)
        t0 = int(w.target_base[lo])
        for k in np.flatnonzero(sure):
            tb, gb = int(s.target_base[k]), int(s.gammas[k])
            np.testing.assert_array_equal(g["out_tokens"][tb: tb + gb + 1],
                                          full["out_tokens"][t0 + tb: t0 + tb + gb + 1])
        np.testing.assert_array_equal(g["num_accepted"][sure], full["num_accepted"][lo:hi][sure])


# ----------------------------------------------------------------------- edge cases

@PATHS
def test_p_equal_q_accepts_everything_on_gpu(path):
    w = workloads.small(B=40, gamma=8, V=3000, dtype="bf16", seed=5, temperatures=0.9,
                        ragged=True)
    for b, (tb, db, g) in enumerate(zip(w.target_base, w.draft_base, w.gammas)):
        w.draft[db: db + g] = w.target[tb: tb + g]
    rng = np.random.default_rng(9)
    w.draft_tokens[:] = workloads.draw_draft_tokens(workloads.decode(w.draft, "bf16"), 0.9, rng)
    w.uniforms[:, 0] = np.float32(np.nextafter(np.float32(1), np.float32(0)))
    g = run(w, path=path)
    np.testing.assert_array_equal(g["num_accepted"], w.gammas)
    _both(w, path=path)


@PATHS
def test_gamma_zero_and_max_gamma(path):
    w0 = workloads.small(B=4, gamma=1, V=500, seed=1)
    # one unused draft row and token keep the (never read) pointers non-NULL
    w0 = workloads.Workload("gamma0", "f32", 4, 0, 500, w0.target[:4].copy(),
                            np.zeros((1, 500), np.float32), np.zeros(1, np.int32),
                            w0.uniforms[:4].copy(), np.array([1.0, 0.0, 0.5, 2.0], np.float32))
    _both(w0, path=path)
    w64 = workloads.small(B=3, gamma=64, V=300, dtype="f32", seed=2, temperatures=1.0,
                          draft_sigma=0.05)
    g, o, _ = _both(w64, path=path)
    assert (o["num_accepted"] >= 32).any()  # long accepted runs exercise the lane loop
    wg = workloads.small(B=3, gamma=64, V=300, dtype="bf16", seed=3, temperatures=0.0,
                         draft_sigma=0.0)
    g, o, _ = _both(wg, greedy=True, path=path)
    assert (o["num_accepted"] == 64).all()   # drafts are the target argmax: all accepted


def test_largest_vocabulary():
    # V = 2^24, the largest the library takes: 1024 tiles per row, chunk sums over 2^21
    # units, the draw's scan over 32768 chunks; sampled and greedy requests
    w = workloads.small(B=2, gamma=2, V=1 << 24, dtype="bf16", seed=24,
                        temperatures=np.array([0.8, 0.0]), target_sigma=3.0, draft_sigma=0.5)
    _both(w)
    _both(w, greedy=True)


@pytest.mark.parametrize("sigma,V,dtype,B,force", [
    (0.02, 4096, "f32", 3000, False), (0.01, 32000, "bf16", 3000, False),
    (0.003, 4096, "f32", 3000, False),
    # q within ~0.1% / 0.03% of p: rejections are forced with accept uniforms near 1, so that
    # every request stops at a row whose residual mass is ~4e-4 / ~1e-4
    (0.001, 4096, "f32", 400, True), (0.0003, 4096, "f32", 400, True),
    (0.001, 20000, "bf16", 800, True),
])
def test_nearly_equal_p_and_q(sigma, V, dtype, B, force):
    # a draft that follows the target closely: the rejections stop at rows whose residual
    # max(p - q, 0), a small mass spread over half the vocabulary, must still be drawn from
    # exactly and its mass reported to 1e-5 relative
    w = workloads.small(B=B, gamma=8, V=V, dtype=dtype, seed=int(sigma * 1e5) + V,
                        temperatures=1.0, target_sigma=2.0, draft_sigma=sigma)
    if force:
        rng = np.random.default_rng(V + B)
        w.uniforms[:, 0] = rng.uniform(0.999, 1.0, size=w.R_t).astype(np.float32)
    print(f"[gpu] nearly equal p and q: sigma {sigma} V={V} {dtype} B={B}", flush=True)
    g = run(w)
    o = oracle.verify(w)
    rej = (o["num_accepted"] < w.gammas) & (o["fallback"] == 0)
    assert rej.sum() >= 20
    rep = parity.compare(w, g, o)
    print(f"[gpu]   {int(rej.sum())} rejections, residual mass there from "
          f"{o['resid_mass'][rej].min():.2e} (median {np.median(o['resid_mass'][rej]):.2e}); "
          f"{rep}", flush=True)


def _small_residual_case(i):
    """Seeded random call whose drafts follow the target within 3e-4 .. 3e-2 (log-uniform):
    residual masses from ~1e-4 to ~1e-2, ragged gamma, masks, temperatures 0.3 .. 3."""
    rng = np.random.default_rng(5100 + i)
    B = int(rng.integers(8, 40))
    V = int(rng.choice([rng.integers(50, 2000), rng.integers(2000, 40000)]))
    dtype = "f32" if rng.random() < 0.6 else "bf16"
    return dict(B=B, gamma=int(rng.integers(1, 9)), V=V, dtype=dtype, seed=5100 + i,
                ragged=True, temperatures=rng.uniform(0.3, 3.0, B),
                target_sigma=float(rng.uniform(1.0, 4.0)),
                draft_sigma=float(np.exp(rng.uniform(np.log(3e-4), np.log(3e-2)))),
                mask_frac=float(rng.choice([0.0, 0.2])))


@pytest.mark.parametrize("i", range(24))
def test_small_residual_calls_on_both_paths(i):
    # the small-residual regime across shapes, dtypes and temperatures, accept uniforms near 1
    # so that most requests stop at such a row; both launch paths against the oracle
    w = workloads.small(**_small_residual_case(i))
    rng = np.random.default_rng(5200 + i)
    w.uniforms[:, 0] = rng.uniform(0.99, 1.0, size=w.R_t).astype(np.float32)
    o = oracle.verify(w)
    for path in ((TWO, ONE) if _one_launch_tiles(w) <= ONE_FITS else (TWO,)):
        print(f"[gpu] small-residual call {i}: B={w.B} gamma={w.gamma} V={w.V} {w.dtype} "
              f"path={path}", flush=True)
        parity.compare(w, run(w, path=path), o)


@PATHS
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_draws_near_a_cdf_step(path, dtype):
    # The draw's uniform placed 2e-6 .. 5e-6 (in probability) from a step of the running sum
    # the oracle draws from, on either side, at residual masses of all sizes: outside the
    # 1e-6 exemption, so the token must be the oracle's exactly.
    from scipy import special
    w = workloads.small(B=64, gamma=3, V=3000, dtype=dtype, seed=97, ragged=True,
                        temperatures=np.linspace(0.4, 1.6, 64), draft_sigma=0.6)
    o = oracle.verify(w)
    zt, zd = workloads.decode(w.target, dtype), workloads.decode(w.draft, dtype)
    rng = np.random.default_rng(98)
    for b in range(w.B):
        tb, db, n = int(w.target_base[b]), int(w.draft_base[b]), int(o["num_accepted"][b])
        T = float(w.temperatures[b])
        p = special.softmax(zt[tb + n] / T)
        r = np.maximum(p - special.softmax(zd[db + n] / T), 0.0) if n < w.gammas[b] else p
        C = np.cumsum(r) / r.sum()
        steps = C[(r > 0) & (C > 1e-3) & (C < 1 - 1e-3)]
        u = steps[rng.integers(len(steps))] + rng.choice([-1, 1]) * rng.uniform(2e-6, 5e-6)
        w.uniforms[tb + n, 1] = np.float32(u)
    o = oracle.verify(w)
    assert (o["cdf_gap"] > 1e-6).mean() > 0.9
    _both(w, path=path)


@PATHS
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_masked_logits(path, dtype):
    # Vocabulary masks (logit -inf, shared by a request's rows): 30% of the entries plus a run
    # of 20000, so some 16K tiles are masked whole; temperatures across the range (the
    # temperature constant's low part, kept positive, must not turn -inf into NaN)
    temps = np.array([0.05, 0.3, 0.0, 0.7, 1.0, 1.3, 0.0, 2.5, 0.9, 0.6, 1.7, 0.45, np.inf])
    w = workloads.small(B=13, gamma=5, V=40000, dtype=dtype, seed=31, temperatures=temps,
                        ragged=True, draft_sigma=0.8, mask_frac=0.3, mask_span=20000)
    _both(w, path=path)
    _both(w, greedy=True, path=path)


def test_requests_beyond_one_grid_dimension():
    # 528280 requests: more row slots (1584840) than one grid dimension holds, and more groups
    # of eight requests (66035) than the finishing launch's y dimension, so the z dimension
    # carries the rest in both launches
    B = 8 * 65535 + 4000
    w = workloads.small(B=B, gamma=1, V=16, dtype="f32", seed=70, draft_sigma=0.8,
                        temperatures=np.where(np.arange(B) % 3 == 0, 0.0, 0.9))
    _both(w)
    _both(w, greedy=True)


@PATHS
def test_ragged_with_empty_requests(path):
    base = workloads.small(B=6, gamma=5, V=777, dtype="bf16", seed=4, ragged=True,
                           temperatures=np.array([0.8, 0, 1.1, 0.5, 0, 0.3]))
    # make requests 1 and 4 have no drafts: drop their draft rows and rebuild CSR
    g = base.gammas.copy()
    keep_d = np.ones(base.R_d, bool)
    keep_t = np.ones(base.R_t, bool)
    for b in (1, 4):
        db, tb = base.draft_base[b], base.target_base[b]
        keep_d[db: db + g[b]] = False
        keep_t[tb + 1: tb + g[b] + 1] = False
        g[b] = 0
    cu = np.concatenate([[0], np.cumsum(g)]).astype(np.int32)
    w = workloads.Workload("empty-requests", "bf16", 6, int(g.max()), 777,
                           base.target[keep_t].copy(), base.draft[keep_d].copy(),
                           base.draft_tokens[keep_d].copy(), base.uniforms[keep_t].copy(),
                           base.temperatures.copy(), cu)
    _both(w, path=path)


@PATHS
def test_single_token_vocabulary(path):
    w = workloads.small(B=5, gamma=3, V=1, dtype="f32", seed=6, ragged=True,
                        temperatures=np.array([1.0, 0.0, 0.5, 0.0, 2.0]))
    g, o, _ = _both(w, path=path)
    np.testing.assert_array_equal(g["num_accepted"], w.gammas)


@PATHS
def test_extreme_temperatures(path):
    # tiny and huge T; with logits near +-10 the smaller temperatures take the row
    # statistics' overflow-safe exponent form, the others the two-FMA form; T = +inf is the
    # uniform distribution (every draft accepted, the bonus drawn uniformly)
    temps = np.array([1e-30, 1e-6, 1e-3, 50.0, 1e4, 0.0, np.inf, 1e30], dtype=np.float32)
    w = workloads.small(B=8, gamma=4, V=2048, dtype="bf16", seed=8, temperatures=temps)
    _both(w, path=path)


@PATHS
def test_large_logits(path):
    # logits of magnitude ~1e4 at T = 1: |max| c is above the two-FMA limit
    w = workloads.small(B=4, gamma=3, V=3000, dtype="f32", seed=9, temperatures=1.0,
                        target_sigma=1.0, draft_sigma=0.5)
    w.target += np.float32(-2.0e4)
    w.draft += np.float32(-2.0e4)
    _both(w, path=path)


@PATHS
def test_draft_ids_outside_vocabulary(path):
    w = workloads.small(B=6, gamma=4, V=900, dtype="f32", seed=10,
                        temperatures=np.array([1.0, 0.0, 0.6, 0.0, 1.2, 0.9]))
    w.draft_tokens[1::3] = 900
    w.draft_tokens[2::5] = -3
    _both(w, path=path)
    _both(w, greedy=True, path=path)


@PATHS
def test_unaligned_rows_take_the_element_path(path):
    # a row stride that is not a multiple of 16 bytes, and a base offset by one element
    import torch
    w = workloads.small(B=4, gamma=3, V=1001, dtype="bf16", seed=12, temperatures=0.9)
    o = oracle.verify(w)
    d = to_device(w)
    for k in ("target", "draft"):
        t = d[k]
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device="cuda")
        buf[1:] = t.reshape(-1)
        d[k] = buf[1:].view_as(t)
    g = run(w, dev=d, path=path)
    parity.compare(w, g, o)


@pytest.mark.parametrize("V,path", [(256, TWO), (256, ONE), (200_000, TWO), (100_000, ONE)])
def test_bonus_fallback_when_residual_is_empty(V, path):
    # p = q at a rejected position (uniform at its upper edge): the residual is empty and
    # the draw falls back to p, as the oracle does (both finishing paths).
    w = workloads.small(B=3, gamma=2, V=V, dtype="f32", seed=13, temperatures=1.0)
    w.draft[:] = w.target[np.concatenate([[0, 1], [3, 4], [6, 7]])]
    w.uniforms[:, 0] = 1.0
    g, o, _ = _both(w, path=path)
    assert (o["fallback"] == 1).all()
    sure = o["cdf_gap"] >= parity.AMBIGUOUS
    assert sure.any()
    for b in np.flatnonzero(sure):
        tb = w.target_base[b]
        np.testing.assert_array_equal(g["out_tokens"][tb: tb + 3], o["out_tokens"][tb: tb + 3])


# ----------------------------------------------------------------------- the workloads

@PATHS
def test_workload1_tiny_sampling(path):
    w = workloads.config(1)
    g, o, rep = _both(w, path=path)
    assert rep["ambiguous"] == 0


@PATHS
def test_workload2_greedy_bit_exact(path):
    w = workloads.config(2)
    g, o, _ = _both(w, greedy=True, path=path)
    g2, _, _ = _both(w, greedy=False, path=path)    # the same step through the mixed entry point
    np.testing.assert_array_equal(g["out_tokens"], g2["out_tokens"])


def test_workload3_llama3_vocab_sampling():
    # (its 1024 one-launch workgroups exceed three quarters of the device's capacity for that
    # kernel, so it takes two launches only)
    w = workloads.config(3)
    _, _, rep = _both(w)
    assert rep["sampled"] == 64


def test_workload4_full_size_every_request():
    w = workloads.config(4)
    _, _, rep = _both(w)
    assert rep["sampled"] == 256


def test_workload5_full_size_every_request():
    w = workloads.config(5)
    _, _, rep = _both(w)
    assert rep["greedy"] == 102 and rep["sampled"] == 410


@PATHS
def test_repeated_calls_are_bit_identical(path):
    w = workloads.small(B=32, gamma=6, V=20000, dtype="bf16", seed=14, ragged=True,
                        temperatures=np.linspace(0, 1.2, 32))
    d = to_device(w)
    a = run(w, dev=d, path=path)
    b = run(w, dev=d, path=path)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


def test_one_workspace_across_shapes_and_paths():
    # one workspace, zero in its counter region (the one-launch counters) and 0xff beyond, is
    # reused by calls of different sizes on both launch paths, which must all match the
    # oracle; every call leaves the counters at zero
    import torch
    shapes = [(40, 5, 30000, "bf16", ONE), (3, 8, 70001, "f32", TWO), (64, 2, 4096, "bf16", ONE),
              (40, 5, 30000, "bf16", TWO), (3, 8, 70001, "f32", ONE), (64, 2, 4096, "bf16", TWO),
              (40, 5, 30000, "bf16", ONE)]
    need = max(sv.spec_verify_workspace_size(B, g, V, sv.SPEC_BF16 if dt == "bf16" else sv.SPEC_F32)
               for B, g, V, dt, _ in shapes)
    ws = torch.full((need,), 0xff, dtype=torch.uint8, device="cuda")
    ws[:sv.COUNTER_BYTES] = 0
    for i, (B, gamma, V, dtype, path) in enumerate(shapes):
        temps = np.where(np.arange(B) % 5 == 2, 0.0, np.linspace(0.5, 1.3, B))
        w = workloads.small(B=B, gamma=gamma, V=V, dtype=dtype, seed=300 + i, ragged=True,
                            temperatures=temps, draft_sigma=1.0)
        print(f"[gpu] shared workspace call {i}: B={B} gamma={gamma} V={V} {dtype} path={path}",
              flush=True)
        g = run(w, workspace=ws, path=path)
        parity.compare(w, g, oracle.verify(w))
        assert int(ws[:sv.COUNTER_BYTES].count_nonzero()) == 0


def test_prepared_call_repeats_the_entry_point():
    # a call marshalled once and run twice gives what the plain call gives
    import torch
    import speculative_sampling_verification_spec_amd as sv
    w = workloads.small(B=20, gamma=4, V=9000, dtype="bf16", seed=88, ragged=True,
                        temperatures=np.linspace(0.0, 1.1, 20))
    d = to_device(w)
    ref = run(w, dev=d, probe=False)
    ws = sv.alloc_workspace(w.B, w.gamma, w.V, sv.SPEC_BF16)
    out = torch.full((w.R_t,), -7, dtype=torch.int32, device="cuda")
    nacc = torch.full((w.B,), -7, dtype=torch.int32, device="cuda")
    call = sv.prepare_sample(d["target"], d["draft"], d["tokens"], d["uniforms"], d["temps"],
                             w.gamma, out, nacc, ws, cu_draft=d["cu"])
    for _ in range(2):
        out.fill_(-7)
        call()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(out.cpu().numpy(), ref["out_tokens"])
        np.testing.assert_array_equal(nacc.cpu().numpy(), ref["num_accepted"])
    g = w.as_greedy()
    dg = to_device(g)
    refg = run(g, greedy=True, dev=dg, probe=False)
    callg = sv.prepare_greedy(dg["target"], dg["tokens"], g.gamma, out, nacc, ws, cu_draft=dg["cu"])
    callg()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out.cpu().numpy(), refg["out_tokens"])
    np.testing.assert_array_equal(nacc.cpu().numpy(), refg["num_accepted"])


def _commit_subset(o, w, keep, gamma, seq, length, stats, hist):
    """The oracle's commit of the requests in `keep` only (the others' rows untouched and
    uncounted), built by committing a batch made of those requests alone."""
    keep = np.flatnonzero(keep)
    g = w.gammas[keep]
    cu = np.concatenate([[0], np.cumsum(g)]).astype(np.int32)
    out = np.concatenate([o["out_tokens"][w.target_base[b]: w.target_base[b] + w.gammas[b] + 1]
                          for b in keep]).astype(np.int32)
    sub_seq, sub_len = seq[keep].copy(), length[keep].copy()
    oracle.commit(out, o["num_accepted"][keep], gamma, sub_seq, sub_len, cu_draft=cu,
                  stats=stats, hist=hist)
    seq[keep], length[keep] = sub_seq, sub_len


@pytest.mark.parametrize("capacity,fill,negative", [(64, "low", False), (14, "high", False),
                                                    (64, "low", True)])
def test_commit_matches_oracle(capacity, fill, negative):
    # the GPU commit of a verification step's outputs against the oracle's commit of the
    # same outputs (histories and counters bit-exact).  With `negative`, every seventh
    # request carries an accepted count of -1, outside the entry point's precondition
    # [0, gamma_b]: the GPU commit leaves such a request alone and uncounted (memory safety on
    # device data it cannot check), which the expected state reproduces by committing the
    # other requests alone through the oracle (the oracle rejects a negative count)
    import torch
    import speculative_sampling_verification_spec_amd as sv
    B, gamma = 300, 6
    temps = np.where(np.arange(B) % 4 == 0, 0.0, np.linspace(0.3, 1.3, B))
    w = workloads.small(B=B, gamma=gamma, V=5000, dtype="bf16", seed=capacity, ragged=True,
                        temperatures=temps, draft_sigma=0.7)
    o = oracle.verify(w)   # both commits take the oracle's step as input
    keep = np.ones(B, dtype=bool)
    if negative:
        keep[::7] = False
    n_dev = np.where(keep, o["num_accepted"], -1).astype(np.int32)
    rng = np.random.default_rng(capacity)
    hi = capacity if fill == "high" else capacity - gamma - 1
    seq0 = rng.integers(0, 5000, size=(B, capacity)).astype(np.int32)
    len0 = rng.integers(0, hi + 1, size=B).astype(np.int32)
    seq_o, len_o = seq0.copy(), len0.copy()
    st_o = np.zeros(5, dtype=np.uint64)
    hi_o = np.zeros(gamma + 1, dtype=np.uint64)
    for _ in range(2):   # the counters accumulate; the histories take the second step too
        _commit_subset(o, w, keep, gamma, seq_o, len_o, st_o, hi_o)
    dev = dict(out=torch.from_numpy(o["out_tokens"]).cuda(),
               n=torch.from_numpy(n_dev).cuda(),
               cu=torch.from_numpy(w.cu_draft.astype(np.int32)).cuda(),
               seq=torch.from_numpy(seq0).cuda(), len=torch.from_numpy(len0).cuda(),
               st=torch.zeros(5, dtype=torch.int64, device="cuda"),
               hi=torch.zeros(gamma + 1, dtype=torch.int64, device="cuda"))
    for _ in range(2):
        sv.spec_verify_commit(dev["out"], dev["n"], gamma, dev["seq"], dev["len"],
                              cu_draft=dev["cu"], stats=dev["st"], accept_hist=dev["hi"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dev["seq"].cpu().numpy(), seq_o)
    np.testing.assert_array_equal(dev["len"].cpu().numpy(), len_o)
    np.testing.assert_array_equal(dev["st"].cpu().numpy().view(np.uint64), st_o)
    np.testing.assert_array_equal(dev["hi"].cpu().numpy().view(np.uint64), hi_o)
    if fill == "high":
        assert int(st_o[4]) > 0   # the truncation path ran


def test_commit_dense_layout_and_many_requests():
    import torch
    import speculative_sampling_verification_spec_amd as sv
    B, gamma, cap = 5000, 3, 9
    rng = np.random.default_rng(7)
    n = rng.integers(0, gamma + 1, size=B).astype(np.int32)
    out = rng.integers(0, 1000, size=B * (gamma + 1)).astype(np.int32)
    seq0 = np.full((B, cap), -5, dtype=np.int32)
    len0 = rng.integers(0, cap + 1, size=B).astype(np.int32)
    seq_o, len_o = seq0.copy(), len0.copy()
    st_o = np.zeros(5, dtype=np.uint64)
    hi_o = np.zeros(gamma + 1, dtype=np.uint64)
    oracle.commit(out, n, gamma, seq_o, len_o, stats=st_o, hist=hi_o)
    seq = torch.from_numpy(seq0).cuda()
    ln = torch.from_numpy(len0).cuda()
    st = torch.zeros(5, dtype=torch.int64, device="cuda")
    hi = torch.zeros(gamma + 1, dtype=torch.int64, device="cuda")
    sv.spec_verify_commit(torch.from_numpy(out).cuda(), torch.from_numpy(n).cuda(), gamma, seq,
                          ln, stats=st, accept_hist=hi)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(seq.cpu().numpy(), seq_o)
    np.testing.assert_array_equal(ln.cpu().numpy(), len_o)
    np.testing.assert_array_equal(st.cpu().numpy().view(np.uint64), st_o)
    np.testing.assert_array_equal(hi.cpu().numpy().view(np.uint64), hi_o)


def _ngram_gpu(seq, length, n_min, n_max, gamma, packed=True):
    import torch
    import speculative_sampling_verification_spec_amd as sv
    B = len(length)
    d = dict(seq=torch.from_numpy(seq).cuda(), len=torch.from_numpy(length).cuda(),
             counts=torch.full((B,), -7, dtype=torch.int32, device="cuda"),
             dense=torch.full((B * gamma,), -7, dtype=torch.int32, device="cuda"),
             cu=torch.full((B + 1,), -7, dtype=torch.int32, device="cuda") if packed else None,
             packed=torch.full((max(B * gamma, 1),), -7, dtype=torch.int32, device="cuda")
             if packed else None)
    sv.spec_ngram_propose(d["seq"], d["len"], n_min, n_max, gamma, d["counts"], d["dense"],
                          d["cu"], d["packed"])
    torch.cuda.synchronize()
    return d


@pytest.mark.parametrize("alphabet,cap,n_min,n_max,gamma", [
    (2, 300, 1, 1, 4), (3, 300, 2, 4, 8), (8, 1000, 1, 6, 5), (50, 5000, 3, 64, 64),
    (32000, 9000, 2, 5, 8), (5, 100, 1, 3, 0),
    (2, 12000, 1, 64, 8),      # long matches across rounds of the LDS-staged context
])
def test_ngram_matches_oracle(alphabet, cap, n_min, n_max, gamma):
    rng = np.random.default_rng(alphabet + cap)
    B = 257
    seq = rng.integers(0, alphabet, size=(B, cap)).astype(np.int32)
    length = rng.integers(0, cap + 1, size=B).astype(np.int32)
    length[:4] = [0, 1, 2, cap]
    print(f"[gpu] ngram alphabet={alphabet} cap={cap} n={n_min}..{n_max} gamma={gamma}", flush=True)
    o = oracle.ngram(seq, length, n_min, n_max, gamma)
    d = _ngram_gpu(seq, length, n_min, n_max, gamma)
    np.testing.assert_array_equal(d["counts"].cpu().numpy(), o["counts"])
    np.testing.assert_array_equal(d["dense"].cpu().numpy().reshape(B, gamma), o["dense"])
    np.testing.assert_array_equal(d["cu"].cpu().numpy(), o["cu"])
    np.testing.assert_array_equal(d["packed"].cpu().numpy()[: o["cu"][-1]], o["packed"])
    d2 = _ngram_gpu(seq, length, n_min, n_max, gamma, packed=False)
    np.testing.assert_array_equal(d2["counts"].cpu().numpy(), o["counts"])


def test_ngram_on_repetitive_contexts_many_requests():
    seq, length = workloads.token_contexts(3000, 4096, seed=12)
    o = oracle.ngram(seq, length, 2, 5, 8)
    assert (o["counts"] > 0).mean() > 0.3
    d = _ngram_gpu(seq, length, 2, 5, 8)
    np.testing.assert_array_equal(d["counts"].cpu().numpy(), o["counts"])
    np.testing.assert_array_equal(d["cu"].cpu().numpy(), o["cu"])
    np.testing.assert_array_equal(d["packed"].cpu().numpy()[: o["cu"][-1]], o["packed"])


def test_propose_verify_commit_chain_matches_oracle():
    # n-gram proposals -> greedy verification -> commit, all on the device with no host
    # round trip, against the same chain through the oracle.  The target rows are built from
    # the oracle's proposals: argmax = the proposal up to a seeded break, then another token.
    import torch
    import speculative_sampling_verification_spec_amd as sv
    B, cap, gamma, V = 400, 2048, 6, 4096
    seq, length = workloads.token_contexts(B, cap, seed=5, alphabet=V, min_fill=0.4)
    length = np.minimum(length, cap - gamma - 1).astype(np.int32)
    o = oracle.ngram(seq, length, 2, 4, gamma)
    counts = o["counts"]
    rng = np.random.default_rng(9)
    R_t = int(counts.sum()) + B
    target = rng.normal(0.0, 1.0, size=(R_t, V))
    t = 0
    for b in range(B):
        k = int(counts[b])
        brk = int(rng.integers(0, k + 1))
        for i in range(k + 1):
            want = o["dense"][b, i] if i < k and i < brk else int(rng.integers(0, V))
            target[t + i, want] += 10.0
        t += k + 1
    w = workloads.Workload("ngram-chain", "f32", B, gamma, V, workloads.encode(target, "f32"),
                           np.zeros((max(int(counts.sum()), 1), V), dtype=np.float32),
                           o["packed"].astype(np.int32), np.zeros((R_t, 2), dtype=np.float32),
                           np.zeros(B, dtype=np.float32), o["cu"].astype(np.int32))
    ov = oracle.verify(w, greedy=True)
    seq_o, len_o = seq.copy(), length.copy()
    oracle.commit(ov["out_tokens"], ov["num_accepted"], gamma, seq_o, len_o, cu_draft=w.cu_draft)
    # device chain
    d = _ngram_gpu(seq, length, 2, 4, gamma)
    tgt = torch.from_numpy(w.target).cuda()
    out = torch.full((R_t,), -7, dtype=torch.int32, device="cuda")
    nacc = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    ws = sv.alloc_workspace(B, gamma, V, sv.SPEC_F32)
    sv.spec_verify_greedy(tgt, d["packed"], gamma, out, nacc, ws, cu_draft=d["cu"])
    sv.spec_verify_commit(out, nacc, gamma, d["seq"], d["len"], cu_draft=d["cu"])
    torch.cuda.synchronize()
    np.testing.assert_array_equal(nacc.cpu().numpy(), ov["num_accepted"])
    np.testing.assert_array_equal(d["seq"].cpu().numpy(), seq_o)
    np.testing.assert_array_equal(d["len"].cpu().numpy(), len_o)
    assert 0 < ov["num_accepted"].sum() < counts.sum()


# ----------------------------------------------------------------------- distribution

def test_gpu_chi_square_emitted_tokens_follow_p():
    from scipy import special
    from tests.stats_util import chi2_pvalue
    rng = np.random.default_rng(17)
    V, gamma, T = 16, 3, 0.9
    zt = rng.normal(0, 1.5, size=(gamma + 1, V))
    zd = zt[:gamma] + rng.normal(0, 1.0, size=(gamma, V))
    n = 1_000_000
    w = workloads.tiled(zt, zd, n, T=T, seed=170)
    g = run(w, probe=False)
    toks = g["out_tokens"].reshape(n, gamma + 1)
    nacc = g["num_accepted"]
    zt_s = workloads.decode(w.target[: gamma + 1], "f32")
    T32 = float(np.float32(T))
    for k in range(gamma + 1):
        reached = nacc >= k
        obs = np.bincount(toks[reached, k], minlength=V)
        pval, x2, df = chi2_pvalue(obs, special.softmax(zt_s[k] / T32))
        assert pval > 1e-3, (k, pval, x2, df)
