"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a library routine
(scipy softmax, numpy argmax), a closed form, an invariant the pages state, a case whose
answer follows by hand from the definition, the pages' worked example, or the distribution
of the output (chi-square, and exact stratified grids).  Between them a dropped term, a
wrong sign, a swapped operand (p/q vs q/p, (p-q)+ vs (q-p)+), a wrong row or uniform
index, a wrong temperature placement or a non-strict comparison fails at least one test.
"""
import json
from pathlib import Path

import numpy as np
import pytest
from scipy import special

import oracle
import workloads
from workloads import Workload
from tests.stats_util import chi2_pvalue

GOLDEN = Path(__file__).resolve().parent / "golden"


def _softmax(z, T):
    return special.softmax(np.asarray(z, dtype=np.float64) / T)


def _explicit(target, draft, tokens, uniforms, T, gamma, dtype="f32", cu=None):
    """Workload from explicit float64 rows (encoded to ``dtype``)."""
    target = workloads.encode(np.asarray(target, dtype=np.float64), dtype)
    draft = workloads.encode(np.asarray(draft, dtype=np.float64).reshape(-1, target.shape[1]),
                             dtype)
    uniforms = np.asarray(uniforms, dtype=np.float32).reshape(-1, 2)
    B = target.shape[0] - draft.shape[0]
    temps = np.broadcast_to(np.asarray(T, dtype=np.float32), (B,)).copy()
    return Workload("explicit", dtype, B, gamma, target.shape[1], target, draft,
                    np.asarray(tokens, dtype=np.int32), uniforms, temps,
                    None if cu is None else np.asarray(cu, dtype=np.int32))


# --------------------------------------------------------------------------- library routines

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [0.05, 0.7, 1.0, 3.0])
def test_row_statistics_and_probabilities_match_scipy_softmax(dtype, T):
    w = workloads.small(B=5, gamma=3, V=257, dtype=dtype, seed=11, temperatures=T)
    r = oracle.verify(w)
    T = float(np.float32(T))    # temperatures are passed as float32
    zt = workloads.decode(w.target, dtype)
    zd = workloads.decode(w.draft, dtype)
    for row in range(w.R_t):
        m = zt[row].max()
        assert r["row_max_t"][row] == m
        S_ref = np.exp(special.logsumexp((zt[row] - m) / T))
        assert r["row_sum_t"][row] == pytest.approx(S_ref, rel=1e-12)
    for row in range(w.R_d):
        assert r["row_max_d"][row] == zd[row].max()
    tb, db = w.target_base, w.draft_base
    for b in range(w.B):
        for i in range(w.gamma):
            x = w.draft_tokens[db[b] + i]
            p_ref = _softmax(zt[tb[b] + i], T)[x]
            q_ref = _softmax(zd[db[b] + i], T)[x]
            assert r["p_x"][db[b] + i] == pytest.approx(p_ref, rel=1e-12, abs=1e-300)
            assert r["q_x"][db[b] + i] == pytest.approx(q_ref, rel=1e-12, abs=1e-300)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_masked_logits_have_zero_probability(dtype):
    # Logits of -inf (a vocabulary mask, shared by a request's target and draft rows, with a
    # long masked run) take probability 0: the statistics and p(x), q(x) are scipy's softmax
    # over the same rows (which maps -inf to 0), no emitted token is a masked one, and greedy
    # requests decode the argmax of the unmasked logits.
    temps = np.array([0.7, 0.0, 1.3, 0.25, 1.0, 0.0])
    w = workloads.small(B=6, gamma=4, V=3000, dtype=dtype, seed=13, temperatures=temps,
                        ragged=True, mask_frac=0.4, mask_span=1200)
    zt = workloads.decode(w.target, dtype)
    zd = workloads.decode(w.draft, dtype)
    assert np.isinf(zt).mean() > 0.5 and np.isinf(zd).any()
    r = oracle.verify(w)
    T32 = w.temperatures
    tb_all, db_all = w.target_base, w.draft_base
    for b, (tb, db, g) in enumerate(zip(tb_all, db_all, w.gammas)):
        n = r["num_accepted"][b]
        k = r["out_tokens"][tb + n]
        assert np.isfinite(zt[tb + n, k])                   # never a masked token
        if T32[b] > 0:
            for i in range(g):
                x = w.draft_tokens[db + i]
                assert np.isfinite(zd[db + i, x])           # drawn from the masked q
                p_ref = _softmax(zt[tb + i], T32[b])[x]
                q_ref = _softmax(zd[db + i], T32[b])[x]
                assert r["p_x"][db + i] == pytest.approx(p_ref, rel=1e-12, abs=1e-300)
                assert r["q_x"][db + i] == pytest.approx(q_ref, rel=1e-12, abs=1e-300)
            S_ref = np.exp(special.logsumexp((zt[tb] - zt[tb].max()) / T32[b]))
            assert r["row_sum_t"][tb] == pytest.approx(S_ref, rel=1e-12)
    out, nacc = _argmax_decoding(w)
    greedy = T32 == 0
    np.testing.assert_array_equal(r["num_accepted"][greedy], nacc[greedy])


def _argmax_decoding(w):
    """Greedy verification written as target-argmax decoding with numpy.argmax
    (first occurrence of the maximum)."""
    zt = workloads.decode(w.target, w.dtype)
    out = np.full(w.R_t, -1, dtype=np.int32)
    nacc = np.zeros(w.B, dtype=np.int32)
    for b, (tb, db, g) in enumerate(zip(w.target_base, w.draft_base, w.gammas)):
        am = [int(np.argmax(zt[tb + i])) for i in range(g + 1)]
        n = g
        for i in range(g):
            if w.draft_tokens[db + i] != am[i]:
                n = i
                break
        out[tb: tb + n] = w.draft_tokens[db: db + n]
        out[tb + n] = am[n]
        nacc[b] = n
    return out, nacc


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ragged", [False, True])
def test_greedy_equals_target_argmax_decoding(dtype, ragged):
    # Speculative Decoding : accélérer l'inférence des LLM, 'Pourquoi la qualité est
    # préservée' (temperature zero); Speculative Decoding wiki, '実装上の注意'.
    w = workloads.small(B=300, gamma=5, V=50, dtype=dtype, seed=3, temperatures=0.0,
                        draft_sigma=0.5, ragged=ragged)
    ref_out, ref_n = _argmax_decoding(w)
    for greedy_flag in (False, True):
        r = oracle.verify(w, greedy=greedy_flag)
        np.testing.assert_array_equal(r["out_tokens"], ref_out)
        np.testing.assert_array_equal(r["num_accepted"], ref_n)
    # the mix must contain both full acceptance and early rejection
    assert (ref_n == w.gammas).any() and (ref_n < w.gammas).any()


def test_greedy_ties_resolve_to_lowest_index():
    V = 12
    t = np.full((3, V), -1.0)
    t[0, [7, 3]] = 2.5          # tie at the maximum: argmax is 3
    t[1, :] = -2.0
    t[1, 9] = 0.0               # +0.0 and -0.0 tie at the maximum: argmax is 5
    t[1, 5] = -0.0
    t[2, [0, 11]] = 4.0         # bonus row: argmax 0
    for dtype in ("f32", "bf16"):
        # draft 3 (lowest tied index) accepted, then draft 9 rejected in favour of 5
        w = _explicit(t, np.zeros((2, V)), [3, 9], np.zeros((3, 2)), 0.0, 2, dtype)
        r = oracle.verify(w)
        assert list(r["out_tokens"]) == [3, 5, -1] and r["num_accepted"][0] == 1
        # draft 7 is a maximum too, but not the lowest-index one: rejected, 3 emitted
        w = _explicit(t, np.zeros((2, V)), [7, 5], np.zeros((3, 2)), 0.0, 2, dtype)
        r = oracle.verify(w)
        assert list(r["out_tokens"]) == [3, -1, -1] and r["num_accepted"][0] == 0
        # both accepted: bonus is the bonus row's lowest-index argmax
        w = _explicit(t, np.zeros((2, V)), [3, 5], np.zeros((3, 2)), 0.0, 2, dtype)
        r = oracle.verify(w)
        assert list(r["out_tokens"]) == [3, 5, 0] and r["num_accepted"][0] == 2


# --------------------------------------------------------------------------- invariants

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_p_equal_q_accepts_every_draft(dtype):
    # min(1, p/q) = 1 when p = q, and u < 1 always.
    w = workloads.small(B=64, gamma=6, V=300, dtype=dtype, seed=5, temperatures=0.8,
                        ragged=True)
    for b, (tb, db, g) in enumerate(zip(w.target_base, w.draft_base, w.gammas)):
        w.draft[db: db + g] = w.target[tb: tb + g]
    # draft tokens drawn from the new q (= p)
    rng = np.random.default_rng(99)
    w.draft_tokens[:] = workloads.draw_draft_tokens(workloads.decode(w.draft, dtype), 0.8, rng)
    w.uniforms[:, 0] = np.float32(np.nextafter(np.float32(1), np.float32(0)))  # worst case u
    r = oracle.verify(w)
    np.testing.assert_array_equal(r["num_accepted"], w.gammas)


@pytest.mark.parametrize("seed", [1, 2])
def test_emitted_count_prefix_and_residual_support(seed):
    # Between 1 and gamma_b + 1 tokens per step; the accepted prefix is the drafts; the
    # replacement is drawn where p > q, so never the rejected draft itself.
    temps = np.where(np.arange(40) % 5 == 0, 0.0, np.linspace(0.3, 1.5, 40))
    w = workloads.small(B=40, gamma=7, V=120, dtype="bf16", seed=seed, temperatures=temps,
                        ragged=True, draft_sigma=1.0)
    r = oracle.verify(w)
    zt = workloads.decode(w.target, w.dtype)
    zd = workloads.decode(w.draft, w.dtype)
    for b, (tb, db, g) in enumerate(zip(w.target_base, w.draft_base, w.gammas)):
        n = r["num_accepted"][b]
        slots = r["out_tokens"][tb: tb + g + 1]
        assert 0 <= n <= g
        assert (slots[: n + 1] >= 0).all() and (slots[n + 1:] == -1).all()
        np.testing.assert_array_equal(slots[:n], w.draft_tokens[db: db + n])
        T = w.temperatures[b]
        if T > 0 and n < g:
            k = slots[n]
            p = _softmax(zt[tb + n], T)
            q = _softmax(zd[db + n], T)
            assert p[k] > q[k]
            assert k != w.draft_tokens[db + n]


def test_ragged_layout_equals_requests_run_alone():
    w = workloads.small(B=12, gamma=6, V=90, dtype="f32", seed=8, ragged=True,
                        temperatures=np.linspace(0.0, 1.2, 12))
    r = oracle.verify(w)
    for b, (tb, db, g) in enumerate(zip(w.target_base, w.draft_base, w.gammas)):
        one = Workload("one", w.dtype, 1, int(g), w.V, w.target[tb: tb + g + 1],
                       w.draft[db: db + g], w.draft_tokens[db: db + g],
                       w.uniforms[tb: tb + g + 1], w.temperatures[b: b + 1], None)
        r1 = oracle.verify(one)
        np.testing.assert_array_equal(r1["out_tokens"], r["out_tokens"][tb: tb + g + 1])
        assert r1["num_accepted"][0] == r["num_accepted"][b]


def test_request_subset_leaves_other_requests_untouched():
    w = workloads.small(B=10, gamma=3, V=64, seed=4)
    full = oracle.verify(w)
    part = oracle.verify(w, requests=[2, 7])
    for b in range(10):
        tb = w.target_base[b]
        if b in (2, 7):
            np.testing.assert_array_equal(part["out_tokens"][tb: tb + 4],
                                          full["out_tokens"][tb: tb + 4])
        else:
            assert (part["out_tokens"][tb: tb + 4] == -2).all()


# --------------------------------------------------------------------------- cases by hand

def test_residual_supported_on_one_token():
    # target row 0: logits (0,0,0,3) -> p(3) ~ 0.864, the others ~ 0.045; draft row 0
    # uniform (q = 1/4 each).  p - q > 0 only at token 3, so after any rejection the
    # replacement is 3 whatever the uniform.  Draft x = 0: ratio p(0)/q(0) ~ 0.18.
    t = [[0, 0, 0, 3], [5, 0, 0, 0]]
    d = [[0, 0, 0, 0]]
    for u_sample in (0.0, 0.3, 0.999):
        w = _explicit(t, d, [0], [[0.5, u_sample], [0.0, 0.5]], 1.0, 1)
        r = oracle.verify(w)
        assert list(r["out_tokens"]) == [3, -1] and r["num_accepted"][0] == 0
    # u = 0.1 < 0.18: accepted; the bonus comes from target row 1, where p(0) ~ 0.98, so a
    # sample draw of 0.5 lands on token 0.
    w = _explicit(t, d, [0], [[0.1, 0.99], [0.99, 0.5]], 1.0, 1)
    r = oracle.verify(w)
    assert list(r["out_tokens"]) == [0, 0] and r["num_accepted"][0] == 1


def test_uniform_roles_and_strict_inverse_cdf():
    # target row 0: logits (0,0,2,2); draft row 0 uniform.  p = (a,a,c,c) with a ~ 0.0596,
    # c ~ 0.4404; q = 1/4.  (p-q)+ = (0,0,r,r): the residual puts exactly 1/2 on tokens 2 and
    # 3.  Draft x = 0 has ratio a/(1/4) ~ 0.238.
    t = [[0, 0, 2, 2], [0, 0, 2, 2]]
    d = [[0, 0, 0, 0]]
    # accept test uses u[0][0] = 0.9 -> reject (using u[0][1] = 0.2 would accept);
    # the draw uses u[0][1] = 0.2 -> token 2 (using u[0][0] = 0.9 would give 3)
    r = oracle.verify(_explicit(t, d, [0], [[0.9, 0.2], [0.0, 0.0]], 1.0, 1))
    assert list(r["out_tokens"]) == [2, -1]
    r = oracle.verify(_explicit(t, d, [0], [[0.9, 0.7], [0.0, 0.0]], 1.0, 1))
    assert list(r["out_tokens"]) == [3, -1]
    # u exactly at the CDF step (1/2): the strict C_k > u R picks the next token, 3
    r = oracle.verify(_explicit(t, d, [0], [[0.9, 0.5], [0.0, 0.0]], 1.0, 1))
    assert list(r["out_tokens"]) == [3, -1]
    assert r["cdf_gap"][0] == 0.0
    # accepted (0.1 < 0.238): the bonus draw is u[1][1] = 0.3 on p of row 1, whose CDF is
    # (0.06, 0.12, 0.56, 1.0) -> token 2 (u[0][1] = 0.05 would give 0, u[1][0] = 0.99 would
    # give 3)
    r = oracle.verify(_explicit(t, d, [0], [[0.1, 0.05], [0.99, 0.3]], 1.0, 1))
    assert list(r["out_tokens"]) == [0, 2]


def test_temperature_divides_logits():
    # p = softmax(z / T): with logits (0, ln 3) and T = 0.5 the target gives p = (1/10, 9/10)
    # (softmax(z * T) would give (0.366, 0.634)); draft logits (0, 0) give q = 1/2.
    # Draft x = 0: ratio = 0.1/0.5 = 0.2; u = 0.25 rejects, u = 0.15 accepts.
    t = [[0.0, np.log(3.0)], [0.0, 0.0]]
    d = [[0.0, 0.0]]
    r = oracle.verify(_explicit(t, d, [0], [[0.25, 0.0], [0.0, 0.0]], 0.5, 1))
    assert r["num_accepted"][0] == 0 and r["out_tokens"][0] == 1
    assert r["p_x"][0] == pytest.approx(0.1, rel=1e-6)   # ln 3 is stored as float32
    r = oracle.verify(_explicit(t, d, [0], [[0.15, 0.0], [0.0, 0.0]], 0.5, 1))
    assert r["num_accepted"][0] == 1


def test_draft_ids_outside_vocabulary_are_rejected():
    t = [[0, 1, 2], [0, 1, 2], [0, 1, 2]]
    d = [[0, 1, 2], [0, 1, 2]]
    for bad in (-1, 3):
        r = oracle.verify(_explicit(t, d, [2, bad], [[0.0, 0.0], [0.0, 0.9], [0.0, 0.0]],
                                    1.0, 2))
        assert r["num_accepted"][0] == 1 and r["out_tokens"][0] == 2
        assert r["p_x"][1] == 0.0 and r["q_x"][1] == 0.0
        # p = q at row 1 so the residual is empty: the fallback samples from p
        assert r["fallback"][0] == 1 and r["out_tokens"][1] == 2
        rg = oracle.verify(_explicit(t, d, [2, bad], np.zeros((3, 2)), 0.0, 2))
        assert list(rg["out_tokens"]) == [2, 2, -1]


def test_low_temperature_sampling_reduces_to_greedy():
    # As T -> 0+, p and q tend to one-hot vectors at the argmaxes: acceptance, residual and
    # bonus all return the target argmax, which is the greedy result.
    T = 1e-6
    w = workloads.small(B=200, gamma=5, V=40, dtype="f32", seed=21, temperatures=T,
                        draft_sigma=0.5)
    for rows in (w.target, w.draft):     # every row's maximum is clear at this temperature
        srt = np.sort(workloads.decode(rows, "f32"), axis=1)
        assert (srt[:, -1] - srt[:, -2]).min() > 50 * T
    rs = oracle.verify(w)
    rg = oracle.verify(w, greedy=True)
    np.testing.assert_array_equal(rs["out_tokens"], rg["out_tokens"])
    np.testing.assert_array_equal(rs["num_accepted"], rg["num_accepted"])


# --------------------------------------------------------------------------- distributions

def test_acceptance_probability_is_min_one_ratio():
    # Stratified grid of N uniforms: the accepted fraction equals min(1, p(x)/q(x)) to 1/N.
    V, N = 5, 4000
    zt = np.array([[0.3, -1.0, 1.2, 0.0, 0.7], [0.0] * V])
    zd = np.array([[1.0, -0.5, 0.2, 0.4, 0.7]])
    T = 0.8
    p, q = _softmax(zt[0], T), _softmax(zd[0], T)
    grid = ((np.arange(N) + 0.5) / N).astype(np.float32)
    for x in range(V):
        w = Workload("grid", "f32", N, 1, V, np.tile(zt.astype(np.float32), (N, 1)),
                     np.tile(zd.astype(np.float32), (N, 1)), np.full(N, x, np.int32),
                     _grid_uniforms(grid), np.full(N, T, np.float32))
        r = oracle.verify(w)
        frac = (r["num_accepted"] == 1).mean()
        assert abs(frac - min(1.0, p[x] / q[x])) <= 1.0 / N + 1e-7


def _grid_uniforms(grid):
    """Uniform rows for a gamma = 1 request per grid point: [u, 0.5] then [0.5, 0.5]."""
    n = len(grid)
    u = np.full((n, 2, 2), 0.5, dtype=np.float32)
    u[:, 0, 0] = grid
    return u.reshape(2 * n, 2)


def test_exact_marginal_on_a_stratified_grid():
    # V = 3, gamma = 1.  For each draft x (weight q(x)) and an N x N stratified grid over
    # (u_accept, u_sample), the token emitted at position 0 must be distributed as p to
    # O(1/N): the exactness claim of the pages, without sampling noise.
    V, N, T = 3, 600, 1.0
    zt = np.array([[0.2, 1.1, -0.4], [0.0, 0.0, 0.0]])
    zd = np.array([[0.9, 0.1, 0.3]])
    p, q = _softmax(zt[0], T), _softmax(zd[0], T)
    g = ((np.arange(N) + 0.5) / N).astype(np.float32)
    ua, us = np.meshgrid(g, g, indexing="ij")
    n = N * N
    uni = np.full((n, 2, 2), 0.5, dtype=np.float32)
    uni[:, 0, 0] = ua.ravel()
    uni[:, 0, 1] = us.ravel()
    dist = np.zeros(V)
    for x in range(V):
        w = Workload("grid2", "f32", n, 1, V, np.tile(zt.astype(np.float32), (n, 1)),
                     np.tile(zd.astype(np.float32), (n, 1)), np.full(n, x, np.int32),
                     uni.reshape(2 * n, 2), np.full(n, T, np.float32))
        r = oracle.verify(w)
        tok0 = r["out_tokens"].reshape(n, 2)[:, 0]
        dist += q[x] * np.bincount(tok0, minlength=V) / n
    np.testing.assert_allclose(dist, p, atol=3.0 / N)


def _chi2_trials(seed, V=16, gamma=3, T=0.9, n_total=1_000_000, chunk=250_000):
    T = float(np.float32(T))
    rng = np.random.default_rng(seed)
    zt = rng.normal(0, 1.5, size=(gamma + 1, V))
    zd = zt[:gamma] + rng.normal(0, 1.0, size=(gamma, V))
    toks, nacc = [], []
    for c in range(n_total // chunk):
        w = workloads.tiled(zt, zd, chunk, T=T, seed=seed * 100 + c)
        r = oracle.verify(w)
        toks.append(r["out_tokens"].reshape(chunk, gamma + 1))
        nacc.append(r["num_accepted"])
        zt_s = workloads.decode(w.target[: gamma + 1], "f32")
        zd_s = workloads.decode(w.draft[:gamma], "f32")
    return np.concatenate(toks), np.concatenate(nacc), zt_s, zd_s, T


def test_chi_square_emitted_tokens_follow_p():
    # 10^6 trials, V = 16, gamma = 3, a different p and q at every position.  Conditional
    # on reaching position k, the emitted token there must be distributed as p_k (accepted
    # drafts, residual draws and the bonus together).
    toks, nacc, zt, zd, T = _chi2_trials(seed=7)
    gamma = zd.shape[0]
    for k in range(gamma + 1):
        reached = nacc >= k
        assert reached.sum() > 50_000
        obs = np.bincount(toks[reached, k], minlength=zt.shape[1])
        pval, x2, df = chi2_pvalue(obs, _softmax(zt[k], T))
        assert pval > 1e-3, (k, pval, x2, df)
    # acceptance rate at position 0 is sum_x min(p, q)
    beta0 = np.minimum(_softmax(zt[0], T), _softmax(zd[0], T)).sum()
    assert abs((nacc >= 1).mean() - beta0) < 5 * np.sqrt(beta0 * (1 - beta0) / len(nacc))


def test_chi_square_residual_follows_p_corr():
    # Conditional on a rejection at position 0, the replacement follows
    # max(p - q, 0) / sum max(p - q, 0) (Speculative Decoding wiki, p_corr).
    toks, nacc, zt, zd, T = _chi2_trials(seed=9)
    p, q = _softmax(zt[0], T), _softmax(zd[0], T)
    rej = nacc == 0
    obs = np.bincount(toks[rej, 0], minlength=zt.shape[1])
    pval, x2, df = chi2_pvalue(obs, np.maximum(p - q, 0.0))
    assert pval > 1e-3, (pval, x2, df)


def test_worked_example_tokens_per_pass():
    g = json.loads((GOLDEN / "tokens_per_pass.json").read_text())
    alpha, gamma = g["alpha"], g["gamma"]
    closed = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    assert abs(closed - g["tokens_per_pass_printed"]) <= g["printed_resolution"]
    accepted_closed = sum(alpha ** k for k in range(1, gamma + 1))
    assert accepted_closed == pytest.approx(closed - 1, rel=1e-12)
    # p = (0.9, 0.1), q = (0.7, 0.3) at every position: sum min(p, q) = 0.8 = alpha
    zt = np.log(np.array([[0.9, 0.1]] * (gamma + 1)))
    zd = np.log(np.array([[0.7, 0.3]] * gamma))
    n = 1_000_000
    w = workloads.tiled(zt, zd, n, T=1.0, seed=31)
    r = oracle.verify(w)
    emitted = r["num_accepted"].astype(np.float64) + 1
    se = emitted.std() / np.sqrt(n)
    assert abs(emitted.mean() - closed) < 4 * se, (emitted.mean(), closed, se)
    assert abs(r["num_accepted"].mean() - accepted_closed) < 4 * se
    assert abs(emitted.mean() - g["tokens_per_pass_printed"]) <= g["printed_resolution"]


# --------------------------------------------------------------------------- commit step

def _commit_case(B=9, gamma=5, V=300, seed=5, temps=None, capacity=40):
    temps = np.linspace(0.0, 1.2, B) if temps is None else temps
    w = workloads.small(B=B, gamma=gamma, V=V, dtype="f32", seed=seed, ragged=True,
                        temperatures=temps, draft_sigma=0.6)
    r = oracle.verify(w)
    rng = np.random.default_rng(seed)
    seq = rng.integers(0, V, size=(B, capacity)).astype(np.int32)
    length = rng.integers(0, capacity - gamma - 1, size=B).astype(np.int32)
    return w, r, seq, length


def test_commit_appends_accepted_drafts_then_the_emitted_token():
    # The accepted prefix is the drafts themselves (aimpact, "Il meccanismo"), followed by
    # the one token drawn at the stop row; the rest of each history is untouched.
    w, r, seq, length = _commit_case()
    before, len0 = seq.copy(), length.copy()
    oracle.commit(r["out_tokens"], r["num_accepted"], w.gamma, seq, length, cu_draft=w.cu_draft)
    for b in range(w.B):
        n = int(r["num_accepted"][b])
        drafts = w.draft_tokens[w.draft_base[b]: w.draft_base[b] + n]
        L = int(len0[b])
        assert length[b] == L + n + 1
        np.testing.assert_array_equal(seq[b, L: L + n], drafts)
        assert seq[b, L + n] == r["out_tokens"][w.target_base[b] + n]
        np.testing.assert_array_equal(seq[b, :L], before[b, :L])
        np.testing.assert_array_equal(seq[b, L + n + 1:], before[b, L + n + 1:])


def test_commit_of_a_greedy_step_appends_target_argmax_decoding():
    # At temperature zero the committed tokens are the target's own argmax decoding up to the
    # first disagreement, computed here with numpy (first occurrence on ties).
    w, r, seq, length = _commit_case(temps=np.zeros(9), seed=8)
    len0 = length.copy()
    oracle.commit(r["out_tokens"], r["num_accepted"], w.gamma, seq, length, cu_draft=w.cu_draft)
    zt = workloads.decode(w.target, w.dtype)
    for b in range(w.B):
        t0, d0, gb = w.target_base[b], w.draft_base[b], int(w.gammas[b])
        ref = []
        for i in range(gb + 1):
            g = int(np.argmax(zt[t0 + i]))
            ref.append(g)
            if i == gb or w.draft_tokens[d0 + i] != g:
                break
        L = int(len0[b])
        assert length[b] == L + len(ref)
        np.testing.assert_array_equal(seq[b, L: L + len(ref)], ref)


def test_commit_rejects_counts_outside_the_step():
    # a step accepts between 0 and gamma_b drafts: any other count is refused, nothing written
    out = np.array([7, 8, 9, 4, 5, -1], dtype=np.int32)   # two requests, gamma 2
    seq = np.zeros((2, 10), dtype=np.int32)
    ln = np.array([3, 2], dtype=np.int32)
    for bad in ([-1, 1], [3, 1], [0, -2]):
        with pytest.raises(ValueError):
            oracle.commit(out, np.array(bad, dtype=np.int32), 2, seq, ln)
    oracle.commit(out, np.array([0, 1], dtype=np.int32), 2, seq, ln)
    assert list(ln) == [4, 4] and seq[0, 3] == 7 and list(seq[1, 2:4]) == [4, 5]


def test_commit_truncates_at_capacity_and_never_writes_past_it():
    w, r, seq, length = _commit_case(B=7, gamma=6, seed=11, capacity=12)
    length[:] = np.array([12, 11, 10, 8, 5, 0, 12], dtype=np.int32)[: w.B]
    before, len0 = seq.copy(), length.copy()
    stats = np.zeros(5, dtype=np.uint64)
    oracle.commit(r["out_tokens"], r["num_accepted"], w.gamma, seq, length,
                  cu_draft=w.cu_draft, stats=stats)
    lost = 0
    for b in range(w.B):
        n = int(r["num_accepted"][b])
        L = int(len0[b])
        assert length[b] == min(L + n + 1, 12)
        lost += max(0, L + n + 1 - 12)
        np.testing.assert_array_equal(seq[b, :L], before[b, :L])
    assert int(stats[4]) == lost
    assert int(stats[2]) == int(r["num_accepted"].sum()) + w.B


def test_commit_counters_accumulate_and_match_the_step():
    w, r, seq, length = _commit_case(seed=21)
    stats = np.zeros(5, dtype=np.uint64)
    hist = np.zeros(w.gamma + 1, dtype=np.uint64)
    for _ in range(2):
        s2, l2 = seq.copy(), length.copy()
        oracle.commit(r["out_tokens"], r["num_accepted"], w.gamma, s2, l2,
                      cu_draft=w.cu_draft, stats=stats, hist=hist)
    n = r["num_accepted"].astype(np.int64)
    assert list(stats[:4]) == [2 * int(w.gammas.sum()), 2 * int(n.sum()),
                               2 * int(n.sum() + w.B), 2 * w.B]
    np.testing.assert_array_equal(hist, 2 * np.bincount(n, minlength=w.gamma + 1))


def test_commit_telemetry_reproduces_the_worked_example():
    # blent.ai, "Quel gain espérer ?": at acceptance rate 0.8 and 4 drafts the target pass
    # yields (1 - 0.8^5) / 0.2 = 3.36 (printed: about 3.4) tokens on average; the counters
    # must show it, and the accepted lengths must follow P(n = k) = a^k (1 - a) for k < 4,
    # P(n = 4) = a^4 (i.i.d. acceptance at rate a).
    g = json.loads((GOLDEN / "tokens_per_pass.json").read_text())
    alpha, gamma = g["alpha"], g["gamma"]
    zt = np.log(np.array([[0.9, 0.1]] * (gamma + 1)))
    zd = np.log(np.array([[0.7, 0.3]] * gamma))
    n = 200_000
    w = workloads.tiled(zt, zd, n, T=1.0, seed=41)
    r = oracle.verify(w)
    seq = np.zeros((n, gamma + 1), dtype=np.int32)
    length = np.zeros(n, dtype=np.int32)
    stats = np.zeros(5, dtype=np.uint64)
    hist = np.zeros(gamma + 1, dtype=np.uint64)
    oracle.commit(r["out_tokens"], r["num_accepted"], gamma, seq, length, stats=stats, hist=hist)
    proposed, accepted, emitted, requests, lost = (int(v) for v in stats)
    assert (proposed, requests, lost) == (gamma * n, n, 0)
    per_pass = emitted / requests
    closed = (1 - alpha ** (gamma + 1)) / (1 - alpha)
    assert abs(per_pass - closed) < 4 * 1.25 / np.sqrt(n)
    assert abs(per_pass - g["tokens_per_pass_printed"]) <= g["printed_resolution"]
    law = np.array([alpha ** k * (1 - alpha) for k in range(gamma)] + [alpha ** gamma])
    pval, x2, df = chi2_pvalue(hist.astype(np.int64), law)
    assert pval > 1e-3, (pval, x2, df)
    assert accepted / proposed == pytest.approx(sum(alpha ** k for k in range(1, gamma + 1)) / gamma,
                                                abs=4 * 1.4 / gamma / np.sqrt(n))


# --------------------------------------------------------------------------- n-gram drafter

def _find_reference(h, n_min, n_max, gamma):
    """Prompt lookup through Python's substring search (lowest index): tokens become
    fixed-width text, the pattern is the last n tokens, searched in the context without its
    last token (so only proper earlier occurrences, possibly overlapping the suffix)."""
    L = len(h)
    text = "".join(f"|{t:08x}" for t in h[: max(L - 1, 0)])
    for n in range(n_max, n_min - 1, -1):
        if n >= L:
            continue
        pat = "".join(f"|{t:08x}" for t in h[L - n:])
        pos = text.find(pat)
        if pos >= 0:
            j = pos // 9
            return list(h[j + n: min(j + n + gamma, L)]), j, n
    return [], -1, 0


def _ngram_one(h, n_min, n_max, gamma, capacity=None):
    cap = capacity or max(len(h), 1)
    seq = np.zeros((1, cap), dtype=np.int32)
    seq[0, : len(h)] = h
    return oracle.ngram(seq, np.array([len(h)], dtype=np.int32), n_min, n_max, gamma)


@pytest.mark.parametrize("h,n_min,n_max,gamma,expect", [
    ([1, 2, 3, 9, 1, 2, 3], 1, 3, 2, [9, 1]),        # the 3-gram 1 2 3 seen at 0
    ([5, 8, 6, 7, 2, 6, 7], 1, 2, 3, [2, 6, 7]),     # longest first: 2-gram 6 7 beats 1-gram 7
    ([1, 2, 3, 4], 1, 3, 4, []),                     # nothing recurs
    ([4, 4], 1, 1, 5, [4]),                          # proposals stop at the context's end
    ([7, 7, 7, 7], 1, 3, 4, [7]),                    # overlapping occurrence at 0
    ([3, 1, 3, 2, 3], 1, 1, 2, [1, 3]),              # earliest of several occurrences
    ([9], 1, 4, 3, []),                              # too short to hold any earlier n-gram
    ([2, 5, 2, 5, 2], 2, 2, 1, [5]),                 # n fixed at 2: 5 2 at 1, then 5
])
def test_ngram_hand_cases(h, n_min, n_max, gamma, expect):
    r = _ngram_one(h, n_min, n_max, gamma)
    assert r["counts"][0] == len(expect)
    assert list(r["dense"][0, : len(expect)]) == expect
    assert all(v == -1 for v in r["dense"][0, len(expect):])
    assert list(r["packed"]) == expect and list(r["cu"]) == [0, len(expect)]


@pytest.mark.parametrize("alphabet", [2, 3, 8, 50])
def test_ngram_matches_substring_search(alphabet):
    rng = np.random.default_rng(alphabet)
    B, cap, gamma = 200, 80, 5
    seq = rng.integers(0, alphabet, size=(B, cap)).astype(np.int32)
    length = rng.integers(0, cap + 1, size=B).astype(np.int32)
    for n_min, n_max in ((1, 1), (2, 4), (1, 6)):
        r = oracle.ngram(seq, length, n_min, n_max, gamma)
        off = 0
        assert r["cu"][0] == 0
        for b in range(B):
            h = list(seq[b, : length[b]])
            ref, j, n = _find_reference(h, n_min, n_max, gamma)
            assert list(r["dense"][b, : r["counts"][b]]) == ref
            assert (r["match_j"][b], r["match_n"][b]) == (j, n)
            assert r["cu"][b + 1] - r["cu"][b] == len(ref)
            assert list(r["packed"][off: off + len(ref)]) == ref
            off += len(ref)


def test_ngram_proposals_continue_the_matched_window():
    # invariants: the matched window equals the pattern, the proposals are what followed it
    rng = np.random.default_rng(3)
    B, cap, gamma = 100, 200, 7
    base = rng.integers(0, 1000, size=(B, cap)).astype(np.int32)
    for b in range(B):   # plant a copy of an earlier span at the end of the context
        a = rng.integers(0, 60)
        base[b, 150:170] = base[b, a: a + 20]
    length = np.full(B, 170, dtype=np.int32)
    r = oracle.ngram(base, length, 2, 5, gamma)
    assert (r["match_n"] == 5).all()
    for b in range(B):
        j, n, c = r["match_j"][b], r["match_n"][b], r["counts"][b]
        assert c == min(gamma, 170 - (j + n)) and c >= 1
        np.testing.assert_array_equal(base[b, j: j + n], base[b, 170 - n: 170])
        np.testing.assert_array_equal(r["dense"][b, :c], base[b, j + n: j + n + c])


# --------------------------------------------------------------------------- exact enumeration

def _intervals(edges):
    """Sub-intervals of [0, 1) cut at ``edges``: (midpoint, length) pairs."""
    e = np.unique(np.clip(np.concatenate([[0.0], np.asarray(edges, dtype=np.float64), [1.0]]), 0, 1))
    return [((a + b) / 2, b - a) for a, b in zip(e[:-1], e[1:]) if b - a > 1e-6]


@pytest.mark.parametrize("V,seed", [(3, 1), (4, 2), (4, 3)])
def test_exact_composition_by_enumeration(V, seed):
    # gamma = 2.  Every draft pair (x0, x1), weighted q0(x0) q1(x1), and every interval of the
    # three uniforms that matter (accept at 0, accept at 1, the stop row's draw) cut at the
    # analytic thresholds min(1, p/q) and the CDF steps of the distribution drawn from.  The
    # oracle is run once at each interval's midpoint and weighted by its length: this is the
    # exact distribution of its output.  It must emit p0 at position 0, given n >= 1 p1 at
    # position 1, and given n = 2 p2 at position 2 (to 1e-12), with
    # P(n >= k) = prod_{i<k} sum_x min(p_i, q_i).
    rng = np.random.default_rng(seed)
    zt = rng.normal(0, 1.0, size=(3, V))
    zd = rng.normal(0, 1.0, size=(2, V))
    tr = workloads.decode(workloads.encode(zt, "f32"), "f32")
    dr = workloads.decode(workloads.encode(zd, "f32"), "f32")
    p = [_softmax(tr[i], 1.0) for i in range(3)]
    q = [_softmax(dr[i], 1.0) for i in range(2)]

    def cdf_edges(w):
        c = np.cumsum(w)
        return c / c[-1]

    cases = []   # (weight, x0, x1, u rows)
    for x0 in range(V):
        for x1 in range(V):
            wx = q[0][x0] * q[1][x1]
            r0 = p[0][x0] / q[0][x0]
            for ua0, la0 in _intervals([r0]):
                if ua0 >= r0:   # rejected at 0: draw from (p0 - q0)+
                    for us0, ls0 in _intervals(cdf_edges(np.maximum(p[0] - q[0], 0))):
                        cases.append((wx * la0 * ls0, x0, x1, [[ua0, us0], [0.5, 0.5], [0.5, 0.5]]))
                    continue
                r1 = p[1][x1] / q[1][x1]
                for ua1, la1 in _intervals([r1]):
                    if ua1 >= r1:
                        edges = cdf_edges(np.maximum(p[1] - q[1], 0))
                        for us1, ls1 in _intervals(edges):
                            cases.append((wx * la0 * la1 * ls1, x0, x1,
                                          [[ua0, 0.5], [ua1, us1], [0.5, 0.5]]))
                    else:
                        for us2, ls2 in _intervals(cdf_edges(p[2])):
                            cases.append((wx * la0 * la1 * ls2, x0, x1,
                                          [[ua0, 0.5], [ua1, 0.5], [0.5, us2]]))
    n = len(cases)
    wts = np.array([c[0] for c in cases])
    assert abs(wts.sum() - 1.0) < 1e-12
    w = Workload("enum", "f32", n, 2, V, np.tile(workloads.encode(zt, "f32"), (n, 1)),
                 np.tile(workloads.encode(zd, "f32"), (n, 1)),
                 np.array([[c[1], c[2]] for c in cases], np.int32).ravel(),
                 np.array([c[3] for c in cases], np.float32).reshape(3 * n, 2),
                 np.ones(n, np.float32))
    r = oracle.verify(w)
    toks = r["out_tokens"].reshape(n, 3)
    nacc = r["num_accepted"]
    first = np.bincount(toks[:, 0], weights=wts, minlength=V)
    np.testing.assert_allclose(first, p[0], rtol=0, atol=1e-12)
    reach1 = nacc >= 1
    beta = [np.minimum(p[i], q[i]).sum() for i in range(2)]
    assert abs(wts[reach1].sum() - beta[0]) < 1e-12
    assert abs(wts[nacc >= 2].sum() - beta[0] * beta[1]) < 1e-12
    second = np.bincount(toks[reach1, 1], weights=wts[reach1], minlength=V) / wts[reach1].sum()
    np.testing.assert_allclose(second, p[1], rtol=0, atol=1e-12)
    reach2 = nacc >= 2   # every draft accepted: the bonus token comes from p2
    third = np.bincount(toks[reach2, 2], weights=wts[reach2], minlength=V) / wts[reach2].sum()
    np.testing.assert_allclose(third, p[2], rtol=0, atol=1e-12)
    # accepted prefixes are the drafts themselves
    d = w.draft_tokens.reshape(n, 2)
    assert (toks[reach1, 0] == d[reach1, 0]).all()


@pytest.mark.parametrize("T", [0.3, 1.0, 2.5])
def test_inverse_cdf_matches_searchsorted(T):
    # p = q accepts every draft, so the token at row gamma is the inverse CDF of p there with
    # the row's draw uniform: numpy's searchsorted(cumsum(w), u * sum(w), 'right') is the first
    # index whose running sum exceeds u R, in index order, skipping zero weights.
    rng = np.random.default_rng(int(T * 10))
    B, gamma, V = 3000, 1, 97
    z = rng.normal(0, 2.0, size=(B * (gamma + 1), V))
    z[:, ::7] = -1e4          # zero-weight tokens in exp: never drawn
    T32 = float(np.float32(T))
    tgt = workloads.encode(z, "f32")
    dft = tgt.reshape(B, gamma + 1, V)[:, :gamma].reshape(B * gamma, V).copy()
    tok = rng.integers(0, V, size=B * gamma).astype(np.int32)
    tok[tok % 7 == 0] += 1
    uni = rng.random((B * (gamma + 1), 2), dtype=np.float32)
    w = Workload("icdf", "f32", B, gamma, V, tgt, dft, tok, uni, np.full(B, T32, np.float32))
    r = oracle.verify(w)
    assert (r["num_accepted"] == gamma).all()
    zs = workloads.decode(tgt, "f32").reshape(B, gamma + 1, V)[:, gamma]
    wts = np.exp((zs - zs.max(axis=1, keepdims=True)) / T32)
    C = np.cumsum(wts, axis=1)
    u = uni.reshape(B, gamma + 1, 2)[:, gamma, 1].astype(np.float64)
    expect = np.array([np.searchsorted(C[b], u[b] * C[b, -1], side="right") for b in range(B)])
    got = r["out_tokens"].reshape(B, gamma + 1)[:, gamma]
    clear = r["cdf_gap"] > 1e-12          # ties within rounding of a CDF step: either is valid
    assert clear.mean() > 0.99
    np.testing.assert_array_equal(got[clear], expect[clear])
    assert not np.isin(got, np.arange(0, V, 7)).any()


# --------------------------------------------------------------------------- decision diagnostics
#
# The parity rule between the GPU and the oracle rests on three of the oracle's diagnostics:
# the accept-test margin |u - p(x)/q(x)| at every decision up to the stop, the CDF gap of the
# stop row's draw, and the residual mass sum_k max(p_k - q_k, 0) (wiki page, section
# "数式で見る speculative decoding の正しさ": alpha(x) and p_corr; blent.ai page, section
# "Pourquoi la qualité est préservée").  They are pinned twice: element by element against a
# computation from scipy's softmax and numpy's cumsum / searchsorted, and by their meaning (a
# uniform moved by less than the margin or gap leaves the oracle's output unchanged, one
# moved past it changes it).

def _reference_decisions(w, b):
    """Request b's decisions from scipy softmax and numpy: (margins up to the stop, stop row,
    weights drawn from, R, fallback, token, gap below u, gap above u)."""
    T = float(w.temperatures[b])
    tb, db, g = int(w.target_base[b]), int(w.draft_base[b]), int(w.gammas[b])
    zt = workloads.decode(w.target[tb: tb + g + 1], w.dtype)
    zd = workloads.decode(w.draft[db: db + g], w.dtype)
    margins, stop = [], g
    for i in range(g):
        x = int(w.draft_tokens[db + i])
        p = _softmax(zt[i], T)[x] if 0 <= x < w.V else 0.0
        q = _softmax(zd[i], T)[x] if 0 <= x < w.V else 0.0
        ratio = p / q if q > 0 else (np.inf if p > 0 else 0.0)
        u = float(w.uniforms[tb + i, 0])
        margins.append(abs(u - ratio))
        if not u < ratio:
            stop = i
            break
    p_stop = _softmax(zt[stop], T)
    r = np.maximum(p_stop - _softmax(zd[stop], T), 0.0) if stop < g else p_stop
    fallback = not r.sum() > 0
    if fallback:
        r = p_stop
    R = r.sum()
    u1 = float(w.uniforms[tb + stop, 1])
    C = np.cumsum(r)
    k = int(np.searchsorted(C, u1 * R, side="right"))
    below = u1 - (C[k - 1] / R if k > 0 else 0.0)
    above = C[k] / R - u1
    return dict(margins=np.array(margins), stop=stop, R=R, fallback=fallback, token=k,
                below=below, above=above)


DIAG_CASES = [  # (B, gamma, V, dtype, seed, temperature, draft noise)
    (40, 6, 300, "f32", 101, 1.0, 0.6),
    (40, 5, 257, "bf16", 102, 0.7, 1.0),
    (30, 8, 120, "f32", 103, 0.3, 0.2),
    (30, 4, 500, "bf16", 104, 2.5, 1.5),
]


@pytest.mark.parametrize("B,gamma,V,dtype,seed,T,sigma", DIAG_CASES)
def test_diagnostics_match_scipy_and_numpy(B, gamma, V, dtype, seed, T, sigma):
    w = workloads.small(B=B, gamma=gamma, V=V, dtype=dtype, seed=seed, temperatures=T,
                        draft_sigma=sigma, ragged=True)
    w.draft_tokens[::11] = V        # outside the vocabulary: p = q = 0, ratio 0, rejected
    r = oracle.verify(w)
    for b in range(w.B):
        ref = _reference_decisions(w, b)
        db, g, n = int(w.draft_base[b]), int(w.gammas[b]), int(r["num_accepted"][b])
        assert n == ref["stop"]
        m = r["margin"][db: db + g]
        np.testing.assert_allclose(m[: n + 1 if n < g else g], ref["margins"], rtol=1e-11,
                                   atol=1e-13)
        assert np.isnan(m[n + 1:]).all()     # nothing recorded past the stop
        assert r["fallback"][b] == int(ref["fallback"])
        assert r["resid_mass"][b] == pytest.approx(ref["R"], rel=1e-11, abs=1e-15)
        assert r["cdf_gap"][b] == pytest.approx(min(ref["below"], ref["above"]), abs=1e-11)
        if min(ref["below"], ref["above"]) > 1e-9:
            assert r["out_tokens"][int(w.target_base[b]) + n] == ref["token"]


def test_residual_mass_is_one_for_the_bonus_and_the_fallback():
    # Every draft accepted (draft = target, accept uniforms 0): the bonus is drawn from p,
    # whose mass is 1.  Draft = target and accept uniforms at the top: the first draft is
    # rejected with p = q, the residual is empty, and the draw falls back to p (mass 1).
    w = workloads.small(B=20, gamma=3, V=200, dtype="f32", seed=7, temperatures=0.8)
    for b in range(w.B):
        tb, db = int(w.target_base[b]), int(w.draft_base[b])
        w.draft[db: db + 3] = w.target[tb: tb + 3]
    w.uniforms[:, 0] = 0.0
    r = oracle.verify(w)
    assert (r["num_accepted"] == 3).all() and (r["fallback"] == 0).all()
    np.testing.assert_allclose(r["resid_mass"], 1.0, rtol=1e-13)
    w.uniforms[:, 0] = np.float32(np.nextafter(np.float32(1), np.float32(0)))
    w.draft_tokens[:] = 0
    w.target[:, 0] = w.target.max()      # token 0 has the row's largest p (= q): ratio 1
    w.draft[:, 0] = w.target[0, 0]
    r = oracle.verify(w)
    assert (r["num_accepted"] == 3).all()     # ratio exactly 1 > u: accepted
    w.draft_tokens[:] = 1                     # ratio 1 as well, but u = 1 - 2^-24 < 1 ...
    w.uniforms[:, 0] = 1.0                    # ... so take u = 1: rejected, p = q, empty
    r = oracle.verify(w)
    assert (r["num_accepted"] == 0).all() and (r["fallback"] == 1).all()
    np.testing.assert_allclose(r["resid_mass"], 1.0, rtol=1e-13)
    for b in range(w.B):
        assert min(_reference_decisions(w, b)["below"], _reference_decisions(w, b)["above"]) \
            == pytest.approx(r["cdf_gap"][b], abs=1e-11)


def _one(w, b):
    tb, db, g = int(w.target_base[b]), int(w.draft_base[b]), int(w.gammas[b])
    return Workload("one", w.dtype, 1, g, w.V, w.target[tb: tb + g + 1].copy(),
                    w.draft[db: db + g].copy(), w.draft_tokens[db: db + g].copy(),
                    w.uniforms[tb: tb + g + 1].copy(), w.temperatures[b: b + 1].copy(), None)


def test_margin_is_the_distance_to_the_accept_boundary():
    # Moving an accept uniform by half its margin toward the boundary leaves every decision
    # as it was; moving it one and a half margins (past the boundary) flips that decision.
    w = workloads.small(B=60, gamma=5, V=400, dtype="f32", seed=61, temperatures=0.9,
                        draft_sigma=0.8, ragged=True)
    r = oracle.verify(w)
    flipped = 0
    for b in range(w.B):
        one = _one(w, b)
        g, n = one.gamma, int(r["num_accepted"][b])
        last = n if n < g else g - 1
        for i in range(last + 1):
            m = float(r["margin"][int(w.draft_base[b]) + i])
            u = float(one.uniforms[i, 0])
            if m < 1e-4:
                continue
            toward = -1.0 if i == n else 1.0     # rejected: u above the ratio; accepted: below
            for scale, same in ((0.5, True), (1.5, False)):
                v = u + toward * scale * m
                if not 0.0 <= v < 1.0:
                    continue
                o = _one(w, b)
                o.uniforms[i, 0] = np.float32(v)
                n2 = int(oracle.verify(o)["num_accepted"][0])
                if same:
                    assert n2 == n, (b, i, scale)
                else:
                    assert (n2 > i) if i == n else (n2 == i), (b, i, scale, n, n2)
                    flipped += 1
    assert flipped > 40


def test_cdf_gap_is_the_distance_to_the_nearest_cdf_step():
    # Moving the draw's uniform by half the gap, either way, keeps the token; moving it by
    # one and a half gaps toward the nearer CDF step gives the neighbouring token.  A gap
    # taken on one side only fails where the other side's step is the nearer one.
    w = workloads.small(B=80, gamma=3, V=60, dtype="f32", seed=62, temperatures=1.1,
                        draft_sigma=1.2, ragged=True)
    r = oracle.verify(w)
    sides = {"below": 0, "above": 0}
    for b in range(w.B):
        ref = _reference_decisions(w, b)
        gap = float(r["cdf_gap"][b])
        if gap < 1e-4:
            continue
        tb, n = int(w.target_base[b]), int(r["num_accepted"][b])
        tok = int(r["out_tokens"][tb + n])
        u = float(w.uniforms[tb + n, 1])
        near = "below" if ref["below"] <= ref["above"] else "above"
        sign = -1.0 if near == "below" else 1.0
        for delta, same in ((0.5 * gap, True), (-0.5 * gap, True), (1.5 * sign * gap, False)):
            v = u + delta
            if not 0.0 <= v < 1.0:
                continue
            o = _one(w, b)
            o.uniforms[n, 1] = np.float32(v)
            t2 = int(oracle.verify(o)["out_tokens"][n])
            if same:
                assert t2 == tok, (b, delta)
            else:
                assert (t2 < tok) if near == "below" else (t2 > tok), (b, near, tok, t2)
                sides[near] += 1
    assert sides["below"] > 5 and sides["above"] > 5


def test_infinite_temperature_is_uniform_over_unmasked_tokens():
    # T = +inf: softmax(z / T) is uniform (its limit as T grows), so p = q = 1/V' over the V'
    # unmasked tokens, every draft is accepted (ratio 1 > u) and the bonus is the inverse CDF
    # of the uniform distribution, floor(u V') among the unmasked ids (numpy searchsorted).
    for mask_frac in (0.0, 0.4):
        w = workloads.small(B=30, gamma=4, V=333, dtype="bf16", seed=71, ragged=True,
                            temperatures=np.inf, mask_frac=mask_frac)
        r = oracle.verify(w)
        assert (r["num_accepted"] == w.gammas).all()
        zt = workloads.decode(w.target, "bf16")
        for b in range(w.B):
            tb, db, g = int(w.target_base[b]), int(w.draft_base[b]), int(w.gammas[b])
            live = np.isfinite(zt[tb])
            n_live = int(live.sum())
            np.testing.assert_allclose(r["p_x"][db: db + g], 1.0 / n_live, rtol=1e-14)
            np.testing.assert_allclose(r["q_x"][db: db + g], 1.0 / n_live, rtol=1e-14)
            np.testing.assert_allclose(r["row_sum_t"][tb: tb + g + 1], n_live, rtol=1e-15)
            u = float(w.uniforms[tb + g, 1])
            C = np.cumsum(live.astype(np.float64) / n_live)
            if r["cdf_gap"][b] > 1e-9:
                assert r["out_tokens"][tb + g] == np.searchsorted(C, u * C[-1], side="right")
            assert live[r["out_tokens"][tb + g]]
