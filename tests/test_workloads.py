"""The seeded input generators: encoding, layout and the workloads' shapes."""
import numpy as np
import pytest
import torch

import workloads


def test_bf16_encoding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(0, 3, 100_000), rng.normal(0, 1e-3, 1000),
                        [0.0, -0.0, 1.0, -2.5, 3.0e38, 1e-40]]).astype(np.float32)
    ours = workloads.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = workloads.bf16_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(ours.view(np.int16)).view(
        torch.bfloat16).float().numpy())


@pytest.mark.parametrize("cid,shape", [(1, (5, 4, 1000, "f32", 36_000, 4)),
                                       (2, (48, 40, 32000, "bf16", 3_072_000, 40)),
                                       (3, (320, 256, 128256, "bf16", 147_750_912, 256))])
def test_small_workload_shapes_and_compulsory_bytes(cid, shape):
    R_t, R_d, V, dtype, nbytes, pos = shape
    w = workloads.config(cid)
    assert (w.R_t, w.R_d, w.V, w.dtype) == (R_t, R_d, V, dtype)
    assert w.compulsory_bytes == nbytes and w.positions == pos
    assert w.uniforms.shape == (R_t, 2) and w.uniforms.dtype == np.float32
    assert ((w.uniforms >= 0) & (w.uniforms < 1)).all()
    assert ((w.draft_tokens >= 0) & (w.draft_tokens < V)).all()


def test_generation_is_deterministic_and_layout_consistent():
    a = workloads.small(B=9, gamma=5, V=77, dtype="bf16", seed=4, ragged=True,
                        temperatures=np.linspace(0, 1, 9))
    b = workloads.small(B=9, gamma=5, V=77, dtype="bf16", seed=4, ragged=True,
                        temperatures=np.linspace(0, 1, 9))
    for f in ("target", "draft", "draft_tokens", "uniforms", "temperatures", "cu_draft"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert a.cu_draft[0] == 0 and a.cu_draft[-1] == a.R_d and a.R_t == a.R_d + a.B
    np.testing.assert_array_equal(a.target_base, a.cu_draft[:-1] + np.arange(9))
    # greedy requests' drafts are the draft-row argmax
    zd = workloads.decode(a.draft, "bf16")
    for bi in np.flatnonzero(a.temperatures == 0):
        db, g = a.draft_base[bi], a.gammas[bi]
        np.testing.assert_array_equal(a.draft_tokens[db: db + g], np.argmax(zd[db: db + g], 1))


def test_gumbel_draft_draw_follows_the_tempered_softmax():
    from scipy import special
    from tests.stats_util import chi2_pvalue
    rng = np.random.default_rng(5)
    z = rng.normal(0, 1.0, 12)
    toks = workloads.draw_draft_tokens(np.broadcast_to(z, (400_000, 12)), 0.6,
                                       np.random.default_rng(6))
    pval, _, _ = chi2_pvalue(np.bincount(toks, minlength=12), special.softmax(z / 0.6))
    assert pval > 1e-3


def test_vocabulary_masks_are_shared_by_a_request_and_leave_a_finite_logit():
    w = workloads.small(B=6, gamma=3, V=500, dtype="bf16", seed=4, ragged=True,
                        temperatures=0.8, mask_frac=0.4, mask_span=200)
    zt = workloads.decode(w.target, "bf16")
    zd = workloads.decode(w.draft, "bf16")
    for b, (tb, db, g) in enumerate(zip(w.target_base, w.draft_base, w.gammas)):
        m = np.isinf(zt[tb])
        assert 0.4 < m.mean() < 0.9 and not m.all()
        for i in range(g + 1):
            np.testing.assert_array_equal(np.isinf(zt[tb + i]), m)
        for i in range(g):
            np.testing.assert_array_equal(np.isinf(zd[db + i]), m)
            assert not m[w.draft_tokens[db + i]]      # drafts are drawn from the masked q
    # a mask that would cover a row keeps entry 0
    w = workloads.small(B=2, gamma=1, V=50, dtype="f32", seed=5, mask_frac=1.0)
    zt = workloads.decode(w.target, "f32")
    assert np.isfinite(zt[:, 0]).all() and np.isinf(zt[:, 1:]).all()


@pytest.mark.parametrize("ragged", [False, True])
def test_a_range_of_requests_verifies_as_the_batch_slice(ragged):
    # Requests are independent: verifying requests [lo, hi) on their own (the share one GPU
    # gets when a batch is split by requests) gives exactly the whole batch's results for them.
    import oracle
    temps = np.where(np.arange(11) % 3 == 0, 0.0, np.linspace(0.4, 1.3, 11))
    w = workloads.small(B=11, gamma=5, V=300, dtype="bf16", seed=21, ragged=ragged,
                        temperatures=temps, draft_sigma=0.8)
    full = oracle.verify(w)
    for lo, hi in [(0, 11), (0, 4), (4, 5), (5, 11), (10, 11)]:
        s = w.requests(lo, hi)
        assert s.B == hi - lo and s.positions == int(w.gammas[lo:hi].sum())
        assert s.compulsory_bytes == int(w.request_bytes()[lo:hi].sum())
        part = oracle.verify(s)
        t0 = int(w.target_base[lo])
        np.testing.assert_array_equal(part["num_accepted"], full["num_accepted"][lo:hi])
        np.testing.assert_array_equal(part["out_tokens"],
                                      full["out_tokens"][t0:t0 + s.R_t])
        np.testing.assert_array_equal(part["resid_mass"], full["resid_mass"][lo:hi])


def test_shard_ranges_cover_the_batch_and_balance_its_bytes():
    w = workloads.small(B=40, gamma=8, V=128, dtype="bf16", seed=5, ragged=True,
                        temperatures=np.where(np.arange(40) % 5 == 0, 0.0, 0.9))
    rb = w.request_bytes()
    assert int(rb.sum()) == w.compulsory_bytes
    for G in (1, 2, 3, 8, 40):
        r = workloads.shard_ranges(w, G)
        assert len(r) == G and r[0][0] == 0 and r[-1][1] == w.B
        assert all(a < b for a, b in r) and all(r[k][1] == r[k + 1][0] for k in range(G - 1))
        # contiguous ranges cut where the running bytes reach k / G of the total: no range
        # holds more than its share plus one request
        assert max(int(rb[a:b].sum()) for a, b in r) <= rb.sum() / G + rb.max()
