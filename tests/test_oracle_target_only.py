"""Pins for the oracle's target-only verify (oracle/mtp.py), none of which re-types it:

* the greedy draft token against NumPy's argmax of softmax(draft) from SciPy, with
  ties going to the smallest index;
* exact brute force at V = 4 with rational p: over the 2^24-point grid of u', the
  pages' acceptance probability p(yhat) and otherwise the oracle's residual
  sample gives the emitted token's law p (target-only sampling as rejection
  sampling with a point-mass draft keeps the target distribution);
* closed forms: a one-hot target at yhat always accepts and its residual is empty;
  p = q gives TV = 0 and the RS-better flag exactly when p(yhat) < 1;
  RS-better is equivalent to overlap > p(yhat) (paperlayer Sec. 7: the boundary
  d_TV < 1 - p(yhat) with 1 - d_TV the rejection-sampling acceptance);
* Monte-Carlo: the acceptance rate equals p(yhat) (paperlayer App. D.2), the mean
  accepted length is the sum of products of p(yhat_k), a rejected row never emits
  yhat, and a chi-square test of the first emitted token against p;
* the uniforms are the rejection-sampling path's position-addressed ones.
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy import special, stats

from oracle import mtp
from oracle.philox import verify_uniforms


def _count_below(pred, n_bits=24):
    """Number of k in [0, 2^n) with pred(k * 2^-n) true, for a predicate true on a
    prefix of the grid: bisection over the oracle's own decision."""
    lo, hi = 0, 1 << n_bits
    if not pred(0.0):
        return 0
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if pred(mid * 2.0 ** -n_bits):
            lo = mid
        else:
            hi = mid
    return hi


def test_greedy_token_is_argmax_of_q_with_smallest_index_on_ties():
    rng = np.random.default_rng(21)
    for V in (2, 17, 1000, 151936):
        x = rng.normal(0, 2, V)
        q = special.softmax(x)
        assert mtp.greedy_draft_token(x) == int(np.flatnonzero(q == q.max())[0])
    x = np.array([0.5, 3.0, -1.0, 3.0, 3.0])
    assert mtp.greedy_draft_token(x) == 1
    x = np.full(9, -np.inf)
    x[6] = 0.0
    x[2] = 0.0
    assert mtp.greedy_draft_token(x) == 2


@pytest.mark.parametrize("p16,yhat", [
    ((5, 3, 6, 2), 2),
    ((8, 4, 2, 2), 0),
    ((1, 1, 1, 13), 1),
    ((4, 4, 4, 4), 3),
    ((0, 8, 0, 8), 1),
    ((0, 0, 16, 0), 2),
])
def test_bruteforce_v4_marginal_is_p(p16, yhat):
    """Sum over the 2^24 values of u' of the oracle's target-only residual sample,
    accepting with probability p(yhat): the emitted token's law is p."""
    p = np.array(p16, dtype=np.float64) / 16.0        # dyadic: exact in float64
    pf = [Fraction(x, 16) for x in p16]
    V = 4
    dr = np.full(V, -3.0)
    dr[yhat] = 2.0                                     # argmax q = yhat
    grid = Fraction(1, 1 << 24)
    res = [Fraction(0)] * V
    for v in range(V):
        n_le = _count_below(lambda up: mtp.target_only_row_sample(p, yhat, up)[0] <= v)
        n_lt = _count_below(lambda up: mtp.target_only_row_sample(p, yhat, up)[0] < v) if v else 0
        res[v] = (n_le - n_lt) * grid
    assert sum(res) == 1
    if pf[yhat] < 1:
        assert res[yhat] == 0                         # the residual never emits yhat
    assert mtp.greedy_draft_token(dr) == yhat
    # acceptance with probability p(yhat) (the pages' rule; the oracle's own accept
    # decision is pinned by the Monte-Carlo test below)
    acc = pf[yhat]
    emit = [(1 - acc) * res[v] for v in range(V)]
    emit[yhat] += acc
    for v in range(V):
        assert abs(emit[v] - pf[v]) <= 2 * grid, (v, float(emit[v]), float(pf[v]))


def test_verify_decision_matches_forced_uniform_rule():
    """Consistency (not a pin): verify_target_only's flags, tokens and p(yhat) agree
    with SciPy's softmax and NumPy's argmax applied to its own uniforms."""
    rng = np.random.default_rng(22)
    B, G, V = 40, 3, 64
    tgt = rng.normal(0, 1.5, (B, G + 1, V))
    dr = tgt[:, :G] + rng.normal(0, 0.7, (B, G, V))
    out = mtp.verify_target_only(tgt, dr, seed=5, offset=11)
    u, _ = verify_uniforms(5, 11, np.arange(B * (G + 1), dtype=np.uint64).reshape(B, G + 1))
    for b in range(B):
        for k in range(G):
            p = special.softmax(tgt[b, k])
            yh = int(np.argmax(dr[b, k]))
            assert out["draft_token"][b, k] == yh
            assert abs(out["p_yhat"][b, k] - p[yh]) < 1e-14
            assert out["accept"][b, k] == (1 if u[b, k] < p[yh] else 0)


def test_one_hot_target_always_accepts_and_has_empty_residual():
    rng = np.random.default_rng(23)
    B, G, V = 8, 3, 100
    tgt = np.full((B, G + 1, V), -np.inf)
    dr = rng.normal(0, 1, (B, G, V))
    yh = np.argmax(dr, axis=-1)
    for b in range(B):
        for k in range(G):
            tgt[b, k, yh[b, k]] = 1.0
        tgt[b, G, 3] = 0.0
    out = mtp.verify_target_only(tgt, dr, seed=1, offset=0)
    assert out["accept"].all() and (out["accepted_len"] == G).all()
    assert np.all(out["p_yhat"] == 1.0)
    assert np.all(out["row_status"][:, :G] & mtp.RESIDUAL_EMPTY)
    np.testing.assert_array_equal(out["row_token"][:, :G], yh)    # empty residual: from p
    assert not out["rs_better"].any()                # 1 - p(yhat) = 0: TO never worse
    np.testing.assert_array_equal(out["next_token"], 3)


def test_p_equals_q_and_the_boundary_identity():
    rng = np.random.default_rng(24)
    B, G, V = 12, 3, 300
    tgt = rng.normal(0, 2, (B, G + 1, V))
    out = mtp.verify_target_only(tgt, tgt[:, :G].copy(), seed=2, offset=5)
    assert np.all(out["tv"] == 0.0)
    assert np.all(out["rs_better"] == (out["p_yhat"] < 1.0))
    # random pairs: RS-better <=> overlap > p(yhat)  (1 - TV is the RS acceptance)
    dr = tgt[:, :G] + rng.normal(0, 2.0, (B, G, V))
    # half the rows: a peaked target whose mode the draft ranks first while spreading
    # the rest of its mass (target-only accepts more often there)
    pk = tgt[: B // 2, :G] * 4.0
    tgt[: B // 2, :G] = pk
    dr[: B // 2] = rng.normal(0, 0.5, (B // 2, G, V))
    np.put_along_axis(dr[: B // 2], np.argmax(pk, axis=-1)[..., None], 4.0, axis=-1)
    out = mtp.verify_target_only(tgt, dr, seed=2, offset=5)
    both = out["rs_better"].astype(bool)
    np.testing.assert_array_equal(both, out["overlap"] > out["p_yhat"])
    np.testing.assert_allclose(out["overlap"] + out["tv"], 1.0, atol=1e-12)
    assert both.any() and not both.all()


def _mc(seed, B, G, V, sigma):
    rng = np.random.default_rng(seed)
    bt = rng.normal(0, 1.2, (G + 1, V))
    bd = bt[:G] + rng.normal(0, sigma, (G, V))
    return np.broadcast_to(bt, (B, G + 1, V)), np.broadcast_to(bd, (B, G, V)), bt, bd


def test_monte_carlo_acceptance_length_and_residual():
    B, G, V = 6000, 3, 10
    tgt, dr, bt, bd = _mc(31, B, G, V, 0.6)
    out = mtp.verify_target_only(tgt, dr, seed=8, offset=0)
    py = np.array([special.softmax(bt[k])[int(np.argmax(bd[k]))] for k in range(G)])
    rate = out["accept"].mean(axis=0)
    sd = np.sqrt(py * (1 - py) / B)
    assert np.all(np.abs(rate - py) < 5 * sd), (rate, py)
    en = np.sum(np.cumprod(py))
    n = out["accepted_len"].astype(np.float64)
    assert abs(n.mean() - en) < 5 * n.std() / np.sqrt(B), (n.mean(), en)
    yh = out["draft_token"][0]
    for k in range(G):
        assert not np.any(out["row_token"][:, k] == yh[k])


def test_monte_carlo_first_token_distribution_chi_square():
    B, G, V = 8000, 1, 8
    tgt, dr, bt, _ = _mc(32, B, G, V, 1.0)
    out = mtp.verify_target_only(tgt, dr, seed=9, offset=300)
    first = np.where(out["accept"][:, 0] == 1, out["draft_token"][:, 0], out["row_token"][:, 0])
    p0 = special.softmax(bt[0])
    counts = np.bincount(first, minlength=V)
    assert stats.chisquare(counts, p0 * B).pvalue > 1e-4


def test_uniforms_and_bonus_row_follow_the_rejection_sampling_path():
    rng = np.random.default_rng(25)
    B, G, V = 5, 3, 40
    tgt = rng.normal(0, 1, (B, G + 1, V))
    dr = tgt[:, :G] + rng.normal(0, 0.5, (B, G, V))
    y = np.argmax(dr, axis=-1)
    to = mtp.verify_target_only(tgt, dr, seed=77, offset=9)
    rs = mtp.verify(tgt, dr, y, seed=77, offset=9)
    np.testing.assert_array_equal(to["u"], rs["u"])
    np.testing.assert_array_equal(to["row_token"][:, G], rs["row_token"][:, G])
    np.testing.assert_array_equal(to["entropy"], rs["entropy"])
    np.testing.assert_array_equal(to["overlap"], rs["overlap"])
    sub = mtp.verify_target_only(tgt[3:4], dr[3:4], seed=77, offset=9 + 3 * (G + 1))
    for key in ("accept", "row_token", "accepted_len", "next_token", "draft_token"):
        np.testing.assert_array_equal(sub[key][0], to[key][3])


def test_status_rows():
    rng = np.random.default_rng(26)
    B, G, V = 2, 2, 30
    tgt = rng.normal(0, 1, (B, G + 1, V))
    dr = tgt[:, :G] + rng.normal(0, 0.3, (B, G, V))
    tgt[0, 1, :] = -np.inf
    dr[1, 0, 4] = np.nan
    out = mtp.verify_target_only(tgt, dr, seed=1, offset=0)
    assert out["row_status"][0, 1] & mtp.BAD_TARGET and out["draft_token"][0, 1] == -1
    assert out["accept"][0, 1] == 0 and out["row_token"][0, 1] == -1 and np.isnan(out["p_yhat"][0, 1])
    assert out["row_status"][1, 0] & mtp.BAD_DRAFT and out["accept"][1, 0] == 0
    assert out["accepted_len"][1] == 0 and out["row_token"][1, 0] == -1
