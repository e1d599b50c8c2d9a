"""Pins for the oracle's verify step (oracle/mtp.py), none of which re-types it:

* log-softmax and entropy against SciPy's routines, and their closed forms
  (uniform row: log V; one-hot row: 0) and the bound max p >= exp(-H)
  (paperlayer App. D.2);
* overlap = 1 - TV with TV from its own definition (paperlayer Sec. 8; rainbus
  "Total Variation Distance"), and the special cases p = q and disjoint supports;
* exact brute force at V = 4 with rational p, q: the emitted token's marginal is
  p (paperlayer Sec. 2: rejection sampling preserves the target distribution
  exactly), to within the 2^-24 grid of the uniforms;
* Monte-Carlo: the acceptance rate equals the overlap (paperlayer Sec. 3), the
  expected accepted length is the sum of products of per-step overlaps
  (paperlayer Sec. 4), and a chi-square test of the first emitted token against p.
"""
from fractions import Fraction

import numpy as np
import pytest
from scipy import special, stats

from oracle import mtp
from oracle.philox import verify_uniforms


def _rows(rng, V, scale=2.0):
    return rng.normal(0.0, scale, V)


def test_log_softmax_matches_scipy():
    rng = np.random.default_rng(1)
    for V in (1, 7, 1024, 151936):
        x = _rows(rng, V, 3.0)
        logp, lse = mtp.log_softmax(x)
        np.testing.assert_allclose(logp, special.log_softmax(x), rtol=0, atol=1e-12)
        assert abs(lse - special.logsumexp(x)) < 1e-12 * max(1.0, abs(lse))
    x = _rows(rng, 64)
    x[::3] = -np.inf
    logp, _ = mtp.log_softmax(x)
    assert np.all(np.exp(logp[::3]) == 0.0)
    np.testing.assert_allclose(np.exp(logp).sum(), 1.0, atol=1e-14)
    assert mtp.log_softmax(np.full(8, -np.inf))[0] is None
    assert mtp.log_softmax(np.array([0.0, np.nan]))[0] is None
    assert mtp.log_softmax(np.array([0.0, np.inf]))[0] is None


def test_entropy_matches_scipy_and_closed_forms():
    rng = np.random.default_rng(2)
    for V in (2, 100, 151936):
        logp, _ = mtp.log_softmax(_rows(rng, V))
        assert abs(mtp.entropy(logp) - stats.entropy(np.exp(logp))) < 1e-10
    for V in (1024, 151936, 262144):
        logp, _ = mtp.log_softmax(np.full(V, 0.37))
        assert abs(mtp.entropy(logp) - np.log(V)) < 1e-10
    assert abs(mtp.entropy(mtp.log_softmax(np.full(151936, 0.0))[0]) - 11.9312146585) < 1e-9
    x = np.full(50, -np.inf)
    x[17] = 4.0
    assert mtp.entropy(mtp.log_softmax(x)[0]) == 0.0
    for _ in range(50):   # max_y p(y) >= exp(-H(p))
        logp, _ = mtp.log_softmax(_rows(rng, 300, rng.uniform(0.1, 5)))
        assert np.exp(logp).max() >= np.exp(-mtp.entropy(logp)) * (1 - 1e-12)


def test_overlap_tv_identities_and_special_cases():
    rng = np.random.default_rng(3)
    for _ in range(20):
        a = _rows(rng, 1000)
        p = np.exp(mtp.log_softmax(a)[0])
        q = np.exp(mtp.log_softmax(a + rng.normal(0, rng.uniform(0.01, 3), 1000))[0])
        alpha, tv = mtp.overlap(p, q), mtp.tv_distance(p, q)
        assert abs(alpha + tv - 1.0) < 1e-12
        assert abs(mtp.residual(p, q).sum() - tv) < 1e-12
        assert 0.0 <= alpha <= 1.0 + 1e-15
    p = np.exp(mtp.log_softmax(_rows(rng, 500))[0])
    assert mtp.overlap(p, p) == pytest.approx(1.0, abs=1e-13) and mtp.tv_distance(p, p) == 0.0
    x = _rows(rng, 500)
    xp, xq = x.copy(), x.copy()
    xp[::2] = -np.inf
    xq[1::2] = -np.inf
    p, q = np.exp(mtp.log_softmax(xp)[0]), np.exp(mtp.log_softmax(xq)[0])
    assert mtp.overlap(p, q) == 0.0
    assert mtp.tv_distance(p, q) == pytest.approx(1.0, abs=1e-14)


def test_accept_decision_cases():
    for u in (0.0, 0.5, 1.0 - 2.0 ** -24):
        assert mtp.accept_decision(u, -3.0, -3.0) == (1, 1.0)        # ratio exactly 1
    assert mtp.accept_decision(0.99, -2.0, -np.inf)[0] == 1          # q(y) = 0 < p(y)
    assert mtp.accept_decision(0.0, -np.inf, -np.inf)[0] == 0        # p(y) = q(y) = 0
    assert mtp.accept_decision(0.0, -np.inf, -1.0)[0] == 0           # p(y) = 0: u < 0 never
    assert mtp.accept_decision(0.25, np.log(0.25), np.log(1.0))[0] == 0   # u == ratio: reject
    assert mtp.accept_decision(0.25 - 2 ** -24, np.log(0.25), 0.0)[0] == 1


def test_inverse_cdf_rules():
    r = np.array([0.0, 0.25, 0.0, 0.5, 0.25])
    assert mtp.inverse_cdf(r, 0.0)[0] == 1            # zero-mass entry 0 never chosen
    assert mtp.inverse_cdf(r, 0.25)[0] == 3           # t on a boundary: strict '>'
    assert mtp.inverse_cdf(r, 0.7499)[0] == 3
    assert mtp.inverse_cdf(r, 0.75)[0] == 4
    assert mtp.inverse_cdf(r, 1.0)[0] == 4            # rounding fallback: last positive
    assert mtp.inverse_cdf(np.array([0, 0, 1.0, 0]), 0.999)[0] == 2


def _perturbed_inverse_cdf(r, t, delta):
    """Inverse CDF of r evaluated with every cumulative sum at a positive-mass token
    moved by delta[v] (a zero-mass token repeats the previous sum, as any summation
    does): the first positive-mass v whose perturbed sum exceeds t, else the last."""
    last = None
    c = np.cumsum(r)
    for v in np.flatnonzero(r > 0):
        last = v
        if c[v] + delta[v] > t:
            return int(v)
    return int(last)


def test_cdf_allowed_is_the_set_of_perturbed_inverse_cdf_tokens():
    """Brute force on tiny rows: every inverse CDF whose cumulative sums each carry an
    error of at most `band` returns a token of cdf_allowed (random perturbations,
    also at the band's edges), and every token of cdf_allowed is returned by some
    such perturbation (the set is tight)."""
    rng = np.random.default_rng(21)
    for trial in range(300):
        V = int(rng.integers(1, 9))
        r = rng.uniform(0, 1, V) * (rng.uniform(0, 1, V) < 0.7)
        if not r.sum() > 0:
            r[rng.integers(V)] = 1.0
        if trial % 3 == 0:   # intervals narrower than the band
            r = r * rng.uniform(0, 1e-3, V)
        band = float(rng.choice([0.0, 1e-4, 0.05, 0.3])) * r.sum()
        t = rng.uniform(0, r.sum())
        if trial % 5 == 0:   # t exactly on a boundary
            pos = np.cumsum(r)[r > 0]
            t = float(pos[rng.integers(pos.size)]) if pos.size > 1 else t
            t = min(t, np.nextafter(r.sum(), 0))
        allowed = set(int(v) for v in mtp.cdf_allowed(r, t, band))
        assert mtp.inverse_cdf(r, t)[0] in allowed
        seen = set()
        for _ in range(200):
            delta = rng.choice([-band, band, 0.0], V) if rng.uniform() < 0.5 else rng.uniform(-band, band, V)
            tok = _perturbed_inverse_cdf(r, t, delta)
            assert tok in allowed, (r, t, band, delta, tok, allowed)
            seen.add(tok)
        c = np.cumsum(r)
        for w in allowed:   # the perturbation that makes w the answer
            delta = np.where(np.arange(V) < w, -band, band)
            assert _perturbed_inverse_cdf(r, t, delta) == w
            assert c[w] > t - band and (c[w - 1] if w else 0.0) <= t + band


def test_cdf_tie_probability_is_the_flag_rate():
    """Monte-Carlo over t uniform on [0, sum r): the share of t whose cdf_allowed has
    more than one token equals cdf_tie_probability, for wide intervals (windows
    apart), heavy-tailed ones (windows overlapping: most intervals are narrower
    than a band) and zeros between positive tokens."""
    rng = np.random.default_rng(22)
    for V, band_rel, wide in ((40, 2e-3, True), (40, 2e-3, False), (300, 1e-4, True), (200, 5e-3, False)):
        r = rng.uniform(0.5, 1.5, V) if wide else np.exp(rng.normal(0, 3, V))
        r[rng.integers(V, size=3)] = 0.0
        band = band_rel * r.sum()
        prob = mtp.cdf_tie_probability(r, band)
        n = 20000
        ts = rng.uniform(0, r.sum(), n)
        hits = sum(mtp.cdf_allowed(r, t, band).size > 1 for t in ts)
        assert abs(hits / n - prob) <= 5 * np.sqrt(prob * (1 - prob) / n) + 1e-4, (V, hits / n, prob)
    assert mtp.cdf_tie_probability(np.array([0.0, 1.0, 0.0]), 0.1) == 0.0


def test_cdf_tie_probability_closed_forms():
    """Four unit intervals (boundaries 1, 2, 3 on [0, 4)): windows of half-width
    0.25 are apart, 3 x 0.5 / 4; of half-width 0.6 they merge into [0.4, 3.6),
    3.2 / 4; of half-width 2 they cover everything.  Zeros between the tokens
    change nothing."""
    r = np.ones(4)
    assert mtp.cdf_tie_probability(r, 0.25) == pytest.approx(0.375)
    assert mtp.cdf_tie_probability(r, 0.6) == pytest.approx(0.8)
    assert mtp.cdf_tie_probability(r, 2.0) == pytest.approx(1.0)
    assert mtp.cdf_tie_probability(np.array([1.0, 0.0, 1.0, 0.0, 0.0, 1.0, 1.0]), 0.25) == pytest.approx(0.375)


def test_cdf_band_scales_with_the_p_mass_of_the_support():
    """The band of a residual row is CDF_TIE_BAND times the p mass on the
    residual's support, not times the residual's own mass: r = (1e-3, 1e-3, 0)
    from p = (0.3, 0.3, 0.4) has M = 0.6, a band of 6e-7 around the boundary at
    1e-3, so t = 1e-3 + 4e-7 admits both tokens and t = 1e-3 + 8e-7 only the
    second."""
    p = np.array([0.3, 0.3, 0.4])
    q = np.array([0.3 - 1e-3, 0.3 - 1e-3, 0.4 + 2e-3])
    assert mtp.support_mass(p, mtp.residual(p, q)) == pytest.approx(0.6)
    tok, empty, allowed = mtp.row_sample(p, q, (1e-3 + 4e-7) / 2e-3)
    assert tok == 1 and not empty and list(allowed) == [0, 1]
    tok, empty, allowed = mtp.row_sample(p, q, (1e-3 + 8e-7) / 2e-3)
    assert tok == 1 and list(allowed) == [1]
    tok, empty, allowed = mtp.row_sample(p, q, (1e-3 - 4e-7) / 2e-3)
    assert tok == 0 and list(allowed) == [0, 1]


def test_row_sample_allowed_sets():
    """row_sample's allowed set: the exact token alone away from boundaries; the
    token on either side near one; every token with p > 0 for a residual whose mass
    is below the band; an empty residual samples p, and only the rows made of the
    same logits pin its token exactly."""
    p = np.array([0.25, 0.25, 0.25, 0.25])
    tok, empty, allowed = mtp.row_sample(p, None, 0.6)
    assert tok == 2 and not empty and list(allowed) == [2]
    tok, empty, allowed = mtp.row_sample(p, None, 0.5 + 1e-9)
    assert tok == 2 and list(allowed) == [1, 2]
    tok, empty, allowed = mtp.row_sample(p, None, 0.5 - 1e-9)
    assert tok == 1 and list(allowed) == [1, 2]
    q = p.copy()
    tok, empty, allowed = mtp.row_sample(p, q, 0.3, identical=True)   # the same logits: exactly empty
    assert empty and tok == 1 and list(allowed) == [1]
    tok, empty, allowed = mtp.row_sample(p, q, 0.3)          # p = q from different logits
    assert empty and tok == 1 and list(allowed) == [0, 1, 2, 3]
    q = np.array([0.25 - 1e-8, 0.25 + 1e-8, 0.25, 0.25])   # residual of mass 1e-8 on token 0
    tok, empty, allowed = mtp.row_sample(p, q, 0.3)
    assert not empty and tok == 0 and list(allowed) == [0, 1, 2, 3]


def _count_below(pred, n_bits=24):
    """Number of k in [0, 2^n) with pred(k * 2^-n) true, for a predicate true on a
    prefix of the grid (monotone decreasing in k): bisection over the oracle's own
    decision function."""
    lo, hi = 0, 1 << n_bits           # pred true on [0, lo), false on [hi, ...)
    if not pred(0.0):
        return 0
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if pred(mid * 2.0 ** -n_bits):
            lo = mid
        else:
            hi = mid
    return hi


@pytest.mark.parametrize("p16,q16", [
    ((5, 3, 6, 2), (2, 5, 3, 6)),
    ((8, 4, 2, 2), (1, 1, 7, 7)),
    ((1, 1, 1, 13), (4, 4, 4, 4)),
    ((4, 4, 4, 4), (4, 4, 4, 4)),
    ((0, 8, 0, 8), (8, 0, 8, 0)),
])
def test_bruteforce_v4_marginal_is_p(p16, q16):
    """Sum over the draft token y ~ q, the 2^24 values of u and the 2^24 values of u'
    of the oracle's accept rule and row sample; the emitted token's law is p."""
    p = np.array(p16, dtype=np.float64) / 16.0        # dyadic: exact in float64
    q = np.array(q16, dtype=np.float64) / 16.0
    V = 4
    pf = [Fraction(x, 16) for x in p16]
    qf = [Fraction(x, 16) for x in q16]
    logp = np.log(p, where=p > 0, out=np.full(V, -np.inf))
    logq = np.log(q, where=q > 0, out=np.full(V, -np.inf))
    grid = Fraction(1, 1 << 24)
    # token law of the row sample, over the u' grid
    res = [Fraction(0)] * V
    for v in range(V):
        n_le = _count_below(lambda up: mtp.row_sample(p, q, up)[0] <= v)
        n_lt = _count_below(lambda up: mtp.row_sample(p, q, up)[0] < v) if v else 0
        res[v] = (n_le - n_lt) * grid
    assert sum(res) == 1
    emit = [Fraction(0)] * V
    for y in range(V):
        if qf[y] == 0:
            continue
        acc = _count_below(lambda u: mtp.accept_decision(u, logp[y], logq[y])[0] == 1) * grid
        emit[y] += qf[y] * acc
        for v in range(V):
            emit[v] += qf[y] * (1 - acc) * res[v]
    alpha = sum(min(a, b) for a, b in zip(pf, qf))
    for v in range(V):
        # continuous-u identity: q min(1, p/q) + (1 - alpha) r / R = p exactly
        r = max(pf[v] - qf[v], Fraction(0))
        R = 1 - alpha
        cont = min(pf[v], qf[v]) + (r if R else 0)
        assert cont == pf[v] or (R == 0 and pf[v] == qf[v])
        assert abs(emit[v] - pf[v]) <= 2 * grid, (v, float(emit[v]), float(pf[v]))


def _sample_tokens(rng, draft):
    """y ~ softmax(draft) per row (inverse transform on float64 q)."""
    q = np.exp(draft - special.logsumexp(draft, axis=-1, keepdims=True))
    c = np.cumsum(q, axis=-1)
    u = rng.random(q.shape[:-1] + (1,)) * c[..., -1:]
    return np.minimum((c <= u).sum(-1), q.shape[-1] - 1)


def test_verify_p_equals_q_accepts_everything():
    rng = np.random.default_rng(4)
    B, G, V = 16, 3, 200
    tgt = rng.normal(0, 2, (B, G + 1, V))
    dr = tgt[:, :G].copy()
    y = _sample_tokens(rng, dr)
    out = mtp.verify(tgt, dr, y, seed=9, offset=0)
    assert out["accept"].all() and (out["accepted_len"] == G).all()
    assert np.all(out["tv"] == 0.0)
    np.testing.assert_allclose(out["overlap"], 1.0, atol=1e-13)
    assert np.all(out["row_status"][:, :G] == mtp.RESIDUAL_EMPTY)
    np.testing.assert_array_equal(out["next_token"], out["row_token"][:, G])


def test_verify_disjoint_supports_rejects_everything():
    rng = np.random.default_rng(5)
    B, G, V = 16, 3, 200
    tgt = rng.normal(0, 2, (B, G + 1, V))
    dr = rng.normal(0, 2, (B, G, V))
    tgt[:, :, ::2] = -np.inf
    dr[:, :, 1::2] = -np.inf
    y = _sample_tokens(rng, dr)
    out = mtp.verify(tgt, dr, y, seed=3, offset=77)
    assert not out["accept"].any() and (out["accepted_len"] == 0).all()
    assert np.all(out["overlap"] == 0.0)
    np.testing.assert_allclose(out["tv"], 1.0, atol=1e-14)
    assert np.all(out["next_token"] % 2 == 1)          # inside the target's support


def test_verify_status_rows():
    rng = np.random.default_rng(6)
    B, G, V = 3, 2, 50
    tgt = rng.normal(0, 1, (B, G + 1, V))
    dr = tgt[:, :G] + rng.normal(0, 0.3, (B, G, V))
    y = _sample_tokens(rng, dr)
    y[0, 0] = V                      # out of range
    tgt[1, 1, :] = -np.inf           # target row with no mass
    dr[2, 0, 5] = np.nan             # NaN in a draft row
    out = mtp.verify(tgt, dr, y, seed=1, offset=0)
    assert out["row_status"][0, 0] & mtp.BAD_TOKEN and out["accept"][0, 0] == 0
    assert out["accepted_len"][0] == 0
    assert out["row_status"][1, 1] & mtp.BAD_TARGET and out["row_token"][1, 1] == -1
    assert np.isnan(out["entropy"][1, 1]) and np.isnan(out["overlap"][1, 1])
    assert out["row_status"][2, 0] & mtp.BAD_DRAFT and out["accept"][2, 0] == 0
    assert out["row_token"][2, 0] == -1


def _mc_inputs(seed, B, G, V, sigma):
    rng = np.random.default_rng(seed)
    base_t = rng.normal(0, 1.5, (G + 1, V))
    base_d = base_t[:G] + rng.normal(0, sigma, (G, V))
    tgt = np.broadcast_to(base_t, (B, G + 1, V))
    dr = np.broadcast_to(base_d, (B, G, V))
    y = _sample_tokens(rng, dr)
    return tgt, dr, y, base_t, base_d


def test_monte_carlo_acceptance_rate_and_length():
    B, G, V = 6000, 3, 12
    tgt, dr, y, bt, bd = _mc_inputs(11, B, G, V, 0.8)
    out = mtp.verify(tgt, dr, y, seed=42, offset=0)
    alphas = np.array([mtp.overlap(np.exp(mtp.log_softmax(bt[k])[0]),
                                   np.exp(mtp.log_softmax(bd[k])[0])) for k in range(G)])
    rate = out["accept"].mean(axis=0)
    sd = np.sqrt(alphas * (1 - alphas) / B)
    assert np.all(np.abs(rate - alphas) < 5 * sd), (rate, alphas)
    # E[n] = sum_k prod_{j<=k} alpha_j for independent steps
    en = np.sum(np.cumprod(alphas))
    n = out["accepted_len"].astype(np.float64)
    assert abs(n.mean() - en) < 5 * n.std() / np.sqrt(B), (n.mean(), en)


def test_monte_carlo_first_token_distribution_chi_square():
    B, G, V = 8000, 1, 8
    tgt, dr, y, bt, _ = _mc_inputs(12, B, G, V, 1.0)
    out = mtp.verify(tgt, dr, y, seed=7, offset=1000)
    first = np.where(out["accept"][:, 0] == 1, y[:, 0], out["row_token"][:, 0])
    p0 = np.exp(mtp.log_softmax(bt[0])[0])
    counts = np.bincount(first, minlength=V)
    assert stats.chisquare(counts, p0 * B).pvalue > 1e-4


def test_verify_uses_position_addressed_uniforms():
    rng = np.random.default_rng(13)
    B, G, V = 4, 3, 30
    tgt = rng.normal(0, 1, (B, G + 1, V))
    dr = tgt[:, :G] + rng.normal(0, 0.5, (B, G, V))
    y = _sample_tokens(rng, dr)
    out = mtp.verify(tgt, dr, y, seed=123, offset=456)
    u, up = verify_uniforms(123, 456, np.arange(B * (G + 1)).reshape(B, G + 1))
    np.testing.assert_array_equal(out["u"], u)
    # the sequence b=2 alone, at offset + 2*(G+1), gives the same results
    sub = mtp.verify(tgt[2:3], dr[2:3], y[2:3], seed=123, offset=456 + 2 * (G + 1))
    for key in ("accept", "row_token", "accepted_len", "next_token"):
        np.testing.assert_array_equal(sub[key][0], out[key][2])
