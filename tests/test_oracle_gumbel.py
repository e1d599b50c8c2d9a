"""Pins for the oracle's Gumbel-max sampling and tempered verify (oracle/mtp.py,
oracle/philox.py), none of which re-types it:

* the per-element uniforms are uniform on (0, 1) (Kolmogorov-Smirnov against
  SciPy) and never 0 or 1; the Gumbel noise -log(-log U) follows SciPy's
  standard Gumbel law;
* the Gumbel-max trick samples w / sum w (paperlayer App. G.2): chi-square over
  independent rows; zero weights never win; ties go to the smallest index;
* the tempered verify reduces to the plain verify of logits divided by T (accept
  flags, overlap, TV, entropy), an empty residual samples p by the inverse CDF
  with the row's u' (numpy's searchsorted on SciPy's softmax), and the first
  emitted token of the full pipeline follows the tempered p (chi-square);
* the Gumbel-max draft tokens follow the tempered q (chi-square).
"""
import numpy as np
from scipy import special, stats

from oracle import mtp
from oracle.philox import element_uniforms, verify_uniforms


def test_element_uniforms_are_uniform_and_open():
    U = element_uniforms(seed=17, offset=3, position=5, V=200003)
    assert U.min() > 0.0 and U.max() < 1.0
    assert stats.kstest(U, "uniform").pvalue > 1e-4
    # a different row or seed gives an independent stream
    U2 = element_uniforms(seed=17, offset=3, position=6, V=200003)
    assert abs(np.corrcoef(U, U2)[0, 1]) < 0.02
    # the row uniforms (u, u') sit on the grid k * 2^-24, the element uniforms on
    # (k + 1/2) * 2^-24, strictly inside (0, 1)
    u, up = verify_uniforms(17, 3, np.arange(8))
    assert np.all(np.modf(u * 2 ** 24)[0] == 0) and np.all(np.modf(U * 2 ** 24)[0] == 0.5)


def test_gumbel_noise_has_the_standard_gumbel_law():
    U = element_uniforms(seed=5, offset=0, position=1, V=100000)
    G = -np.log(-np.log(U))
    assert stats.kstest(G, stats.gumbel_r.cdf).pvalue > 1e-4


def test_gumbel_max_samples_w_over_sum_w():
    rng = np.random.default_rng(3)
    V, N = 8, 40000
    w = rng.uniform(0.1, 2.0, V)
    w[3] = 0.0
    toks = np.array([mtp.gumbel_argmax(np.log(w, where=w > 0, out=np.full(V, -np.inf)),
                                       element_uniforms(11, 0, r, V))[0] for r in range(N)])
    assert not np.any(toks == 3)
    counts = np.bincount(toks, minlength=V)
    keep = w > 0
    assert stats.chisquare(counts[keep], (w / w.sum() * N)[keep]).pvalue > 1e-4


def test_gumbel_max_ties_and_zero_weights():
    U = np.full(6, 0.5)
    assert mtp.gumbel_argmax(np.log(np.array([1.0, 2.0, 2.0, 0.5, 2.0, 1.0])), U)[0] == 1
    assert mtp.gumbel_argmax(np.array([-np.inf, -np.inf, 0.0, -np.inf]), np.full(4, 0.999))[0] == 2
    tok, allowed = mtp.gumbel_argmax(np.log(np.array([1.0, 1.0 + 1e-9])), np.full(2, 0.3))
    assert tok == 1 and list(allowed) == [0, 1]
    tok, allowed = mtp.gumbel_argmax(np.log(np.array([1.0, 2.0, 1.0])), np.array([0.3, 0.3, 0.9]))
    assert list(allowed) == [tok]
    tok, allowed = mtp.gumbel_argmax(np.full(3, -np.inf), np.full(3, 0.5))
    assert tok == 0 and list(allowed) == [0]


def test_gumbel_gap_probability_bound():
    """The chance that the runner-up key lies within a gap g of the winner is at
    most e^g - 1 (the bound verify_gumbel reports per row): Monte-Carlo over many
    uniform vectors, for skewed weights, and for n equal weights, where the chance is
    exactly (n - 1) c / (n + (n - 1) c) with c = e^g - 1 (the winner's clock is
    Exp(n), the runner-up's lead an independent Exp(n - 1))."""
    rng = np.random.default_rng(12)
    g = 0.05
    for w in (np.ones(40), np.exp(rng.normal(0, 2, 40))):
        n, hits = 20000, 0
        for r in range(n):
            _, allowed = mtp.gumbel_argmax(np.log(w), element_uniforms(99, 1, r, w.size), gap_band=g)
            hits += allowed.size > 1
        bound = np.expm1(g)
        assert hits / n <= bound + 5 * np.sqrt(bound / n)
        if np.all(w == 1.0):
            m = w.size
            exact = (m - 1) * bound / (m + (m - 1) * bound)
            assert abs(hits / n - exact) <= 5 * np.sqrt(exact / n)


def test_tempered_verify_reduces_to_plain_verify_of_scaled_logits():
    rng = np.random.default_rng(8)
    B, G, V = 6, 3, 500
    tgt = rng.normal(0, 1.5, (B, G + 1, V))
    dr = tgt[:, :G] + rng.normal(0, 0.6, (B, G, V))
    y = rng.integers(0, V, (B, G))
    for T in (0.5, 1.0, 2.5):
        g = mtp.verify_gumbel(tgt, dr, y, seed=4, offset=10, temperature=T)
        p = mtp.verify(tgt / T, dr / T, y, seed=4, offset=10)
        for key in ("accept", "accepted_len", "row_status"):
            np.testing.assert_array_equal(g[key], p[key])
        for key in ("overlap", "tv", "entropy"):
            np.testing.assert_allclose(g[key], p[key], rtol=1e-12, atol=1e-14)


def test_identical_rows_sample_p():
    """An empty residual (the same logits on both sides) samples the tempered p by
    the inverse CDF with the row's u' (the smallest v whose cumulative probability
    exceeds u'); a bonus row takes the Gumbel-max of p."""
    rng = np.random.default_rng(9)
    B, G, V = 4, 2, 64
    tgt = rng.normal(0, 1, (B, G + 1, V))
    out = mtp.verify_gumbel(tgt, tgt[:, :G].copy(), np.zeros((B, G), int), seed=2, offset=0, temperature=0.8)
    assert np.all(out["row_status"][:, :G] & mtp.RESIDUAL_EMPTY)
    _, up = verify_uniforms(2, 0, np.arange(B * (G + 1), dtype=np.uint64).reshape(B, G + 1))
    for b in range(B):
        for k in range(G + 1):
            logp = special.log_softmax(tgt[b, k] / 0.8)
            if k < G:
                want = int(np.searchsorted(np.cumsum(np.exp(logp)), up[b, k], side="right"))
            else:
                U = element_uniforms(2, 0, b * (G + 1) + k, V)
                want = int(np.argmax(logp - np.log(-np.log(U))))
            assert out["row_token"][b, k] == want, (b, k)


def test_first_emitted_token_follows_tempered_p():
    B, G, V, T = 12000, 1, 8, 0.7
    rng = np.random.default_rng(10)
    bt = rng.normal(0, 1.0, (G + 1, V))
    bd = bt[:G] + rng.normal(0, 0.9, (G, V))
    tgt = np.broadcast_to(bt, (B, G + 1, V))
    dr = np.broadcast_to(bd, (B, G, V))
    y, _ = mtp.gumbel_draft_tokens(dr, seed=31, offset=0, temperature=T)
    out = mtp.verify_gumbel(tgt, dr, y, seed=32, offset=0, temperature=T)
    first = np.where(out["accept"][:, 0] == 1, y[:, 0], out["row_token"][:, 0])
    p = special.softmax(bt[0] / T)
    assert stats.chisquare(np.bincount(first, minlength=V), p * B).pvalue > 1e-4


def test_gumbel_draft_tokens_follow_tempered_q():
    N, V, T = 20000, 10, 1.6
    rng = np.random.default_rng(12)
    z = rng.normal(0, 1.2, V)
    toks, _ = mtp.gumbel_draft_tokens(np.broadcast_to(z, (N, V)), seed=7, offset=100, temperature=T)
    q = special.softmax(z / T)
    assert stats.chisquare(np.bincount(toks, minlength=V), q * N).pvalue > 1e-4
