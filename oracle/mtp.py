"""Plain float64 reference for the MTP verify step and the end-to-end TV loss.

TEST INFRASTRUCTURE ONLY (see the package docstring).  One row at a time,
NumPy float64, every quantity from its definition; no blocking, no fusion.

Notation follows the pages: target distribution p (the policy), draft
distribution q (an MTP head), gamma draft positions, vocabulary V.

Readings taken where the pages leave a step open are marked READING.
"""
import numpy as np

from .philox import element_uniforms, verify_uniforms

# Row status flags.  READING: the pages define no error handling; these name the
# data conditions that make a row's result undefined or that change its rule.
BAD_TOKEN = 1        # draft token outside [0, V): treated as a rejection
BAD_TARGET = 2       # target row has no finite log-sum-exp (NaN, +inf, all -inf)
BAD_DRAFT = 4        # same for the draft row
RESIDUAL_EMPTY = 8   # max(0, p - q) sums to zero: the row samples from p instead


def log_softmax(x):
    """(log p, lse) of one logit row.

    paperlayer Sec. 2 and App. A: p = softmax(target logits), q = softmax(draft
    logits z).  lse = m + log sum_v exp(x_v - m) with m = max x.  Entries at -inf
    give p = 0.  Returns (None, lse) when lse is not finite.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.isnan(x).any():
        return None, float("nan")
    m = x.max()
    if not np.isfinite(m):
        return None, float("nan")
    lse = m + np.log(np.sum(np.exp(x - m)))
    return x - lse, float(lse)


def entropy(logp):
    """H(p) = -sum_v p_v log p_v in nats, with 0 log 0 = 0.

    rainbus prerequisite "Entropy" (H is the negated sum of p log p).
    READING: natural logarithm.
    """
    p = np.exp(logp)
    nz = p > 0
    return float(-np.sum(p[nz] * logp[nz]))


def overlap(p, q):
    """alpha = sum_v min(p_v, q_v): the acceptance probability of rejection
    sampling (paperlayer Sec. 3 "Rejection Sampling"; Sec. 8, alpha = 1 - d_TV)."""
    return float(np.sum(np.minimum(p, q)))


def tv_distance(p, q):
    """d_TV(p, q) = 1/2 sum_v |p_v - q_v| (rainbus prerequisite "Total Variation
    Distance")."""
    return 0.5 * float(np.sum(np.abs(p - q)))


def residual(p, q):
    """r_v = max(0, p_v - q_v), the unnormalised residual distribution sampled on a
    rejection (EntMTP page, Related Work "Speculative Decoding"; paperlayer
    App. G.1)."""
    return np.maximum(p - q, 0.0)


def inverse_cdf(r, t):
    """Smallest v (in vocabulary order) whose cumulative mass C_v = sum_{w<=v} r_w
    exceeds t; if rounding leaves none, the last v with r_v > 0.

    paperlayer App. G.1 draws the residual sample by inverting its cumulative
    distribution.  READING: the
    cumulative sum runs in vocabulary index order and the comparison is strict,
    so a token with r_v = 0 is never chosen.
    Returns (token, lower boundary C_{v-1}, upper boundary C_v).
    """
    c = np.cumsum(r)
    v = int(np.searchsorted(c, t, side="right"))
    if v >= len(r):
        pos = np.nonzero(r > 0)[0]
        v = int(pos[-1])
    lo = float(c[v - 1]) if v > 0 else 0.0
    return v, lo, float(c[v])


# READING (near-ties of the inverse CDF): a float32 evaluation carries rounding in
# its cumulative sums, so where t lies within a band of a boundary C_v it may pick
# the token on the other side.  Each residual entry max(0, p_v - q_v) is formed
# from operands of size up to p_v, so the rounding of the cumulative sums is of the
# order of 2^-24 times the p mass they span, however small the residual is: the
# band is CDF_TIE_BAND * M, M = sum of p_v over the tokens with r_v > 0 (M = sum r
# for a row sampled from p itself, or p without one token).  The tokens it admits
# are listed exactly (cdf_allowed), so a flagged row still has at most a few
# correct answers.
CDF_TIE_BAND = 1e-6
# READING: an acceptance decision whose |u - min(1, ratio)| is within this band may
# go either way in a float evaluation of the ratio.
ACCEPT_TIE_BAND = 1e-6


def cdf_allowed(r, t, band):
    """Every token an inverse CDF of r whose cumulative sums are each off by at most
    `band` (absolute) may return for t: the v with r_v > 0 whose interval
    [C_{v-1}, C_v) meets [t - band, t + band].  Contains inverse_cdf(r, t)'s token
    (t < sum r); with a small band it adds only the nearest positive-mass token
    across a boundary that t lies near.  Sorted int64 array."""
    c = np.cumsum(r)
    lo_edge = np.concatenate(([0.0], c[:-1]))
    return np.flatnonzero((r > 0) & (lo_edge <= t + band) & (c > t - band))


def cdf_tie_probability(r, band):
    """The chance, over t uniform on [0, sum r), that cdf_allowed(r, t, band)
    admits more than one token: t lies within `band` (absolute) of a boundary
    between two positive-mass tokens, i.e. in [b - band, b + band) for such a
    boundary b.  The union of those windows is measured exactly: the boundaries
    are sorted, so each window adds what lies beyond the end of the one before."""
    r = np.asarray(r, dtype=np.float64)
    c = np.cumsum(r)
    total = float(c[-1]) if c.size else 0.0
    pos = np.flatnonzero(r > 0)
    if not total > 0 or pos.size < 2:
        return 0.0
    b = c[pos[:-1]]
    lo = np.clip(b - band, 0.0, total)
    hi = np.clip(b + band, 0.0, total)
    prev_hi = np.concatenate(([0.0], hi[:-1]))
    covered = float(np.sum(np.maximum(hi - np.maximum(lo, prev_hi), 0.0)))
    return min(1.0, covered / total)


def support_mass(p, r):
    """M = sum of p_v over the tokens with r_v > 0: the size of the operands the
    residual's entries on its support are formed from (see CDF_TIE_BAND)."""
    return float(np.sum(np.where(np.asarray(r) > 0, p, 0.0)))


def accept_decision(u, logp_y, logq_y):
    """Accept iff u < min(1, p(y)/q(y)) (paperlayer Sec. 2 "Acceptance methods",
    App. G.1; rainbus "Rejection Sampling").

    The ratio is exp(log p(y) - log q(y)); q(y) = 0 < p(y) gives +inf (accept);
    p(y) = q(y) = 0 gives NaN, taken as a rejection.  READING: strict '<', so a
    ratio of exactly 1 always accepts (u < 1).  Returns (flag 0/1, ratio).
    """
    with np.errstate(invalid="ignore", over="ignore"):
        ratio = float(np.exp(np.float64(logp_y) - np.float64(logq_y)))
    if np.isnan(ratio):
        return 0, 0.0
    return (1 if u < min(1.0, ratio) else 0), ratio


def row_sample(p, q, u_prime, cdf_tie_band=CDF_TIE_BAND, identical=False):
    """The token a row emits when it is the first rejection (or the bonus row).

    r = max(0, p - q) when q is given, else r = p (bonus row).  READING: if the
    residual has no mass (p = q exactly) the row samples from p instead.
    t = u' * sum r; the token is inverse_cdf(r, t).
    Returns (token, residual_was_empty, allowed): `allowed` lists the tokens a
    float32 evaluation may return (cdf_allowed with band cdf_tie_band * M, M the
    p mass on the support of r).
    READING: a residual whose mass is below cdf_tie_band is below what a float32
    sum resolves: such an evaluation may find it empty (and sample p) or form it
    from rounding noise, so every token with p > 0 is allowed there -- unless the
    two rows are the same logits (`identical`), which any evaluation turns into the
    same p and q, so that the residual is exactly empty there too.
    """
    empty = False
    near_empty = False
    if q is None:
        r = p
    else:
        r = residual(p, q)
        mass = float(np.sum(r))
        near_empty = mass < cdf_tie_band and not identical
        if not mass > 0:
            empty = True
            r = p
    total = float(np.cumsum(r)[-1])
    t = u_prime * total
    tok, _, _ = inverse_cdf(r, t)
    allowed = cdf_allowed(r, t, cdf_tie_band * support_mass(p, r))
    if near_empty:
        allowed = np.flatnonzero(p > 0)
    assert tok in allowed
    return tok, empty, allowed


def _near_empty(p, q, cdf_tie_band, identical):
    """The residual max(0, p - q) is below what a float32 sum resolves (see
    row_sample)."""
    return float(np.sum(residual(p, q))) < cdf_tie_band and not identical


def _row_tie_bound(p, q, cdf_tie_band, identical=False):
    """cdf_tie_probability of the distribution a row samples (1 for a near-empty
    residual, whose row is always flagged)."""
    if q is None:
        return cdf_tie_probability(p, cdf_tie_band * support_mass(p, p))
    r = residual(p, q)
    mass = float(np.sum(r))
    if _near_empty(p, q, cdf_tie_band, identical):
        return 1.0
    r = r if mass > 0 else p
    return cdf_tie_probability(r, cdf_tie_band * support_mass(p, r))


def _accept_tie_bound(ratio, tie_band):
    """Chance, over u uniform on [0, 1), that |u - min(1, ratio)| <= tie_band."""
    return min(1.0, tie_band if ratio >= 1.0 else 2.0 * tie_band)


def _new_outputs(B, G, u, up):
    G1 = G + 1
    return dict(
        accept=np.zeros((B, G), np.uint8), accepted_len=np.zeros(B, np.int32),
        next_token=np.full(B, -1, np.int32), row_token=np.full((B, G1), -1, np.int32),
        overlap=np.full((B, G), np.nan), tv=np.full((B, G), np.nan),
        entropy=np.full((B, G1), np.nan), row_status=np.zeros((B, G1), np.int32),
        ratio=np.full((B, G), np.nan), u=u, u_prime=up,
        accept_tie=np.zeros((B, G), bool), accept_tie_bound=np.zeros((B, G)),
        token_tie=np.zeros((B, G1), bool), token_tie_bound=np.zeros((B, G1)),
        token_allowed=np.empty((B, G1), object), near_empty=np.zeros((B, G1), bool),
        lse_p=np.full((B, G1), np.nan), lse_q=np.full((B, G), np.nan),
    )


def _set_token(out, b, k, tok, allowed, bound):
    out["row_token"][b, k] = tok
    out["token_allowed"][b, k] = allowed
    out["token_tie"][b, k] = allowed.size > 1
    out["token_tie_bound"][b, k] = bound


def verify(target, draft, tokens, seed, offset, tie_band=ACCEPT_TIE_BAND, cdf_tie_band=CDF_TIE_BAND):
    """Rejection-sampling verification of gamma drafted tokens per sequence.

    target: float64 [B, gamma+1, V] -- target logits at the gamma draft positions
            plus the bonus position.
    draft:  float64 [B, gamma, V]   -- cached draft logits (q = softmax).
    tokens: int [B, gamma]          -- draft tokens y_k, sampled from q_k.
    seed, offset: Philox key and counter base (see philox.verify_uniforms).

    Steps (paperlayer Sec. 2 "Acceptance methods", App. G.1; rainbus
    "Rejection Sampling"; EntMTP Related Work):
      1. p_k = softmax(target_k), q_k = softmax(draft_k).
      2. H(p_k) for every row, k = 0..gamma.
      3. alpha_k = sum min(p_k, q_k); TV_k = 1/2 sum |p_k - q_k|.
      4. u_k, u'_k from Philox at position b*(gamma+1)+k.
      5. accept_k = u_k < min(1, p_k(y_k) / q_k(y_k)).  READING: strict '<'; the
         decision is reported for every k, the sequence stops at the first 0.
      6. n_b = number of leading accepts (0..gamma).
      7. Row sample: r = max(0, p_k - q_k) for k < gamma; r = p_gamma for the
         bonus row (READING: when all gamma are accepted the next token comes
         from the bonus target row).  If sum r = 0, r = p_k (READING; flagged).
         t = u'_k * sum r; token = inverse_cdf(r, t).
      8. next_token_b = row_token[b, n_b].

    Near-ties: accept_tie marks |u - min(1, ratio)| <= tie_band, where a float
    evaluation may decide the other way; token_allowed[b, k] lists every token a
    float32 inverse CDF may return (row_sample), token_tie marks rows with more
    than one.  accept_tie_bound / token_tie_bound are each flag's probability bound
    over the uniforms, for bounding how many flags a batch may carry.
    """
    target = np.asarray(target, dtype=np.float64)
    draft = np.asarray(draft, dtype=np.float64)
    tokens = np.asarray(tokens, dtype=np.int64)
    B, G1, V = target.shape
    G = G1 - 1
    assert draft.shape == (B, G, V) and tokens.shape == (B, G)

    pos = np.arange(B * G1, dtype=np.uint64).reshape(B, G1)
    u, up = verify_uniforms(seed, offset, pos)

    out = _new_outputs(B, G, u, up)
    for b in range(B):
        for k in range(G1):
            logp, lse_p = log_softmax(target[b, k])
            out["lse_p"][b, k] = lse_p
            if logp is None:
                out["row_status"][b, k] |= BAD_TARGET
                out["token_allowed"][b, k] = np.array([-1])
            else:
                out["entropy"][b, k] = entropy(logp)
            if k == G:                                   # bonus row: r = p
                if logp is not None:
                    p = np.exp(logp)
                    tok, _, allowed = row_sample(p, None, up[b, k], cdf_tie_band)
                    _set_token(out, b, k, tok, allowed, _row_tie_bound(p, None, cdf_tie_band))
                continue
            logq, lse_q = log_softmax(draft[b, k])
            out["lse_q"][b, k] = lse_q
            y = int(tokens[b, k])
            if logq is None:
                out["row_status"][b, k] |= BAD_DRAFT
                out["token_allowed"][b, k] = np.array([-1])
            if not (0 <= y < V):
                out["row_status"][b, k] |= BAD_TOKEN
            if logp is None or logq is None:
                continue
            p, q = np.exp(logp), np.exp(logq)
            out["overlap"][b, k] = overlap(p, q)
            out["tv"][b, k] = tv_distance(p, q)
            if 0 <= y < V:
                flag, ratio = accept_decision(u[b, k], logp[y], logq[y])
                out["ratio"][b, k] = ratio
                out["accept"][b, k] = flag
                out["accept_tie"][b, k] = abs(u[b, k] - min(1.0, ratio)) <= tie_band
                out["accept_tie_bound"][b, k] = _accept_tie_bound(ratio, tie_band)
            same = bool(np.array_equal(target[b, k], draft[b, k]))
            tok, empty, allowed = row_sample(p, q, up[b, k], cdf_tie_band, identical=same)
            if empty:
                out["row_status"][b, k] |= RESIDUAL_EMPTY
            out["near_empty"][b, k] = _near_empty(p, q, cdf_tie_band, same)
            _set_token(out, b, k, tok, allowed, _row_tie_bound(p, q, cdf_tie_band, same))
        n = 0
        while n < G and out["accept"][b, n] == 1:
            n += 1
        out["accepted_len"][b] = n
        out["next_token"][b] = out["row_token"][b, n]
    return out


def greedy_draft_token(draft_logits):
    """yhat = argmax_y q(y): the draft token chosen greedily (paperlayer Sec. 2
    "Preliminaries", acceptance methods; App. D.2 "Target-Only Sampling").  q is a
    softmax of the draft logits, so this is the argmax of the logits.  READING:
    among equal maxima the smallest index."""
    return int(np.argmax(np.asarray(draft_logits, dtype=np.float64)))


def target_only_residual(p, yhat):
    """p with the greedy token removed: the residual max(0, p - delta_yhat) of the
    point-mass draft at yhat (see target_only_row_sample)."""
    r = np.array(p, dtype=np.float64)
    r[yhat] = 0.0
    return r


def target_only_row_sample(p, yhat, u_prime, cdf_tie_band=CDF_TIE_BAND):
    """The token a rejected target-only row emits.

    READING: the pages give target-only acceptance (probability p(yhat)) but not the
    token emitted on a rejection.  Target-only sampling is rejection sampling whose
    draft distribution is the point mass at yhat: the acceptance probability
    min(1, p(yhat)/1) is the pages' p(yhat), and the residual max(0, p - delta_yhat)
    is p with yhat removed, which keeps the emitted token's law exactly p.  If that
    residual has no mass (p(yhat) = 1) the row samples from p (flagged, as in
    row_sample).  t = u' * sum r; the token is inverse_cdf(r, t).
    Returns (token, residual_was_empty, allowed) as row_sample does.
    """
    r = target_only_residual(p, yhat)
    mass = float(np.sum(r))
    near_empty = 0.0 < mass < cdf_tie_band
    empty = not mass > 0
    if empty:
        r = np.asarray(p, dtype=np.float64)
    total = float(np.cumsum(r)[-1])
    t = u_prime * total
    tok, _, _ = inverse_cdf(r, t)
    allowed = cdf_allowed(r, t, cdf_tie_band * support_mass(p, r))
    if near_empty:
        allowed = np.flatnonzero(np.asarray(p) > 0)
    assert tok in allowed
    return tok, empty, allowed


def verify_target_only(target, draft, seed, offset, tie_band=ACCEPT_TIE_BAND, cdf_tie_band=CDF_TIE_BAND):
    """Target-only verification of gamma draft positions per sequence, with the
    rejection-sampling statistics and the RS/TO diagnostic.

    target: float64 [B, gamma+1, V]; draft: float64 [B, gamma, V]; no draft tokens:
    each draft position proposes its greedy token.

    Steps (paperlayer Sec. 2 "Preliminaries", acceptance methods; Sec. 7
    "Discussion", robustness of acceptance methods; App. D.2 "Target-Only
    Sampling"):
      1. p_k = softmax(target_k), q_k = softmax(draft_k); H(p_k) for every row.
      2. yhat_k = greedy_draft_token(draft_k).
      3. accept_k = u_k < p_k(yhat_k).  READING: strict '<' as for rejection
         sampling, with the same position-addressed uniforms.
      4. n_b = number of leading accepts; next_token_b = row_token[b, n_b].
      5. Row sample: target_only_row_sample(p_k, yhat_k, u'_k) for k < gamma;
         p_gamma for the bonus row.
      6. alpha_k = sum min(p_k, q_k) and TV_k = d_TV(p_k, q_k) as for rejection
         sampling; rs_better_k = TV_k < 1 - p_k(yhat_k), the boundary below which
         rejection sampling accepts more often than target-only sampling
         (1 - TV_k > p_k(yhat_k)).
    Near-ties as in verify; rs_tie marks |TV_k - (1 - p_k(yhat_k))| <= tie_band.
    """
    target = np.asarray(target, dtype=np.float64)
    draft = np.asarray(draft, dtype=np.float64)
    B, G1, V = target.shape
    G = G1 - 1
    assert draft.shape == (B, G, V)

    pos = np.arange(B * G1, dtype=np.uint64).reshape(B, G1)
    u, up = verify_uniforms(seed, offset, pos)

    out = _new_outputs(B, G, u, up)
    out.update(draft_token=np.full((B, G), -1, np.int32), p_yhat=np.full((B, G), np.nan),
               rs_better=np.zeros((B, G), np.uint8), rs_tie=np.zeros((B, G), bool))
    for b in range(B):
        for k in range(G1):
            logp, _ = log_softmax(target[b, k])
            if logp is None:
                out["row_status"][b, k] |= BAD_TARGET
                out["token_allowed"][b, k] = np.array([-1])
            else:
                out["entropy"][b, k] = entropy(logp)
            if k == G:                                   # bonus row: r = p
                if logp is not None:
                    p = np.exp(logp)
                    tok, _, allowed = row_sample(p, None, up[b, k], cdf_tie_band)
                    _set_token(out, b, k, tok, allowed, _row_tie_bound(p, None, cdf_tie_band))
                continue
            logq, _ = log_softmax(draft[b, k])
            if logq is None:
                out["row_status"][b, k] |= BAD_DRAFT
                out["token_allowed"][b, k] = np.array([-1])
            if logp is None or logq is None:
                continue
            p, q = np.exp(logp), np.exp(logq)
            yhat = greedy_draft_token(draft[b, k])
            py = float(p[yhat])
            out["draft_token"][b, k] = yhat
            out["p_yhat"][b, k] = py
            out["accept"][b, k] = 1 if u[b, k] < py else 0
            out["accept_tie"][b, k] = abs(u[b, k] - py) <= tie_band
            out["accept_tie_bound"][b, k] = _accept_tie_bound(py, tie_band)
            out["overlap"][b, k] = overlap(p, q)
            tv = tv_distance(p, q)
            out["tv"][b, k] = tv
            out["rs_better"][b, k] = 1 if tv < 1.0 - py else 0
            out["rs_tie"][b, k] = abs(tv - (1.0 - py)) <= tie_band
            tok, empty, allowed = target_only_row_sample(p, yhat, up[b, k], cdf_tie_band)
            if empty:
                out["row_status"][b, k] |= RESIDUAL_EMPTY
            r = target_only_residual(p, yhat)
            mass = float(np.sum(r))
            out["near_empty"][b, k] = 0.0 < mass < cdf_tie_band
            rs = r if mass > 0 else p
            bound = 1.0 if out["near_empty"][b, k] else cdf_tie_probability(rs, cdf_tie_band * support_mass(p, rs))
            _set_token(out, b, k, tok, allowed, bound)
        n = 0
        while n < G and out["accept"][b, n] == 1:
            n += 1
        out["accepted_len"][b] = n
        out["next_token"][b] = out["row_token"][b, n]
    return out


# READING (near-ties of the Gumbel-max argmax): keys within this gap of the winner
# (natural-log units) may be ordered differently by a float32 evaluation.
GUMBEL_GAP_BAND = 1e-4


def gumbel_argmax(logw, U, gap_band=GUMBEL_GAP_BAND):
    """argmax_v (log w_v + G_v) with G_v = -log(-log U_v): the Gumbel-max trick, a
    sample from w / sum w (paperlayer App. G.2 "Gumbel-Max Trick (vLLM)").  Entries
    with w_v = 0 (log w_v = -inf) never win.  READING: ties go to the smallest index.
    Returns (token, allowed): `allowed` lists the tokens whose key lies within
    gap_band of the winner's (the winner included), any of which a float32
    evaluation of the keys may choose.
    """
    keys = np.asarray(logw, dtype=np.float64) - np.log(-np.log(np.asarray(U, dtype=np.float64)))
    tok = int(np.argmax(keys))
    top = keys[tok]
    allowed = np.flatnonzero(np.isfinite(keys) & (keys >= top - gap_band))
    if tok not in allowed:         # no finite key: argmax is index 0 of an all -inf row
        allowed = np.array([tok])
    return tok, allowed


def gumbel_draft_tokens(draft, seed, offset, temperature=1.0):
    """Draft tokens by the Gumbel-max trick at temperature T: y = argmax_v
    (z_v / T + G_v) for each row of draft logits z [..., V] (App. G.2: argmax of
    log q / T + G, and log q differs from z / T by a constant).  Row r (in
    row-major order) uses element_uniforms(seed, offset, r, V).  Returns (tokens,
    allowed) of the leading shape, `allowed` an object array of the tokens
    gumbel_argmax admits per row."""
    z = np.asarray(draft, dtype=np.float64)
    lead, V = z.shape[:-1], z.shape[-1]
    flat = z.reshape(-1, V)
    tok = np.zeros(flat.shape[0], np.int32)
    allowed = np.empty(flat.shape[0], object)
    for r in range(flat.shape[0]):
        tok[r], allowed[r] = gumbel_argmax(flat[r] / temperature, element_uniforms(seed, offset, r, V))
    return tok.reshape(lead), allowed.reshape(lead)


def verify_gumbel(target, draft, tokens, seed, offset, temperature=1.0, tie_band=ACCEPT_TIE_BAND,
                  cdf_tie_band=CDF_TIE_BAND, gap_band=GUMBEL_GAP_BAND):
    """Rejection-sampling verification at temperature T with Gumbel-max sampling of
    the emitted tokens (paperlayer App. G.2, "Gumbel-Max Trick (vLLM)").

    Steps as in verify, except:
      1. p_k = softmax(target_k / T), q_k = softmax(draft_k / T).  READING: the
         temperature scales both the target and the cached draft logits.
      7. Row sample: r = max(0, p_k - q_k) (k < gamma) or p_gamma (bonus row); the
         token is gumbel_argmax(log r, U) with U = element_uniforms(seed, offset,
         b*(gamma+1) + k, V).  READING: the pages leave the empty residual open; a
         row whose residual is empty samples p by the inverse CDF with its u'
         (row_sample of p, flagged) -- any exact sample of p keeps the law; the
         inverse CDF needs no key of p for rows that have a residual.
    Acceptance uses the same u as verify; token_allowed lists the tokens within the
    key gap band of the winner (every token with p > 0 for a residual below
    cdf_tie_band, as in row_sample; the CDF near-ties for an empty residual's inverse
    CDF).  token_tie_bound is e^gap_band - 1 per Gumbel-max row: in
    the exponential-race form of the trick the winner's clock T1 ~ Exp(sum w) and
    the runner-up arrives an independent Exp(sum w - w_win) later (memoryless
    clocks), so the chance that log T2 - log T1 < gap_band is at most
    e^gap_band - 1.
    """
    target = np.asarray(target, dtype=np.float64) / temperature
    draft = np.asarray(draft, dtype=np.float64) / temperature
    out = verify(target, draft, tokens, seed, offset, tie_band, cdf_tie_band)
    B, G1, V = target.shape
    G = G1 - 1
    for b in range(B):
        for k in range(G1):
            logp, _ = log_softmax(target[b, k])
            if logp is None:
                continue
            p = np.exp(logp)
            near_empty = False
            w = p
            if k < G:
                logq, _ = log_softmax(draft[b, k])
                if logq is None:
                    continue
                r = residual(p, np.exp(logq))
                mass = float(np.sum(r))
                near_empty = _near_empty(p, np.exp(logq), cdf_tie_band, bool(np.array_equal(target[b, k], draft[b, k])))
                w = r if mass > 0 else None
            if w is None:      # empty residual: the inverse CDF of p with the row's u'
                tok, _, allowed = row_sample(p, None, out["u_prime"][b, k], cdf_tie_band)
                bound = _row_tie_bound(p, None, cdf_tie_band)
            else:
                U = element_uniforms(seed, offset, b * G1 + k, V)
                with np.errstate(divide="ignore"):
                    tok, allowed = gumbel_argmax(np.log(w), U, gap_band)
                bound = float(np.expm1(gap_band))
            if near_empty:
                allowed = np.flatnonzero(p > 0)
                bound = 1.0
            _set_token(out, b, k, tok, allowed, bound)
        n = out["accepted_len"][b]
        out["next_token"][b] = out["row_token"][b, n]
    return out


def _head_targets(target, G):
    """Target rows per (position, head): a [T, V] target is shared by all heads."""
    target = np.asarray(target, dtype=np.float64)
    if target.ndim == 2:
        return np.broadcast_to(target[:, None, :], (target.shape[0], G, target.shape[1]))
    return target


def tv_stats(target, draft):
    """Per (position t, head k): lse_p, lse_q, alpha, S.

    alpha_{t,k} = clamp(sum_v min(p_v, q_v), 0, 1)   (paperlayer App. F: the
        forward pass accumulates the overlap; READING: tau_max = 1, so the clamp
        only guards rounding).
    S_{t,k} = sum_v 1[q_v <= p_v] q_v              (paperlayer App. A).
    READING: the indicator is evaluated on log-probabilities, ties count as 1.
    READING: a row without a finite normaliser (all -inf, or a NaN) is a data error,
    as in verify: that head's alpha and S are NaN (and so are the position's loss and
    the mean).
    target: [T, V] (shared by all heads) or [T, gamma, V]; draft: [T, gamma, V].
    Returns float64 [T, gamma, 4].
    """
    draft = np.asarray(draft, dtype=np.float64)
    T, G, V = draft.shape
    tgt = _head_targets(target, G)
    saved = np.empty((T, G, 4))
    for t in range(T):
        for k in range(G):
            logp, lse_p = log_softmax(tgt[t, k])
            logq, lse_q = log_softmax(draft[t, k])
            if logp is None or logq is None:
                saved[t, k] = (lse_p, lse_q, np.nan, np.nan)
                continue
            p, q = np.exp(logp), np.exp(logq)
            alpha = min(max(overlap(p, q), 0.0), 1.0)
            s = float(np.sum(q[logq <= logp]))
            saved[t, k] = (lse_p, lse_q, alpha, s)
    return saved


def e2e_position_loss(alpha):
    """l_t = -sum_{k=1..gamma} prod_{j<=k} alpha_{t,j}.

    paperlayer Sec. 4 "End-to-end TV loss": the loss optimises the expected
    acceptance length, which multiplies per-step acceptances, so earlier steps
    weigh more; rainbus "Method steps" (first step) and "Technical novelty"
    (fourth point).  READING: no normalising constant (any would only scale it).
    alpha: [T, gamma] -> [T].
    """
    alpha = np.asarray(alpha, dtype=np.float64)
    return -np.sum(np.cumprod(alpha, axis=1), axis=1)


def tv_loss(target, draft):
    """Mean over positions of the end-to-end multi-step TV loss.

    Returns (loss, pos_loss [T], saved [T, gamma, 4] = (lse_p, lse_q, alpha, S)).
    READING: the loss is averaged over the T positions.
    """
    saved = tv_stats(target, draft)
    pos_loss = e2e_position_loss(saved[:, :, 2])
    return float(np.mean(pos_loss)), pos_loss, saved


def e2e_weights(alpha, g, T):
    """w_{t,j} = dL/d alpha_{t,j} for L = (g/T) sum_t l_t.

    d l_t / d alpha_j = -sum_{k>=j} prod_{i<=k, i != j} alpha_i, written as
    products without division so that alpha = 0 is safe.
    """
    alpha = np.asarray(alpha, dtype=np.float64)
    Tn, G = alpha.shape
    w = np.zeros((Tn, G))
    for t in range(Tn):
        for j in range(G):
            acc = 0.0
            for k in range(j, G):
                prod = 1.0
                for i in range(k + 1):
                    if i != j:
                        prod *= alpha[t, i]
                acc += prod
            w[t, j] = -(g / T) * acc
    return w


def tv_loss_grad(target, draft, g=1.0):
    """Gradient of g * tv_loss with respect to the draft logits.

    paperlayer App. A: with p detached, d alpha / d z_v = q_v (1[q_v <= p_v] - S),
    bounded by q_v; rainbus "Technical novelty": the TV gradient is -q times
    (indicator - S).  Chained through the end-to-end weights:
        grad_{t,j,v} = w_{t,j} q_v (1[q_v <= p_v] - S_{t,j}).
    The target gets no gradient.  Returns float64 [T, gamma, V] and the
    per-element indicator-tie mask is not computed here (see indicator_margin).
    """
    draft = np.asarray(draft, dtype=np.float64)
    T, G, V = draft.shape
    tgt = _head_targets(target, G)
    saved = tv_stats(target, draft)
    w = e2e_weights(saved[:, :, 2], g, T)
    grad = np.empty((T, G, V))
    for t in range(T):
        for k in range(G):
            logp, _ = log_softmax(tgt[t, k])
            logq, _ = log_softmax(draft[t, k])
            if logp is None or logq is None:   # data error (see tv_stats)
                grad[t, k] = np.nan
                continue
            q = np.exp(logq)
            ind = (logq <= logp).astype(np.float64)
            grad[t, k] = w[t, k] * q * (ind - saved[t, k, 3])
    return grad


def indicator_margin(target, draft):
    """|log q_v - log p_v| per element: where it is tiny, a float32 evaluation of
    the indicator 1[q_v <= p_v] may legitimately flip.  [T, gamma, V]."""
    draft = np.asarray(draft, dtype=np.float64)
    T, G, V = draft.shape
    tgt = _head_targets(target, G)
    m = np.empty((T, G, V))
    for t in range(T):
        for k in range(G):
            logp, _ = log_softmax(tgt[t, k])
            logq, _ = log_softmax(draft[t, k])
            m[t, k] = np.abs(logq - logp)
    return m


def _head_topk(x, G):
    """Top-K target entries per (position, head): a [T, K] input is shared by all heads."""
    x = np.asarray(x)
    if x.ndim == 2:
        return np.broadcast_to(x[:, None, :], (x.shape[0], G, x.shape[1]))
    return x


def tv_topk_stats(idx, val, draft):
    """Per (position t, head k) for the top-K path: lse_A, lse_q, alpha, S.

    paperlayer App. F ("Fused TV Loss Kernel"): an optional top-K path keeps O(K)
    of the target instead of O(V).  READING: the target is given by K entries per
    row, vocabulary indices I_j and target logits A_j, and stands for the target
    truncated to those entries and renormalised, p_j = exp(A_j - lse_A); the
    draft stays the full softmax q = softmax(z) over V.  Then, entry by entry,
        alpha = clamp(sum_j min(p_j, q_{I_j}), 0, 1),
        S = sum_j 1[log q_{I_j} <= log p_j] q_{I_j},
    which for distinct indices are the full path's alpha and S against the
    truncated target (p = 0 off the K entries, where the indicator is 0).
    READING: an entry whose index is outside [0, V) has no mass (as A_j = -inf);
    repeated indices are taken entry by entry (each its own point mass), which is
    no longer a distance between distributions over V.
    idx: int [T, K] (shared by the heads) or [T, gamma, K]; val: the same shape;
    draft: [T, gamma, V].  Returns float64 [T, gamma, 4].
    """
    draft = np.asarray(draft, dtype=np.float64)
    T, G, V = draft.shape
    I = _head_topk(idx, G)
    A = _head_topk(np.asarray(val, dtype=np.float64), G)
    saved = np.empty((T, G, 4))
    for t in range(T):
        for k in range(G):
            ii = np.asarray(I[t, k], dtype=np.int64)
            ok = (ii >= 0) & (ii < V)
            a = np.where(ok, A[t, k], -np.inf)
            logp, lse_a = log_softmax(a)
            logq, lse_q = log_softmax(draft[t, k])
            if logp is None or logq is None:
                saved[t, k] = (lse_a, lse_q, np.nan, np.nan)
                continue
            lq = np.where(ok, logq[np.where(ok, ii, 0)], -np.inf)
            qj, pj = np.exp(lq), np.exp(logp)
            alpha = min(max(float(np.sum(np.minimum(pj, qj))), 0.0), 1.0)
            s = float(np.sum(qj[lq <= logp]))
            saved[t, k] = (lse_a, lse_q, alpha, s)
    return saved


def tv_topk_loss(idx, val, draft):
    """Mean over positions of the end-to-end TV loss with top-K targets (the
    position loss and the mean as in tv_loss).  Returns (loss, pos_loss, saved)."""
    saved = tv_topk_stats(idx, val, draft)
    pos_loss = e2e_position_loss(saved[:, :, 2])
    return float(np.mean(pos_loss)), pos_loss, saved


def tv_topk_loss_grad(idx, val, draft, g=1.0):
    """Gradient of g * tv_topk_loss with respect to the draft logits (paperlayer
    App. A with the truncated target): d alpha / d z_v = q_v (c_v - S) with c_v the
    number of entries j with I_j = v and log q_v <= log p_j (0 or 1 for distinct
    indices), chained through the end-to-end weights.  Returns float64 [T, gamma, V].
    """
    draft = np.asarray(draft, dtype=np.float64)
    T, G, V = draft.shape
    I = _head_topk(idx, G)
    A = _head_topk(np.asarray(val, dtype=np.float64), G)
    saved = tv_topk_stats(idx, val, draft)
    w = e2e_weights(saved[:, :, 2], g, T)
    grad = np.empty((T, G, V))
    for t in range(T):
        for k in range(G):
            ii = np.asarray(I[t, k], dtype=np.int64)
            ok = (ii >= 0) & (ii < V)
            logp, _ = log_softmax(np.where(ok, A[t, k], -np.inf))
            logq, _ = log_softmax(draft[t, k])
            if logp is None or logq is None:
                grad[t, k] = np.nan
                continue
            q = np.exp(logq)
            c = np.zeros(V)
            for j in np.flatnonzero(ok):
                if logq[ii[j]] <= logp[j]:
                    c[ii[j]] += 1.0
            grad[t, k] = w[t, k] * q * (c - saved[t, k, 3])
    return grad


def tv_topk_indicator_margin(idx, val, draft):
    """|log q_{I_j} - log p_j| per entry [T, gamma, K] (inf for entries out of
    range): where it is tiny a float32 indicator may flip."""
    draft = np.asarray(draft, dtype=np.float64)
    T, G, V = draft.shape
    I = _head_topk(idx, G)
    A = _head_topk(np.asarray(val, dtype=np.float64), G)
    K = I.shape[-1]
    m = np.full((T, G, K), np.inf)
    for t in range(T):
        for k in range(G):
            ii = np.asarray(I[t, k], dtype=np.int64)
            ok = (ii >= 0) & (ii < V)
            logp, _ = log_softmax(np.where(ok, A[t, k], -np.inf))
            logq, _ = log_softmax(draft[t, k])
            if logp is None or logq is None:
                continue
            m[t, k, ok] = np.abs(logq[ii[ok]] - logp[ok])
    return m
