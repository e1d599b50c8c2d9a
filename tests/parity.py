"""Comparison helpers for GPU-vs-oracle parity tests.

Tolerances (the verify and loss statistics): float32 inputs |d| <= 1e-5 |ref| +
2^-21 (the relative bar, with a floor of four float32 ulps of 1: a mass formed in
float32 from distributions that each sum to 1 carries absolute rounding of that
order, so a statistic whose exact value is 0 cannot meet a purely relative bar);
bfloat16 inputs |d| <= 1e-3.  Accept flags must equal the oracle's except
where |u - min(1, ratio)| <= 1e-6 (the oracle's accept_tie).  Every row token
must be one of the tokens the oracle lists for that row (token_allowed: the
exact inverse-CDF token, plus, where t lies within the band of a boundary, the
nearest positive-mass token across it; for Gumbel-max rows the tokens whose key
is within the gap band of the winner's).  Accepted lengths must be equal unless
a tied decision actually flipped at or before the first rejection; next tokens
follow from the row tokens.  The number of flagged decisions and rows is
bounded by the oracle's per-flag probability bounds (mean + 5 sigma + 3).
"""
import numpy as np
import torch

from oracle import mtp as omtp
from oracle.bf16 import bf16_bits_to_f64, f64_to_bf16_bits

STAT_RTOL_F32, STAT_ATOL_F32 = 1e-5, 2.0 ** -21
STAT_ATOL_BF16 = 1e-3


def to_f64(t):
    """Exact float64 copy of a float32 / bfloat16 tensor."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(t.contiguous().view(torch.int16).numpy().view(np.uint16))
    return t.to(torch.float64).numpy()


def stat_close(gpu, ref, dtype):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    both_nan = np.isnan(gpu) & np.isnan(ref)
    if dtype == torch.float32:
        ok = np.abs(gpu - ref) <= STAT_RTOL_F32 * np.abs(ref) + STAT_ATOL_F32
    else:
        ok = np.abs(gpu - ref) <= STAT_ATOL_BF16
    return ok | both_nan


def oracle_verify(target, draft, tokens, seed, offset):
    return omtp.verify(to_f64(target), to_f64(draft), tokens.cpu().numpy(), seed, offset)


def _flag_bound(probs):
    """Upper bound on the number of flags whose probabilities are at most `probs`
    (independent): mean + 5 sigma + 3."""
    probs = np.asarray(probs, dtype=np.float64)
    mean = probs.sum()
    return mean + 5.0 * np.sqrt(max(mean, 0.0)) + 3.0


def check_tokens(got, ref_tok, allowed):
    """Every token equals the oracle's or is one of its allowed tokens for that row.
    Returns the number of rows where the GPU chose another allowed token."""
    got = np.asarray(got)
    mism = np.argwhere(got != ref_tok)
    for idx in mism:
        idx = tuple(idx)
        al = allowed[idx]
        assert al is not None and got[idx] in al, (
            f"token at {idx}: {got[idx]} is not among the allowed {list(al)[:8] if al is not None else None} "
            f"(oracle {ref_tok[idx]})")
    return len(mism)


def compare_verify(out, ref, dtype, rows=None):
    """Assert GPU verify outputs equal the oracle's (`rows` selects the sequences of
    `out` the oracle ran on).  Returns the flag and mismatch counts."""
    def g(name):
        v = out[name].cpu().numpy()
        return v if rows is None else v[rows]

    acc, ref_acc, acc_tie = g("accept"), ref["accept"], ref["accept_tie"]
    flips = acc != ref_acc
    assert not (flips & ~acc_tie).any(), f"accept mismatch at {np.argwhere(flips & ~acc_tie)[:10]}"
    rt = g("row_token")
    tok_mism = check_tokens(rt, ref["row_token"], ref["token_allowed"])
    B, G1 = ref["row_token"].shape
    G = G1 - 1
    al, nt = g("accepted_len"), g("next_token")
    for b in range(B):
        n = 0
        while n < G and acc[b, n] == 1:
            n += 1
        assert al[b] == n and nt[b] == rt[b, n], f"sequence {b}: outputs not self-consistent"
        if al[b] != ref["accepted_len"][b]:
            first = min(al[b], ref["accepted_len"][b])
            assert flips[b, :first + 1].any(), f"sequence {b}: accepted length {al[b]} vs {ref['accepted_len'][b]}"
    # the RESIDUAL_EMPTY bit is a float decision only where the residual is near-empty
    st, rst = g("row_status"), ref["row_status"]
    mask = np.where(ref["near_empty"], ~omtp.RESIDUAL_EMPTY, -1)
    np.testing.assert_array_equal(st & mask, rst & mask)
    for name in ("overlap", "tv", "entropy"):
        ok = stat_close(g(name), ref[name], dtype)
        assert ok.all(), f"{name}: max err {np.nanmax(np.abs(g(name) - ref[name]))} at {np.argwhere(~ok)[:5]}"
    n_acc_tie, n_tok_tie = int(acc_tie.sum()), int(ref["token_tie"].sum())
    assert n_acc_tie <= _flag_bound(ref["accept_tie_bound"]), ("accept near-ties", n_acc_tie)
    assert n_tok_tie <= _flag_bound(ref["token_tie_bound"]), ("token near-ties", n_tok_tie)
    return dict(accept_ties=n_acc_tie, accept_flips=int(flips.sum()), token_ties=n_tok_tie,
                token_mismatches=tok_mism, rows=int(rt.size))


def oracle_target_only(target, draft, seed, offset):
    return omtp.verify_target_only(to_f64(target), to_f64(draft), seed, offset)


# The RS/TO flag compares a float32 TV with 1 - p(yhat); rows whose float64 values
# lie within this band of the boundary may flip.
RS_FLAG_BAND = 1e-4


def compare_target_only(out, ref, dtype, rows=None):
    """compare_verify's checks for a target-only call, plus the greedy tokens (exact:
    both sides compare the same input values), p(yhat) within the statistic
    tolerance and the RS/TO flags away from the boundary.  Returns tie counts."""
    ties = compare_verify(out, ref, dtype, rows)

    def g(name):
        v = out[name].cpu().numpy()
        return v if rows is None else v[rows]

    np.testing.assert_array_equal(g("draft_token"), ref["draft_token"])
    ok = stat_close(g("p_yhat"), ref["p_yhat"], dtype)
    assert ok.all(), f"p_yhat: {g('p_yhat')[~ok][:5]} vs {ref['p_yhat'][~ok][:5]}"
    near = np.abs(ref["tv"] - (1.0 - ref["p_yhat"])) <= RS_FLAG_BAND
    bad = (g("rs_better") != ref["rs_better"]) & ~near
    assert not bad.any(), f"rs_better mismatch at {np.argwhere(bad)[:10]}"
    return ties


def bf16_ulp_distance(a_bits, b_bits):
    """|a - b| in units of bfloat16 spacing (ordered-integer distance)."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + x)
    return np.abs(ordered(a_bits) - ordered(b_bits))


def bf16_bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def compare_grad_bf16(grad_gpu, grad_ref, margin, tie_band=1e-5):
    """grad_gpu: bf16 tensor [..., V]; grad_ref: float64.  Elements must agree to
    1 bf16 ulp except where `margin` < tie_band (the indicator may flip there; a
    caller may also zero the margin of elements it accounts for otherwise).
    Returns the number of excluded elements."""
    ref_bits = f64_to_bf16_bits(grad_ref)
    d = bf16_ulp_distance(bf16_bits(grad_gpu), ref_bits)
    tie = margin < tie_band
    bad = (d > 1) & ~tie
    assert not bad.any(), (f"{bad.sum()} gradient elements differ by more than 1 bf16 ulp; "
                           f"first at {np.argwhere(bad)[:5]}")
    return int(tie.sum())
