"""Comparison helpers for GPU-vs-oracle parity tests.

Tolerances (the verify and loss statistics): float32 inputs |d| <= 1e-5 |ref| +
1e-7; bfloat16 inputs |d| <= 1e-3.  Accept flags and token ids must be equal
except where the oracle marks a near-tie (|u - min(1, ratio)| <= 1e-6, or t
within 1e-6 * sum r of an inverse-CDF boundary); those are counted and reported.
"""
import numpy as np
import torch

from oracle import mtp as omtp
from oracle.bf16 import bf16_bits_to_f64, f64_to_bf16_bits

STAT_RTOL_F32, STAT_ATOL_F32 = 1e-5, 1e-7
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


def compare_verify(out, ref, dtype, rows=None):
    """Assert GPU verify outputs equal the oracle's.  `rows` selects sequences of
    `out` (the oracle ran on that subset).  Returns tie counts."""
    def g(name):
        v = out[name].cpu().numpy()
        return v if rows is None else v[rows]

    acc_tie = ref["accept_tie"]
    tok_tie = ref["token_tie"]
    acc = g("accept")
    bad = (acc != ref["accept"]) & ~acc_tie
    assert not bad.any(), f"accept mismatch at {np.argwhere(bad)[:10]}"
    rt = g("row_token")
    bad = (rt != ref["row_token"]) & ~tok_tie
    assert not bad.any(), f"row_token mismatch at {np.argwhere(bad)[:10]}: {rt[bad][:10]} vs {ref['row_token'][bad][:10]}"
    B, G1 = ref["row_token"].shape
    G = G1 - 1
    seq_tie = acc_tie.any(axis=1) | tok_tie.any(axis=1)
    al = g("accepted_len")
    nt = g("next_token")
    assert np.all((al == ref["accepted_len"]) | seq_tie), "accepted_len mismatch"
    assert np.all((nt == ref["next_token"]) | seq_tie), "next_token mismatch"
    # self-consistency holds everywhere, ties included
    for b in range(B):
        n = 0
        while n < G and acc[b, n] == 1:
            n += 1
        assert al[b] == n and nt[b] == rt[b, n]
    # the RESIDUAL_EMPTY bit is a float decision where the residual mass is ~0
    st, rst = g("row_status"), ref["row_status"].copy()
    near = tok_tie & ((rst & omtp.RESIDUAL_EMPTY) | (st & omtp.RESIDUAL_EMPTY)).astype(bool)
    mask = np.where(near, ~omtp.RESIDUAL_EMPTY, -1)
    np.testing.assert_array_equal(st & mask, rst & mask)
    for name in ("overlap", "tv", "entropy"):
        ok = stat_close(g(name), ref[name], dtype)
        assert ok.all(), f"{name}: max err {np.nanmax(np.abs(g(name) - ref[name]))} at {np.argwhere(~ok)[:5]}"
    return int(acc_tie.sum()), int(tok_tie.sum())


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
