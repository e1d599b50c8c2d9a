"""The GPU-vs-oracle comparison helpers (tests/parity.py), checked on the CPU with
the oracle's own outputs standing in for a GPU call: they accept them, accept a
token the oracle lists as an allowed neighbour, and reject planted mistakes (a
token outside the allowed set, a flipped decision outside the tie band, an
accepted length that no tied decision explains, a statistic off by more than the
tolerance)."""
import numpy as np
import pytest
import torch

from oracle import mtp as omtp
from parity import compare_verify


def _case(B=6, G=3, V=400, seed=3):
    rng = np.random.default_rng(seed)
    tgt = rng.normal(0, 1.3, (B, G + 1, V))
    dr = tgt[:, :G] + rng.normal(0, 0.4, (B, G, V))
    y = rng.integers(0, V, (B, G))
    return tgt, dr, y


def _as_gpu(ref):
    keys = ("accept", "accepted_len", "next_token", "row_token", "overlap", "tv", "entropy", "row_status")
    return {k: torch.from_numpy(np.array(ref[k], copy=True)) for k in keys}


def test_oracle_outputs_pass_and_counts_are_reported():
    tgt, dr, y = _case()
    ref = omtp.verify(tgt, dr, y, seed=5, offset=9)
    res = compare_verify(_as_gpu(ref), ref, torch.float32)
    assert res["token_mismatches"] == 0 and res["accept_flips"] == 0


def test_allowed_neighbour_passes_and_other_tokens_fail():
    tgt, dr, y = _case()
    # a band wide enough that some rows admit two tokens
    ref = omtp.verify(tgt, dr, y, seed=5, offset=9, cdf_tie_band=2e-3)
    flagged = np.argwhere(ref["token_tie"])
    assert flagged.size
    b, k = flagged[0]
    out = _as_gpu(ref)
    alt = [v for v in ref["token_allowed"][b, k] if v != ref["row_token"][b, k]][0]
    out["row_token"][b, k] = int(alt)
    n = int(out["accepted_len"][b])
    if n == k:
        out["next_token"][b] = int(alt)
    assert compare_verify(out, ref, torch.float32)["token_mismatches"] == 1
    out["row_token"][b, k] = int(max(ref["token_allowed"][b, k]) + 1)
    if n == k:
        out["next_token"][b] = out["row_token"][b, k]
    with pytest.raises(AssertionError):
        compare_verify(out, ref, torch.float32)


def test_planted_decision_length_and_statistic_mistakes_fail():
    tgt, dr, y = _case()
    ref = omtp.verify(tgt, dr, y, seed=5, offset=9)
    out = _as_gpu(ref)
    out["accept"][0, 0] ^= 1                      # outside the tie band
    with pytest.raises(AssertionError):
        compare_verify(out, ref, torch.float32)
    out = _as_gpu(ref)
    out["accepted_len"][1] = (int(out["accepted_len"][1]) + 1) % 4
    with pytest.raises(AssertionError):
        compare_verify(out, ref, torch.float32)
    out = _as_gpu(ref)
    out["overlap"][2, 1] += 1e-4
    with pytest.raises(AssertionError):
        compare_verify(out, ref, torch.float32)
