"""GPU parity of mtp_verify_gumbel and mtp_gumbel_sample against the float64 oracle.

Cases follow the other verify tests: the tiny float32 workload at three
temperatures; ragged vocabularies (both dtypes, gamma up to 8); float32 rows of
more than 64 chunks; every row of the rollout workload with draft tokens from
the GPU sampler; sampled sequences of the long-tail workload; temperature 1
against the plain verify's flags and statistics; edge cases (p = q, a wave where
q outweighs p by more than 2^64, bad rows); workspace reuse across the three
verify modes; position-addressed noise; the sampler on ragged rows and rows
with one or no finite logit; and chi-square tests of the sampler against the
tempered q and of the first emitted token against the tempered p.

Tokens must equal the oracle's except where it marks a near-tie of the Gumbel
keys (runner-up within 1e-4 in natural-log units, far above the float32 key
error) or a near-empty residual; accept flags as for the plain verify.
"""
import numpy as np
import pytest
import torch
from scipy import special, stats

import synthetic
import tv_loss_amd as mtp
from oracle import mtp as omtp
from parity import (check_tokens, compare_target_only, compare_verify, oracle_target_only, oracle_verify,
                    stat_close, to_f64)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mtp.load()


def _say(*a):
    print(*a, flush=True)


def _run(target, draft, tokens, T, seed, offset):
    out = mtp.verify_gumbel(target, draft, tokens, T, seed, offset)
    torch.cuda.synchronize()
    return out


def _oracle(target, draft, tokens, T, seed, offset):
    return omtp.verify_gumbel(to_f64(target), to_f64(draft), tokens.cpu().numpy(), seed, offset, temperature=T)


def _pad(t, d, V, dtype, fill=30.0):
    """Rows must start 16-byte aligned: pad the vocabulary dimension, by default
    with a large finite logit (exact in bf16), so a read past V would change every
    statistic and token."""
    pv = 16 // (torch.finfo(dtype).bits // 8)
    pad = (-V) % pv
    if not pad:
        return t, d
    tp = torch.full(t.shape[:-1] + (V + pad,), fill, dtype=dtype, device=DEV)
    dp = torch.full(d.shape[:-1] + (V + pad,), fill, dtype=dtype, device=DEV)
    tp[..., :V] = t
    dp[..., :V] = d
    return tp[..., :V], dp[..., :V]


def _compare_sampler(tokens, draft, T, seed, offset):
    ref, allowed = omtp.gumbel_draft_tokens(to_f64(draft), seed, offset, temperature=T)
    check_tokens(tokens.cpu().numpy(), ref, allowed)
    return int(sum(a.size > 1 for a in allowed.ravel()))


@pytest.mark.parametrize("T", [0.6, 1.0, 1.7])
@pytest.mark.parametrize("seed", range(4))
def test_tiny_float32(seed, T):
    w = synthetic.VERIFY_WORKLOADS["tiny"]
    t, d, y = synthetic.verify_inputs(w, DEV, seed=seed)
    _say("gm tiny seed", seed, "T", T)
    out = _run(t, d, y, T, seed=900 + seed, offset=5 * seed)
    compare_verify(out, _oracle(t, d, y, T, 900 + seed, 5 * seed), torch.float32)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V,G,B", [(1, 1, 3), (7, 2, 2), (1000, 3, 3), (8193, 3, 2), (50003, 3, 3),
                                   (70000, 8, 2)])
def test_ragged_vocab(V, G, B, dtype):
    w = dict(B=B, G=G, V=V, dtype=dtype, kind="normal", scale=1.5, sigma=0.4, seed=13)
    t, d, y = synthetic.verify_inputs(w, DEV, seed=V + 5 * G)
    t, d = _pad(t, d, V, dtype)
    _say("gm ragged", V, G, B, dtype)
    out = _run(t, d, y, 0.8, seed=7, offset=123)
    compare_verify(out, _oracle(t, d, y, 0.8, 7, 123), dtype)


def test_many_chunks_float32():
    """More than 64 chunks per row: key words beyond the first 64 lanes' share."""
    B, G, V = 2, 2, 262144
    w = dict(B=B, G=G, V=V, dtype=torch.float32, kind="normal", scale=1.2, sigma=0.5, seed=15)
    t, d, y = synthetic.verify_inputs(w, DEV, seed=V + 2)
    _say("gm many chunks")
    out = _run(t, d, y, 1.3, seed=10, offset=40)
    compare_verify(out, _oracle(t, d, y, 1.3, 10, 40), torch.float32)


def test_rollout_all_rows_with_gpu_draft_tokens():
    """Draft tokens from the GPU sampler at T (its own counter range), then the
    tempered verify; both against the oracle on every row."""
    w = synthetic.VERIFY_WORKLOADS["rollout"]
    T = 0.7
    t, d, _ = synthetic.verify_inputs(w, DEV)          # the full bench batch: 64 x (3 + 1) rows
    B, G = d.shape[0], d.shape[1]
    _say("gm rollout shape")
    y = mtp.gumbel_sample(d, T, seed=41, offset=1 << 40)
    torch.cuda.synchronize()
    assert y.shape == (B, G) and y.dtype == torch.int32
    near = _compare_sampler(y, d, T, 41, 1 << 40)
    out = _run(t, d, y, T, seed=42, offset=0)
    ties = compare_verify(out, _oracle(t, d, y, T, 42, 0), torch.bfloat16)
    _say("sampler near-ties", near, "verify ties", ties, "accept", out["accept"].float().mean().item())


def test_long_tail_sampled():
    w = synthetic.VERIFY_WORKLOADS["long_tail"]
    t, d, y = synthetic.verify_inputs(w, DEV, B=96)
    _say("gm long tail")
    out = _run(t, d, y, 1.2, seed=6, offset=0)
    G1 = w["G"] + 1
    for b in (0, 1, 50, 95):
        ref = _oracle(t[b:b + 1], d[b:b + 1], y[b:b + 1], 1.2, 6, b * G1)
        compare_verify(out, ref, torch.bfloat16, rows=[b])


def test_temperature_one_keeps_the_plain_verify_decisions():
    """At T = 1 the accept decisions, accepted lengths and statistics are those of
    mtp_verify (same uniforms u); only the row samples differ in method."""
    w = synthetic.VERIFY_WORKLOADS["rollout"]
    t, d, y = synthetic.verify_inputs(w, DEV, B=16, V=80000)
    gm = _run(t, d, y, 1.0, seed=3, offset=77)
    rs = mtp.verify(t, d, y, 3, 77)
    torch.cuda.synchronize()
    assert torch.equal(gm["accept"], rs["accept"]) and torch.equal(gm["accepted_len"], rs["accepted_len"])
    for k in ("overlap", "entropy", "tv"):
        ok = stat_close(gm[k].cpu().numpy(), rs[k].cpu().numpy(), torch.float32)
        assert ok.all(), k
    compare_verify(gm, _oracle(t, d, y, 1.0, 3, 77), torch.bfloat16)


def test_identical_rows_sample_tempered_p():
    B, G, V = 4, 3, 30000
    g = torch.Generator(device=DEV).manual_seed(5)
    t = torch.randn((B, G + 1, V), generator=g, device=DEV).to(torch.bfloat16)
    d = t[:, :G].clone()
    y = torch.randint(0, V, (B, G), generator=g, device=DEV, dtype=torch.int32)
    out = _run(t, d, y, 0.9, seed=12, offset=0)
    assert out["accept"].all() and (out["accepted_len"] == G).all()
    assert ((out["row_status"][:, :G] & mtp.ROW_RESIDUAL_EMPTY) != 0).all()
    assert (out["tv"] == 0).all()
    compare_verify(out, _oracle(t, d, y, 0.9, 12, 0), torch.bfloat16)


def test_q_outweighs_p_by_more_than_2_to_the_64_in_a_wave():
    """In the first 4096 entries p is ~2^-86 of its row maximum while q sits at its
    own maximum: those waves take the residual in q's units."""
    B, G, V = 3, 2, 20000
    g = torch.Generator(device=DEV).manual_seed(8)
    t = torch.randn((B, G + 1, V), generator=g, device=DEV)
    d = torch.randn((B, G, V), generator=g, device=DEV)
    t[:, :G, :4096] = -60.0
    d[:, :, :4096] += 5.0
    d[:, :, 4096:] = -60.0
    t, d = t.contiguous(), d.contiguous()
    y = synthetic.gumbel_tokens(d, torch.Generator(device=DEV).manual_seed(9))
    out = _run(t, d, y, 1.0, seed=2, offset=0)
    compare_verify(out, _oracle(t, d, y, 1.0, 2, 0), torch.float32)


def test_bad_rows():
    w = dict(B=3, G=3, V=9000, dtype=torch.bfloat16, kind="normal", scale=1.0, sigma=0.3, seed=4)
    t, d, y = synthetic.verify_inputs(w, DEV)
    t[1, 2, :] = float("-inf")
    d[2, 0, 17] = float("nan")
    y[0, 1] = 9000                                      # out of range
    out = _run(t, d, y, 0.5, seed=8, offset=0)
    st = out["row_status"].cpu().numpy()
    assert st[1, 2] & mtp.ROW_BAD_TARGET and out["row_token"][1, 2] == -1 and out["accept"][1, 2] == 0
    assert st[2, 0] & mtp.ROW_BAD_DRAFT and out["accept"][2, 0] == 0 and out["accepted_len"][2] == 0
    assert st[0, 1] & mtp.ROW_BAD_TOKEN and out["accept"][0, 1] == 0
    compare_verify(out, _oracle(t, d, y, 0.5, 8, 0), torch.bfloat16)


def test_workspace_shared_across_verify_modes():
    """Gumbel, rejection-sampling and target-only calls alternate on one workspace:
    each repeats bit for bit and the error word stays clear."""
    w = synthetic.VERIFY_WORKLOADS["rollout"]
    t, d, y = synthetic.verify_inputs(w, DEV, B=8, V=60000)
    first = _run(t, d, y, 0.8, seed=4, offset=0)
    rs_first = mtp.verify(t, d, y, 4, 0)
    to_first = mtp.verify_target_only(t, d, 4, 0)
    for _ in range(4):
        rs = mtp.verify(t, d, y, 4, 0)
        again = _run(t, d, y, 0.8, seed=4, offset=0)
        to = mtp.verify_target_only(t, d, 4, 0)
        torch.cuda.synchronize()
        for ref, cur in ((first, again), (rs_first, rs), (to_first, to)):
            for k in ref:
                assert torch.equal(torch.nan_to_num(ref[k].float()), torch.nan_to_num(cur[k].float())), k
    assert mtp.workspace_error(mtp.workspace(DEV, 1)) == 0
    compare_verify(first, _oracle(t, d, y, 0.8, 4, 0), torch.bfloat16)
    compare_verify(rs_first, oracle_verify(t, d, y, 4, 0), torch.bfloat16)
    compare_target_only(to_first, oracle_target_only(t, d, 4, 0), torch.bfloat16)


def test_offset_addresses_the_noise():
    w = synthetic.VERIFY_WORKLOADS["rollout"]
    t, d, y = synthetic.verify_inputs(w, DEV, B=5, V=30000)
    full = _run(t, d, y, 1.4, seed=71, offset=500)
    for b in range(5):
        one = _run(t[b:b + 1], d[b:b + 1], y[b:b + 1], 1.4, seed=71, offset=500 + 4 * b)
        for k in ("accept", "row_token", "accepted_len", "next_token"):
            assert torch.equal(one[k][0], full[k][b]), (b, k)
    toks = mtp.gumbel_sample(d, 1.4, seed=3, offset=20)
    for b in range(5):
        one = mtp.gumbel_sample(d[b], 1.4, seed=3, offset=20 + 3 * b)
        assert torch.equal(one, toks[b]), b


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V", [1, 5, 8, 1000, 4099, 151936, 262147])
def test_sampler_matches_oracle(V, dtype):
    rows = 37 if V < 200000 else 9
    g = torch.Generator(device=DEV).manual_seed(V)
    x = (1.3 * torch.randn((rows, V), generator=g, device=DEV)).to(dtype)
    x, _ = _pad(x, x, V, dtype)
    _say("sampler", V, dtype)
    for T in (0.5, 1.3):
        toks = mtp.gumbel_sample(x, T, seed=V + 1, offset=7)
        torch.cuda.synchronize()
        _compare_sampler(toks, x, T, V + 1, 7)


def test_sampler_one_and_no_finite_logit():
    V = 5000
    x = torch.full((4, V), float("-inf"), device=DEV)
    x[0, 4321] = 3.0                                    # one finite entry: always it
    x[1, 0] = -1e30                                     # one very negative finite entry
    x[3, :] = float("nan")                              # no comparable key
    toks = mtp.gumbel_sample(x, 0.7, seed=1, offset=0).cpu().numpy()
    assert toks[0] == 4321 and toks[1] == 0 and toks[2] == -1 and toks[3] == -1


def test_chi_square_sampler_and_first_token():
    """Over 200000 sequences at T = 0.8: the sampler's tokens follow softmax(z / T)
    and the first emitted token follows softmax(target / T) (App. G.2: the
    tempered rejection sampler keeps the tempered target law)."""
    V, B, T = 16, 200000, 0.8
    g = torch.Generator(device=DEV).manual_seed(23)
    base_t = 1.3 * torch.randn((1, 2, V), generator=g, device=DEV)
    base_d = base_t[:, :1] + 0.8 * torch.randn((1, 1, V), generator=g, device=DEV)
    t = base_t.expand(B, 2, V).contiguous()
    d = base_d.expand(B, 1, V).contiguous()
    y = mtp.gumbel_sample(d, T, seed=99, offset=1 << 33)
    q = special.softmax(to_f64(base_d[0, 0]) / T)
    cy = torch.bincount(y[:, 0].long(), minlength=V).cpu().numpy()
    assert stats.chisquare(cy, q * B).pvalue > 1e-4
    out = _run(t, d, y, T, seed=2026, offset=0)
    first = torch.where(out["accept"][:, 0] == 1, y[:, 0], out["row_token"][:, 0])
    counts = torch.bincount(first.long(), minlength=V).cpu().numpy()
    p = special.softmax(to_f64(base_t[0, 0]) / T)
    assert stats.chisquare(counts, p * B).pvalue > 1e-4
    n = 2000
    _compare_sampler(y[:n], d[:n], T, 99, 1 << 33)
    compare_verify({k: v[:n] for k, v in out.items()}, _oracle(t[:n], d[:n], y[:n], T, 2026, 0), torch.float32)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_sampler_equal_logits_pick_the_largest_noise(dtype):
    """Equal logits: the token is the element with the largest Gumbel noise (U
    nearest 1), where the exponential variate is smallest; checks the noise's
    accuracy in its upper tail against the float64 oracle."""
    rows, V = 24, 262144
    x = torch.full((rows, V), 0.25, dtype=dtype, device=DEV)
    toks = mtp.gumbel_sample(x, 1.0, seed=1234, offset=55)
    torch.cuda.synchronize()
    assert _compare_sampler(toks, x, 1.0, 1234, 55) <= 2


def test_sampler_leaves_the_shared_workspace_zeroed():
    """The sampler's partial maxima are cleared by its second kernel, so a verify
    call on the same (shared) workspace right after it sees a clean one."""
    w = synthetic.VERIFY_WORKLOADS["rollout"]
    t, d, y = synthetic.verify_inputs(w, DEV, B=6, V=50000)
    toks = mtp.gumbel_sample(d, 0.9, seed=8, offset=1 << 36)
    torch.cuda.synchronize()
    ws = mtp.workspace(DEV, 1)
    assert int(torch.count_nonzero(ws)) == 0
    out = _run(t, d, toks, 0.9, seed=8, offset=0)
    assert mtp.workspace_error(ws) == 0 and int(torch.count_nonzero(ws)) == 0
    _compare_sampler(toks, d, 0.9, 8, 1 << 36)
    compare_verify(out, _oracle(t, d, toks, 0.9, 8, 0), torch.bfloat16)
