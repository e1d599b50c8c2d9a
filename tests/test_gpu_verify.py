"""GPU parity of mtp_verify against the float64 oracle, on identical seeded inputs.

Sizes: the tiny float32 workload; ragged vocabularies spanning several chunks (4096
bfloat16 or 3072 float32 logits each) with a partial last vector; the full rollout workload (64 x 4 rows of
151936, every row checked); 64 sampled sequences of the long-tail workload (512 x 5
rows of 262144, the last super-group's included) and 16 of each of the 15
entropy-sweep cells; edge cases; determinism and
workspace reuse; and 10^6 sequences at V = 8 and 16 (2 x 10^6 Philox counters) whose
every decision and token equals the oracle's, with a chi-square test of the
emitted token against p.
"""
import numpy as np
import pytest
import torch
from scipy import stats

import synthetic
import tv_loss_amd as mtp
from oracle import mtp as omtp
from oracle.philox import verify_uniforms
from parity import compare_verify, oracle_verify, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
PAD_LOGIT = 30.0   # fills the padding past V in ragged rows


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mtp.load()


def _run(target, draft, tokens, seed, offset):
    out = mtp.verify(target, draft, tokens, seed, offset)
    torch.cuda.synchronize()
    return out


def _say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("seed", range(12))
def test_tiny_float32(seed):
    w = synthetic.VERIFY_WORKLOADS["tiny"]
    t, d, y = synthetic.verify_inputs(w, DEV, seed=seed)
    _say("tiny seed", seed)
    out = _run(t, d, y, seed=1000 + seed, offset=7 * seed)
    ref = oracle_verify(t, d, y, 1000 + seed, 7 * seed)
    compare_verify(out, ref, torch.float32)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V,G,B", [(1, 1, 3), (7, 2, 2), (8, 3, 2), (1000, 3, 3), (8191, 1, 2), (8193, 3, 2),
                                   (50003, 3, 3), (70000, 8, 2)])
def test_ragged_vocab(V, G, B, dtype):
    """Vocabulary sizes around vector and chunk boundaries; padded row strides."""
    w = dict(B=B, G=G, V=V, dtype=dtype, kind="normal", scale=1.5, sigma=0.4, seed=11)
    t, d, y = synthetic.verify_inputs(w, DEV, seed=V + G)
    pad = (-V) % (16 // t.element_size())
    if pad:   # rows must start 16-byte aligned: pad the vocabulary dimension with a
        # large finite logit (exact in bf16), so a read past V would change every
        # statistic and token
        tp = torch.full((B, G + 1, V + pad), PAD_LOGIT, dtype=dtype, device=DEV)
        dp = torch.full((B, G, V + pad), PAD_LOGIT, dtype=dtype, device=DEV)
        tp[..., :V] = t
        dp[..., :V] = d
        t, d = tp[..., :V], dp[..., :V]
    _say("ragged", V, G, B, dtype)
    out = _run(t, d, y, seed=5, offset=123)
    ref = oracle_verify(t, d, y, 5, 123)
    compare_verify(out, ref, dtype)


@pytest.mark.parametrize("V", [262144, 400003])
def test_many_chunks_float32(V):
    """More than 64 (V = 262144) and more than 128 (V = 400003) chunks per row for
    float32 rows: records beyond the first 64 per lane batch, and chunk masses the
    finish re-reads instead of keeping in registers."""
    B, G = 2, 2
    w = dict(B=B, G=G, V=V, dtype=torch.float32, kind="normal", scale=1.2, sigma=0.5, seed=13)
    t, d, y = synthetic.verify_inputs(w, DEV, seed=V)
    pad = (-V) % 4
    if pad:
        tp = torch.full((B, G + 1, V + pad), PAD_LOGIT, dtype=torch.float32, device=DEV)
        dp = torch.full((B, G, V + pad), PAD_LOGIT, dtype=torch.float32, device=DEV)
        tp[..., :V] = t
        dp[..., :V] = d
        t, d = tp[..., :V], dp[..., :V]
    _say("many chunks", V)
    out = _run(t, d, y, seed=8, offset=40)
    compare_verify(out, oracle_verify(t, d, y, 8, 40), torch.float32)


@pytest.mark.parametrize("extra", [-28, -4, 0, 4, 8])
def test_item_split_around_four_items_per_super_group(extra):
    """Super-groups take contiguous, unequal item ranges once every one of them has at
    least four items (N >= 4 S), round-robin items below: V = 151936 (38 chunks per
    row), N = B (G + 1) around four items per super-group of the full chip, every
    output against the oracle."""
    G, V = 3, 151936
    smax = torch.cuda.get_device_properties(0).multi_processor_count * 4 // 38
    B = max(1, smax + extra // 4)
    w = dict(B=B, G=G, V=V, dtype=torch.bfloat16, kind="normal", scale=1.3, sigma=0.4, seed=17)
    t, d, y = synthetic.verify_inputs(w, DEV, seed=B)
    _say("item split", B, "x", G + 1, "items, super-groups at most", smax)
    out = _run(t, d, y, seed=3, offset=B)
    compare_verify(out, oracle_verify(t, d, y, 3, B), torch.bfloat16)


def test_rollout_full():
    w = synthetic.VERIFY_WORKLOADS["rollout"]
    t, d, y = synthetic.verify_inputs(w, DEV)
    _say("rollout full")
    out = _run(t, d, y, seed=2, offset=0)
    ref = oracle_verify(t, d, y, 2, 0)
    ties = compare_verify(out, ref, torch.bfloat16)
    _say("rollout ties (accept, token):", ties, "mean overlap", ref["overlap"].mean())


def test_long_tail_sampled():
    w = synthetic.VERIFY_WORKLOADS["long_tail"]
    t, d, y = synthetic.verify_inputs(w, DEV)
    _say("long tail")
    out = _run(t, d, y, seed=5, offset=0)
    G1 = w["G"] + 1
    # 64 sequences: both ends (the last ones sit in the last super-group) and a seeded sample
    rng = np.random.default_rng(17)
    fixed = [0, 1, 2, 3, 255, 256, 400, 508, 509, 510, 511]
    rows = sorted(fixed + rng.choice(np.setdiff1d(np.arange(512), fixed), 64 - len(fixed), replace=False).tolist())
    for b in rows:
        ref = oracle_verify(t[b:b + 1], d[b:b + 1], y[b:b + 1], 5, b * G1)
        compare_verify(out, ref, torch.bfloat16, rows=[b])
    # whole-batch properties
    rt = out["row_token"].cpu().numpy()
    assert rt.min() >= 0 and rt.max() < w["V"]
    ov, tv = out["overlap"].cpu().numpy(), out["tv"].cpu().numpy()
    np.testing.assert_allclose(ov + tv, 1.0, atol=2e-3)
    assert (out["row_status"].cpu().numpy() == 0).all()


@pytest.mark.parametrize("i_tau", range(5))
@pytest.mark.parametrize("i_sigma", range(3))
def test_entropy_sweep_cell(i_tau, i_sigma):
    w = synthetic.sweep_cell(i_tau, i_sigma)
    t, d, y = synthetic.verify_inputs(w, DEV)
    seed = w["seed"]
    _say("sweep cell", i_tau, i_sigma)
    out = _run(t, d, y, seed=seed, offset=0)
    G1 = w["G"] + 1
    # 16 sequences per cell: both ends and a seeded sample
    rng = np.random.default_rng(1000 + 10 * i_tau + i_sigma)
    fixed = [0, 37, 127]
    seqs = sorted(fixed + rng.choice(np.setdiff1d(np.arange(128), fixed), 13, replace=False).tolist())
    for b in seqs:
        ref = oracle_verify(t[b:b + 1], d[b:b + 1], y[b:b + 1], seed, b * G1)
        compare_verify(out, ref, torch.bfloat16, rows=[b])
    _say(f"tau={synthetic.SWEEP_TAUS[i_tau]} sigma={synthetic.SWEEP_SIGMAS[i_sigma]}: "
         f"accept {out['accept'].float().mean().item():.4f}, mean n {out['accepted_len'].float().mean().item():.3f}, "
         f"H {out['entropy'].mean().item():.3f}")


def test_identical_rows_accept_everything():
    w = synthetic.VERIFY_WORKLOADS["rollout"]
    t, _, _ = synthetic.verify_inputs(w, DEV, B=8)
    d = t[:, :3].clone()
    y = synthetic.gumbel_tokens(d, torch.Generator(device=DEV).manual_seed(3))
    out = _run(t, d, y, seed=4, offset=0)
    assert out["accept"].all() and (out["accepted_len"] == 3).all()
    assert (out["tv"] == 0).all()                       # same bytes -> same p, q bits
    assert torch.allclose(out["overlap"], torch.ones_like(out["overlap"]), atol=1e-3)
    assert (out["row_status"][:, :3] == mtp.ROW_RESIDUAL_EMPTY).all()
    assert torch.equal(out["next_token"], out["row_token"][:, 3])
    ref = oracle_verify(t, d, y, 4, 0)
    compare_verify(out, ref, torch.bfloat16)


def test_disjoint_supports_reject_everything():
    B, G, V = 4, 3, 20000
    g = torch.Generator(device=DEV).manual_seed(9)
    t = torch.randn((B, G + 1, V), generator=g, device=DEV).to(torch.bfloat16)
    d = torch.randn((B, G, V), generator=g, device=DEV).to(torch.bfloat16)
    t[:, :, 0::2] = float("-inf")
    d[:, :, 1::2] = float("-inf")
    y = synthetic.gumbel_tokens(d, g)
    out = _run(t, d, y, seed=1, offset=0)
    assert not out["accept"].any() and (out["accepted_len"] == 0).all()
    assert (out["overlap"] == 0).all()
    assert torch.allclose(out["tv"], torch.ones_like(out["tv"]), atol=1e-3)
    assert (out["next_token"] % 2 == 1).all()
    compare_verify(out, oracle_verify(t, d, y, 1, 0), torch.bfloat16)


def test_bad_rows_and_tokens():
    w = dict(B=4, G=3, V=9000, dtype=torch.bfloat16, kind="normal", scale=1.0, sigma=0.3, seed=1)
    t, d, y = synthetic.verify_inputs(w, DEV)
    y[0, 1] = -1
    y[1, 0] = 9000
    t[2, 2, :] = float("-inf")
    d[3, 0, 17] = float("nan")
    out = _run(t, d, y, seed=8, offset=0)
    st = out["row_status"].cpu().numpy()
    assert st[0, 1] & mtp.ROW_BAD_TOKEN and out["accept"][0, 1] == 0
    assert st[1, 0] & mtp.ROW_BAD_TOKEN and out["accepted_len"][1] == 0
    assert st[2, 2] & mtp.ROW_BAD_TARGET and out["row_token"][2, 2] == -1
    assert torch.isnan(out["entropy"][2, 2]) and torch.isnan(out["overlap"][2, 2])
    assert st[3, 0] & mtp.ROW_BAD_DRAFT and out["accept"][3, 0] == 0 and out["row_token"][3, 0] == -1
    compare_verify(out, oracle_verify(t, d, y, 8, 0), torch.bfloat16)


def test_empty_batch():
    t = torch.zeros((0, 4, 64), dtype=torch.bfloat16, device=DEV)
    out = mtp.verify(t, t[:, :3], torch.zeros((0, 3), dtype=torch.int32, device=DEV), 0)
    assert out["accepted_len"].numel() == 0


def test_deterministic_and_workspace_reuse():
    w = synthetic.VERIFY_WORKLOADS["rollout"]
    t, d, y = synthetic.verify_inputs(w, DEV, B=16)
    small = synthetic.verify_inputs(dict(w, B=3, V=9000), DEV)
    first = _run(t, d, y, seed=3, offset=0)
    for i in range(10):
        # alternate shapes on the same workspace; every call must leave it clean
        s_out = _run(*small, seed=1, offset=i)
        again = _run(t, d, y, seed=3, offset=0)
        for k in first:
            assert torch.equal(torch.nan_to_num(first[k].float()), torch.nan_to_num(again[k].float())), k
    ws = mtp.workspace(DEV, 1)
    assert mtp.workspace_error(ws) == 0
    compare_verify(s_out, oracle_verify(*small, 1, 9), torch.bfloat16)


def test_offset_addresses_the_uniform_stream():
    """Sequence b alone at offset + b*(gamma+1) reproduces its results in the batch."""
    w = synthetic.VERIFY_WORKLOADS["rollout"]
    t, d, y = synthetic.verify_inputs(w, DEV, B=6, V=30000)
    full = _run(t, d, y, seed=77, offset=1000)
    for b in range(6):
        one = _run(t[b:b + 1], d[b:b + 1], y[b:b + 1], seed=77, offset=1000 + 4 * b)
        for k in ("accept", "row_token", "accepted_len", "next_token"):
            assert torch.equal(one[k][0], full[k][b]), (b, k)


@pytest.mark.parametrize("V", [8, 16])
def test_million_sequences_match_the_oracle_and_emit_p(V):
    """10^6 sequences of one (p, q) pair at V = 8 and 16, each with its own Philox
    counters (2 x 10^6 counters): every acceptance decision, row token and next
    token equals the one the oracle's rules give with its uniforms, near-ties (the
    oracle's tie bands) excepted and counted; the first emitted token is distributed
    as p (rejection sampling, paperlayer Sec. 2: chi-square p-value > 1e-4); and the
    acceptance rate is the overlap within 5 sigma."""
    B = 10 ** 6
    g = torch.Generator(device=DEV).manual_seed(31 + V)
    base_t = 1.5 * torch.randn((1, 2, V), generator=g, device=DEV)
    base_d = base_t[:, :1] + 0.9 * torch.randn((1, 1, V), generator=g, device=DEV)
    t = base_t.expand(B, 2, V).contiguous()
    d = base_d.expand(B, 1, V).contiguous()
    y = synthetic.gumbel_tokens(d, g)
    seed, offset = 4242 + V, 17
    _say("verify 1e6 sequences V", V)
    out = _run(t, d, y, seed=seed, offset=offset)
    acc = out["accept"][:, 0].cpu().numpy()
    rt = out["row_token"].cpu().numpy()
    nxt = out["next_token"].cpu().numpy()
    yy = y[:, 0].cpu().numpy()
    del t, d
    torch.cuda.empty_cache()
    # the oracle's rules, sequence by sequence, with its uniforms
    lp0, _ = omtp.log_softmax(to_f64(base_t[0, 0]))
    lp1, _ = omtp.log_softmax(to_f64(base_t[0, 1]))
    lq0, _ = omtp.log_softmax(to_f64(base_d[0, 0]))
    p0, p1, q0 = np.exp(lp0), np.exp(lp1), np.exp(lq0)
    u, up = verify_uniforms(seed, offset, np.arange(2 * B, dtype=np.uint64).reshape(B, 2))
    ref_acc = np.empty(B, np.uint8)
    tie_a = np.empty(B, bool)
    # the two rows' samples depend only on u' (one (p, q) pair for every sequence):
    # the oracle's token and allowed set, per distinct u'
    memo = {}

    def sample(row, upv):
        key = (row, float(upv))
        if key not in memo:
            memo[key] = omtp.row_sample(p0, q0, upv) if row == 0 else omtp.row_sample(p1, None, upv)
        return memo[key]

    bad = []
    n_flag = np.zeros(2, np.int64)
    n_mism = np.zeros(2, np.int64)
    for i in range(B):
        ref_acc[i], ratio = omtp.accept_decision(u[i, 0], lp0[yy[i]], lq0[yy[i]])
        tie_a[i] = abs(u[i, 0] - min(1.0, ratio)) <= omtp.ACCEPT_TIE_BAND
        for row in (0, 1):
            tok, _, allowed = sample(row, up[i, row])
            n_flag[row] += allowed.size > 1
            if rt[i, row] != tok:
                n_mism[row] += 1
                if rt[i, row] not in allowed:
                    bad.append((i, row, rt[i, row], tok))
    assert not bad, bad[:5]
    assert ((acc == ref_acc) | tie_a).all(), np.argwhere((acc != ref_acc) & ~tie_a)[:5]
    # next token: the first rejection's sample, or the bonus row's
    assert (nxt == np.where(acc == 1, rt[:, 1], rt[:, 0])).all()
    # the flag counts stay within the bound their probabilities give
    for row, pp, r in ((0, p0, omtp.residual(p0, q0)), (1, p1, p1)):
        pr = omtp.cdf_tie_probability(r, omtp.CDF_TIE_BAND * omtp.support_mass(pp, r))
        assert n_flag[row] <= B * pr + 5 * np.sqrt(B * pr) + 3, (row, n_flag[row], B * pr)
    assert tie_a.sum() <= B * 2e-6 + 5 * np.sqrt(B * 2e-6) + 3
    _say("near-ties: accept", int(tie_a.sum()), "token rows flagged", n_flag.tolist(),
         "GPU chose the other allowed token", n_mism.tolist())
    first = np.where(acc == 1, yy, rt[:, 0])
    counts = np.bincount(first, minlength=V)
    assert stats.chisquare(counts, p0 * B).pvalue > 1e-4
    alpha = omtp.overlap(p0, q0)
    rate = acc.mean()
    assert abs(rate - alpha) < 5 * np.sqrt(alpha * (1 - alpha) / B)


def test_mean_accepted_length_is_the_product_of_overlaps():
    """The expected number of accepted drafts is sum_k prod_{j<=k} alpha_j for
    independent positions (paperlayer Sec. 4: the acceptance length multiplies the
    per-step overlaps): 200000 sequences of three fixed (p, q) pairs, each with its
    own uniforms, against the overlaps of the oracle, within 5 sigma."""
    B, G, V = 200000, 3, 16
    g = torch.Generator(device=DEV).manual_seed(57)
    base_t = 1.2 * torch.randn((1, G + 1, V), generator=g, device=DEV)
    base_d = base_t[:, :G] + torch.tensor([0.3, 0.6, 1.0], device=DEV)[None, :, None] * torch.randn(
        (1, G, V), generator=g, device=DEV)
    t = base_t.expand(B, G + 1, V).contiguous()
    d = base_d.expand(B, G, V).contiguous()
    y = synthetic.gumbel_tokens(d, g)
    out = _run(t, d, y, seed=99, offset=5)
    n = out["accepted_len"].double().cpu().numpy()
    alphas = []
    for k in range(G):
        lp, _ = omtp.log_softmax(to_f64(base_t[0, k]))
        lq, _ = omtp.log_softmax(to_f64(base_d[0, k]))
        alphas.append(omtp.overlap(np.exp(lp), np.exp(lq)))
    expect = sum(np.prod(alphas[:k + 1]) for k in range(G))
    _say("alphas", alphas, "E[n]", expect, "mean n", n.mean())
    assert abs(n.mean() - expect) < 5 * n.std() / np.sqrt(B)
    # each flag's rate is its overlap, independently of the others
    rates = out["accept"].double().mean(0).cpu().numpy()
    for k in range(G):
        assert abs(rates[k] - alphas[k]) < 5 * np.sqrt(alphas[k] * (1 - alphas[k]) / B)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_largest_vocabulary(dtype):
    """The largest vocabulary one GPU verifies (every workgroup of the row resident
    at once), checked against the oracle; one vector more is refused."""
    V = mtp.verify_max_vocab(dtype)
    per = 4096 if dtype == torch.bfloat16 else 3072
    assert V % per == 0 and V >= 256 * per
    w = dict(B=1, G=1, V=V, dtype=dtype, kind="normal", scale=1.5, sigma=0.5, seed=21)
    t, d, y = synthetic.verify_inputs(w, DEV, seed=21)
    _say("verify largest vocabulary", V, dtype)
    out = _run(t, d, y, seed=4, offset=0)
    compare_verify(out, oracle_verify(t, d, y, 4, 0), dtype)
    pv = 16 // t.element_size()
    big = torch.zeros((1, 2, V + pv), dtype=dtype, device=DEV)
    with pytest.raises(mtp.MtpError, match="MTP_ERR_SHAPE"):
        mtp.verify(big, big[:, :1], torch.zeros((1, 1), dtype=torch.int32, device=DEV), 0)
    with pytest.raises(mtp.MtpError, match="MTP_ERR_SHAPE"):
        mtp.verify_gumbel(big, big[:, :1], torch.zeros((1, 1), dtype=torch.int32, device=DEV), 1.0, 0)
