"""GPU parity of mtp_verify_target_only against the float64 oracle.

Sizes and cases follow the rejection-sampling verify tests: the tiny float32
workload; ragged vocabularies around vector and chunk boundaries (both dtypes,
gamma up to 8); float32 rows of more than 64 chunks; every row of the rollout
batch; sampled sequences of the long-tail workload; edge cases (equal maxima of q
in different chunks and in the partial last vector, a one-hot target, bad rows);
workspace reuse alternating with rejection-sampling calls; position-addressed
uniforms; and a chi-square test of the first emitted token against p.
"""
import numpy as np
import pytest
import torch
from scipy import stats

import synthetic
import tv_loss_amd as mtp
from oracle import mtp as omtp
from parity import compare_target_only, compare_verify, oracle_target_only, oracle_verify, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mtp.load()


def _run(target, draft, seed, offset):
    out = mtp.verify_target_only(target, draft, seed, offset)
    torch.cuda.synchronize()
    return out


def _say(*a):
    print(*a, flush=True)


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


@pytest.mark.parametrize("seed", range(6))
def test_tiny_float32(seed):
    w = synthetic.VERIFY_WORKLOADS["tiny"]
    t, d, _ = synthetic.verify_inputs(w, DEV, seed=seed)
    _say("to tiny seed", seed)
    out = _run(t, d, seed=500 + seed, offset=3 * seed)
    compare_target_only(out, oracle_target_only(t, d, 500 + seed, 3 * seed), torch.float32)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V,G,B", [(1, 1, 3), (7, 2, 2), (1000, 3, 3), (8193, 3, 2), (50003, 3, 3),
                                   (70000, 8, 2)])
def test_ragged_vocab(V, G, B, dtype):
    w = dict(B=B, G=G, V=V, dtype=dtype, kind="normal", scale=1.5, sigma=0.4, seed=12)
    t, d, _ = synthetic.verify_inputs(w, DEV, seed=V + 3 * G)
    t, d = _pad(t, d, V, dtype)
    _say("to ragged", V, G, B, dtype)
    out = _run(t, d, seed=6, offset=321)
    compare_target_only(out, oracle_target_only(t, d, 6, 321), dtype)


def test_many_chunks_float32():
    """More than 64 chunks per row: argmax words and records beyond the first 64."""
    B, G, V = 2, 2, 262144
    w = dict(B=B, G=G, V=V, dtype=torch.float32, kind="normal", scale=1.2, sigma=0.5, seed=14)
    t, d, _ = synthetic.verify_inputs(w, DEV, seed=V + 1)
    _say("to many chunks")
    out = _run(t, d, seed=9, offset=17)
    compare_target_only(out, oracle_target_only(t, d, 9, 17), torch.float32)


def test_rollout_all_rows():
    w = synthetic.VERIFY_WORKLOADS["rollout"]
    t, d, _ = synthetic.verify_inputs(w, DEV)          # the full bench batch: 64 x (3 + 1) rows
    _say("to rollout shape")
    out = _run(t, d, seed=2, offset=0)
    ref = oracle_target_only(t, d, 2, 0)
    ties = compare_target_only(out, ref, torch.bfloat16)
    _say("ties", ties, "TO accept", ref["accept"].mean(), "RS-better share", ref["rs_better"].mean())


def test_long_tail_sampled():
    w = synthetic.VERIFY_WORKLOADS["long_tail"]
    t, d, _ = synthetic.verify_inputs(w, DEV, B=96)
    _say("to long tail")
    out = _run(t, d, seed=5, offset=0)
    G1 = w["G"] + 1
    for b in (0, 1, 47, 95):
        ref = oracle_target_only(t[b:b + 1], d[b:b + 1], 5, b * G1)
        compare_target_only(out, ref, torch.bfloat16, rows=[b])


def test_equal_maxima_take_the_smallest_index():
    """q's maximum at several indices: in different chunks, in one vector, and in
    the partial last vector; the greedy token is the smallest of them."""
    B, G, V = 4, 3, 40001
    g = torch.Generator(device=DEV).manual_seed(31)
    t = torch.randn((B, G + 1, V), generator=g, device=DEV).to(torch.bfloat16)
    d = torch.randn((B, G, V), generator=g, device=DEV).to(torch.bfloat16)
    d[0, 0, [30000, 9000, 39999]] = 8.0                 # different chunks
    d[0, 1, [40000, 17]] = 8.0                          # partial last vector and an early one
    d[0, 2, 40000] = 8.0                                # the last element alone
    d[1, 0, [4096, 4097, 4099]] = 8.0                   # one vector
    d[1, 1, [8191, 8192]] = 8.0                         # across a chunk boundary
    t, d = _pad(t, d, V, torch.bfloat16)
    out = _run(t, d, seed=3, offset=0)
    yh = out["draft_token"].cpu().numpy()
    assert yh[0, 0] == 9000 and yh[0, 1] == 17 and yh[0, 2] == 40000
    assert yh[1, 0] == 4096 and yh[1, 1] == 8191
    compare_target_only(out, oracle_target_only(t, d, 3, 0), torch.bfloat16)


def test_one_hot_target_accepts_and_samples_p():
    B, G, V = 4, 3, 20000
    g = torch.Generator(device=DEV).manual_seed(7)
    d = torch.randn((B, G, V), generator=g, device=DEV).to(torch.bfloat16)
    t = torch.full((B, G + 1, V), float("-inf"), device=DEV).to(torch.bfloat16)
    yh = d.float().argmax(-1)
    for b in range(B):
        for k in range(G):
            t[b, k, yh[b, k]] = 2.0
    t[:, G] = torch.randn((B, V), generator=g, device=DEV).to(torch.bfloat16)
    out = _run(t, d, seed=11, offset=0)
    assert out["accept"].all() and (out["accepted_len"] == G).all()
    assert torch.equal(out["draft_token"], yh.int())
    assert (out["p_yhat"] == 1.0).all() and not out["rs_better"].any()
    assert ((out["row_status"][:, :G] & mtp.ROW_RESIDUAL_EMPTY) != 0).all()
    assert torch.equal(out["row_token"][:, :G], yh.int())
    compare_target_only(out, oracle_target_only(t, d, 11, 0), torch.bfloat16)


def test_bad_rows():
    w = dict(B=3, G=3, V=9000, dtype=torch.bfloat16, kind="normal", scale=1.0, sigma=0.3, seed=2)
    t, d, _ = synthetic.verify_inputs(w, DEV)
    t[1, 2, :] = float("-inf")
    d[2, 0, 17] = float("nan")
    out = _run(t, d, seed=8, offset=0)
    st = out["row_status"].cpu().numpy()
    assert st[1, 2] & mtp.ROW_BAD_TARGET and out["draft_token"][1, 2] == -1 and out["row_token"][1, 2] == -1
    assert torch.isnan(out["p_yhat"][1, 2]) and out["accept"][1, 2] == 0
    assert st[2, 0] & mtp.ROW_BAD_DRAFT and out["accept"][2, 0] == 0 and out["accepted_len"][2] == 0
    compare_target_only(out, oracle_target_only(t, d, 8, 0), torch.bfloat16)


def test_workspace_shared_with_rejection_sampling():
    """Alternate target-only and rejection-sampling calls (different record layouts)
    on one workspace: every call leaves it clean and repeats bit for bit."""
    w = synthetic.VERIFY_WORKLOADS["rollout"]
    t, d, y = synthetic.verify_inputs(w, DEV, B=8, V=60000)
    first = _run(t, d, seed=4, offset=0)
    rs_first = mtp.verify(t, d, y, 4, 0)
    for i in range(6):
        rs = mtp.verify(t, d, y, 4, 0)
        again = _run(t, d, seed=4, offset=0)
        torch.cuda.synchronize()
        for k in first:
            assert torch.equal(torch.nan_to_num(first[k].float()), torch.nan_to_num(again[k].float())), k
        for k in rs_first:
            assert torch.equal(torch.nan_to_num(rs_first[k].float()), torch.nan_to_num(rs[k].float())), k
    assert mtp.workspace_error(mtp.workspace(DEV, 1)) == 0
    compare_target_only(first, oracle_target_only(t, d, 4, 0), torch.bfloat16)
    compare_verify(rs_first, oracle_verify(t, d, y, 4, 0), torch.bfloat16)


def test_offset_addresses_the_uniform_stream():
    w = synthetic.VERIFY_WORKLOADS["rollout"]
    t, d, _ = synthetic.verify_inputs(w, DEV, B=5, V=30000)
    full = _run(t, d, seed=70, offset=900)
    for b in range(5):
        one = _run(t[b:b + 1], d[b:b + 1], seed=70, offset=900 + 4 * b)
        for k in ("accept", "row_token", "accepted_len", "next_token", "draft_token"):
            assert torch.equal(one[k][0], full[k][b]), (b, k)


def test_chi_square_first_token_is_p():
    """Target-only sampling with the point-mass residual emits tokens distributed
    as p: over 200000 sequences, the first emitted token against p, and the
    acceptance rate against p(yhat) (paperlayer App. D.2)."""
    V, B = 16, 200000
    g = torch.Generator(device=DEV).manual_seed(22)
    base_t = 1.3 * torch.randn((1, 2, V), generator=g, device=DEV)
    base_d = base_t[:, :1] + 0.8 * torch.randn((1, 1, V), generator=g, device=DEV)
    t = base_t.expand(B, 2, V).contiguous()
    d = base_d.expand(B, 1, V).contiguous()
    out = _run(t, d, seed=2025, offset=0)
    first = torch.where(out["accept"][:, 0] == 1, out["draft_token"][:, 0], out["row_token"][:, 0])
    counts = torch.bincount(first.long(), minlength=V).cpu().numpy()
    p = np.exp(omtp.log_softmax(to_f64(base_t[0, 0]))[0])
    assert stats.chisquare(counts, p * B).pvalue > 1e-4
    py = p[int(np.argmax(to_f64(base_d[0, 0])))]
    rate = out["accept"].float().mean().item()
    assert abs(rate - py) < 5 * np.sqrt(py * (1 - py) / B)
    ref = oracle_target_only(t[:2000], d[:2000], 2025, 0)
    compare_target_only({k: v[:2000] for k, v in out.items()}, ref, torch.float32)
