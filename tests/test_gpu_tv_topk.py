"""GPU parity of mtp_tv_topk_fwd / mtp_tv_topk_bwd against the float64 oracle
(oracle.mtp.tv_topk_*), with the tolerances of the full-vocabulary TV tests:
saved statistics and losses within the statistic tolerances (S also within the
draft mass of entries whose indicator is within 1e-5 of flipping), the bfloat16
gradient within 1 bf16 ulp of the oracle's rounded value and the float32 gradient
within 1e-3 norm-relative per row.  Cases: the tiny float32 workload; ragged
vocabularies and K (both dtypes, shared and per-head targets, gamma up to 8);
K = V against the full-vocabulary path; indices out of range, repeated indices
and -inf logits; rows with no finite normaliser; sampled positions of the
T = 8192, V = 151936, K = 256 workload; the autograd wrapper.
"""
import numpy as np
import pytest
import torch

import synthetic
import tv_loss_amd as mtp
from oracle import mtp as omtp
from parity import compare_grad_bf16, stat_close, to_f64

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TIE_BAND = 1e-5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mtp.load()


def _say(*a):
    print(*a, flush=True)


def _np(idx, val, draft, positions=None):
    i, v, d = idx.cpu().numpy().astype(np.int64), val.cpu().numpy().astype(np.float64), to_f64(draft)
    if positions is not None:
        i, v, d = i[positions], v[positions], d[positions]
    return i, v, d


def _softmax(d):
    with np.errstate(invalid="ignore"):   # a row of -inf gives NaN, as the oracle's
        m = d.max(-1, keepdims=True)
        return np.exp(d - m - np.log(np.sum(np.exp(d - m), -1, keepdims=True)))


def _tie_mass(i, v, d):
    """Per row: the draft mass at entries whose indicator is within TIE_BAND of
    flipping (S may differ from the oracle's by up to it), and the per-element
    tie mask of the gradient (elements that are such an entry)."""
    margin = omtp.tv_topk_indicator_margin(i, v, d)
    q = _softmax(d)
    T, G, V = d.shape
    ib = np.broadcast_to(i[:, None, :], (T, G, i.shape[-1])) if i.ndim == 2 else i
    ok = (ib >= 0) & (ib < V)
    qi = np.where(ok, np.take_along_axis(q, np.where(ok, ib, 0), -1), 0.0)
    tie = margin < TIE_BAND
    elem_tie = np.zeros((T, G, V), bool)
    for t in range(T):
        for k in range(G):
            elem_tie[t, k, ib[t, k][tie[t, k] & ok[t, k]]] = True
    return np.where(tie, qi, 0.0).sum(-1), elem_tie, q


def _check_forward(idx, val, draft, loss, pos, saved, dtype, positions=None):
    i, v, d = _np(idx, val, draft, positions)
    ref_loss, ref_pos, ref_saved = omtp.tv_topk_loss(i, v, d)
    tie_mass, _, _ = _tie_mass(i, v, d)
    sv = saved.cpu().numpy().astype(np.float64)
    ps = pos.cpu().numpy().astype(np.float64)
    if positions is not None:
        sv, ps = sv[positions], ps[positions]
    for c, name in enumerate(("lse_A", "lse_q", "alpha", "S")):
        a, r = sv[..., c], ref_saved[..., c]
        nonfinite = ~np.isfinite(a) & ~np.isfinite(r)
        d_ = np.abs(a - r)
        if name.startswith("lse"):
            ok = d_ <= 1e-6 * np.abs(r) + 1e-5
        elif name == "S":
            ok = stat_close(a, r, dtype) | (d_ <= tie_mass * (1 + 1e-3) + 1e-6)
        else:
            ok = stat_close(a, r, dtype)
        assert (ok | nonfinite).all(), f"saved {name}: max err {np.nanmax(d_)}"
    okp = stat_close(ps, ref_pos, dtype) | (np.isnan(ps) & np.isnan(ref_pos))
    assert okp.all(), f"pos_loss max err {np.nanmax(np.abs(ps - ref_pos))}"
    if positions is None:
        assert (stat_close(loss.cpu().numpy(), [ref_loss], dtype) | (np.isnan(loss.cpu().numpy()) & np.isnan(ref_loss))).all()
    return ref_saved


def _check_backward(idx, val, draft, saved, g, gb, gf, positions=None):
    i, v, d = _np(idx, val, draft, positions)
    if positions is not None:
        gb, gf = gb[positions], gf[positions]
    gs = g * d.shape[0] / saved.shape[0]
    ref = omtp.tv_topk_loss_grad(i, v, d, gs)
    tie_mass, elem_tie, q = _tie_mass(i, v, d)
    _, _, ref_saved = omtp.tv_topk_loss(i, v, d)
    w = omtp.e2e_weights(ref_saved[:, :, 2], gs, d.shape[0])
    slack = np.abs(w)[..., None] * q * tie_mass[..., None] * 1.01
    gbf = to_f64(gb)
    # excluded: elements at a tied entry, and elements within the slack of an S shift
    margin = np.where(elem_tie | (np.abs(gbf - ref) <= slack), 0.0, 1.0)
    ties = compare_grad_bf16(gb, ref, margin, TIE_BAND)
    g32 = gf.cpu().numpy().astype(np.float64)
    err = np.where(elem_tie, 0.0, np.maximum(np.abs(g32 - ref) - slack, 0.0))
    den = np.linalg.norm(np.where(elem_tie, 0.0, ref), axis=-1)
    rel = np.linalg.norm(err, axis=-1) / np.maximum(den, 1e-30)
    assert (rel <= 1e-3).all(), f"float32 gradient rel err {rel.max()}"
    return ties


def _run(idx, val, draft, g=1.0):
    loss, pos, saved = mtp.tv_topk_fwd(idx, val, draft)
    gl = torch.tensor([g], dtype=torch.float32, device=DEV)
    gb = mtp.tv_topk_bwd(idx, val, draft, saved, gl, grad_dtype=torch.bfloat16)
    gf = mtp.tv_topk_bwd(idx, val, draft, saved, gl, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    return loss, pos, saved, gb, gf


@pytest.mark.parametrize("seed", range(4))
def test_tiny_float32(seed):
    w = synthetic.TV_WORKLOADS["tiny"]
    i, v, d = synthetic.topk_inputs(w, 64, DEV, seed=seed)
    _say("topk tiny seed", seed)
    loss, pos, saved, gb, gf = _run(i, v, d, g=1.0 + 0.2 * seed)
    _check_forward(i, v, d, loss, pos, saved, torch.float32)
    _check_backward(i, v, d, saved, 1.0 + 0.2 * seed, gb, gf)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shared", [True, False])
@pytest.mark.parametrize("T,G,V,K", [(1, 1, 7, 3), (5, 3, 1000, 50), (3, 4, 8200, 300), (6, 3, 50003, 1000),
                                     (2, 8, 20000, 17), (4, 2, 1, 1)])
def test_ragged(T, G, V, K, shared, dtype):
    w = dict(T=T, G=G, V=V, dtype=dtype, scale=1.2, sigma=0.3, shared=shared, seed=5)
    i, v, d = synthetic.topk_inputs(w, K, DEV, seed=T * 7 + V)
    if V % (16 // d.element_size()):   # rows must start 16-byte aligned: pad the vocabulary
        pv = 16 // d.element_size()
        dp = torch.full((T, G, V + (-V) % pv), float("-inf"), dtype=dtype, device=DEV)
        dp[..., :V] = d
        d = dp[..., :V]
    _say("topk ragged", T, G, V, K, shared, dtype)
    loss, pos, saved = mtp.tv_topk_fwd(i, v, d)
    gl = torch.tensor([0.7], dtype=torch.float32, device=DEV)
    pad = (-V) % 8                      # gradient rows 16-byte aligned for both dtypes
    gpad = torch.zeros((T, G, V + pad), dtype=torch.bfloat16, device=DEV)
    gfpad = torch.zeros((T, G, V + pad), dtype=torch.float32, device=DEV)
    gb = mtp.tv_topk_bwd(i, v, d, saved, gl, out=gpad[..., :V])
    gf = mtp.tv_topk_bwd(i, v, d, saved, gl, out=gfpad[..., :V])
    torch.cuda.synchronize()
    _check_forward(i, v, d, loss, pos, saved, dtype)
    _check_backward(i, v, d, saved, 0.7, gb, gf)
    if pad:   # nothing written past the vocabulary
        assert (gpad[..., V:] == 0).all() and (gfpad[..., V:] == 0).all()


def test_k_equal_v_is_the_full_vocabulary_path():
    w = dict(T=4, G=3, V=12000, dtype=torch.bfloat16, scale=1.2, sigma=0.3, shared=True, seed=6)
    t, d = synthetic.tv_inputs(w, DEV)
    val, idx = torch.sort(t.float(), dim=-1, descending=True)
    idx = idx.to(torch.int32).contiguous()
    loss, pos, saved, gb, gf = _run(idx, val.contiguous(), d)
    floss, fpos, fsaved = mtp.tv_loss_fwd(t, d)
    fgf = mtp.tv_loss_bwd(t, d, fsaved, torch.ones(1, device=DEV), grad_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.allclose(saved[..., 1:], fsaved[..., 1:], rtol=1e-5, atol=1e-6)
    assert torch.allclose(pos, fpos, rtol=1e-5, atol=1e-6)
    rel = (gf - fgf).norm(dim=-1) / fgf.norm(dim=-1)
    assert rel.max().item() < 1e-4
    _check_forward(idx, val, d, loss, pos, saved, torch.bfloat16)


def test_out_of_range_repeated_and_masked_entries():
    T, G, V, K = 3, 3, 9000, 40
    w = dict(T=T, G=G, V=V, dtype=torch.bfloat16, scale=1.2, sigma=0.3, shared=False, seed=7)
    i, v, d = synthetic.topk_inputs(w, K, DEV)
    i[0, 0, 3], i[0, 1, 7], i[2, 2, 0] = -5, V, 1 << 30       # out of range: no mass
    i[1, 0, 5] = i[1, 0, 6]                                    # a repeated index
    i[1, 1, 2], i[1, 1, 9] = 4095, 4095
    v[2, 0, 4] = float("-inf")                                 # an entry without mass
    loss, pos, saved, gb, gf = _run(i, v, d, g=1.1)
    _check_forward(i, v, d, loss, pos, saved, torch.bfloat16)
    _check_backward(i, v, d, saved, 1.1, gb, gf)


def test_rows_without_a_finite_normaliser():
    T, G, V, K = 2, 2, 5000, 8
    w = dict(T=T, G=G, V=V, dtype=torch.float32, scale=1.0, sigma=0.3, shared=False, seed=8)
    i, v, d = synthetic.topk_inputs(w, K, DEV)
    i[0, 1, :] = -1                      # no entry in range
    d[1, 0, :] = float("-inf")           # a draft row without mass
    loss, pos, saved, gb, gf = _run(i, v, d)
    sv = saved.cpu()
    assert torch.isnan(sv[0, 1, 2]) and torch.isnan(sv[1, 0, 2])
    assert torch.isfinite(sv[0, 0, 2]) and torch.isfinite(sv[1, 1, 2])
    assert torch.isnan(loss).all()
    _check_forward(i, v, d, loss, pos, saved, torch.float32)


def test_bench_workload_sampled_positions():
    w = synthetic.TV_WORKLOADS["tv_loss"]
    i, v, d = synthetic.topk_inputs(w, 256, DEV)
    _say("topk full workload", tuple(d.shape))
    loss, pos, saved, gb, gf = _run(i, v, d)
    positions = [0, 1, 2047, 4096, 8191]
    _check_forward(i, v, d, loss, pos, saved, torch.bfloat16, positions)
    _check_backward(i, v, d, saved, 1.0, gb, gf, positions)
    assert torch.isfinite(loss).all()
    del gb, gf, d
    torch.cuda.empty_cache()


def test_autograd_wrapper():
    w = dict(T=6, G=3, V=30000, dtype=torch.float32, scale=1.2, sigma=0.3, shared=True, seed=9)
    i, v, d = synthetic.topk_inputs(w, 100, DEV)
    z = d.clone().requires_grad_(True)
    L = mtp.tv_topk_loss(z, i, v)
    (2.5 * L).backward()
    _, _, saved = mtp.tv_topk_fwd(i, v, d)
    ref = mtp.tv_topk_bwd(i, v, d, saved, torch.tensor([2.5], device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(z.grad, ref)


def test_plan_matches_the_functional_calls():
    w = dict(synthetic.TV_WORKLOADS["tv_loss"], T=16, V=20000)
    i, v, d = synthetic.topk_inputs(w, 128, DEV, seed=3)
    plan = mtp.TVTopKPlan(i, v, d, grad_dtype=torch.bfloat16)
    loss, pos, saved = mtp.tv_topk_fwd(i, v, d)
    g = mtp.tv_topk_bwd(i, v, d, saved, torch.ones(1, device=DEV), grad_dtype=torch.bfloat16)
    plan.forward()
    plan.backward()
    torch.cuda.synchronize()
    assert torch.equal(plan.saved, saved) and torch.equal(plan.loss, loss)
    assert torch.equal(plan.grad, g)
