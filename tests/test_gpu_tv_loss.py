"""GPU parity of mtp_tv_loss_fwd / mtp_tv_loss_bwd against the float64 oracle.

Forward: loss, per-position loss and the saved statistics (lse_p, lse_q, alpha, S)
within the statistic tolerances.  Backward: the bfloat16 gradient within 1 bf16
ulp of the oracle's value rounded to nearest even (indicator near-ties excepted),
and the float32 gradient within 1e-3 norm-relative per (position, head) row.
Sizes: the tiny float32 workload, ragged vocabularies over several chunks, shared
and per-head targets, and 256 sampled positions of the full T = 8192 workload
(with properties checked at every position).
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


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mtp.load()


def _say(*a):
    print(*a, flush=True)


TIE_BAND = 1e-5   # |log q - log p| below which a float32 indicator may flip


def _tie_mass(tf, df):
    """Per (position, head): the draft mass q of elements whose indicator is within
    TIE_BAND of flipping.  A float32 evaluation may count them on either side, so S
    may legitimately differ from the oracle's by up to this mass."""
    margin = omtp.indicator_margin(tf, df)
    q = np.exp(df - np.log(np.sum(np.exp(df - df.max(-1, keepdims=True)), -1, keepdims=True))
               - df.max(-1, keepdims=True))
    return margin, q, np.where(margin < TIE_BAND, q, 0.0).sum(-1)


def _check_forward(target, draft, loss, pos, saved, dtype, positions=None):
    tf, df = to_f64(target), to_f64(draft)
    if positions is not None:
        tf, df = tf[positions], df[positions]
    ref_loss, ref_pos, ref_saved = omtp.tv_loss(tf, df)
    _, _, tie_mass = _tie_mass(tf, df)
    sv = saved.cpu().numpy().astype(np.float64)
    ps = pos.cpu().numpy().astype(np.float64)
    if positions is not None:
        sv, ps = sv[positions], ps[positions]
    for i, name in enumerate(("lse_p", "lse_q", "alpha", "S")):
        d = np.abs(sv[..., i] - ref_saved[..., i])
        if name.startswith("lse"):   # compare log-sum-exp relative to its size
            ok = d <= 1e-6 * np.abs(ref_saved[..., i]) + 1e-5
        elif name == "S":
            ok = stat_close(sv[..., i], ref_saved[..., i], dtype) | (d <= tie_mass * (1 + 1e-3) + 1e-6)
        else:
            ok = stat_close(sv[..., i], ref_saved[..., i], dtype)
        assert ok.all(), f"saved {name}: max err {d.max()}"
    assert stat_close(ps, ref_pos, dtype).all(), f"pos_loss max err {np.abs(ps - ref_pos).max()}"
    if positions is None:
        assert stat_close(loss.cpu().numpy(), [ref_loss], dtype).all()
    return ref_saved


def _check_backward(target, draft, saved, g, grad_bf16, grad_f32, positions=None):
    tf, df = to_f64(target), to_f64(draft)
    if positions is not None:
        tf, df = tf[positions], df[positions]
        grad_bf16, grad_f32 = grad_bf16[positions], grad_f32[positions]
    # The oracle's gradient for the sampled positions, scaled as in the full mean.
    T_full = saved.shape[0]
    gs = g * tf.shape[0] / T_full
    ref = omtp.tv_loss_grad(tf, df, gs)
    margin, q, tie_mass = _tie_mass(tf, df)
    _, _, ref_saved = omtp.tv_loss(tf, df)
    w = omtp.e2e_weights(ref_saved[:, :, 2], gs, tf.shape[0])
    # a shift of S by up to the tie mass moves every element by up to |w| q tie_mass
    slack = np.abs(w)[..., None] * q * tie_mass[..., None] * 1.01
    gb = to_f64(grad_bf16)
    ties = compare_grad_bf16(grad_bf16, ref, np.where(np.abs(gb - ref) <= slack, 0.0, margin), TIE_BAND)
    gf = grad_f32.cpu().numpy().astype(np.float64)
    err = np.where(margin < TIE_BAND, 0.0, np.maximum(np.abs(gf - ref) - slack, 0.0))
    den = np.linalg.norm(np.where(margin < TIE_BAND, 0.0, ref), axis=-1)
    rel = np.linalg.norm(err, axis=-1) / np.maximum(den, 1e-30)
    assert (rel <= 1e-3).all(), f"float32 gradient rel err {rel.max()}"
    # sum_v q_v (1[q_v <= p_v] - S) = S - S = 0: every gradient row sums to zero, up
    # to the mass of elements whose indicator the gradient's evaluation may decide
    # otherwise than the one that produced the saved S
    rs = np.abs(gf.sum(-1))
    assert (rs <= 1e-4 * np.abs(gf).sum(-1) + np.abs(w) * tie_mass * 1.01 + 1e-12).all(), \
        f"gradient row sums {rs.max()}"
    return ties


def _run(target, draft, g=1.0):
    loss, pos, saved = mtp.tv_loss_fwd(target, draft)
    gl = torch.tensor([g], dtype=torch.float32, device=DEV)
    gb = mtp.tv_loss_bwd(target, draft, saved, gl, grad_dtype=torch.bfloat16)
    gf = mtp.tv_loss_bwd(target, draft, saved, gl, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    return loss, pos, saved, gb, gf


@pytest.mark.parametrize("seed", range(6))
def test_tiny_float32(seed):
    w = synthetic.TV_WORKLOADS["tiny"]
    t, d = synthetic.tv_inputs(w, DEV, seed=seed)
    _say("tiny tv seed", seed)
    loss, pos, saved, gb, gf = _run(t, d, g=1.0 + 0.1 * seed)
    _check_forward(t, d, loss, pos, saved, torch.float32)
    _check_backward(t, d, saved, 1.0 + 0.1 * seed, gb, gf)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shared", [True, False])
@pytest.mark.parametrize("T,G,V", [(1, 1, 7), (5, 3, 1000), (3, 4, 8200), (17, 3, 50003), (2, 8, 20000),
                                   (4, 2, 1)])
def test_ragged(T, G, V, shared, dtype):
    w = dict(T=T, G=G, V=V, dtype=dtype, scale=1.2, sigma=0.3, shared=shared, seed=3)
    t, d = synthetic.tv_inputs(w, DEV, seed=T * 100 + V)
    pad = (-V) % 8
    if pad:
        tp = torch.zeros(t.shape[:-1] + (V + pad,), dtype=dtype, device=DEV)
        dp = torch.zeros(d.shape[:-1] + (V + pad,), dtype=dtype, device=DEV)
        tp[..., :V] = t
        dp[..., :V] = d
        t, d = tp[..., :V], dp[..., :V]
    _say("tv ragged", T, G, V, shared, dtype)
    loss, pos, saved = mtp.tv_loss_fwd(t, d)
    gl = torch.tensor([0.7], dtype=torch.float32, device=DEV)
    gpad = torch.zeros((T, G, V + pad), dtype=torch.bfloat16, device=DEV)
    gfpad = torch.zeros((T, G, V + pad), dtype=torch.float32, device=DEV)
    gb = mtp.tv_loss_bwd(t, d, saved, gl, out=gpad[..., :V])
    gf = mtp.tv_loss_bwd(t, d, saved, gl, out=gfpad[..., :V])
    torch.cuda.synchronize()
    _check_forward(t, d, loss, pos, saved, dtype)
    _check_backward(t, d, saved, 0.7, gb, gf)
    if pad:   # nothing written past the vocabulary
        assert (gpad[..., V:] == 0).all() and (gfpad[..., V:] == 0).all()


def _check_all_positions(loss, pos, saved):
    """Properties of every position of a call: 0 <= S <= alpha <= 1 (S sums q over
    the elements where q < p, each at most min(p, q)), finite normalisers, the
    position loss is -sum_k prod_{j<=k} alpha_j of its saved overlaps, and the loss
    is the mean of the position losses."""
    sv = saved.double().cpu().numpy()
    a, S = sv[..., 2], sv[..., 3]
    assert np.isfinite(sv[..., :2]).all()
    assert (S >= 0).all() and (a <= 1 + 1e-6).all() and (S <= a + 1e-6).all()
    expect = -np.cumprod(a, axis=1).sum(axis=1)
    p = pos.double().cpu().numpy()
    np.testing.assert_allclose(p, expect, rtol=1e-5, atol=1e-6)
    assert abs(loss.item() - p.mean()) <= 1e-6 * abs(p.mean()) + 1e-7


def test_full_workload_sampled_positions():
    w = synthetic.TV_WORKLOADS["tv_loss"]
    t, d = synthetic.tv_inputs(w, DEV)
    _say("tv full workload")
    loss, pos, saved, gb, gf = _run(t, d, g=1.0)
    # 256 positions against the oracle: both ends, the middle and a seeded sample
    rng = np.random.default_rng(123)
    fixed = [0, 1, 2, 1000, 4095, 4096, 8190, 8191]
    positions = sorted(fixed + rng.choice(np.setdiff1d(np.arange(8192), fixed), 248, replace=False).tolist())
    ref_saved = _check_forward(t, d, loss, pos, saved, torch.bfloat16, positions)
    ties = _check_backward(t, d, saved, 1.0, gb, gf, positions)
    _check_all_positions(loss, pos, saved)
    _say("alpha per head:", ref_saved[:, :, 2].mean(0), "indicator ties:", ties)


def test_identical_heads_give_zero_gradient():
    V, T, G = 30000, 3, 3
    g = torch.Generator(device=DEV).manual_seed(5)
    t = torch.randn((T, V), generator=g, device=DEV).to(torch.bfloat16)
    d = t[:, None, :].expand(T, G, V).contiguous()
    loss, pos, saved, gb, gf = _run(t, d)
    assert torch.allclose(saved[:, :, 2], torch.ones_like(saved[:, :, 2]), atol=1e-3)
    assert abs(loss.item() + G) < 3e-3
    # every indicator is 1 and S = sum q, so the gradient is q (1 - S) ~ 1e-7 q
    qmax = gf.abs().max().item()
    assert qmax < 1e-5, qmax


def test_autograd_function_matches_explicit_backward():
    w = synthetic.TV_WORKLOADS["tiny"]
    t, d = synthetic.tv_inputs(w, DEV, seed=9)
    z = d.clone().requires_grad_(True)
    loss = mtp.tv_loss(z, t)
    (2.5 * loss).backward()
    _, _, saved = mtp.tv_loss_fwd(t, d)
    ref = mtp.tv_loss_bwd(t, d, saved, torch.tensor([2.5], device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(z.grad, ref)


def test_forward_is_deterministic_and_reuses_workspace():
    w = synthetic.TV_WORKLOADS["tv_loss"]
    t, d = synthetic.tv_inputs(w, DEV, T=256)
    small = synthetic.tv_inputs(dict(w, shared=False), DEV, T=5, V=5000)
    a = mtp.tv_loss_fwd(t, d)
    for _ in range(5):
        mtp.tv_loss_fwd(*small)
        b = mtp.tv_loss_fwd(t, d)
        for x, y in zip(a, b):
            assert torch.equal(x, y)
    torch.cuda.synchronize()
    assert mtp.workspace_error(mtp.workspace(DEV, 1)) == 0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_largest_vocabulary_closed_form(dtype):
    """V = 2^30 (the largest the API takes; a float32 row spans 4 GiB), T = 1,
    gamma = 1: a uniform target and a draft that is uniform but for its last logit,
    a = 30 (so that a misread last element would change every statistic).  With
    n = V - 1 + e^a: q_o = 1/n < 1/V < q_j = e^a/n, alpha = (V - 1)/n + 1/V,
    S = (V - 1)/n, lse_p = ln V, lse_q = ln n, and the gradient (g = 1) is
    -q_o (1 - S) off j and q_j S at j."""
    V, a = 1 << 30, 30.0
    j = V - 1
    t = torch.zeros((1, V), dtype=dtype, device=DEV)
    d = torch.zeros((1, 1, V), dtype=dtype, device=DEV)
    d[0, 0, j] = a
    _say("tv largest vocabulary", dtype)
    loss, pos, saved = mtp.tv_loss_fwd(t, d)
    g = mtp.tv_loss_bwd(t, d, saved, torch.ones(1, device=DEV), grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    n = (V - 1) + np.exp(a)
    alpha, S = (V - 1) / n + 1 / V, (V - 1) / n
    sv = saved[0, 0].double().cpu().numpy()
    assert abs(sv[0] - np.log(V)) < 1e-6 * np.log(V)
    assert abs(sv[1] - np.log(n)) < 1e-6 * np.log(n)
    assert abs(sv[2] - alpha) < 1e-4 * alpha and abs(sv[3] - S) < 1e-4 * S
    assert abs(loss.item() + alpha) < 1e-4 * alpha
    qo, qj = 1 / n, np.exp(a) / n
    for v, ref in ((0, -qo * (1 - S)), (j - 1, -qo * (1 - S)), (V // 2, -qo * (1 - S)), (j, qj * S)):
        got = g[0, 0, v].double().item()
        assert abs(got - ref) <= 2 ** -7 * abs(ref), (v, got, ref)
    del t, d, g
    torch.cuda.empty_cache()


@pytest.mark.parametrize("extra", [0, 8])
def test_single_read_forward_at_the_co_residency_limit(extra):
    """The single-read forward holds every chunk of a row on chip at once: the
    largest vocabulary it takes is (co-resident workgroups) x 4096 bf16 logits, one
    super-group for the whole call.  At that vocabulary it runs with a single
    super-group; one vector more falls back to the two streaming passes.  Both must
    match the oracle, and no bounded wait may time out."""
    props = torch.cuda.get_device_properties(0)
    V = 2 * props.multi_processor_count * 4096 + extra
    w = dict(T=2, G=3, V=V, dtype=torch.bfloat16, scale=1.25, sigma=0.3, shared=True, seed=6)
    t, d = synthetic.tv_inputs(w, DEV)
    _say("tv co-residency limit", V)
    loss, pos, saved, gb, gf = _run(t, d, g=1.0)
    _check_forward(t, d, loss, pos, saved, torch.bfloat16)
    _check_backward(t, d, saved, 1.0, gb, gf)
    assert mtp.workspace_error(mtp.workspace(DEV, 1)) == 0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shared,G", [(True, 3), (False, 2), (False, 3)])
def test_masked_supports(shared, G, dtype):
    """-inf logits (masking) on both sides: partly overlapping windows, equal
    supports, a head disjoint from the target (alpha = 0, S = 0, zero gradient),
    a narrow target window (most wave segments hold no target mass) and narrow
    draft windows (most hold no draft mass).  shared gamma = 3 and per-head gamma = 2
    take the single-read forward, per-head gamma = 3 the two streaming passes."""
    T, V = 4, 50000
    w = dict(T=T, G=G, V=V, dtype=dtype, scale=1.2, sigma=0.3, shared=shared, seed=11)
    t, d = synthetic.tv_inputs(w, DEV, seed=77)
    t, d = t.clone(), d.clone()
    ninf = float("-inf")

    def keep(x, lo, hi):   # mask a row outside [lo, hi)
        x[..., :lo] = ninf
        x[..., hi:] = ninf

    tgt = (lambda pos: [t[pos]]) if shared else (lambda pos: [t[pos, k] for k in range(G)])
    for row in tgt(0):
        keep(row, 1000, 30000)
    keep(d[0, 0], 20000, 45000)           # partial overlap
    keep(d[0, 1], 1000, 30000)            # the target's support
    if G > 2:
        keep(d[0, 2], 35000, V)           # disjoint from the target
    for row in tgt(1):
        keep(row, 12345, 12845)           # narrow target window
    for k in range(G):
        keep(d[2, k], 7000 + 3000 * k, 7300 + 3000 * k)   # narrow draft windows
    _say("tv masked supports", shared, G, dtype)
    loss, pos, saved, gb, gf = _run(t, d, g=0.9)
    ref_saved = _check_forward(t, d, loss, pos, saved, dtype)
    _check_backward(t, d, saved, 0.9, gb, gf)
    if G > 2:   # the disjoint head
        assert saved[0, 2, 2].item() == 0.0 and saved[0, 2, 3].item() == 0.0
        assert ref_saved[0, 2, 2] == 0.0
        assert (gf[0, 2] == 0).all() and (gb[0, 2] == 0).all()
    # masked draft elements get no gradient
    dm = torch.isinf(d.float())
    assert (gf[dm] == 0).all() and (gb[dm] == 0).all()


@pytest.mark.parametrize("shared,G", [(True, 3), (False, 3)])
def test_position_without_a_finite_target_normaliser(shared, G):
    """A target row of -inf only has no normaliser: its position's statistics are
    NaN (a data error), and every other position still matches the oracle."""
    T, V = 5, 20000
    w = dict(T=T, G=G, V=V, dtype=torch.bfloat16, scale=1.2, sigma=0.3, shared=shared, seed=12)
    t, d = synthetic.tv_inputs(w, DEV, seed=78)
    t = t.clone()
    t[2] = float("-inf")
    loss, pos, saved = mtp.tv_loss_fwd(t, d)
    torch.cuda.synchronize()
    sv = saved.cpu()
    assert torch.isnan(sv[2, :, 2]).all() and torch.isnan(sv[2, :, 3]).all()
    assert torch.isnan(pos[2]).item() and torch.isnan(loss).item()
    keep = [0, 1, 3, 4]
    tf, df = to_f64(t)[keep], to_f64(d)[keep]
    _, ref_pos, ref_saved = omtp.tv_loss(tf, df)
    for i in (2, 3):
        assert stat_close(sv[keep][..., i].double().numpy(), ref_saved[..., i], torch.bfloat16).all()
    assert stat_close(pos.cpu()[keep].double().numpy(), ref_pos, torch.bfloat16).all()
    assert mtp.workspace_error(mtp.workspace(DEV, 1)) == 0
