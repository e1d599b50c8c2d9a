"""GPU parity of mtp_tv_loss_fwd_bwd (forward and backward in one sweep) against
the float64 oracle, with the tolerances of the separate calls: loss, per-position
loss and saved statistics as the forward's; the bfloat16 gradient within 1 bf16 ulp
of the oracle's RNE value and the float32 gradient within 1e-3 norm-relative per
row, indicator near-ties excepted.  Sizes: the tiny float32 workload, ragged
vocabularies over several chunks (rows padded past V with a large finite logit,
so an over-read would show, and gradient padding that must stay untouched),
shared and per-head targets (shapes the one-sweep kernel does not take go through
the forward and backward calls), masked supports with a head disjoint from the
target, identical heads, 256 sampled positions of the full T = 8192 workload,
and repeated calls on one workspace."""
import numpy as np
import pytest
import torch

import synthetic
import tv_loss_amd as mtp
from test_gpu_tv_loss import _check_all_positions, _check_backward, _check_forward

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PAD_LOGIT = 30.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mtp.load()


def _say(*a):
    print(*a, flush=True)


def _run(t, d, g, outs=None):
    gl = torch.tensor([g], dtype=torch.float32, device=DEV)
    ob, of = outs if outs else (None, None)
    loss, pos, saved, gb = mtp.tv_loss_fwd_bwd(t, d, gl, grad_dtype=torch.bfloat16, out=ob)
    loss2, pos2, saved2, gf = mtp.tv_loss_fwd_bwd(t, d, gl, grad_dtype=torch.float32, out=of)
    torch.cuda.synchronize()
    # the float32-gradient call computed the same forward (bit for bit when both calls
    # take the same path; gamma = 1 with bf16 logits and gradient takes the two calls)
    assert torch.allclose(torch.nan_to_num(saved), torch.nan_to_num(saved2), rtol=1e-6, atol=1e-7)
    return loss, pos, saved, gb, gf


@pytest.mark.parametrize("seed", range(4))
def test_tiny_float32(seed):
    w = synthetic.TV_WORKLOADS["tiny"]
    t, d = synthetic.tv_inputs(w, DEV, seed=seed)
    _say("fused tiny seed", seed)
    g = 1.0 + 0.1 * seed
    loss, pos, saved, gb, gf = _run(t, d, g)
    _check_forward(t, d, loss, pos, saved, torch.float32)
    _check_backward(t, d, saved, g, gb, gf)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shared", [True, False])
@pytest.mark.parametrize("T,G,V", [(1, 1, 7), (5, 3, 1000), (3, 4, 8200), (17, 3, 50003), (2, 5, 20000),
                                   (4, 2, 1), (9, 2, 151939)])
def test_ragged(T, G, V, shared, dtype):
    w = dict(T=T, G=G, V=V, dtype=dtype, scale=1.2, sigma=0.3, shared=shared, seed=3)
    t, d = synthetic.tv_inputs(w, DEV, seed=T * 100 + V + 7)
    pv = 16 // t.element_size()
    pad = (-V) % pv
    if pad:
        tp = torch.full(t.shape[:-1] + (V + pad,), PAD_LOGIT, dtype=dtype, device=DEV)
        dp = torch.full(d.shape[:-1] + (V + pad,), PAD_LOGIT, dtype=dtype, device=DEV)
        tp[..., :V] = t
        dp[..., :V] = d
        t, d = tp[..., :V], dp[..., :V]
    gpad = torch.zeros((T, G, (V + 7) // 8 * 8 + 8), dtype=torch.bfloat16, device=DEV)
    gfpad = torch.zeros((T, G, (V + 3) // 4 * 4 + 4), dtype=torch.float32, device=DEV)
    _say("fused ragged", T, G, V, shared, dtype)
    loss, pos, saved, gb, gf = _run(t, d, 0.7, (gpad[..., :V], gfpad[..., :V]))
    _check_forward(t, d, loss, pos, saved, dtype)
    _check_backward(t, d, saved, 0.7, gb, gf)
    assert (gpad[..., V:] == 0).all() and (gfpad[..., V:] == 0).all()


def test_full_workload_sampled_positions():
    w = synthetic.TV_WORKLOADS["tv_loss"]
    t, d = synthetic.tv_inputs(w, DEV)
    _say("fused full workload")
    loss, pos, saved, gb, gf = _run(t, d, 1.0)
    rng = np.random.default_rng(321)
    fixed = [0, 1, 2, 4095, 4096, 8190, 8191]
    positions = sorted(fixed + rng.choice(np.setdiff1d(np.arange(8192), fixed), 249, replace=False).tolist())
    _check_forward(t, d, loss, pos, saved, torch.bfloat16, positions)
    ties = _check_backward(t, d, saved, 1.0, gb, gf, positions)
    _check_all_positions(loss, pos, saved)
    # every gradient row sums to zero (sum_v q_v (1[q_v < p_v] - S) = S - S)
    for s in range(0, gf.shape[0], 1024):
        rows = gf[s:s + 1024].double()
        assert (rows.sum(-1).abs() <= 1e-4 * rows.abs().sum(-1)).all()
    _say(len(positions), "positions checked; indicator ties", ties)


def test_matches_the_separate_calls_within_tolerance():
    w = dict(synthetic.TV_WORKLOADS["tv_loss"], T=64)
    t, d = synthetic.tv_inputs(w, DEV, seed=9)
    loss, pos, saved, gb, gf = _run(t, d, 1.3)
    loss2, pos2, saved2 = mtp.tv_loss_fwd(t, d)
    torch.cuda.synchronize()
    assert torch.allclose(saved[..., :3], saved2[..., :3], atol=1e-5, rtol=1e-5)
    assert abs(loss.item() - loss2.item()) < 1e-5


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shared,G", [(True, 3), (False, 2), (False, 3)])
def test_masked_supports_and_a_disjoint_head(shared, G, dtype):
    """-inf logits on both sides: overlapping and equal windows, a head disjoint from
    the target (alpha = S = 0 and a zero gradient, exactly), narrow target and
    draft windows; masked draft elements get no gradient."""
    T, V = 4, 50000
    w = dict(T=T, G=G, V=V, dtype=dtype, scale=1.2, sigma=0.3, shared=shared, seed=11)
    t, d = synthetic.tv_inputs(w, DEV, seed=77)
    t, d = t.clone(), d.clone()
    ninf = float("-inf")

    def keep(x, lo, hi):
        x[..., :lo] = ninf
        x[..., hi:] = ninf

    tgt = (lambda pos: [t[pos]]) if shared else (lambda pos: [t[pos, k] for k in range(G)])
    for row in tgt(0):
        keep(row, 1000, 30000)
    keep(d[0, 0], 20000, 45000)
    keep(d[0, 1], 1000, 30000)
    if G > 2:
        keep(d[0, 2], 35000, V)
    for row in tgt(1):
        keep(row, 12345, 12845)
    for k in range(G):
        keep(d[2, k], 7000 + 3000 * k, 7300 + 3000 * k)
    _say("fused masked supports", shared, G, dtype)
    loss, pos, saved, gb, gf = _run(t, d, 0.9)
    _check_forward(t, d, loss, pos, saved, dtype)
    _check_backward(t, d, saved, 0.9, gb, gf)
    if G > 2:
        assert saved[0, 2, 2].item() == 0.0 and saved[0, 2, 3].item() == 0.0
        assert (gf[0, 2] == 0).all() and (gb[0, 2] == 0).all()
    dm = torch.isinf(d.float())
    assert (gf[dm] == 0).all() and (gb[dm] == 0).all()


@pytest.mark.parametrize("extra", [0, 8])
def test_at_the_co_residency_limit(extra):
    """The one-sweep kernel holds every chunk of a row on chip: at (co-resident
    workgroups) x 4096 bf16 logits it runs as one super-group; one vector more
    goes through the forward and backward calls.  Both match the oracle."""
    props = torch.cuda.get_device_properties(0)
    V = 2 * props.multi_processor_count * 4096 + extra
    w = dict(T=2, G=3, V=V, dtype=torch.bfloat16, scale=1.25, sigma=0.3, shared=True, seed=6)
    t, d = synthetic.tv_inputs(w, DEV)
    _say("fused co-residency limit", V)
    loss, pos, saved, gb, gf = _run(t, d, 1.0)
    _check_forward(t, d, loss, pos, saved, torch.bfloat16)
    _check_backward(t, d, saved, 1.0, gb, gf)


def test_identical_heads_give_zero_gradient():
    V, T, G = 30000, 3, 3
    g = torch.Generator(device=DEV).manual_seed(5)
    t = torch.randn((T, V), generator=g, device=DEV).to(torch.bfloat16)
    d = t[:, None, :].expand(T, G, V).contiguous()
    loss, pos, saved, gb, gf = _run(t, d, 1.0)
    assert torch.allclose(saved[:, :, 2], torch.ones_like(saved[:, :, 2]), atol=1e-3)
    assert (saved[:, :, 3] > 1 - 1e-3).all()
    assert gf.abs().max().item() < 1e-5


def test_repeated_calls_are_deterministic_and_leave_the_workspace_clean():
    w = dict(synthetic.TV_WORKLOADS["tv_loss"], T=40, V=70000)
    t, d = synthetic.tv_inputs(w, DEV, seed=5)
    first = _run(t, d, 1.0)
    small = dict(synthetic.TV_WORKLOADS["tv_loss"], T=3, V=9000)
    ts, ds = synthetic.tv_inputs(small, DEV, seed=6)
    for _ in range(3):
        _run(ts, ds, 2.0)
        again = _run(t, d, 1.0)
        for a, b in zip(first, again):
            assert torch.equal(torch.nan_to_num(a.float()), torch.nan_to_num(b.float()))
    assert mtp.workspace_error(mtp.workspace(DEV, 1)) == 0


def test_plan_matches_the_functional_call():
    w = dict(synthetic.TV_WORKLOADS["tv_loss"], T=16, V=20000)
    t, d = synthetic.tv_inputs(w, DEV, seed=3)
    plan = mtp.TVPlan(t, d, grad_dtype=torch.bfloat16)
    plan.fused()
    loss, pos, saved, g = mtp.tv_loss_fwd_bwd(t, d, torch.ones(1, device=DEV), grad_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(plan.saved, saved) and torch.equal(plan.loss, loss)
    assert torch.equal(plan.grad, g)
