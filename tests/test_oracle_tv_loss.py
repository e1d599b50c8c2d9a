"""Pins for the oracle's end-to-end TV loss and its gradient (oracle/mtp.py):

* closed forms: equal per-step overlaps a give l = -(a + a^2 + ... + a^gamma);
  at gamma = 1 the loss is -alpha = TV - 1 (paperlayer App. F's single-step
  loss 1 - overlap, up to the constant);
* the end-to-end weights against torch autograd of the loss in alpha;
* the gradient against central finite differences of the oracle's own loss
  (float64), and against torch float64 autograd of the plain formula (a library
  differentiation of softmax / min / cumprod);
* invariants from paperlayer App. A: sum_v grad = 0 per row, |grad_v| <= |w| q_v,
  p = q gives a zero gradient, S in [0, 1].
"""
import numpy as np
import pytest
import torch

from oracle import mtp


def _case(seed, T, G, V, shared, sig=0.6, min_margin=1e-3):
    """Random logits whose |log q - log p| stays above min_margin (no indicator
    ties, so finite differences see a smooth loss)."""
    rng = np.random.default_rng(seed)
    while True:
        tgt = rng.normal(0, 1.5, (T, V) if shared else (T, G, V))
        base = tgt[:, None, :] if shared else tgt
        dr = base + rng.normal(0, sig, (T, G, V))
        if mtp.indicator_margin(tgt, dr).min() > min_margin:
            return tgt, dr


def test_closed_form_equal_overlaps():
    rng = np.random.default_rng(0)
    V, G = 300, 3
    t = rng.normal(0, 1, V)
    d = t + rng.normal(0, 0.5, V)
    tgt = np.stack([t, t])                      # [T=2, V], shared by heads
    dr = np.stack([np.stack([d] * G)] * 2)      # identical heads
    loss, pos, saved = mtp.tv_loss(tgt, dr)
    a = saved[0, 0, 2]
    assert np.allclose(saved[:, :, 2], a)
    np.testing.assert_allclose(pos, -(a + a ** 2 + a ** 3), rtol=1e-14)
    assert loss == pytest.approx(-(a + a ** 2 + a ** 3), rel=1e-14)


def test_single_step_is_tv_minus_one():
    rng = np.random.default_rng(1)
    tgt = rng.normal(0, 1, (4, 1, 100))
    dr = tgt + rng.normal(0, 0.7, (4, 1, 100))
    _, pos, saved = mtp.tv_loss(tgt, dr)
    for t in range(4):
        p = np.exp(mtp.log_softmax(tgt[t, 0])[0])
        q = np.exp(mtp.log_softmax(dr[t, 0])[0])
        assert pos[t] == pytest.approx(mtp.tv_distance(p, q) - 1.0, abs=1e-14)


def test_weights_match_autograd():
    rng = np.random.default_rng(2)
    for G in (1, 2, 3, 4, 6):
        alpha = rng.uniform(0, 1, (5, G))
        alpha[0, 0] = 0.0                        # a zero overlap is allowed
        g = 1.7
        a = torch.tensor(alpha, requires_grad=True)
        L = g * (-torch.cumprod(a, dim=1).sum(dim=1)).mean()
        L.backward()
        np.testing.assert_allclose(mtp.e2e_weights(alpha, g, 5), a.grad.numpy(), rtol=1e-13,
                                   atol=1e-15)


@pytest.mark.parametrize("shared", [True, False])
def test_gradient_matches_finite_differences(shared):
    T, G, V = 2, 3, 16
    tgt, dr = _case(3, T, G, V, shared)
    g = 1.3
    grad = mtp.tv_loss_grad(tgt, dr, g)
    h = 1e-6
    num = np.empty_like(dr)
    for idx in np.ndindex(dr.shape):
        zp, zm = dr.copy(), dr.copy()
        zp[idx] += h
        zm[idx] -= h
        num[idx] = g * (mtp.tv_loss(tgt, zp)[0] - mtp.tv_loss(tgt, zm)[0]) / (2 * h)
    # central differences carry a rounding error of about eps * |L| / h ~ 4e-10
    np.testing.assert_allclose(grad, num, rtol=1e-6, atol=2e-9)
    assert np.abs(grad).max() > 1e-3


@pytest.mark.parametrize("shared", [True, False])
def test_gradient_matches_torch_autograd(shared):
    T, G, V = 3, 3, 257
    tgt, dr = _case(4, T, G, V, shared, min_margin=1e-4)
    g = 0.9
    p = torch.softmax(torch.tensor(tgt), dim=-1)
    if shared:
        p = p[:, None, :]
    z = torch.tensor(dr, requires_grad=True)
    q = torch.softmax(z, dim=-1)
    alpha = torch.clamp(torch.minimum(p, q).sum(-1), 0.0, 1.0)
    L = g * (-torch.cumprod(alpha, dim=1).sum(1)).mean()
    L.backward()
    np.testing.assert_allclose(mtp.tv_loss_grad(tgt, dr, g), z.grad.numpy(), rtol=1e-9,
                               atol=1e-15)
    loss, _, _ = mtp.tv_loss(tgt, dr)
    assert g * loss == pytest.approx(L.item(), rel=1e-13)


def test_gradient_invariants():
    T, G, V = 4, 3, 500
    tgt, dr = _case(5, T, G, V, True, sig=0.8, min_margin=0)
    g = 1.0
    grad = mtp.tv_loss_grad(tgt, dr, g)
    _, _, saved = mtp.tv_loss(tgt, dr)
    w = mtp.e2e_weights(saved[:, :, 2], g, T)
    assert np.all((saved[:, :, 3] >= 0) & (saved[:, :, 3] <= 1))
    np.testing.assert_allclose(grad.sum(-1), 0.0, atol=1e-15)
    for t in range(T):
        for k in range(G):
            q = np.exp(mtp.log_softmax(dr[t, k])[0])
            assert np.all(np.abs(grad[t, k]) <= np.abs(w[t, k]) * q * (1 + 1e-12))
    # p = q: every indicator is 1 and S = 1, so the gradient vanishes
    same = np.stack([tgt] * G, axis=1)
    gz = mtp.tv_loss_grad(tgt, same, 1.0)
    assert np.abs(gz).max() < 1e-15
    # disjoint supports: alpha = 0, loss 0, finite weights
    x = np.random.default_rng(6).normal(0, 1, (1, 40))
    xp, xq = x.copy(), x.copy()
    xp[:, ::2] = -np.inf
    xq[:, 1::2] = -np.inf
    loss, pos, saved = mtp.tv_loss(xp, np.stack([xq] * 2, axis=1))
    assert loss == 0.0 and np.all(saved[:, :, 2] == 0.0)
    assert np.all(np.isfinite(mtp.e2e_weights(saved[:, :, 2], 1.0, 1)))


def test_row_without_a_finite_normaliser_is_a_data_error():
    """READING (as in verify): a target or draft row of -inf only, or one holding a
    NaN, has no normaliser; that head's alpha and S are NaN, so are its position's
    loss and the mean, and the other positions are unaffected."""
    rng = np.random.default_rng(3)
    t = rng.normal(size=(3, 40))
    d = t[:, None, :] + 0.3 * rng.normal(size=(3, 2, 40))
    t_bad, d_bad = t.copy(), d.copy()
    t_bad[1] = -np.inf
    d_bad[2, 1, 5] = np.nan
    loss, pos, saved = mtp.tv_loss(t_bad, d_bad)
    assert np.isnan(loss)
    assert np.isnan(saved[1, :, 2:]).all() and np.isnan(pos[1])
    assert np.isnan(saved[2, 1, 2:]).all() and np.isnan(pos[2])
    assert np.isfinite(saved[2, 0]).all()
    _, pos_ok, saved_ok = mtp.tv_loss(t, d)
    assert np.allclose(saved[0], saved_ok[0]) and np.isclose(pos[0], pos_ok[0])
    g = mtp.tv_loss_grad(t_bad, d_bad)
    assert np.isnan(g[1]).all() and np.isfinite(g[0]).all()


def test_indicator_margin_closed_forms():
    """indicator_margin = |log q_v - log p_v| (the TV tests excuse indicator flips
    where it is tiny), pinned by closed forms: a draft equal to the target shifted
    by a constant has q = p (margin 0); a draft that raises one logit j by d has
    log q_v - log p_v = -log(1 + p_j (e^d - 1)) off j and d plus that at j."""
    rng = np.random.default_rng(40)
    T, G, V = 2, 3, 50
    tgt = rng.normal(0, 1.5, (T, V))
    dr = tgt[:, None, :] + np.array([0.0, 2.5, -7.0])[None, :, None]
    assert np.abs(mtp.indicator_margin(tgt, dr)).max() < 1e-12
    j, d = 17, 0.8
    dr = np.repeat(tgt[:, None, :], G, axis=1)
    dr[:, 1, j] += d
    m = mtp.indicator_margin(tgt, dr)
    p = np.exp(tgt - np.log(np.exp(tgt).sum(-1, keepdims=True)))
    shift = np.log1p(p[:, j] * np.expm1(d))
    for t in range(T):
        expect = np.full(V, shift[t])
        expect[j] = abs(d - shift[t])
        np.testing.assert_allclose(m[t, 1], expect, rtol=1e-10, atol=1e-13)
        assert np.abs(m[t, 0]).max() < 1e-12 and np.abs(m[t, 2]).max() < 1e-12
