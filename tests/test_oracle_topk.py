"""Pins for the oracle's top-K TV path (oracle/mtp.py: tv_topk_*):

* with distinct indices it equals the full-vocabulary TV loss, saved statistics
  and gradient against the target truncated to the K entries (logits -inf
  elsewhere), for K = 1, a few, and K = V (a permutation: the full target);
* K = 1 closed forms: alpha = S = q(I), grad = w q (1[v = I] - q(I));
* the gradient against torch float64 autograd of the plain formula (softmax over
  the K entries scattered into V, min, clamp, cumprod);
* an index outside [0, V) acts as an entry with no mass.
Repeated indices follow the entry-by-entry reading, which has no outside
reference (parity unpinned for that case; only its invariance under a
reordering of the entries is checked).
"""
import numpy as np
import pytest
import torch

from oracle import mtp


def _topk_case(seed, T, G, V, K, shared, sig=0.6, min_margin=1e-3):
    rng = np.random.default_rng(seed)
    while True:
        shape = (T, K) if shared else (T, G, K)
        idx = np.stack([rng.permutation(V)[:K] for _ in range(int(np.prod(shape[:-1])))]).reshape(shape)
        val = rng.normal(0, 1.5, shape)
        dr = rng.normal(0, 1.5, (T, G, V))
        base = np.broadcast_to(idx[:, None, :], (T, G, K)) if shared else idx
        bval = np.broadcast_to(val[:, None, :], (T, G, K)) if shared else val
        for t in range(T):
            for k in range(G):
                dr[t, k, base[t, k]] = bval[t, k] + rng.normal(0, sig, K)
        if mtp.tv_topk_indicator_margin(idx, val, dr).min() > min_margin:
            return idx, val, dr


def _masked(idx, val, V):
    """The truncated target as full rows: the K logits at their indices, -inf elsewhere."""
    out = np.full(idx.shape[:-1] + (V,), -np.inf)
    np.put_along_axis(out, idx, val, axis=-1)
    return out


@pytest.mark.parametrize("shared", [True, False])
@pytest.mark.parametrize("K", [1, 3, 17, 40])
def test_distinct_indices_equal_the_full_path_on_the_truncated_target(K, shared):
    T, G, V = 3, 3, 40
    idx, val, dr = _topk_case(10 + K, T, G, V, K, shared, min_margin=0)
    tgt = _masked(idx, val, V)
    loss, pos, saved = mtp.tv_topk_loss(idx, val, dr)
    floss, fpos, fsaved = mtp.tv_loss(tgt, dr)
    assert loss == pytest.approx(floss, rel=1e-13, abs=1e-15)
    np.testing.assert_allclose(pos, fpos, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(saved[..., 1:], fsaved[..., 1:], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(saved[..., 0], fsaved[..., 0], rtol=1e-13)   # lse of the K logits
    np.testing.assert_allclose(mtp.tv_topk_loss_grad(idx, val, dr, 1.4), mtp.tv_loss_grad(tgt, dr, 1.4),
                               rtol=1e-12, atol=1e-16)


def test_k_equal_v_is_the_full_target():
    rng = np.random.default_rng(3)
    T, G, V = 2, 2, 64
    tgt = rng.normal(0, 1, (T, V))
    dr = tgt[:, None, :] + rng.normal(0, 0.5, (T, G, V))
    perm = np.stack([rng.permutation(V) for _ in range(T)])
    loss, _, saved = mtp.tv_topk_loss(perm, np.take_along_axis(tgt, perm, -1), dr)
    floss, _, fsaved = mtp.tv_loss(tgt, dr)
    assert loss == pytest.approx(floss, rel=1e-13)
    np.testing.assert_allclose(saved, fsaved, rtol=1e-12, atol=1e-15)


def test_k1_closed_form():
    rng = np.random.default_rng(4)
    T, G, V = 3, 2, 30
    idx = rng.integers(0, V, (T, 1))
    val = rng.normal(0, 1, (T, 1))
    dr = rng.normal(0, 1, (T, G, V))
    _, pos, saved = mtp.tv_topk_loss(idx, val, dr)
    q = np.exp(dr - np.log(np.exp(dr).sum(-1, keepdims=True)))
    qi = np.take_along_axis(q, np.broadcast_to(idx[:, None, :], (T, G, 1)), -1)[..., 0]
    np.testing.assert_allclose(saved[..., 2], qi, rtol=1e-13)
    np.testing.assert_allclose(saved[..., 3], qi, rtol=1e-13)
    np.testing.assert_allclose(pos, -(qi[:, 0] + qi[:, 0] * qi[:, 1]), rtol=1e-13)
    w = mtp.e2e_weights(qi, 1.0, T)
    onehot = np.zeros((T, G, V))
    for t in range(T):
        onehot[t, :, idx[t, 0]] = 1.0
    np.testing.assert_allclose(mtp.tv_topk_loss_grad(idx, val, dr), w[..., None] * q * (onehot - qi[..., None]),
                               rtol=1e-12, atol=1e-17)


@pytest.mark.parametrize("shared", [True, False])
def test_gradient_matches_torch_autograd(shared):
    T, G, V, K = 3, 3, 300, 24
    idx, val, dr = _topk_case(5, T, G, V, K, shared, min_margin=1e-4)
    g = 0.8
    pk = torch.softmax(torch.tensor(val), dim=-1)
    ii = torch.tensor(idx, dtype=torch.int64)
    if shared:
        pk, ii = pk[:, None, :].expand(T, G, K), ii[:, None, :].expand(T, G, K)
    p = torch.zeros(T, G, V, dtype=torch.float64).scatter(-1, ii, pk)
    z = torch.tensor(dr, requires_grad=True)
    q = torch.softmax(z, dim=-1)
    alpha = torch.clamp(torch.minimum(p, q).sum(-1), 0.0, 1.0)
    L = g * (-torch.cumprod(alpha, dim=1).sum(1)).mean()
    L.backward()
    np.testing.assert_allclose(mtp.tv_topk_loss_grad(idx, val, dr, g), z.grad.numpy(), rtol=1e-9, atol=1e-16)
    assert g * mtp.tv_topk_loss(idx, val, dr)[0] == pytest.approx(L.item(), rel=1e-13)


def test_out_of_range_indices_have_no_mass():
    T, G, V, K = 2, 2, 50, 8
    idx, val, dr = _topk_case(6, T, G, V, K, True, min_margin=0)
    bad = idx.copy()
    bad[0, 2], bad[1, 5] = -1, V + 3
    ref_idx, ref_val = idx.copy(), val.copy()
    ref_val[0, 2], ref_val[1, 5] = -np.inf, -np.inf
    a = mtp.tv_topk_loss(bad, val, dr)
    b = mtp.tv_topk_loss(ref_idx, ref_val, dr)
    # equal up to summation order (numpy's pairwise sums see one more zero term)
    assert a[0] == pytest.approx(b[0], rel=1e-14)
    np.testing.assert_allclose(a[2], b[2], rtol=1e-14, atol=1e-17)
    np.testing.assert_allclose(mtp.tv_topk_loss_grad(bad, val, dr), mtp.tv_topk_loss_grad(ref_idx, ref_val, dr),
                               rtol=1e-13, atol=1e-18)


def test_repeated_indices_entry_by_entry_is_order_free():
    T, G, V, K = 2, 2, 30, 6
    rng = np.random.default_rng(7)
    idx = rng.integers(0, 4, (T, K))              # many repeats
    val = rng.normal(0, 1, (T, K))
    dr = rng.normal(0, 1, (T, G, V))
    perm = rng.permutation(K)
    a = mtp.tv_topk_loss(idx, val, dr)
    b = mtp.tv_topk_loss(idx[:, perm], val[:, perm], dr)
    assert a[0] == pytest.approx(b[0], rel=1e-14)
    np.testing.assert_allclose(mtp.tv_topk_loss_grad(idx, val, dr), mtp.tv_topk_loss_grad(idx[:, perm], val[:, perm], dr),
                               rtol=1e-13, atol=1e-17)


def test_indicator_margin_closed_form():
    """tv_topk_indicator_margin = |log q(I_j) - log p_j| per entry, pinned by a closed
    form: when the K target logits are the draft logits at their indices plus a
    constant, the truncated target is q restricted to the entries and renormalised,
    so every entry's margin is |log Q| with Q the draft mass on the entries; an
    entry out of range gets inf."""
    rng = np.random.default_rng(41)
    T, G, V, K = 2, 2, 40, 7
    dr = rng.normal(0, 1.2, (T, G, V))
    idx = np.stack([np.stack([rng.choice(V, K, replace=False) for _ in range(G)]) for _ in range(T)])
    val = np.take_along_axis(dr, idx, -1) + 3.25
    idx = idx.copy()
    idx[0, 1, 4] = V + 5
    val[0, 1, 4] = 0.0
    m = mtp.tv_topk_indicator_margin(idx, val, dr)
    q = np.exp(dr - np.log(np.exp(dr).sum(-1, keepdims=True)))
    for t in range(T):
        for k in range(G):
            ok = idx[t, k] < V
            Q = q[t, k, idx[t, k][ok]].sum()
            np.testing.assert_allclose(m[t, k][ok], abs(np.log(Q)), rtol=1e-10)
            assert np.all(np.isinf(m[t, k][~ok]))
