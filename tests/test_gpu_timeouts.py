"""Bounded waits that give up are reported, not hidden.

The verify kernels and the single-read TV forward exchange row statistics between
workgroups and wait for them with a bound (mtp_set_wait_limit).  With the bound
set to 0 from the host, every wait that finds a record missing gives up at once
(no kernel stalls: each wave moves on), so the failure path runs on purpose:
the workspace error word is set, verify rows whose pass 2 ran without their
statistics carry MTP_ROW_SYNC_TIMEOUT with token -1, NaN overlap / TV and a
rejection, TV-loss positions get NaN alpha, S and loss -- and every row or
position without the flag still matches the oracle.
"""
import numpy as np
import pytest
import torch

import synthetic
import tv_loss_amd as mtp
from oracle import mtp as omtp
from parity import compare_verify, oracle_verify, stat_close, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DEFAULT_WAIT_TICKS = 100_000_000   # one second of the 100 MHz clock


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mtp.load()


@pytest.fixture
def zero_wait_limit():
    old = mtp.set_wait_limit(0)
    try:
        yield
    finally:
        mtp.set_wait_limit(old)


def _clear_error(ws):
    word = mtp.workspace_error(ws)
    ws[:4].zero_()
    torch.cuda.synchronize()
    return word


def test_verify_reports_timed_out_rows(zero_wait_limit):
    # the full rollout batch: with about ten items per super-group, a large share of
    # the record polls find a record not yet published (a few polls of a smaller
    # batch may all find their records in place, and then nothing gives up)
    w = synthetic.VERIFY_WORKLOADS["rollout"]
    t, d, y = synthetic.verify_inputs(w, DEV, B=64)
    print("verify with wait limit 0", flush=True)
    out = mtp.verify(t, d, y, seed=2, offset=0)
    torch.cuda.synchronize()
    word = _clear_error(mtp.workspace(DEV, 1))
    st = out["row_status"].cpu().numpy()
    flagged = (st & mtp.ROW_SYNC_TIMEOUT) != 0
    print("error word", word, "rows flagged", int(flagged.sum()), "of", flagged.size, flush=True)
    assert word != 0 and flagged.any()
    rt = out["row_token"].cpu().numpy()
    acc = out["accept"].cpu().numpy()
    G = d.shape[1]
    assert (rt[flagged] == -1).all()
    fl_pair = flagged[:, :G]
    assert np.isnan(out["overlap"].cpu().numpy()[fl_pair]).all()
    assert np.isnan(out["tv"].cpu().numpy()[fl_pair]).all() and (acc[fl_pair] == 0).all()
    # sequences without a flagged row match the oracle
    clean = np.flatnonzero(~flagged.any(axis=1))
    for b in clean[:4]:
        ref = oracle_verify(t[b:b + 1], d[b:b + 1], y[b:b + 1], 2, b * (G + 1))
        compare_verify(out, ref, torch.bfloat16, rows=[b])
    # the next call, with the default bound again, is clean
    mtp.set_wait_limit(DEFAULT_WAIT_TICKS)
    again = mtp.verify(t, d, y, seed=2, offset=0)
    torch.cuda.synchronize()
    assert mtp.workspace_error(mtp.workspace(DEV, 1)) == 0
    assert ((again["row_status"].cpu().numpy() & mtp.ROW_SYNC_TIMEOUT) == 0).all()


def test_tv_forward_reports_timed_out_positions(zero_wait_limit):
    tw = dict(synthetic.TV_WORKLOADS["tv_loss"], T=64)
    t, d = synthetic.tv_inputs(tw, DEV)
    print("tv forward with wait limit 0", flush=True)
    loss, pos, saved = mtp.tv_loss_fwd(t, d)
    torch.cuda.synchronize()
    word = _clear_error(mtp.workspace(DEV, 1))
    sv = saved.cpu().numpy()
    bad = np.isnan(sv[:, :, 2]).any(axis=1)
    print("error word", word, "positions with NaN alpha", int(bad.sum()), "of", bad.size, flush=True)
    assert word != 0 and bad.any()
    assert np.isnan(loss.item())
    assert np.isnan(pos.cpu().numpy()[bad]).all() and np.isfinite(pos.cpu().numpy()[~bad]).all()
    ok = np.flatnonzero(~bad)[:6]
    _, ref_pos, ref_saved = omtp.tv_loss(to_f64(t[ok]), to_f64(d[ok]))
    assert stat_close(pos.cpu().numpy()[ok], ref_pos, torch.bfloat16).all()
    assert stat_close(sv[ok, :, 2], ref_saved[:, :, 2], torch.bfloat16).all()
