"""GPU parity with small chunks (mtp_set_chunk_vectors): short rows spread over
hundreds of workgroups, so that the exchange of row statistics between them runs
at small vocabularies -- records past the first 64 per row, several rounds of
polling, super-groups of few items, workgroups whose waves cover their chunk in
part or not at all, owner segments that end inside a chunk.  Every verify mode,
the single-read TV forward and the fused forward + backward, against the float64
oracle with the tolerances of the full-size tests; ragged vocabularies padded with
a large finite logit."""
import numpy as np
import pytest
import torch

import synthetic
import tv_loss_amd as mtp
from oracle import mtp as omtp
from parity import compare_target_only, compare_verify, oracle_target_only, oracle_verify, to_f64
from test_gpu_tv_loss import _check_backward, _check_forward

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
PAD_LOGIT = 30.0


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mtp.load()


@pytest.fixture
def chunk():
    """Sets the chunk size for one test and restores the default after it."""
    def set_(n):
        mtp.set_chunk_vectors(n)
    yield set_
    mtp.set_chunk_vectors(0)


def _say(*a):
    print(*a, flush=True)


def _pad_rows(x, V, fill=PAD_LOGIT):
    pv = 16 // x.element_size()
    pad = (-V) % pv
    if not pad:
        return x
    xp = torch.full(x.shape[:-1] + (V + pad,), fill, dtype=x.dtype, device=DEV)
    xp[..., :V] = x
    return xp[..., :V]


# (chunk vectors, V, gamma, B): from one vector per chunk (8 bf16 / 4 fp32 logits) up
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("cv,V,G,B", [(1, 2003, 3, 2), (3, 8200, 3, 3), (7, 20011, 2, 4), (64, 30000, 3, 5),
                                      (200, 151936, 3, 2)])
def test_verify(chunk, cv, V, G, B, dtype):
    chunk(cv)
    w = dict(B=B, G=G, V=V, dtype=dtype, kind="normal", scale=1.3, sigma=0.4, seed=21)
    t, d, y = synthetic.verify_inputs(w, DEV, seed=V + cv)
    t, d = _pad_rows(t, V), _pad_rows(d, V)
    _say("small chunks verify", cv, V, G, B, dtype)
    out = mtp.verify(t, d, y, 13, 5)
    torch.cuda.synchronize()
    compare_verify(out, oracle_verify(t, d, y, 13, 5), dtype)


@pytest.mark.parametrize("cv,V,G,B", [(1, 2003, 3, 2), (5, 9001, 2, 3), (64, 40000, 3, 2)])
def test_target_only(chunk, cv, V, G, B):
    chunk(cv)
    w = dict(B=B, G=G, V=V, dtype=torch.bfloat16, kind="normal", scale=1.3, sigma=0.4, seed=22)
    t, d, _ = synthetic.verify_inputs(w, DEV, seed=V + 2 * cv)
    t, d = _pad_rows(t, V), _pad_rows(d, V)
    _say("small chunks target-only", cv, V, G, B)
    out = mtp.verify_target_only(t, d, 7, 11)
    torch.cuda.synchronize()
    compare_target_only(out, oracle_target_only(t, d, 7, 11), torch.bfloat16)


@pytest.mark.parametrize("cv,V,G,B", [(1, 2003, 3, 2), (5, 9001, 2, 3), (64, 40000, 3, 2)])
def test_gumbel(chunk, cv, V, G, B):
    chunk(cv)
    w = dict(B=B, G=G, V=V, dtype=torch.bfloat16, kind="normal", scale=1.3, sigma=0.4, seed=23)
    t, d, _ = synthetic.verify_inputs(w, DEV, seed=V + 3 * cv)
    t, d = _pad_rows(t, V), _pad_rows(d, V)
    y = synthetic.gumbel_tokens(d.float() / 0.8, torch.Generator(device=DEV).manual_seed(cv))
    _say("small chunks gumbel", cv, V, G, B)
    out = mtp.verify_gumbel(t, d, y, 0.8, 3, 4)
    torch.cuda.synchronize()
    ref = omtp.verify_gumbel(to_f64(t), to_f64(d), y.cpu().numpy(), 3, 4, temperature=0.8)
    compare_verify(out, ref, torch.bfloat16)


def test_max_vocab_follows_the_chunk(chunk):
    full = mtp.verify_max_vocab(torch.bfloat16)
    chunk(16)
    small = mtp.verify_max_vocab(torch.bfloat16)
    assert small * 512 == full * 16
    chunk(0)
    assert mtp.verify_max_vocab(torch.bfloat16) == full


@pytest.mark.parametrize("shared,G", [(True, 3), (False, 2)])
@pytest.mark.parametrize("cv,V,T", [(1, 2003, 3), (7, 9000, 4), (100, 60001, 3)])
def test_tv_forward_and_fused(chunk, cv, V, T, shared, G):
    chunk(cv)
    w = dict(T=T, G=G, V=V, dtype=torch.bfloat16, scale=1.2, sigma=0.3, shared=shared, seed=24)
    t, d = synthetic.tv_inputs(w, DEV, seed=V + cv)
    t, d = _pad_rows(t, V), _pad_rows(d, V)
    _say("small chunks tv", cv, V, T, shared, G)
    loss, pos, saved = mtp.tv_loss_fwd(t, d)
    gl = torch.tensor([0.8], dtype=torch.float32, device=DEV)
    gb = mtp.tv_loss_bwd(t, d, saved, gl, grad_dtype=torch.bfloat16)
    gf = mtp.tv_loss_bwd(t, d, saved, gl, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    _check_forward(t, d, loss, pos, saved, torch.bfloat16)
    _check_backward(t, d, saved, 0.8, gb, gf)
    floss, fpos, fsaved, fgb = mtp.tv_loss_fwd_bwd(t, d, gl, grad_dtype=torch.bfloat16)
    _, _, _, fgf = mtp.tv_loss_fwd_bwd(t, d, gl, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    _check_forward(t, d, floss, fpos, fsaved, torch.bfloat16)
    _check_backward(t, d, fsaved, 0.8, fgb, fgf)
