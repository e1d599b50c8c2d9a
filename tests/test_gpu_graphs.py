"""The C-ABI calls under HIP graph capture: no call allocates, frees or issues a
memset, so a captured verify (all three modes), sampler and TV-loss calls (forward,
backward, the top-K pair and the fused forward + backward) replay to the eager
results.  Every graph is replayed several times
with eager calls of the same entry points (on the same workspace) and host
synchronisations in between, and every replay is compared with the eager run."""
import ctypes

import pytest
import torch

import synthetic
import tv_loss_amd as mtp
from tv_loss_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
P = ctypes.c_void_p


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mtp.load()


def _p(t):
    return P(t.data_ptr())


def _check(status):
    _lib.check(status)


def test_verify_modes_and_sampler_replay_to_the_eager_results():
    lib = mtp.load()
    w = synthetic.VERIFY_WORKLOADS["rollout"]
    t, d, y = synthetic.verify_inputs(w, DEV, B=16, V=50000)
    B, G1, V = t.shape
    G = G1 - 1
    dt = _lib.MTP_BF16
    sizes = []
    for fn in (lib.mtp_verify_workspace_size, lib.mtp_verify_target_only_workspace_size,
               lib.mtp_verify_gumbel_workspace_size):
        n = ctypes.c_size_t()
        _check(fn(B, G, V, dt, ctypes.byref(n)))
        sizes.append(n.value)
    n = ctypes.c_size_t()
    _check(lib.mtp_gumbel_sample_workspace_size(B * G, V, dt, ctypes.byref(n)))
    sizes.append(n.value)
    ws = torch.zeros(max(sizes), dtype=torch.uint8, device=DEV)
    outs = {}

    def alloc(tag):
        o = dict(acc=torch.empty((B, G), dtype=torch.uint8, device=DEV),
                 alen=torch.empty(B, dtype=torch.int32, device=DEV),
                 nxt=torch.empty(B, dtype=torch.int32, device=DEV),
                 rtok=torch.empty((B, G1), dtype=torch.int32, device=DEV),
                 ovl=torch.empty((B, G), dtype=torch.float32, device=DEV),
                 tv=torch.empty((B, G), dtype=torch.float32, device=DEV),
                 ent=torch.empty((B, G1), dtype=torch.float32, device=DEV),
                 rst=torch.empty((B, G1), dtype=torch.int32, device=DEV),
                 dtok=torch.empty((B, G), dtype=torch.int32, device=DEV),
                 pyh=torch.empty((B, G), dtype=torch.float32, device=DEV),
                 rsb=torch.empty((B, G), dtype=torch.uint8, device=DEV),
                 smp=torch.empty(B * G, dtype=torch.int32, device=DEV))
        outs[tag] = o
        return o

    def calls(o, stream):
        s = P(stream.cuda_stream)
        _check(lib.mtp_verify(_p(t), t.stride(1), _p(d), d.stride(1), dt, B, G, V, _p(y), 7, 100,
                              _p(o["acc"]), _p(o["alen"]), _p(o["nxt"]), _p(o["rtok"]), _p(o["ovl"]),
                              _p(o["tv"]), _p(o["ent"]), _p(o["rst"]), _p(ws), ws.numel(), s))
        _check(lib.mtp_verify_target_only(_p(t), t.stride(1), _p(d), d.stride(1), dt, B, G, V, 7, 100,
                                          _p(o["acc"]), _p(o["alen"]), _p(o["nxt"]), _p(o["dtok"]), _p(o["pyh"]),
                                          _p(o["rsb"]), _p(o["rtok"]), _p(o["ovl"]), _p(o["tv"]), _p(o["ent"]),
                                          _p(o["rst"]), _p(ws), ws.numel(), s))
        _check(lib.mtp_gumbel_sample(_p(d), d.stride(1), dt, B * G, V, ctypes.c_float(0.8), 3, 1 << 30,
                                     _p(o["smp"]), _p(ws), ws.numel(), s))
        _check(lib.mtp_verify_gumbel(_p(t), t.stride(1), _p(d), d.stride(1), dt, B, G, V, _p(o["smp"]),
                                     ctypes.c_float(0.8), 7, 100, _p(o["acc"]), _p(o["alen"]), _p(o["nxt"]),
                                     _p(o["rtok"]), _p(o["ovl"]), _p(o["tv"]), _p(o["ent"]), _p(o["rst"]),
                                     _p(ws), ws.numel(), s))

    side = torch.cuda.Stream()
    eager = alloc("eager")
    torch.cuda.synchronize()               # inputs, outputs and the zeroed workspace are ready
    with torch.cuda.stream(side):
        calls(eager, side)
    torch.cuda.synchronize()
    ref = {k: v.clone() for k, v in eager.items()}

    graphed = alloc("graph")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        calls(graphed, side)
    for i in range(4):
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(torch.nan_to_num(graphed[k].float()), torch.nan_to_num(ref[k].float())), (i, k)
            graphed[k].fill_(0)
        with torch.cuda.stream(side):      # eager calls on the same workspace between replays
            calls(eager, side)
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(torch.nan_to_num(eager[k].float()), torch.nan_to_num(ref[k].float())), (i, k)
    assert int(torch.count_nonzero(ws)) == 0


def test_tv_loss_calls_replay_to_the_eager_results():
    """Forward, backward, the top-K pair and the fused call in one graph."""
    lib = mtp.load()
    w = dict(T=64, G=3, V=40000, dtype=torch.bfloat16, scale=1.2, sigma=0.3, shared=True, seed=11)
    t, d = synthetic.tv_inputs(w, DEV)
    i, v, _ = synthetic.topk_inputs(w, 128, DEV)
    T, G, V = d.shape
    dt = _lib.MTP_BF16
    n1, n2 = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.mtp_tv_loss_workspace_size(T, G, V, dt, 1, ctypes.byref(n1)))
    _check(lib.mtp_tv_topk_workspace_size(T, G, V, dt, ctypes.byref(n2)))
    n3 = ctypes.c_size_t()
    _check(lib.mtp_tv_loss_fwd_bwd_workspace_size(T, G, V, dt, 1, ctypes.byref(n3)))
    ws = torch.zeros(max(n1.value, n2.value, n3.value), dtype=torch.uint8, device=DEV)
    gl = torch.ones(1, device=DEV)

    def alloc():
        return dict(loss=torch.empty(1, device=DEV), pos=torch.empty(T, device=DEV),
                    saved=torch.empty((T, G, 4), device=DEV),
                    grad=torch.empty((T, G, V), dtype=torch.bfloat16, device=DEV),
                    kloss=torch.empty(1, device=DEV), ksaved=torch.empty((T, G, 4), device=DEV),
                    kgrad=torch.empty((T, G, V), dtype=torch.float32, device=DEV),
                    floss=torch.empty(1, device=DEV), fpos=torch.empty(T, device=DEV),
                    fsaved=torch.empty((T, G, 4), device=DEV),
                    fgrad=torch.empty((T, G, V), dtype=torch.bfloat16, device=DEV))

    def calls(o, stream):
        s = P(stream.cuda_stream)
        _check(lib.mtp_tv_loss_fwd(_p(t), t.stride(0), 0, _p(d), d.stride(0), d.stride(1), dt, T, G, V,
                                   _p(o["loss"]), _p(o["pos"]), _p(o["saved"]), _p(ws), ws.numel(), s))
        _check(lib.mtp_tv_loss_bwd(_p(t), t.stride(0), 0, _p(d), d.stride(0), d.stride(1), dt, T, G, V,
                                   _p(o["saved"]), _p(gl), _p(o["grad"]), V * G, V, _lib.MTP_BF16, s))
        _check(lib.mtp_tv_topk_fwd(_p(i), _p(v), i.stride(0), 0, i.shape[1], _p(d), d.stride(0), d.stride(1), dt,
                                   T, G, V, _p(o["kloss"]), None, _p(o["ksaved"]), _p(ws), ws.numel(), s))
        _check(lib.mtp_tv_topk_bwd(_p(i), _p(v), i.stride(0), 0, i.shape[1], _p(d), d.stride(0), d.stride(1), dt,
                                   T, G, V, _p(o["ksaved"]), _p(gl), _p(o["kgrad"]), V * G, V, _lib.MTP_F32, s))
        _check(lib.mtp_tv_loss_fwd_bwd(_p(t), t.stride(0), 0, _p(d), d.stride(0), d.stride(1), dt, T, G, V, _p(gl),
                                       _p(o["floss"]), _p(o["fpos"]), _p(o["fsaved"]), _p(o["fgrad"]), V * G, V,
                                       _lib.MTP_BF16, _p(ws), ws.numel(), s))

    side = torch.cuda.Stream()
    eager = alloc()
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        calls(eager, side)
    torch.cuda.synchronize()
    ref = {k: x.clone() for k, x in eager.items()}
    graphed = alloc()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        calls(graphed, side)
    for r in range(4):
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(graphed[k], ref[k]), (r, k)
            graphed[k].zero_()
        with torch.cuda.stream(side):
            calls(eager, side)
        torch.cuda.synchronize()
        for k in ref:
            assert torch.equal(eager[k], ref[k]), (r, k)
    assert int(torch.count_nonzero(ws)) == 0
