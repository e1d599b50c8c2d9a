"""mtp_verify_noalloc (the verify call whose workspace is the library's own
file-scope device array) against mtp_verify with a caller workspace, through the
C ABI: two calls in a row, the second on a smaller input, every output equal to
the workspace call's (same kernels, same inputs) and the small call also against
the oracle; a call whose workspace would exceed the array is refused."""
import ctypes

import numpy as np
import pytest
import torch

import synthetic
import tv_loss_amd as mtp
from tv_loss_amd import _lib
from parity import compare_verify, oracle_verify

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
KEYS = ("accept", "accepted_len", "next_token", "row_token", "overlap", "tv", "entropy", "row_status")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mtp.load()


def _noalloc(target, draft, tokens, seed, offset):
    lib = mtp.load()
    B, G1, V = target.shape
    G = G1 - 1
    dev = target.device
    out = {"accept": torch.empty((B, G), dtype=torch.uint8, device=dev),
           "accepted_len": torch.empty(B, dtype=torch.int32, device=dev),
           "next_token": torch.empty(B, dtype=torch.int32, device=dev),
           "row_token": torch.empty((B, G1), dtype=torch.int32, device=dev),
           "overlap": torch.empty((B, G), dtype=torch.float32, device=dev),
           "tv": torch.empty((B, G), dtype=torch.float32, device=dev),
           "entropy": torch.empty((B, G1), dtype=torch.float32, device=dev),
           "row_status": torch.empty((B, G1), dtype=torch.int32, device=dev)}
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    dt = _lib.MTP_BF16 if target.dtype == torch.bfloat16 else _lib.MTP_F32
    st = lib.mtp_verify_noalloc(p(target), target.stride(1), p(draft), draft.stride(1), dt, B, G, V, p(tokens),
                                ctypes.c_uint64(seed), ctypes.c_uint64(offset), p(out["accept"]),
                                p(out["accepted_len"]), p(out["next_token"]), p(out["row_token"]),
                                p(out["overlap"]), p(out["tv"]), p(out["entropy"]), p(out["row_status"]),
                                ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    return st, out


def _same(a, b):
    for k in KEYS:
        x, y = a[k].cpu().numpy(), b[k].cpu().numpy()
        if x.dtype.kind == "f":
            assert np.array_equal(x, y, equal_nan=True), k
        else:
            assert np.array_equal(x, y), k


def test_noalloc_matches_the_workspace_call_twice_then_refuses_too_much():
    w = synthetic.VERIFY_WORKLOADS["rollout"]
    big = synthetic.verify_inputs(w, DEV, B=24)
    small = synthetic.verify_inputs(w, DEV, B=3, V=9000)
    for i, (t, d, y) in enumerate((big, small)):
        print("noalloc call", i, tuple(t.shape), flush=True)
        st, out = _noalloc(t, d, y, seed=7, offset=100 * i)
        assert st == 0, mtp.load().mtp_last_error()
        ref = mtp.verify(t, d, y, seed=7, offset=100 * i)
        torch.cuda.synchronize()
        _same(out, ref)
    compare_verify(out, oracle_verify(*small, 7, 100), torch.bfloat16)
    # a workspace beyond the array is refused before any launch (real tensors of the
    # refused shape, so that even a call that went ahead would read only its inputs)
    B, G, V = 1024, 4, 262144
    need = ctypes.c_size_t()
    assert mtp.load().mtp_verify_workspace_size(B, G, V, _lib.MTP_BF16, ctypes.byref(need)) == 0
    assert need.value > _lib.VERIFY_NOALLOC_SCRATCH_BYTES
    t = torch.zeros((B, G + 1, V), dtype=torch.bfloat16, device=DEV)
    d = torch.zeros((B, G, V), dtype=torch.bfloat16, device=DEV)
    st, out = _noalloc(t, d, torch.zeros((B, G), dtype=torch.int32, device=DEV), 0, 0)
    assert st == 5 and b"scratch" in mtp.load().mtp_last_error()
