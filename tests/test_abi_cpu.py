"""The C ABI without a GPU: libmtp.so loads, exports every function that
include/mtp.h declares, and rejects bad arguments before any HIP call.

Every call below fails argument validation, so no kernel is launched and no
pointer is dereferenced, with or without a GPU."""
import ctypes
import os
import re

import pytest

import tv_loss_amd
from tv_loss_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mtp.h")

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="libmtp.so not built")

P = ctypes.c_void_p
A16 = P(0x10000)      # an aligned fake address: validation fails before it is used
MIS = P(0x10008)      # 8-byte aligned only


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mtp_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function():
    lib = tv_loss_amd.load()
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"{n} has no ctypes signature"
    assert set(_lib.SIGNATURES) == set(names)


def test_header_constants_match_binding():
    text = open(HEADER).read()
    for name, val in (("MTP_ROW_BAD_TOKEN", _lib.ROW_BAD_TOKEN), ("MTP_ROW_BAD_TARGET", _lib.ROW_BAD_TARGET),
                      ("MTP_ROW_BAD_DRAFT", _lib.ROW_BAD_DRAFT),
                      ("MTP_ROW_RESIDUAL_EMPTY", _lib.ROW_RESIDUAL_EMPTY), ("MTP_MAX_GAMMA", _lib.MAX_GAMMA)):
        assert re.search(rf"#define {name} {val}\b", text), name
    assert "MTP_F32 = 0" in text and "MTP_BF16 = 1" in text


def test_status_strings():
    lib = tv_loss_amd.load()
    for code, name in _lib.STATUS.items():
        assert lib.mtp_status_string(code).decode() == name
    assert lib.mtp_version().decode().startswith("libmtp")


def _verify(lib, **kw):
    a = dict(target=A16, ts=151936, draft=A16, ds=151936, dt=1, B=64, G=3, V=151936, tok=A16, seed=0, off=0,
             acc=A16, alen=A16, nxt=A16, rtok=None, ovl=None, tv=None, ent=None, rst=None, ws=A16,
             wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.mtp_verify(a["target"], a["ts"], a["draft"], a["ds"], a["dt"], a["B"], a["G"], a["V"], a["tok"],
                          a["seed"], a["off"], a["acc"], a["alen"], a["nxt"], a["rtok"], a["ovl"], a["tv"],
                          a["ent"], a["rst"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(target=None), 1), (dict(draft=None), 1), (dict(tok=None), 1), (dict(acc=None), 1),
    (dict(alen=None), 1), (dict(nxt=None), 1),
    (dict(G=0), 2), (dict(G=9), 2), (dict(V=0), 2), (dict(V=-5), 2), (dict(B=-1), 2),
    (dict(ts=151935), 2), (dict(ds=100), 2),
    (dict(dt=2), 3), (dict(dt=-1), 3),
    (dict(target=MIS), 4), (dict(draft=MIS), 4), (dict(ts=151937, ds=151944, V=151937), 4),
    (dict(ws=None), 5), (dict(wsb=1024), 5), (dict(ws=P(0x10010)), 5),
])
def test_verify_rejects_bad_arguments(kw, code):
    lib = tv_loss_amd.load()
    assert _verify(lib, **kw) == code, lib.mtp_last_error()
    assert lib.mtp_last_error()


def test_verify_empty_batch_is_a_noop():
    lib = tv_loss_amd.load()
    assert _verify(lib, B=0, target=None, draft=None, ws=None, wsb=0) == 0
    n = ctypes.c_size_t(123)
    assert lib.mtp_verify_workspace_size(0, 3, 100, 1, ctypes.byref(n)) == 0 and n.value == 0


def test_workspace_sizes_grow_with_the_problem():
    lib = tv_loss_amd.load()
    n = ctypes.c_size_t()
    sizes = []
    for B in (1, 64, 512):
        assert lib.mtp_verify_workspace_size(B, 3, 151936, 1, ctypes.byref(n)) == 0
        sizes.append(n.value)
    assert sizes == sorted(sizes) and sizes[0] > 0 and all(s % 256 == 0 for s in sizes)
    assert lib.mtp_verify_workspace_size(64, 3, 151936, 1, None) == 1
    assert lib.mtp_tv_loss_workspace_size(0, 3, 100, 1, 1, ctypes.byref(n)) == 2
    assert lib.mtp_tv_loss_workspace_size(8192, 3, 151936, 1, 1, ctypes.byref(n)) == 0 and n.value > 0


def _verify_gumbel(lib, **kw):
    a = dict(target=A16, ts=151936, draft=A16, ds=151936, dt=1, B=64, G=3, V=151936, tok=A16, T=0.8, seed=0,
             off=0, acc=A16, alen=A16, nxt=A16, ws=A16, wsb=1 << 30)
    a.update(kw)
    return lib.mtp_verify_gumbel(a["target"], a["ts"], a["draft"], a["ds"], a["dt"], a["B"], a["G"], a["V"],
                                 a["tok"], a["T"], a["seed"], a["off"], a["acc"], a["alen"], a["nxt"], None, None,
                                 None, None, None, a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(tok=None), 1), (dict(acc=None), 1), (dict(G=9), 2), (dict(ds=7), 2),
    (dict(T=0.0), 2), (dict(T=-1.0), 2), (dict(T=float("inf")), 2), (dict(T=float("nan")), 2),
    (dict(dt=3), 3), (dict(draft=MIS), 4), (dict(ws=None), 5), (dict(wsb=4096), 5),
])
def test_verify_gumbel_rejects_bad_arguments(kw, code):
    lib = tv_loss_amd.load()
    assert _verify_gumbel(lib, **kw) == code, lib.mtp_last_error()
    assert lib.mtp_last_error()


def _sample(lib, **kw):
    a = dict(x=A16, rs=151936, dt=1, rows=64, V=151936, T=1.0, seed=0, off=0, tok=A16, ws=A16, wsb=1 << 30)
    a.update(kw)
    return lib.mtp_gumbel_sample(a["x"], a["rs"], a["dt"], a["rows"], a["V"], a["T"], a["seed"], a["off"],
                                 a["tok"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(x=None), 1), (dict(tok=None), 1),
    (dict(rows=-1), 2), (dict(V=0), 2), (dict(V=(1 << 30) + 1), 2), (dict(rs=151935), 2),
    (dict(T=0.0), 2), (dict(T=float("nan")), 2), (dict(T=float("-inf")), 2),
    (dict(dt=9), 3), (dict(x=MIS), 4), (dict(rs=151937, V=151937), 4),
    (dict(rows=1 << 20, rs=1 << 20, V=1 << 20), 2),             # 2^20 rows x 128 chunks: too many
    (dict(ws=None), 5), (dict(wsb=64 * 19 * 8 - 8), 5), (dict(ws=P(0x10080)), 5),
])
def test_gumbel_sample_rejects_bad_arguments(kw, code):
    lib = tv_loss_amd.load()
    assert _sample(lib, **kw) == code, lib.mtp_last_error()


def test_gumbel_entries_empty_inputs_and_workspace():
    lib = tv_loss_amd.load()
    assert _sample(lib, rows=0, x=None, tok=None, ws=None, wsb=0) == 0
    n = ctypes.c_size_t()
    assert lib.mtp_gumbel_sample_workspace_size(64, 151936, 1, ctypes.byref(n)) == 0
    assert n.value == -(-64 * 38 * 8 // 256) * 256                  # 38 chunks of 4096 bf16 per row
    assert lib.mtp_gumbel_sample_workspace_size(64, 151936, 0, ctypes.byref(n)) == 0 and n.value >= 64 * 75 * 8
    assert lib.mtp_gumbel_sample_workspace_size(0, 151936, 1, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.mtp_gumbel_sample_workspace_size(-1, 151936, 1, ctypes.byref(n)) == 2
    assert _verify_gumbel(lib, B=0, target=None, draft=None, tok=None, ws=None, wsb=0) == 0
    n_rs, n_gm = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.mtp_verify_workspace_size(64, 3, 151936, 1, ctypes.byref(n_rs)) == 0
    assert lib.mtp_verify_gumbel_workspace_size(64, 3, 151936, 1, ctypes.byref(n_gm)) == 0
    assert n_gm.value > n_rs.value and n_gm.value % 256 == 0   # adds the per-wave key words
    assert lib.mtp_verify_gumbel_workspace_size(0, 3, 151936, 1, ctypes.byref(n_gm)) == 0 and n_gm.value == 0


def _fwd(lib, **kw):
    a = dict(t=A16, tp=151936, th=0, d=A16, dp=3 * 151936, dh=151936, dt=1, T=8, G=3, V=151936, loss=A16,
             pos=None, saved=A16, ws=A16, wsb=1 << 30, stream=None)
    a.update(kw)
    return lib.mtp_tv_loss_fwd(a["t"], a["tp"], a["th"], a["d"], a["dp"], a["dh"], a["dt"], a["T"], a["G"],
                               a["V"], a["loss"], a["pos"], a["saved"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(t=None), 1), (dict(d=None), 1), (dict(loss=None), 1), (dict(saved=None), 1),
    (dict(T=0), 2), (dict(G=0), 2), (dict(G=9), 2), (dict(V=0), 2), (dict(tp=-1), 2),
    (dict(dt=5), 3),
    (dict(t=MIS), 4), (dict(dp=3 * 151936 + 1), 4),
    (dict(ws=None), 5), (dict(wsb=256), 5),
])
def test_tv_fwd_rejects_bad_arguments(kw, code):
    lib = tv_loss_amd.load()
    assert _fwd(lib, **kw) == code, lib.mtp_last_error()


def _bwd(lib, **kw):
    a = dict(t=A16, tp=151936, th=0, d=A16, dp=3 * 151936, dh=151936, dt=1, T=8, G=3, V=151936, saved=A16,
             gl=A16, g=A16, gp=3 * 151936, gh=151936, gdt=1, stream=None)
    a.update(kw)
    return lib.mtp_tv_loss_bwd(a["t"], a["tp"], a["th"], a["d"], a["dp"], a["dh"], a["dt"], a["T"], a["G"],
                               a["V"], a["saved"], a["gl"], a["g"], a["gp"], a["gh"], a["gdt"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(saved=None), 1), (dict(gl=None), 1), (dict(g=None), 1), (dict(d=None), 1),
    (dict(T=0), 2), (dict(gp=-3), 2),
    (dict(gdt=7), 3), (dict(dt=7), 3),
    (dict(g=MIS), 4), (dict(gh=151937), 4),
])
def test_tv_bwd_rejects_bad_arguments(kw, code):
    lib = tv_loss_amd.load()
    assert _bwd(lib, **kw) == code, lib.mtp_last_error()


def _topk_fwd(lib, **kw):
    a = dict(i=A16, v=A16, kp=256, kh=0, K=256, d=A16, dp=3 * 151936, dh=151936, dt=1, T=8, G=3, V=151936,
             loss=A16, pos=None, saved=A16, ws=A16, wsb=1 << 30)
    a.update(kw)
    return lib.mtp_tv_topk_fwd(a["i"], a["v"], a["kp"], a["kh"], a["K"], a["d"], a["dp"], a["dh"], a["dt"], a["T"],
                               a["G"], a["V"], a["loss"], a["pos"], a["saved"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(i=None), 1), (dict(v=None), 1), (dict(d=None), 1), (dict(loss=None), 1), (dict(saved=None), 1),
    (dict(K=0), 2), (dict(K=(1 << 20) + 1), 2), (dict(T=0), 2), (dict(G=9), 2), (dict(kp=-1), 2),
    (dict(dt=4), 3), (dict(i=P(0x10002)), 4), (dict(v=P(0x10001)), 4), (dict(d=MIS), 4),
    (dict(ws=None), 5), (dict(wsb=256), 5),
])
def test_tv_topk_fwd_rejects_bad_arguments(kw, code):
    lib = tv_loss_amd.load()
    assert _topk_fwd(lib, **kw) == code, lib.mtp_last_error()


def _topk_bwd(lib, **kw):
    a = dict(i=A16, v=A16, kp=256, kh=0, K=256, d=A16, dp=3 * 151936, dh=151936, dt=1, T=8, G=3, V=151936,
             saved=A16, gl=A16, g=A16, gp=3 * 151936, gh=151936, gdt=1)
    a.update(kw)
    return lib.mtp_tv_topk_bwd(a["i"], a["v"], a["kp"], a["kh"], a["K"], a["d"], a["dp"], a["dh"], a["dt"], a["T"],
                               a["G"], a["V"], a["saved"], a["gl"], a["g"], a["gp"], a["gh"], a["gdt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(saved=None), 1), (dict(gl=None), 1), (dict(g=None), 1), (dict(i=None), 1),
    (dict(K=-3), 2), (dict(gh=-1), 2), (dict(gdt=2), 3), (dict(g=MIS), 4), (dict(gp=3 * 151936 + 1), 4),
])
def test_tv_topk_bwd_rejects_bad_arguments(kw, code):
    lib = tv_loss_amd.load()
    assert _topk_bwd(lib, **kw) == code, lib.mtp_last_error()


def test_verify_max_vocab_arguments():
    lib = tv_loss_amd.load()
    v = ctypes.c_int32(-1)
    assert lib.mtp_verify_max_vocab(1, None) == 1
    assert lib.mtp_verify_max_vocab(7, ctypes.byref(v)) == 3
    st = lib.mtp_verify_max_vocab(1, ctypes.byref(v))   # needs a device: MTP_ERR_DEVICE without one
    assert st in (0, 6) and (st != 0 or v.value >= 4096)


def test_tv_topk_workspace_size():
    lib = tv_loss_amd.load()
    n = ctypes.c_size_t()
    assert lib.mtp_tv_topk_workspace_size(8192, 3, 151936, 1, ctypes.byref(n)) == 0
    full = ctypes.c_size_t()
    assert lib.mtp_tv_loss_workspace_size(8192, 3, 151936, 1, 1, ctypes.byref(full)) == 0
    assert 0 < n.value < full.value and n.value % 256 == 0
    assert lib.mtp_tv_topk_workspace_size(0, 3, 151936, 1, ctypes.byref(n)) == 2


def test_python_binding_refuses_cpu_tensors():
    import torch
    t = torch.zeros(1, 4, 16)
    with pytest.raises(ValueError):
        tv_loss_amd.verify(t, t[:, :3], torch.zeros(1, 3, dtype=torch.int32), 0)


def test_chunk_vectors_hook_resizes_the_persistent_layouts():
    """mtp_set_chunk_vectors returns the previous count and changes the chunking,
    hence the workspace sizes, of the verify and single-read TV layouts; 0 or a
    negative count restores the default."""
    lib = tv_loss_amd.load()
    n0, n1 = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.mtp_verify_workspace_size(4, 3, 20000, 1, ctypes.byref(n0)) == 0
    try:
        assert lib.mtp_set_chunk_vectors(3) == 0
        assert lib.mtp_verify_workspace_size(4, 3, 20000, 1, ctypes.byref(n1)) == 0
        # 2500 vectors: 834 chunks of 3 instead of 5 of 512; records and pass-2 words grow
        assert n1.value > 100 * n0.value // 2
        assert lib.mtp_set_chunk_vectors(-5) == 3
        assert lib.mtp_verify_workspace_size(4, 3, 20000, 1, ctypes.byref(n1)) == 0
        assert n1.value == n0.value
    finally:
        lib.mtp_set_chunk_vectors(0)
