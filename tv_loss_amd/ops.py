"""PyTorch-facing wrappers over the libmtp C ABI.

Every computation runs in the HIP kernels behind include/mtp.h; this module only
checks tensor layouts, allocates outputs with torch, passes pointers and the
current stream, and caches one zero-initialised workspace per (device, stream).
There is no CPU fallback: without libmtp.so or a GPU these functions raise.
"""
import ctypes

import torch

from . import _lib
from ._lib import MtpError, check, load

_DTYPES = {torch.float32: _lib.MTP_F32, torch.bfloat16: _lib.MTP_BF16}
_workspaces = {}


def _dtype_code(t):
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"logits must be float32 or bfloat16, got {t.dtype}") from None


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace(device, nbytes):
    """A zero-filled workspace of at least nbytes for the current stream of device.
    The kernels leave it zeroed after each call, so it is reused as is."""
    device = torch.device(device)
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def _grad_buffer(T, G, V, dtype, device):
    """A [T, gamma, V] gradient whose rows start 16 bytes apart (the kernels store
    whole 16-byte vectors): a view of a buffer padded past V when V is ragged."""
    per = 16 // torch.empty((), dtype=dtype).element_size()
    Vp = (V + per - 1) // per * per
    buf = torch.empty((T, G, Vp), dtype=dtype, device=device)
    return buf[..., :V] if Vp != V else buf


def _require_cuda(*ts):
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on a GPU")


def _verify_shape(target, draft):
    if target.dim() != 3 or draft.dim() != 3:
        raise ValueError("target must be [B, gamma+1, V] and draft [B, gamma, V]")
    B, G1, V = target.shape
    G = G1 - 1
    if tuple(draft.shape) != (B, G, V) or draft.dtype != target.dtype:
        raise ValueError("draft must match target: [B, gamma, V], same dtype")
    for name, t, rows in (("target", target, G1), ("draft", draft, G)):
        if t.stride(2) != 1 or (B > 1 and t.stride(0) != rows * t.stride(1)):
            raise ValueError(f"{name} needs unit stride along V and a uniform row stride")
    return B, G1, V


def verify(target, draft, draft_tokens, seed, offset=0, *, stats=True):
    """Rejection-sampling verification (see mtp_verify in include/mtp.h).

    target: [B, gamma+1, V], draft: [B, gamma, V] (float32 or bfloat16, same dtype,
    unit stride along V, uniform row stride); draft_tokens: int32 [B, gamma].
    Returns a dict of tensors: accept (uint8 [B, gamma]), accepted_len, next_token
    (int32 [B]) and, with stats, row_token, row_status (int32 [B, gamma+1]),
    overlap, tv (float [B, gamma]) and entropy (float [B, gamma+1]).
    """
    lib = load()
    _require_cuda(target, draft, draft_tokens)
    B, G1, V = _verify_shape(target, draft)
    G = G1 - 1
    if draft_tokens.dtype != torch.int32 or tuple(draft_tokens.shape) != (B, G):
        raise ValueError("draft_tokens must be int32 [B, gamma]")
    draft_tokens = draft_tokens.contiguous()
    dev = target.device
    dt = _dtype_code(target)
    out = {
        "accept": torch.empty((B, G), dtype=torch.uint8, device=dev),
        "accepted_len": torch.empty(B, dtype=torch.int32, device=dev),
        "next_token": torch.empty(B, dtype=torch.int32, device=dev),
    }
    if stats:
        out.update(row_token=torch.empty((B, G1), dtype=torch.int32, device=dev),
                   row_status=torch.empty((B, G1), dtype=torch.int32, device=dev),
                   overlap=torch.empty((B, G), dtype=torch.float32, device=dev),
                   tv=torch.empty((B, G), dtype=torch.float32, device=dev),
                   entropy=torch.empty((B, G1), dtype=torch.float32, device=dev))
    if B == 0:
        return out
    nbytes = ctypes.c_size_t()
    check(lib.mtp_verify_workspace_size(B, G, V, dt, ctypes.byref(nbytes)))
    ws = workspace(dev, nbytes.value)
    with torch.cuda.device(dev):
        check(lib.mtp_verify(
            _ptr(target), target.stride(1), _ptr(draft), draft.stride(1), dt, B, G, V,
            _ptr(draft_tokens), ctypes.c_uint64(seed), ctypes.c_uint64(offset),
            _ptr(out["accept"]), _ptr(out["accepted_len"]), _ptr(out["next_token"]),
            _ptr(out.get("row_token")), _ptr(out.get("overlap")), _ptr(out.get("tv")),
            _ptr(out.get("entropy")), _ptr(out.get("row_status")),
            _ptr(ws), ws.numel(), _stream(dev)))
    return out


def verify_max_vocab(dtype, device=0):
    """The largest vocabulary the verify calls accept for `dtype` on `device`
    (mtp_verify_max_vocab)."""
    lib = load()
    v = ctypes.c_int32()
    with torch.cuda.device(device):
        check(lib.mtp_verify_max_vocab(_DTYPES[dtype], ctypes.byref(v)))
    return v.value


def verify_target_only(target, draft, seed, offset=0, *, stats=True):
    """Target-only verification with the RS/TO diagnostic (see
    mtp_verify_target_only in include/mtp.h): every draft position proposes its
    greedy token argmax q.  Same inputs as verify() without draft_tokens; the dict
    adds draft_token (int32 [B, gamma]) and, with stats, p_yhat (float) and
    rs_better (uint8) [B, gamma]."""
    lib = load()
    _require_cuda(target, draft)
    B, G1, V = _verify_shape(target, draft)
    G = G1 - 1
    dev = target.device
    dt = _dtype_code(target)
    out = {
        "accept": torch.empty((B, G), dtype=torch.uint8, device=dev),
        "accepted_len": torch.empty(B, dtype=torch.int32, device=dev),
        "next_token": torch.empty(B, dtype=torch.int32, device=dev),
        "draft_token": torch.empty((B, G), dtype=torch.int32, device=dev),
    }
    if stats:
        out.update(row_token=torch.empty((B, G1), dtype=torch.int32, device=dev),
                   row_status=torch.empty((B, G1), dtype=torch.int32, device=dev),
                   overlap=torch.empty((B, G), dtype=torch.float32, device=dev),
                   tv=torch.empty((B, G), dtype=torch.float32, device=dev),
                   entropy=torch.empty((B, G1), dtype=torch.float32, device=dev),
                   p_yhat=torch.empty((B, G), dtype=torch.float32, device=dev),
                   rs_better=torch.empty((B, G), dtype=torch.uint8, device=dev))
    if B == 0:
        return out
    nbytes = ctypes.c_size_t()
    check(lib.mtp_verify_target_only_workspace_size(B, G, V, dt, ctypes.byref(nbytes)))
    ws = workspace(dev, nbytes.value)
    with torch.cuda.device(dev):
        check(lib.mtp_verify_target_only(
            _ptr(target), target.stride(1), _ptr(draft), draft.stride(1), dt, B, G, V,
            ctypes.c_uint64(seed), ctypes.c_uint64(offset),
            _ptr(out["accept"]), _ptr(out["accepted_len"]), _ptr(out["next_token"]), _ptr(out["draft_token"]),
            _ptr(out.get("p_yhat")), _ptr(out.get("rs_better")),
            _ptr(out.get("row_token")), _ptr(out.get("overlap")), _ptr(out.get("tv")),
            _ptr(out.get("entropy")), _ptr(out.get("row_status")),
            _ptr(ws), ws.numel(), _stream(dev)))
    return out


def _tv_layout(target, draft):
    if draft.dim() != 3:
        raise ValueError("draft must be [T, gamma, V]")
    T, G, V = draft.shape
    if target.dim() == 2:
        if tuple(target.shape) != (T, V):
            raise ValueError("a shared target must be [T, V]")
        t_pos, t_head = target.stride(0), 0
        if target.stride(1) != 1:
            raise ValueError("target needs unit stride along V")
    elif target.dim() == 3:
        if tuple(target.shape) != (T, G, V):
            raise ValueError("a per-head target must be [T, gamma, V]")
        t_pos, t_head = target.stride(0), target.stride(1)
        if target.stride(2) != 1:
            raise ValueError("target needs unit stride along V")
        if t_head == 0:
            raise ValueError("a per-head target with head stride 0: pass the [T, V] row instead")
    else:
        raise ValueError("target must be [T, V] or [T, gamma, V]")
    if draft.stride(2) != 1:
        raise ValueError("draft needs unit stride along V")
    if draft.dtype != target.dtype:
        raise ValueError("target and draft must share a dtype")
    return T, G, V, t_pos, t_head


def tv_loss_fwd(target, draft):
    """End-to-end TV loss forward (mtp_tv_loss_fwd).  target: [T, V] shared by the
    heads or [T, gamma, V]; draft: [T, gamma, V].  Returns (loss [1], pos_loss [T],
    saved [T, gamma, 4])."""
    lib = load()
    _require_cuda(target, draft)
    T, G, V, t_pos, t_head = _tv_layout(target, draft)
    dev = draft.device
    dt = _dtype_code(draft)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    pos_loss = torch.empty(T, dtype=torch.float32, device=dev)
    saved = torch.empty((T, G, 4), dtype=torch.float32, device=dev)
    nbytes = ctypes.c_size_t()
    check(lib.mtp_tv_loss_workspace_size(T, G, V, dt, int(t_head == 0), ctypes.byref(nbytes)))
    ws = workspace(dev, nbytes.value)
    with torch.cuda.device(dev):
        check(lib.mtp_tv_loss_fwd(_ptr(target), t_pos, t_head, _ptr(draft), draft.stride(0), draft.stride(1),
                                  dt, T, G, V, _ptr(loss), _ptr(pos_loss), _ptr(saved),
                                  _ptr(ws), ws.numel(), _stream(dev)))
    return loss, pos_loss, saved


def tv_loss_bwd(target, draft, saved, grad_loss, grad_dtype=None, out=None):
    """End-to-end TV loss backward (mtp_tv_loss_bwd): gradient w.r.t. the draft
    logits, [T, gamma, V] in grad_dtype (default: the draft's dtype)."""
    lib = load()
    _require_cuda(target, draft, saved, grad_loss)
    T, G, V, t_pos, t_head = _tv_layout(target, draft)
    dev = draft.device
    dt = _dtype_code(draft)
    grad_dtype = grad_dtype or draft.dtype
    if out is None:
        out = _grad_buffer(T, G, V, grad_dtype, dev)
    if out.stride(2) != 1 or tuple(out.shape) != (T, G, V):
        raise ValueError("grad output must be [T, gamma, V] with unit stride along V")
    gdt = _DTYPES[out.dtype]
    saved = saved.contiguous()
    grad_loss = grad_loss.reshape(1).to(torch.float32).contiguous()
    with torch.cuda.device(dev):
        check(lib.mtp_tv_loss_bwd(_ptr(target), t_pos, t_head, _ptr(draft), draft.stride(0), draft.stride(1),
                                  dt, T, G, V, _ptr(saved), _ptr(grad_loss), _ptr(out), out.stride(0),
                                  out.stride(1), gdt, _stream(dev)))
    return out


def tv_loss_fwd_bwd(target, draft, grad_loss, grad_dtype=None, out=None):
    """End-to-end TV loss forward and backward in one sweep (mtp_tv_loss_fwd_bwd),
    with the upstream gradient grad_loss (float [1]) given up front.  Returns (loss
    [1], pos_loss [T], saved [T, gamma, 4], grad [T, gamma, V] in grad_dtype,
    default the draft's dtype)."""
    lib = load()
    _require_cuda(target, draft, grad_loss)
    T, G, V, t_pos, t_head = _tv_layout(target, draft)
    dev = draft.device
    dt = _dtype_code(draft)
    grad_dtype = grad_dtype or draft.dtype
    if out is None:
        out = _grad_buffer(T, G, V, grad_dtype, dev)
    if out.stride(2) != 1 or tuple(out.shape) != (T, G, V):
        raise ValueError("grad output must be [T, gamma, V] with unit stride along V")
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    pos_loss = torch.empty(T, dtype=torch.float32, device=dev)
    saved = torch.empty((T, G, 4), dtype=torch.float32, device=dev)
    grad_loss = grad_loss.reshape(1).to(torch.float32).contiguous()
    nbytes = ctypes.c_size_t()
    check(lib.mtp_tv_loss_fwd_bwd_workspace_size(T, G, V, dt, int(t_head == 0), ctypes.byref(nbytes)))
    ws = workspace(dev, nbytes.value)
    with torch.cuda.device(dev):
        check(lib.mtp_tv_loss_fwd_bwd(_ptr(target), t_pos, t_head, _ptr(draft), draft.stride(0), draft.stride(1),
                                      dt, T, G, V, _ptr(grad_loss), _ptr(loss), _ptr(pos_loss), _ptr(saved),
                                      _ptr(out), out.stride(0), out.stride(1), _DTYPES[out.dtype],
                                      _ptr(ws), ws.numel(), _stream(dev)))
    return loss, pos_loss, saved, out


class TVLoss(torch.autograd.Function):
    """L = mean_t -sum_k prod_{j<=k} alpha_{t,j}; gradient to the draft logits only
    (the target distribution is detached)."""

    @staticmethod
    def forward(ctx, draft, target):
        loss, _, saved = tv_loss_fwd(target.detach(), draft.detach())
        ctx.save_for_backward(draft.detach(), target.detach(), saved)
        return loss[0]

    @staticmethod
    def backward(ctx, grad_out):
        draft, target, saved = ctx.saved_tensors
        grad = tv_loss_bwd(target, draft, saved, grad_out.reshape(1))
        return grad, None


def tv_loss(draft, target):
    return TVLoss.apply(draft, target)


def _topk_layout(idx, val, draft):
    if draft.dim() != 3:
        raise ValueError("draft must be [T, gamma, V]")
    T, G, V = draft.shape
    if idx.dtype != torch.int32 or val.dtype != torch.float32:
        raise ValueError("target_idx must be int32 and target_val float32")
    if tuple(idx.shape) != tuple(val.shape) or idx.stride() != val.stride():
        raise ValueError("target_idx and target_val must have the same shape and strides")
    if idx.dim() == 2 and idx.shape[0] == T:
        k_pos, k_head = idx.stride(0), 0
    elif idx.dim() == 3 and tuple(idx.shape[:2]) == (T, G):
        k_pos, k_head = idx.stride(0), idx.stride(1)
    else:
        raise ValueError("top-K targets must be [T, K] (shared by the heads) or [T, gamma, K]")
    if idx.stride(-1) != 1:
        raise ValueError("top-K targets need unit stride along K")
    if draft.stride(2) != 1:
        raise ValueError("draft needs unit stride along V")
    return T, G, V, idx.shape[-1], k_pos, k_head


def tv_topk_fwd(target_idx, target_val, draft):
    """End-to-end TV loss forward with top-K targets (mtp_tv_topk_fwd).
    target_idx int32 / target_val float32: [T, K] shared by the heads or
    [T, gamma, K]; draft: [T, gamma, V].  Returns (loss [1], pos_loss [T],
    saved [T, gamma, 4] = (lse_A, lse_q, alpha, S))."""
    lib = load()
    _require_cuda(target_idx, target_val, draft)
    T, G, V, K, k_pos, k_head = _topk_layout(target_idx, target_val, draft)
    dev = draft.device
    dt = _dtype_code(draft)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    pos_loss = torch.empty(T, dtype=torch.float32, device=dev)
    saved = torch.empty((T, G, 4), dtype=torch.float32, device=dev)
    nbytes = ctypes.c_size_t()
    check(lib.mtp_tv_topk_workspace_size(T, G, V, dt, ctypes.byref(nbytes)))
    ws = workspace(dev, nbytes.value)
    with torch.cuda.device(dev):
        check(lib.mtp_tv_topk_fwd(_ptr(target_idx), _ptr(target_val), k_pos, k_head, K, _ptr(draft),
                                  draft.stride(0), draft.stride(1), dt, T, G, V, _ptr(loss), _ptr(pos_loss),
                                  _ptr(saved), _ptr(ws), ws.numel(), _stream(dev)))
    return loss, pos_loss, saved


def tv_topk_bwd(target_idx, target_val, draft, saved, grad_loss, grad_dtype=None, out=None):
    """Backward of the top-K TV loss (mtp_tv_topk_bwd): gradient w.r.t. the draft
    logits, [T, gamma, V] in grad_dtype (default: the draft's dtype)."""
    lib = load()
    _require_cuda(target_idx, target_val, draft, saved, grad_loss)
    T, G, V, K, k_pos, k_head = _topk_layout(target_idx, target_val, draft)
    dev = draft.device
    dt = _dtype_code(draft)
    grad_dtype = grad_dtype or draft.dtype
    if out is None:
        out = _grad_buffer(T, G, V, grad_dtype, dev)
    if out.stride(2) != 1 or tuple(out.shape) != (T, G, V):
        raise ValueError("grad output must be [T, gamma, V] with unit stride along V")
    gdt = _DTYPES[out.dtype]
    saved = saved.contiguous()
    grad_loss = grad_loss.reshape(1).to(torch.float32).contiguous()
    with torch.cuda.device(dev):
        check(lib.mtp_tv_topk_bwd(_ptr(target_idx), _ptr(target_val), k_pos, k_head, K, _ptr(draft),
                                  draft.stride(0), draft.stride(1), dt, T, G, V, _ptr(saved), _ptr(grad_loss),
                                  _ptr(out), out.stride(0), out.stride(1), gdt, _stream(dev)))
    return out


class TVTopKLoss(torch.autograd.Function):
    """The end-to-end TV loss against top-K targets; gradient to the draft logits only."""

    @staticmethod
    def forward(ctx, draft, target_idx, target_val):
        loss, _, saved = tv_topk_fwd(target_idx, target_val, draft.detach())
        ctx.save_for_backward(draft.detach(), target_idx, target_val, saved)
        return loss[0]

    @staticmethod
    def backward(ctx, grad_out):
        draft, idx, val, saved = ctx.saved_tensors
        return tv_topk_bwd(idx, val, draft, saved, grad_out.reshape(1)), None, None


def tv_topk_loss(draft, target_idx, target_val):
    return TVTopKLoss.apply(draft, target_idx, target_val)


def workspace_error(ws):
    """The error word of a workspace (non-zero after a bounded-wait timeout)."""
    lib = load()
    word = ctypes.c_uint32()
    check(lib.mtp_workspace_error(_ptr(ws), ctypes.byref(word), _stream(ws.device)))
    return word.value


def set_wait_limit(ticks):
    """Bound, in ticks of the GPU's 100 MHz clock, on every wait for row statistics
    exchanged between workgroups, for calls launched afterwards (mtp_set_wait_limit);
    returns the previous bound.  0 makes such waits give up at once."""
    return int(load().mtp_set_wait_limit(ctypes.c_uint64(int(ticks))))


def set_chunk_vectors(vectors):
    """Diagnostics: 16-byte vectors per chunk of the persistent verify and TV grids
    (mtp_set_chunk_vectors; 0 restores each kernel's own chunk).  Returns the
    previous count."""
    return int(load().mtp_set_chunk_vectors(int(vectors)))


def _check_temperature(temperature):
    t = float(temperature)
    if not (t > 0.0) or t == float("inf"):
        raise ValueError(f"temperature must be positive and finite, got {temperature}")
    return t


def verify_gumbel(target, draft, draft_tokens, temperature, seed, offset=0, *, stats=True):
    """Rejection-sampling verification at a temperature with Gumbel-max row samples
    (see mtp_verify_gumbel in include/mtp.h).  Inputs and outputs as for verify();
    p and q are the softmax of the logits divided by `temperature`."""
    lib = load()
    _require_cuda(target, draft, draft_tokens)
    B, G1, V = _verify_shape(target, draft)
    G = G1 - 1
    if draft_tokens.dtype != torch.int32 or tuple(draft_tokens.shape) != (B, G):
        raise ValueError("draft_tokens must be int32 [B, gamma]")
    T = _check_temperature(temperature)
    draft_tokens = draft_tokens.contiguous()
    dev = target.device
    dt = _dtype_code(target)
    out = {
        "accept": torch.empty((B, G), dtype=torch.uint8, device=dev),
        "accepted_len": torch.empty(B, dtype=torch.int32, device=dev),
        "next_token": torch.empty(B, dtype=torch.int32, device=dev),
    }
    if stats:
        out.update(row_token=torch.empty((B, G1), dtype=torch.int32, device=dev),
                   row_status=torch.empty((B, G1), dtype=torch.int32, device=dev),
                   overlap=torch.empty((B, G), dtype=torch.float32, device=dev),
                   tv=torch.empty((B, G), dtype=torch.float32, device=dev),
                   entropy=torch.empty((B, G1), dtype=torch.float32, device=dev))
    if B == 0:
        return out
    nbytes = ctypes.c_size_t()
    check(lib.mtp_verify_gumbel_workspace_size(B, G, V, dt, ctypes.byref(nbytes)))
    ws = workspace(dev, nbytes.value)
    with torch.cuda.device(dev):
        check(lib.mtp_verify_gumbel(
            _ptr(target), target.stride(1), _ptr(draft), draft.stride(1), dt, B, G, V,
            _ptr(draft_tokens), ctypes.c_float(T), ctypes.c_uint64(seed), ctypes.c_uint64(offset),
            _ptr(out["accept"]), _ptr(out["accepted_len"]), _ptr(out["next_token"]),
            _ptr(out.get("row_token")), _ptr(out.get("overlap")), _ptr(out.get("tv")),
            _ptr(out.get("entropy")), _ptr(out.get("row_status")),
            _ptr(ws), ws.numel(), _stream(dev)))
    return out


def gumbel_sample(logits, temperature, seed, offset=0):
    """Gumbel-max samples of softmax(logits / temperature) over the last dimension
    (see mtp_gumbel_sample in include/mtp.h): row r of the flattened leading
    dimensions uses Philox counter offset + r.  logits: float32 or bfloat16 [..., V]
    with unit stride along V and a uniform row stride.  Returns int32 [...]."""
    lib = load()
    _require_cuda(logits)
    if logits.dim() < 1:
        raise ValueError("logits must have a vocabulary dimension")
    V = logits.shape[-1]
    lead = tuple(logits.shape[:-1])
    flat = logits.reshape(-1, V)
    if flat.stride(-1) != 1:
        flat = flat.contiguous()
    rows = flat.shape[0]
    T = _check_temperature(temperature)
    dt = _dtype_code(logits)
    tokens = torch.empty(rows, dtype=torch.int32, device=logits.device)
    if rows:
        pv = 16 // flat.element_size()
        vp = -(-V // pv) * pv                     # V rounded up to whole 16-byte vectors
        stride = flat.stride(0) if rows > 1 else vp
        if (stride * flat.element_size()) % 16 or flat.data_ptr() % 16:
            # rows must start 16-byte aligned: copy into a padded buffer
            padded = torch.empty((rows, vp), dtype=flat.dtype, device=flat.device)
            padded[:, :V] = flat
            flat, stride = padded, vp
        nbytes = ctypes.c_size_t()
        check(lib.mtp_gumbel_sample_workspace_size(rows, V, dt, ctypes.byref(nbytes)))
        ws = workspace(logits.device, nbytes.value)
        with torch.cuda.device(logits.device):
            check(lib.mtp_gumbel_sample(_ptr(flat), stride, dt, rows, V, ctypes.c_float(T),
                                        ctypes.c_uint64(seed), ctypes.c_uint64(offset), _ptr(tokens),
                                        _ptr(ws), ws.numel(), _stream(logits.device)))
    return tokens.reshape(lead)


class VerifyPlan:
    """A verify call bound once to fixed input and output tensors, so that repeated
    launches (a decode loop, a benchmark) only pay for the C call.  `run(seed,
    offset)` enqueues mtp_verify on the current stream and returns the outputs
    dict, whose tensors are overwritten by every run."""

    def __init__(self, target, draft, draft_tokens=None, target_only=False, temperature=None):
        self.lib = load()
        B, G1, V = target.shape
        self.shape = (B, G1 - 1, V)
        nbytes = ctypes.c_size_t()
        dt = _dtype_code(target)
        if target_only:                                               # greedy draft tokens
            self.inputs = (target, draft)                             # keeps the pointers alive
            self.out = verify_target_only(target, draft, 0, 0)        # validates, allocates, warms
            check(self.lib.mtp_verify_target_only_workspace_size(B, G1 - 1, V, dt, ctypes.byref(nbytes)))
            self._head = (_ptr(target), target.stride(1), _ptr(draft), draft.stride(1), dt, B, G1 - 1, V)
            o = self.out
            mid = (_ptr(o["accept"]), _ptr(o["accepted_len"]), _ptr(o["next_token"]), _ptr(o["draft_token"]),
                   _ptr(o["p_yhat"]), _ptr(o["rs_better"]))
            self._fn = self.lib.mtp_verify_target_only
        elif temperature is not None:                                 # Gumbel-max row samples
            draft_tokens = draft_tokens.contiguous()
            self.inputs = (target, draft, draft_tokens)
            self.out = verify_gumbel(target, draft, draft_tokens, temperature, 0, 0)
            check(self.lib.mtp_verify_gumbel_workspace_size(B, G1 - 1, V, dt, ctypes.byref(nbytes)))
            self._head = (_ptr(target), target.stride(1), _ptr(draft), draft.stride(1), dt, B, G1 - 1, V,
                          _ptr(draft_tokens), ctypes.c_float(_check_temperature(temperature)))
            o = self.out
            mid = (_ptr(o["accept"]), _ptr(o["accepted_len"]), _ptr(o["next_token"]))
            self._fn = self.lib.mtp_verify_gumbel
        else:
            draft_tokens = draft_tokens.contiguous()
            self.inputs = (target, draft, draft_tokens)
            self.out = verify(target, draft, draft_tokens, 0, 0)
            check(self.lib.mtp_verify_workspace_size(B, G1 - 1, V, dt, ctypes.byref(nbytes)))
            self._head = (_ptr(target), target.stride(1), _ptr(draft), draft.stride(1), dt, B, G1 - 1, V,
                          _ptr(draft_tokens))
            o = self.out
            mid = (_ptr(o["accept"]), _ptr(o["accepted_len"]), _ptr(o["next_token"]))
            self._fn = self.lib.mtp_verify
        self.ws = workspace(target.device, nbytes.value)
        self._tail = mid + (_ptr(o["row_token"]), _ptr(o["overlap"]), _ptr(o["tv"]), _ptr(o["entropy"]),
                            _ptr(o["row_status"]), _ptr(self.ws), self.ws.numel(), _stream(target.device))

    def run(self, seed, offset=0):
        st = self._fn(*self._head, ctypes.c_uint64(seed), ctypes.c_uint64(offset), *self._tail)
        if st:
            check(st)
        return self.out


class TVPlan:
    """Forward and backward TV-loss calls bound to fixed tensors (see VerifyPlan)."""

    def __init__(self, target, draft, grad_dtype=None):
        self.lib = load()
        T, G, V, t_pos, t_head = _tv_layout(target, draft)
        self.inputs = (target, draft)
        dev = draft.device
        dt = _dtype_code(draft)
        self.loss, self.pos_loss, self.saved = tv_loss_fwd(target, draft)
        self.grad_loss = torch.ones(1, dtype=torch.float32, device=dev)
        self.grad = _grad_buffer(T, G, V, grad_dtype or draft.dtype, dev)
        nbytes = ctypes.c_size_t()
        check(self.lib.mtp_tv_loss_workspace_size(T, G, V, dt, int(t_head == 0), ctypes.byref(nbytes)))
        self.ws = workspace(dev, nbytes.value)
        s = _stream(dev)
        common = (_ptr(target), t_pos, t_head, _ptr(draft), draft.stride(0), draft.stride(1), dt, T, G, V)
        self._fwd = common + (_ptr(self.loss), _ptr(self.pos_loss), _ptr(self.saved), _ptr(self.ws),
                              self.ws.numel(), s)
        self._bwd = common + (_ptr(self.saved), _ptr(self.grad_loss), _ptr(self.grad), self.grad.stride(0),
                              self.grad.stride(1), _DTYPES[self.grad.dtype], s)
        check(self.lib.mtp_tv_loss_fwd_bwd_workspace_size(T, G, V, dt, int(t_head == 0), ctypes.byref(nbytes)))
        self.ws_fused = workspace(dev, nbytes.value) if nbytes.value > self.ws.numel() else self.ws
        self._fused = common + (_ptr(self.grad_loss), _ptr(self.loss), _ptr(self.pos_loss), _ptr(self.saved),
                                _ptr(self.grad), self.grad.stride(0), self.grad.stride(1),
                                _DTYPES[self.grad.dtype], _ptr(self.ws_fused), self.ws_fused.numel(), s)

    def forward(self):
        st = self.lib.mtp_tv_loss_fwd(*self._fwd)
        if st:
            check(st)
        return self.loss

    def backward(self):
        st = self.lib.mtp_tv_loss_bwd(*self._bwd)
        if st:
            check(st)
        return self.grad

    def fused(self):
        """Forward and backward in one sweep (loss, saved statistics and gradient)."""
        st = self.lib.mtp_tv_loss_fwd_bwd(*self._fused)
        if st:
            check(st)
        return self.grad


class TVTopKPlan:
    """Forward and backward top-K TV-loss calls bound to fixed tensors (see VerifyPlan)."""

    def __init__(self, target_idx, target_val, draft, grad_dtype=None):
        self.lib = load()
        T, G, V, K, k_pos, k_head = _topk_layout(target_idx, target_val, draft)
        self.inputs = (target_idx, target_val, draft)
        dev = draft.device
        dt = _dtype_code(draft)
        self.loss, self.pos_loss, self.saved = tv_topk_fwd(target_idx, target_val, draft)
        self.grad_loss = torch.ones(1, dtype=torch.float32, device=dev)
        self.grad = _grad_buffer(T, G, V, grad_dtype or draft.dtype, dev)
        nbytes = ctypes.c_size_t()
        check(self.lib.mtp_tv_topk_workspace_size(T, G, V, dt, ctypes.byref(nbytes)))
        self.ws = workspace(dev, nbytes.value)
        s = _stream(dev)
        common = (_ptr(target_idx), _ptr(target_val), k_pos, k_head, K, _ptr(draft), draft.stride(0),
                  draft.stride(1), dt, T, G, V)
        self._fwd = common + (_ptr(self.loss), _ptr(self.pos_loss), _ptr(self.saved), _ptr(self.ws),
                              self.ws.numel(), s)
        self._bwd = common + (_ptr(self.saved), _ptr(self.grad_loss), _ptr(self.grad), self.grad.stride(0),
                              self.grad.stride(1), _DTYPES[self.grad.dtype], s)

    def forward(self):
        st = self.lib.mtp_tv_topk_fwd(*self._fwd)
        if st:
            check(st)
        return self.loss

    def backward(self):
        st = self.lib.mtp_tv_topk_bwd(*self._bwd)
        if st:
            check(st)
        return self.grad


__all__ = ["verify", "verify_max_vocab", "verify_target_only", "verify_gumbel", "gumbel_sample", "tv_loss_fwd", "tv_loss_bwd",
           "tv_loss", "TVLoss", "tv_topk_fwd", "tv_topk_bwd", "tv_topk_loss", "TVTopKLoss", "MtpError",
           "workspace", "workspace_error", "VerifyPlan", "TVPlan", "TVTopKPlan", "tv_loss_fwd_bwd", "set_wait_limit",
           "set_chunk_vectors"]
