"""ctypes declarations for libmtp.so (the C ABI in include/mtp.h)."""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmtp.so")

MTP_F32 = 0
MTP_BF16 = 1

ROW_BAD_TOKEN = 1
ROW_BAD_TARGET = 2
ROW_BAD_DRAFT = 4
ROW_RESIDUAL_EMPTY = 8
ROW_SYNC_TIMEOUT = 16

MAX_GAMMA = 8
VERIFY_NOALLOC_SCRATCH_BYTES = 16 << 20   # MTP_VERIFY_NOALLOC_SCRATCH_BYTES

STATUS = {0: "MTP_OK", 1: "MTP_ERR_NULL", 2: "MTP_ERR_SHAPE", 3: "MTP_ERR_DTYPE", 4: "MTP_ERR_ALIGN",
          5: "MTP_ERR_WORKSPACE", 6: "MTP_ERR_DEVICE", 7: "MTP_ERR_LAUNCH"}

# name -> (restype, argtypes); one entry per function declared in include/mtp.h
_c = ctypes
_P = _c.c_void_p
SIGNATURES = {
    "mtp_verify_workspace_size": (_c.c_int, [_c.c_int32, _c.c_int32, _c.c_int32, _c.c_int,
                                             _c.POINTER(_c.c_size_t)]),
    "mtp_verify": (_c.c_int, [_P, _c.c_int64, _P, _c.c_int64, _c.c_int, _c.c_int32, _c.c_int32, _c.c_int32,
                              _P, _c.c_uint64, _c.c_uint64, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                              _c.c_size_t, _P]),
    "mtp_verify_noalloc": (_c.c_int, [_P, _c.c_int64, _P, _c.c_int64, _c.c_int, _c.c_int32, _c.c_int32, _c.c_int32,
                                      _P, _c.c_uint64, _c.c_uint64, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "mtp_verify_max_vocab": (_c.c_int, [_c.c_int, _c.POINTER(_c.c_int32)]),
    "mtp_verify_target_only_workspace_size": (_c.c_int, [_c.c_int32, _c.c_int32, _c.c_int32, _c.c_int,
                                                         _c.POINTER(_c.c_size_t)]),
    "mtp_verify_target_only": (_c.c_int, [_P, _c.c_int64, _P, _c.c_int64, _c.c_int, _c.c_int32, _c.c_int32,
                                          _c.c_int32, _c.c_uint64, _c.c_uint64, _P, _P, _P, _P, _P, _P, _P, _P,
                                          _P, _P, _P, _P, _c.c_size_t, _P]),
    "mtp_verify_gumbel_workspace_size": (_c.c_int, [_c.c_int32, _c.c_int32, _c.c_int32, _c.c_int,
                                                    _c.POINTER(_c.c_size_t)]),
    "mtp_verify_gumbel": (_c.c_int, [_P, _c.c_int64, _P, _c.c_int64, _c.c_int, _c.c_int32, _c.c_int32,
                                     _c.c_int32, _P, _c.c_float, _c.c_uint64, _c.c_uint64, _P, _P, _P, _P, _P,
                                     _P, _P, _P, _P, _c.c_size_t, _P]),
    "mtp_gumbel_sample_workspace_size": (_c.c_int, [_c.c_int32, _c.c_int32, _c.c_int,
                                                    _c.POINTER(_c.c_size_t)]),
    "mtp_gumbel_sample": (_c.c_int, [_P, _c.c_int64, _c.c_int, _c.c_int32, _c.c_int32, _c.c_float, _c.c_uint64,
                                     _c.c_uint64, _P, _P, _c.c_size_t, _P]),
    "mtp_tv_loss_workspace_size": (_c.c_int, [_c.c_int32, _c.c_int32, _c.c_int32, _c.c_int, _c.c_int32,
                                              _c.POINTER(_c.c_size_t)]),
    "mtp_tv_loss_fwd": (_c.c_int, [_P, _c.c_int64, _c.c_int64, _P, _c.c_int64, _c.c_int64, _c.c_int,
                                   _c.c_int32, _c.c_int32, _c.c_int32, _P, _P, _P, _P, _c.c_size_t, _P]),
    "mtp_tv_loss_bwd": (_c.c_int, [_P, _c.c_int64, _c.c_int64, _P, _c.c_int64, _c.c_int64, _c.c_int,
                                   _c.c_int32, _c.c_int32, _c.c_int32, _P, _P, _P, _c.c_int64, _c.c_int64,
                                   _c.c_int, _P]),
    "mtp_tv_loss_fwd_bwd_workspace_size": (_c.c_int, [_c.c_int32, _c.c_int32, _c.c_int32, _c.c_int, _c.c_int32,
                                                      _c.POINTER(_c.c_size_t)]),
    "mtp_tv_loss_fwd_bwd": (_c.c_int, [_P, _c.c_int64, _c.c_int64, _P, _c.c_int64, _c.c_int64, _c.c_int,
                                       _c.c_int32, _c.c_int32, _c.c_int32, _P, _P, _P, _P, _P, _c.c_int64,
                                       _c.c_int64, _c.c_int, _P, _c.c_size_t, _P]),
    "mtp_tv_topk_workspace_size": (_c.c_int, [_c.c_int32, _c.c_int32, _c.c_int32, _c.c_int,
                                              _c.POINTER(_c.c_size_t)]),
    "mtp_tv_topk_fwd": (_c.c_int, [_P, _P, _c.c_int64, _c.c_int64, _c.c_int32, _P, _c.c_int64, _c.c_int64, _c.c_int,
                                   _c.c_int32, _c.c_int32, _c.c_int32, _P, _P, _P, _P, _c.c_size_t, _P]),
    "mtp_tv_topk_bwd": (_c.c_int, [_P, _P, _c.c_int64, _c.c_int64, _c.c_int32, _P, _c.c_int64, _c.c_int64, _c.c_int,
                                   _c.c_int32, _c.c_int32, _c.c_int32, _P, _P, _P, _c.c_int64, _c.c_int64, _c.c_int,
                                   _P]),
    "mtp_workspace_error": (_c.c_int, [_P, _c.POINTER(_c.c_uint32), _P]),
    "mtp_set_wait_limit": (_c.c_uint64, [_c.c_uint64]),
    "mtp_set_chunk_vectors": (_c.c_int32, [_c.c_int32]),
    "mtp_status_string": (_c.c_char_p, [_c.c_int]),
    "mtp_last_error": (_c.c_char_p, []),
    "mtp_version": (_c.c_char_p, []),
}

_lib = None


class MtpError(RuntimeError):
    def __init__(self, status, detail):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


def load():
    """Load libmtp.so once.  Raises ImportError if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing; build it with `python -m tv_loss_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def check(status):
    if status != 0:
        raise MtpError(status, load().mtp_last_error().decode())
