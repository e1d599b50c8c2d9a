"""tv_loss_amd: MTP rejection-sampling verification and the end-to-end TV loss
for AMD Instinct MI355X (gfx950).

The kernels live in libmtp.so (C ABI declared in include/mtp.h, sources in
csrc/); `tv_loss_amd.ops` is a thin PyTorch binding over it.
"""
from ._lib import (MAX_GAMMA, MTP_BF16, MTP_F32, ROW_BAD_DRAFT, ROW_BAD_TARGET, ROW_BAD_TOKEN,
                   ROW_RESIDUAL_EMPTY, ROW_SYNC_TIMEOUT, LIB_PATH, MtpError, load)
from .ops import (TVLoss, TVPlan, TVTopKLoss, TVTopKPlan, VerifyPlan, gumbel_sample, set_chunk_vectors, set_wait_limit, tv_loss,
                  tv_loss_bwd, tv_loss_fwd, tv_loss_fwd_bwd, tv_topk_bwd, tv_topk_fwd, tv_topk_loss, verify, verify_gumbel, verify_max_vocab,
                  verify_target_only, workspace, workspace_error)

__all__ = ["verify", "verify_max_vocab", "verify_target_only", "verify_gumbel", "gumbel_sample", "tv_topk_fwd", "tv_topk_bwd",
           "tv_topk_loss", "TVTopKLoss", "TVTopKPlan", "tv_loss_fwd", "tv_loss_bwd", "tv_loss_fwd_bwd", "tv_loss", "TVLoss", "MtpError", "load", "workspace",
           "workspace_error", "set_wait_limit", "set_chunk_vectors", "VerifyPlan", "TVPlan", "LIB_PATH", "MTP_F32", "MTP_BF16",
           "ROW_BAD_TOKEN", "ROW_BAD_TARGET", "ROW_BAD_DRAFT", "ROW_RESIDUAL_EMPTY", "ROW_SYNC_TIMEOUT", "MAX_GAMMA"]
