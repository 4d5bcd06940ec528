"""MI355X (gfx950) matmul over MLX-style affine-quantized packed weights.

The public calls mirror the C ABI of libmxq.so (``include/mxq.h``):
``mxq_qmv`` (decode), ``mxq_qmv_grouped`` (several decode projections per
launch), ``mxq_qmm`` (prefill), ``mxq_linear`` (either, plus an output bias),
``mxq_linear_act`` (the same for float16 or bfloat16 activations),
``mxq_linear_a8`` (int8 activations, quantized per row in the kernel),
``mxq_dequant`` (bit-exact standalone dequant) and ``mxq_pack`` (host packer),
plus diagnostics (``mxq_describe``, ``mxq_describe_grouped``) and the split
workspace controls (``mxq_release_workspaces``, ``mxq_workspace_bytes``).
"""

from ._lib import (  # noqa: F401
    MXQ_BF16,
    MXQ_ERR_HIP,
    MXQ_ERR_INVALID_ARG,
    MXQ_ERR_MISALIGNED,
    MXQ_ERR_UNSUPPORTED,
    MXQ_F16,
    MXQ_F32,
    MXQ_OK,
    MxqError,
    load,
    mxq_dequant,
    mxq_describe,
    mxq_describe_grouped,
    mxq_linear,
    mxq_linear_a8,
    mxq_linear_act,
    mxq_pack,
    mxq_qmm,
    mxq_qmm_noalloc,
    mxq_qmv,
    mxq_qmv_grouped,
    mxq_release_workspaces,
    mxq_workspace_bytes,
    QmvProblem,
)
