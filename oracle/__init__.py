"""CPU oracle of the Gated DeltaNet decode block -- TEST INFRASTRUCTURE.

Only the tests under ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The HIP path never imports, links or calls it, and it shares no code with the
HIP path: only the seeded input generator feeds both.

It is a plain, slow, step-by-step restatement of what the block computes, in
float64, with rounding to the storage types (bf16 / f32) at the points the
stock chain of separate kernels rounds them. See ``oracle/gdn.py``.
"""
from .gdn import (  # noqa: F401
    bf16_to_f64,
    f64_to_bf16,
    residual_add,
    gemma_rmsnorm,
    project_bf16,
    mxfp4_quantize,
    mxfp4_dequantize,
    project_mxfp4,
    split_qkvz,
    split_ba,
    conv_update,
    gates,
    l2norm,
    gated_delta_step,
    gated_delta_recurrence,
    gated_rmsnorm,
    decode_block,
    verify_block,
)
