"""k-quant prefill MMQ for MI355X (gfx950).

q4_K / q6_K super-block weights times per-token q8 "pad40" activations,
int8 x int8 -> int32 sub-block dot products on the int8 MFMA, rescaled to
fp32 in a fused epilogue.  The compute is in libqig.so (hand-written HIP,
C ABI declared in include/qig.h); this package is its thin ctypes binding.
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    QigError,
    expand_q6k_dense,
    load,
    mmq_q4k,
    mmq_q4k_partials,
    mmq_q4k_prepared,
    mmq_q4k_prepared_q8t,
    mmq_q4k_prepared_streamk,
    mmq_q4k_q8t,
    mmq_q4k_q8t_noalloc,
    mmq_q4k_streamk,
    mmq_q6k,
    mmq_q6k_partials,
    mmq_q6k_prepared,
    mmq_q6k_prepared_q8t,
    mmq_q6k_prepared_streamk,
    mmq_q6k_q8t,
    mmq_q6k_streamk,
    new_workspace,
    prepare_q4k,
    prepare_q6k,
    prepared_bytes,
    q8_pad40_bytes,
    q8_tiled_bytes,
    quantize_q8_pad40,
    quantize_q8_tiled,
    workspace,
)
