"""FP64 CPU oracle (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library under
``varlen_depthwise_causal_amd`` never imports it.
"""
from .oracle import (  # noqa: F401
    LIBRARY,
    POLICY_BF16,
    POLICY_FP32,
    SOURCE,
    Oracle,
    OracleError,
    backward,
    bf16_rne,
    build,
    compile_library,
    decode_bf16,
    decode_f32,
    decode_param,
    default,
    forward,
    silu,
    silu_grad,
)
