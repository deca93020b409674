"""CPU oracle for exact softmax attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import anything from here.  The GPU library (the
``io_aware_exact_fwd_amd`` package and its C ABI) never imports, links or
executes this code, and this code never imports the library.

``oracle.attention``  -- float64 definition of the forward and backward.
``oracle.bruteforce`` -- scalar pure-Python loops that pin the above.
``oracle.fp8``        -- 8-bit (E4M3) inputs: decoding and the exact result.
"""
from .attention import (attention_backward, attention_forward, attention_probs,
                        backward_dq_rows, check_cu_seqlens, default_scale, forward_rows,
                        probs_rows, to_f64,
                        varlen_backward, varlen_forward, varlen_forward_rows)
from .bruteforce import bf_backward, bf_forward
from .fp8 import dequantize, e4m3_to_f64, fp8_attention_forward

__all__ = [
    "attention_forward", "attention_backward", "attention_probs", "forward_rows",
    "backward_dq_rows", "default_scale", "to_f64", "bf_forward", "bf_backward",
    "varlen_forward", "varlen_backward", "varlen_forward_rows", "check_cu_seqlens",
    "e4m3_to_f64", "dequantize", "fp8_attention_forward", "probs_rows",
]
