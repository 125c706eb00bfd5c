"""CPU oracle of the QoQ W4A8 per-group GEMM path.

Test infrastructure only: the test-suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it; the library never does.
"""
from .qoq_oracle import *  # noqa: F401,F403
from .qoq_oracle import (GROUP, W_QMAX, X_QMAX, U4_MAX, rne_div,  # noqa: F401
                         quantize_weights_level0, quantize_weights_level1,
                         dequantize_level1, quantize_activations, contract,
                         epilogue_fp32, epilogue, pack_weights,
                         quantize_pack_weights, w4a8_reference)
