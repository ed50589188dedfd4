"""CPU oracle of the ViT encoder forward (numpy float64).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the library's compute path, with which
it shares no code.  See oracle/encoder.py (the encoder), oracle/predictor.py
(the masked-latent predictor that follows it), oracle/head.py (the
attentive-pool head and classifier) and oracle/quant.py (the 8-bit block
weight format) for the step-by-step definitions and the
citations of the passages each one follows.

Parity status: every function here is pinned by a -m "not gpu" test against
something other than itself (brute force, a library special case, a closed
form, or a value the pages print), with one exception: the contents of the
sincos2d position *table* (an input, built by the workload generator, not by
this module) are parity unpinned because the pages print no values for it.
"""
from .encoder import *  # noqa: F401,F403
from .predictor import id_positions, predictor_forward  # noqa: F401
from .head import attentive_pool_forward, cross_attention_pool  # noqa: F401
from . import quant  # noqa: F401
