"""CPU oracle (float64) of the Muon optimizer step.

TEST INFRASTRUCTURE ONLY: tests/, the smoke check and the benchmark's CPU
baseline use it; the product path never does. It shares no code with the GPU
library in newton_schulz_step_amd/.
"""
from .muon_oracle import (  # noqa: F401
    ADAM_DEFAULTS, DEFAULT_NS_METHOD, MUON_DEFAULTS, NS_A, NS_B, NS_C, NS_EPS,
    NS_METHODS, NS_STEPS, adamw_step, gram_scale, momentum_update, muon_step,
    newton_schulz_gram, newton_schulz_standard, normalise, orthogonalise, pack,
    partition_windows, problem_blocks, unpack, window_step)
from .rounding import round_to, storer  # noqa: F401
from . import planner  # noqa: F401,E402
