"""Seeded synthetic inputs for BLASST attention (shared by the tests, the oracle checks and the
benchmark).  This package only draws and lays out random inputs: it holds none of the method's
arithmetic (no softmax, no threshold, no skip rule)."""

from .gen import (  # noqa: F401
    PrefillInputs,
    DecodeInputs,
    prefill_inputs,
    decode_inputs,
    to_bf16_rne_numpy,
)
from .configs import CONFIGS, config_seed  # noqa: F401
