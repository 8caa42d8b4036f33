"""The stored input parameters of the workloads, checked against the oracle
(no GPU): the Mistral-shaped stack's clip factor gives the stated rate."""
import numpy as np

from oracle.clip_calibration import coded_bits
from synth import MISTRAL_CLIP_SIGMA, tensor_specs, weights


def test_mistral_clip_factor_gives_the_stated_rate():
    """LazyWeights streams its Mistral-7B at 3.89 bits per weight (LazyWeights
    abstract); the stored clip factor puts the coded stack (one-row chunks,
    64 lanes, stream words plus chunk offsets) at 3.90 +- 0.05 bits per
    weight on a layer the calibration did not search on."""
    ws = [(s.rows, s.cols, weights(s)) for s in tensor_specs("mistral_stack") if s.layer == 2]
    bits = coded_bits(ws, MISTRAL_CLIP_SIGMA, 64, 4096)
    assert abs(bits - 3.90) <= 0.05, bits
    assert abs(bits - 3.90) <= 0.005, bits   # every layer has the same distribution
