"""CPU float64 oracle for sigmoid attention (test infrastructure only).

Imported by tests, the smoke check and the bench's CPU baseline; never by the
library.  See ``sigattn_oracle`` for what it computes and the readings it takes.
"""
from .sigattn_oracle import (BIAS_MODES, attention, bias, head, head_backward,
                             head_forward, logistic, score_scale)

__all__ = ["BIAS_MODES", "attention", "bias", "head", "head_backward",
           "head_forward", "logistic", "score_scale"]
