"""CPU float64 oracles (test infrastructure only): sigmoid attention
(``sigattn_oracle``, re-exported here) and, for the comparison workload,
softmax attention (``softmax_oracle``).

Imported by tests, the smoke check and the bench's CPU baseline; never by the
library.  Each module states what it computes and the readings it takes.
"""
from . import softmax_oracle
from .sigattn_oracle import (BIAS_MODES, attention, bias, head, head_backward,
                             head_forward, logistic, score_scale)

__all__ = ["softmax_oracle", "BIAS_MODES", "attention", "bias", "head", "head_backward",
           "head_forward", "logistic", "score_scale"]
