"""CPU float64 oracle (test infrastructure only; see oracle/logprob.py)."""
from .logprob import (  # noqa: F401
    entropy, linear_logits, linear_logprob_entropy, logprob_entropy, sample_targets,
    tempered_logits,
)
