"""CPU float64 oracle (test infrastructure only; see oracle/logprob.py, oracle/compare.py, oracle/backward.py)."""
from .logprob import (  # noqa: F401
    entropy, linear_logits, linear_logprob_entropy, logprob_entropy, sample_targets,
    tempered_logits,
)
from .compare import METRIC_NAMES, logprob_compare  # noqa: F401
from .backward import linear_grads, linear_grads_sampled, logits_grad  # noqa: F401
