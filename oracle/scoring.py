"""Oracle for the teacher-forced scoring pass over finished experience.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg; the product path never calls it.

After generation, the PPO step needs the log-probability of every generated token
under the actor and under the frozen reference model (DeepSpeed-Chat paper summary,
section on the RLHF pipeline: the training phase of step 3 uses the reference
model's log-probabilities for the KL term, and PPO scores the actor's own tokens).
Both are the same computation on the finished sequence, prompt followed by answer,
with the answer given rather than generated ("teacher forcing").  The pages give no
formula; the reading taken here is the plain one:

    lp[b, j] = log softmax(logits of the prefix seq[b, :S_p + j])[seq[b, S_p + j]]

for j = 0 .. S - S_p - 1, where the logits of a prefix are the LM head at its last
position (the final LayerNorm of that position's hidden state times the tied
embedding), at temperature 1.  Written out by definition: one causal pass over the
whole sequence with no cache (``OracleModel.hidden``), the head at positions
S_p - 1 .. S - 2, log-softmax in float64, and the gather of the next token.
"""
from __future__ import annotations

import numpy as np

from oracle import opt_he as O
from oracle.sampling import logsumexp


def teacher_forced_logprobs(model: O.OracleModel, seq, prompt_len: int) -> np.ndarray:
    """Log-probabilities [B, S - prompt_len] (float64) of seq[:, prompt_len:] given
    everything before each of them; seq is [B, S] with 1 <= prompt_len < S."""
    seq = np.asarray(seq).astype(np.int64)
    B, S = seq.shape
    if not 1 <= prompt_len < S:
        raise ValueError("need 1 <= prompt_len < S")
    h = model.hidden(seq, 0, None)[:, prompt_len - 1:S - 1]        # predicts tokens prompt_len .. S-1
    return logprobs_from_logits(model.lm_logits(h), seq[:, prompt_len:])


def logprobs_from_logits(logits, target) -> np.ndarray:
    """log softmax(logits)[target] along the last axis: logits [..., V], target [...]."""
    logits = np.asarray(logits, dtype=np.float64)
    target = np.asarray(target).astype(np.int64)
    picked = np.take_along_axis(logits, target[..., None], axis=-1)[..., 0]
    return picked - logsumexp(logits, axis=-1)
