"""Plain CPU oracle for the train/rollout numerical-mismatch metric.

TEST INFRASTRUCTURE ONLY. Imported by tests/, by __graft_entry__.smoke() and
by the cpu_baseline leg of bench.py, and by nothing else. The GPU library
never calls it and shares no code with it.

Source: [NV-RL] "NVIDIA强化学习加速实操：10分钟提升2倍训练效率" (nmedialink.com
repost of the NeMo-RL FP8 blog), section "FP8面临的关键挑战：数值分歧": the
rollout engine and the training engine score the same generated tokens, and
their disagreement is measured by the multiplicative probability error, the
mean over the n tokens of exp(|log p_train - log p_infer|) of each token's
log-probability under the two engines.  1 means the two agree exactly; the
page quotes 1.03 to 1.05 as the range usually accepted.

Readings (the page gives the formula only):

R20 A token's log-probability is the log-softmax of the logits of its
    position evaluated at the token's id, in float64:
        log p = logits[id] - log(sum_v exp(logits[v])).
R21 n is the number of scored tokens; the mean is the plain arithmetic mean
    of exp(|difference|) over them.
"""
from __future__ import annotations

import numpy as np


def token_logprobs(logits, ids):
    """R20: log-probabilities [n] of token ids [n] under logits [n, V], float64.

    The log-sum-exp is taken relative to each row's maximum so that large
    logits do not overflow; the result is the same quantity."""
    z = np.asarray(logits, np.float64)
    ids = np.asarray(ids, np.int64)
    if z.ndim != 2 or ids.shape != (z.shape[0],):
        raise ValueError("logits must be [n, V] and ids [n]")
    zmax = np.max(z, axis=1, keepdims=True)
    lse = zmax[:, 0] + np.log(np.sum(np.exp(z - zmax), axis=1))
    return z[np.arange(z.shape[0]), ids] - lse


def token_mult_prob_error(logp_train, logp_infer):
    """R21: (1/n) * sum_i exp(|logp_train_i - logp_infer_i|), float64."""
    a = np.asarray(logp_train, np.float64)
    b = np.asarray(logp_infer, np.float64)
    if a.shape != b.shape or a.ndim != 1 or a.size == 0:
        raise ValueError("two non-empty vectors of the same length are needed")
    return float(np.mean(np.exp(np.abs(a - b))))
