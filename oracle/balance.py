"""Quantile Balancing of the expert selection bias, in fp64 on the CPU.

TEST INFRASTRUCTURE ONLY (part of the oracle; see ``oracle/__init__``).

What the pages state: during training each expert's selection bias is updated
from the distribution of that expert's score margins, so that its routed token
count drifts toward a target load, replacing an auxiliary balancing loss
("Kimi K3 and the New Open-Weights Moat: Inference Efficiency", section "How
the router picks 16 of 896", Fig. 2 and the paragraph after it); allocation is
derived from quantiles of the router scores directly ("What Kimi K3 asks of
the hardware", section "Width: 896 experts and the interconnect").  No formula
is printed.  The reading taken here is the plainest one those sentences
support:

* target load: ``n = round(T * k / E)`` tokens per expert (an exact half
  goes to the even integer), clamped to ``[1, T - 1]`` (a uniform load);
* margin of expert ``e`` on token ``t``: its selection key (sigmoid score plus
  selection bias) minus the k-th largest key among the token's *other*
  experts -- expert ``e`` is routed token ``t`` exactly when its margin is
  positive;
* quantile: ``Q_e`` = the midpoint of ``e``'s n-th and (n+1)-th largest
  margins over the batch, so that shifting ``e``'s bias by ``-Q_e`` alone
  would route exactly ``n`` tokens to it;
* update: ``b_e <- b_e - eta * Q_e`` for every expert at once, step
  ``eta`` in ``(0, 1]``.

Parity unpinned beyond this reading: the checks in
``tests/test_oracle_balance.py`` pin the reading's own consequences (exact
single-expert counts, a bisection search for the bias interval, invariance
to a common bias shift, loads converging on a skewed batch), not a printed
value.
"""

from __future__ import annotations

import numpy as np


def keys(logits: np.ndarray, bias: np.ndarray, decide=np.float32) -> np.ndarray:
    """Selection keys: sigmoid score plus selection bias (the router of the
    Moat page's Fig. 2), rounded to ``decide`` where the GPU rounds."""
    lg = np.asarray(logits, dtype=np.float64)
    s = 1.0 / (1.0 + np.exp(-lg))
    if decide is not None:
        s = s.astype(decide).astype(np.float64)
    kk = s + np.asarray(bias, dtype=np.float64)[None, :]
    if decide is not None:
        kk = kk.astype(decide).astype(np.float64)
    return kk


def margins(key: np.ndarray, k: int) -> np.ndarray:
    """[T][E] margins: each key minus the k-th largest key among the token's
    other experts.  For a routed expert (key at or above the token's k-th
    largest) that is the (k+1)-th largest key of the token, otherwise the k-th."""
    T, E = key.shape
    assert 1 <= k < E
    srt = -np.sort(-key, axis=1)          # descending per token
    kth = srt[:, k - 1][:, None]
    k1th = srt[:, k][:, None]
    return key - np.where(key >= kth, k1th, kth)


def target_load(T: int, E: int, k: int) -> int:
    n = int(round(T * k / E))
    return min(max(n, 1), T - 1)


def quantiles(m: np.ndarray, n: int) -> np.ndarray:
    """Per expert: midpoint of the n-th and (n+1)-th largest margins."""
    srt = -np.sort(-m, axis=0)            # descending per expert (column)
    return 0.5 * (srt[n - 1] + srt[n])


def update(logits: np.ndarray, bias: np.ndarray, k: int, eta: float = 1.0, decide=np.float32):
    """One Quantile Balancing step: returns (new bias, Q) in fp64."""
    key = keys(logits, bias, decide)
    T, E = key.shape
    n = target_load(T, E, k)
    q = quantiles(margins(key, k), n)
    return np.asarray(bias, dtype=np.float64) - eta * q, q


def loads(logits: np.ndarray, bias: np.ndarray, k: int, decide=np.float32) -> np.ndarray:
    """Tokens routed to each expert: top-k of the keys, ties to the lower id."""
    key = keys(logits, bias, decide)
    T, E = key.shape
    eidx = np.arange(E)
    cnt = np.zeros(E, dtype=np.int64)
    for t in range(T):
        order = np.lexsort((eidx, -key[t]))
        cnt[order[:k]] += 1
    return cnt
