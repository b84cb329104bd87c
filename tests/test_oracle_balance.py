"""Pins of the Quantile Balancing oracle (CPU).

The pages give only what the update achieves -- each expert's routed count
moves toward a target load, driven by quantiles of its score margins -- so
these tests pin the consequences of the reading in ``oracle/balance.py``
rather than printed values: the quantile shift of one expert gives it exactly
the target count; a bisection on the routed count finds the same shift
without sorting margins; a common shift of every bias changes nothing; and
repeated updates flatten a skewed load.
"""

import numpy as np

from oracle import balance as qb


def _case(T=240, E=16, k=4, seed=3, skew=0.0):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E))
    if skew:
        ranks = rng.permutation(E) + 1.0
        p = ranks ** -skew
        lg = lg + np.log(E * p / p.sum())[None, :]
    bias = rng.standard_normal(E) * 0.05
    return lg, bias


def _count(key, e, k):
    """Tokens routed to expert e: stable top-k of the keys (ties to the lower id)."""
    order = np.argsort(-key, axis=1, kind="stable")[:, :k]
    return int((order == e).sum())


def test_target_load_of_the_k3_shape():
    assert qb.target_load(16384, 896, 16) == 293      # 16384 * 16 / 896 = 292.57
    assert qb.target_load(8192, 896, 16) == 146
    assert qb.target_load(10, 1000, 1) == 1            # clamped to at least one token


def test_target_load_ties_go_to_the_even_count():
    assert qb.target_load(140, 896, 16) == 2           # 2.5
    assert qb.target_load(20, 8, 1) == 2               # 2.5
    assert qb.target_load(60, 8, 1) == 8               # 7.5


def test_quantile_shift_gives_one_expert_exactly_the_target():
    lg, bias = _case()
    T, E, k = lg.shape[0], lg.shape[1], 4
    n = qb.target_load(T, E, k)
    _, q = qb.update(lg, bias, k, eta=1.0, decide=None)
    for e in range(E):
        b = bias.copy()
        b[e] -= q[e]
        assert _count(qb.keys(lg, b, decide=None), e, k) == n, e


def test_bisection_on_the_routed_count_finds_the_same_shift():
    lg, bias = _case(T=160, E=12, k=3, seed=5)
    k = 3
    key0 = qb.keys(lg, bias, decide=None)
    T, E = key0.shape
    n = qb.target_load(T, E, k)
    _, q = qb.update(lg, bias, k, eta=1.0, decide=None)

    def cnt(e, d):
        key = key0.copy()
        key[:, e] += d
        return _count(key, e, k)

    for e in range(E):
        # lowest shift reaching n tokens, highest shift keeping at most n
        lo, hi = -4.0, 4.0
        for _ in range(80):
            mid = 0.5 * (lo + hi)
            lo, hi = (lo, mid) if cnt(e, mid) >= n else (mid, hi)
        a = hi
        lo, hi = -4.0, 4.0
        for _ in range(80):
            mid = 0.5 * (lo + hi)
            lo, hi = (mid, hi) if cnt(e, mid) <= n else (lo, mid)
        c = lo
        assert a <= c + 1e-12
        assert abs(0.5 * (a + c) + q[e]) < 1e-9, (e, a, c, q[e])


def test_a_common_bias_shift_changes_no_quantile():
    lg, bias = _case(seed=7)
    _, q0 = qb.update(lg, bias, 4, decide=None)
    _, q1 = qb.update(lg, bias + 0.3, 4, decide=None)
    assert np.allclose(q0, q1, rtol=0, atol=1e-12)


def test_repeated_updates_flatten_a_skewed_load():
    lg, bias = _case(T=2048, E=64, k=4, seed=11, skew=1.1)
    k = 4
    n = qb.target_load(2048, 64, k)
    bias = np.zeros(64)
    first = qb.loads(lg, bias, k, decide=None)
    assert first.sum() == 2048 * k
    for _ in range(12):
        bias, _ = qb.update(lg, bias, k, eta=0.5, decide=None)
    last = qb.loads(lg, bias, k, decide=None)
    assert last.sum() == 2048 * k
    assert first.max() > 2.5 * n
    assert last.max() < 1.3 * n
    assert np.std(last) < np.std(first) / 5
