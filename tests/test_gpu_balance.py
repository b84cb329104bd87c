"""Quantile Balancing on the GPU (``moe_quantile_balance``) against the oracle
in ``oracle/balance.py``: the per-expert quantiles and the updated bias, the
single-expert exactness the reading implies, an in-place update, the K3 shape
(16384 tokens x 896 experts, top-16), and repeated updates on a Zipf-skewed
batch."""

import numpy as np
import pytest

from oracle import balance as qb
from tests.gpu_harness import say

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def LY():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from latent_routing_mxfp4_amd import layer
    return layer


def _logits(T, E, seed, skew=0.0):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E))
    if skew:
        ranks = rng.permutation(E) + 1.0
        p = ranks ** -skew
        lg = lg + np.log(E * p / p.sum())[None, :]
    return lg.astype(np.float32), (rng.standard_normal(E) * 0.05).astype(np.float32)


def _gpu(LY, lg, bias, k, eta=1.0, inplace=False):
    L = torch.from_numpy(lg).cuda()
    b = torch.from_numpy(bias).cuda()
    q = torch.empty_like(b)
    out = LY.quantile_balance(L, b, k, eta, out=b if inplace else None, quantiles=q)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64), q.cpu().numpy().astype(np.float64)


# (300, 1280): more experts than the threshold pass keeps in registers (keys in
# LDS); (16500, 24): more tokens than the selection keeps in registers (counts
# re-read from global memory).
@pytest.mark.parametrize("T,E,k", [(240, 16, 4), (1000, 64, 6), (513, 128, 8), (300, 1280, 6), (16500, 24, 2),
                                   (140, 896, 16), (20, 8, 1), (60, 8, 1)])   # the last three: T k / E ends in .5
def test_quantiles_and_bias_match_the_oracle(LY, T, E, k):
    say(f"quantile balance T={T} E={E} k={k}")
    lg, bias = _logits(T, E, seed=T + E)
    nb, q = _gpu(LY, lg, bias, k, eta=0.75)
    nb_ref, q_ref = qb.update(lg, bias, k, eta=0.75)
    assert np.abs(q - q_ref).max() <= 1e-6, np.abs(q - q_ref).max()
    assert np.abs(nb - nb_ref).max() <= 1e-6
    # the reading's defining property, on the GPU's own quantiles
    n = qb.target_load(T, E, k)
    key = qb.keys(lg, bias, decide=None)
    for e in range(E):
        kk = key.copy()
        kk[:, e] -= q[e]
        order = np.argsort(-kk, axis=1, kind="stable")[:, :k]
        assert int((order == e).sum()) == n, e


def test_in_place_update(LY):
    lg, bias = _logits(300, 32, seed=2)
    a, _ = _gpu(LY, lg, bias, 4, eta=0.5)
    b, _ = _gpu(LY, lg, bias, 4, eta=0.5, inplace=True)
    assert np.array_equal(a, b)


def test_k3_shape_16384_tokens_896_experts(LY):
    say("quantile balance at the K3 shape")
    lg, bias = _logits(16384, 896, seed=1004)
    nb, q = _gpu(LY, lg, bias, 16, eta=1.0)
    nb_ref, q_ref = qb.update(lg, bias, 16, eta=1.0)
    assert np.abs(q - q_ref).max() <= 1e-6, np.abs(q - q_ref).max()
    assert np.abs(nb - nb_ref).max() <= 1e-6


def test_repeated_updates_flatten_a_skewed_batch(LY):
    T, E, k = 4096, 128, 8
    lg, _ = _logits(T, E, seed=1005, skew=1.1)
    n = qb.target_load(T, E, k)
    bias = np.zeros(E, np.float32)
    first = qb.loads(lg, bias, k)
    ref = bias.astype(np.float64)
    for _ in range(8):
        gb, _ = _gpu(LY, lg, bias, k, eta=0.5)
        ref, _ = qb.update(lg, ref.astype(np.float32), k, eta=0.5)
        assert np.abs(gb - ref).max() <= 1e-5
        bias = gb.astype(np.float32)
    last = qb.loads(lg, bias, k)
    assert first.max() > 2 * n and last.max() < 1.3 * n
