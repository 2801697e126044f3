"""Pins of the oracle's hash routing and bias-balancing step.

Passage: "Qwen3.5-397B-A17B vs DeepSeek-V4-Pro", component table, router row, DeepSeek-V4-Pro
cell.  In the first three MoE layers a hash of the token id fixes the experts; the other layers
balance the experts without an auxiliary loss, with a bias speed of 0.001.

Readings (the pages give no more than that):
* the hash is a fixed table of k expert ids per token id, and the combine weights stay the
  router's (the same formulas as for the learned choice, on the table's experts, in the
  table's slot order);
* the balancing step is the published sign rule of auxiliary-loss-free balancing,
  b_e <- b_e + 0.001 * sign(mean load - load_e), loads counted over the batch's T*k
  assignments, one fp32 add per expert.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle


# ------------------------------------------------------------------ hash routing

def test_hashed_sqrt_softplus_hand_example():
    # logits [0, 1, -1]: s = sqrt(softplus(l)) = sqrt(ln 2), sqrt(ln(1 + e)), sqrt(ln(1 + 1/e))
    s = [math.sqrt(math.log(2.0)), math.sqrt(math.log(1.0 + math.e)),
         math.sqrt(math.log(1.0 + 1.0 / math.e))]
    ids, w = oracle.route_hashed(np.array([[0.0, 1.0, -1.0]]), [0], np.array([[2, 0]]),
                                 oracle.SQRT_SOFTPLUS, True, 2.5)
    assert ids.tolist() == [[2, 0]]                      # the table's order, not the scores'
    want = [2.5 * s[2] / (s[2] + s[0]), 2.5 * s[0] / (s[2] + s[0])]
    assert np.allclose(w[0], want, rtol=0, atol=1e-14)
    assert abs(w[0, 0] - 1.0050222) < 1e-7 and abs(w.sum() - 2.5) < 1e-14


def test_hashed_softmax_equals_library_softmax_of_the_table_experts():
    rng = np.random.default_rng(3)
    T, E, k, V = 40, 17, 5, 23
    logits = rng.standard_normal((T, E))
    table = np.stack([rng.permutation(E)[:k] for _ in range(V)]).astype(np.int32)
    tok = rng.integers(0, V, T).astype(np.int32)
    ids, w = oracle.route_hashed(logits, tok, table)
    assert np.array_equal(ids, table[tok])
    for t in range(T):
        assert np.allclose(w[t], softmax(logits[t, table[tok[t]]]), rtol=0, atol=1e-15)
    # not renormalised: the full softmax probability of each table expert
    _, w2 = oracle.route_hashed(logits, tok, table, renormalize=False)
    for t in range(T):
        assert np.allclose(w2[t], softmax(logits[t])[table[tok[t]]], rtol=0, atol=1e-15)


@pytest.mark.parametrize("score,gamma", [(oracle.SOFTMAX, 1.0), (oracle.SIGMOID, 1.0),
                                         (oracle.SQRT_SOFTPLUS, 2.5)])
def test_hashed_equals_learned_routing_when_the_table_holds_its_choice(score, gamma):
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((30, 12))
    ids, w, _ = oracle.route(logits, 4, score, True, gamma)
    h_ids, h_w = oracle.route_hashed(logits, np.arange(30), ids, score, True, gamma)
    assert np.array_equal(h_ids, ids)
    assert np.max(np.abs(h_w - w)) < 1e-15


def test_hashed_rejects_bad_tables_and_token_ids():
    l = np.zeros((2, 4))
    with pytest.raises(ValueError):
        oracle.route_hashed(l, [0, 5], np.array([[0, 1]] * 3))       # token id >= vocab
    with pytest.raises(ValueError):
        oracle.route_hashed(l, [0, 1], np.array([[0, 0], [1, 2]]))   # repeated expert
    with pytest.raises(ValueError):
        oracle.route_hashed(l, [0, 1], np.array([[0, 4], [1, 2]]))   # expert >= E


# ------------------------------------------------------------------ bias balancing

def test_bias_step_hand_example():
    # loads [3, 1, 2, 2] over 8 assignments and 4 experts: mean 2
    ids = np.array([[0, 1], [0, 2], [0, 3], [2, 3]])
    b = oracle.bias_update([0.5, -0.25, 0.0, 0.1], ids, 4)
    f = np.float32
    assert b.dtype == np.float32
    assert b[0] == f(0.5) - f(0.001)      # over-loaded: down by one step
    assert b[1] == f(-0.25) + f(0.001)    # under-loaded: up by one step
    assert b[2] == f(0.0) and b[3] == f(0.1)  # at the mean: unchanged


def test_bias_balanced_load_is_a_fixed_point():
    # every expert takes exactly T*k/E assignments (k > 1, so a per-token mean would differ)
    E, k = 6, 3
    ids = np.array([[(t + j) % E for j in range(k)] for t in range(12)])
    b0 = np.linspace(-0.2, 0.3, E).astype(np.float32)
    b0[0] = -0.0
    assert np.array_equal(oracle.bias_update(b0, ids, E).view(np.int32), b0.view(np.int32))


def test_bias_fractional_mean_and_idle_expert():
    # E = 3, T*k = 4: mean 4/3; loads [2, 2, 0]
    b = oracle.bias_update(np.zeros(3, np.float32), np.array([[0, 1], [0, 1]]), 3)
    s = np.float32(0.001)
    assert b.tolist() == [-s, -s, s]


def test_bias_steps_balance_a_skewed_router():
    # the point of the method: with a fixed skewed router, repeated steps flatten the load
    rng = np.random.default_rng(9)
    T, E, k = 512, 8, 2
    skew = np.log(np.arange(1, E + 1, dtype=np.float64) ** -1.1)
    logits = rng.standard_normal((T, E)) * 0.5 + skew
    b = np.zeros(E, np.float32)

    def imbalance(bias):
        ids, _, _ = oracle.route(logits, k, oracle.SQRT_SOFTPLUS, True, 2.5, bias)
        return np.bincount(ids.ravel(), minlength=E).max() / (T * k / E), ids

    start, _ = imbalance(b)
    for _ in range(400):
        _, ids = imbalance(b)
        b = oracle.bias_update(b, ids, E)
    end, _ = imbalance(b)
    assert start > 2.0 and end < 1.25, (start, end)
    assert b[0] < 0 < b[-1]   # the hot expert is pushed down, the cold one up


def test_bias_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.bias_update(np.zeros(4, np.float32), np.array([[0, 4]]), 4)


@pytest.mark.parametrize("kind", [oracle.SIGMOID, oracle.SQRT_SOFTPLUS])
def test_hashed_sigma_family_without_renormalising(kind):
    # the table's experts in its order, each weighted by gamma times its own unbiased score
    l = np.array([[0.0, 1.0, -1.0], [0.5, -2.0, 3.0]])
    table = np.array([[2, 0], [1, 2]], np.int32)
    ids, w = oracle.route_hashed(l, [0, 1], table, kind, False, 2.5)
    assert ids.tolist() == [[2, 0], [1, 2]]
    if kind == oracle.SIGMOID:
        sc = lambda v: 1.0 / (1.0 + math.exp(-v))  # noqa: E731
        assert w[0].tolist() == pytest.approx([2.5 * 0.2689414213699951, 1.25], abs=1e-15)
    else:
        sc = lambda v: math.sqrt(math.log1p(math.exp(v)))  # noqa: E731
        assert w[0].tolist() == pytest.approx([2.5 * 0.5596978537731075,
                                               2.5 * 0.8325546111576977], abs=1e-15)
    for t in range(2):
        want = [2.5 * sc(l[t, e]) for e in table[t]]
        assert np.allclose(w[t], want, rtol=1e-15, atol=0)
    # and the renormalised variant is the same vector over its sum, times gamma
    _, wr = oracle.route_hashed(l, [0, 1], table, kind, True, 2.5)
    assert np.allclose(wr, 2.5 * w / w.sum(axis=1, keepdims=True), rtol=1e-14, atol=0)
