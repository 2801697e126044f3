"""Pins of the oracle's router (logits, scores, top-k, weights) and permutation.

Passages (archdiff.com, "Qwen3.5-397B-A17B vs DeepSeek-V4-Pro", component table, router row):
Qwen3.5 cell -- one linear map gives a logit per expert, then softmax, the k largest kept and
renormalised, no selection bias; DeepSeek-V4-Pro cell -- sqrt-softplus scores, a per-expert
bias that only affects which k are picked, the picked scores normalised and multiplied by 2.5.
Blueprint router box: sigma or sqrt-softplus scores balanced by a bias.  The tie-break (lower
expert index wins) is a reading: the pages are silent on it.
"""
import itertools
import math

import numpy as np
import pytest
from scipy.special import softmax

import oracle

LN2 = math.log(2.0)


def test_logits_match_numpy_matmul():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((9, 40))
    wr = rng.standard_normal((40, 12)).astype(np.float32)
    z = rng.standard_normal(12).astype(np.float32)
    got = oracle.router_logits(x, wr, z)
    ref = x @ wr.astype(np.float64) + z.astype(np.float64)
    assert np.max(np.abs(got - ref)) < 1e-12
    # bf16 storage: the top 16 bits of fp32
    wb = (rng.standard_normal((40, 12)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    wb_val = (wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = oracle.router_logits(x, wb)
    assert np.max(np.abs(got - x @ wb_val)) < 1e-12
    # non-symmetric shape check: transposing W_r would not even fit
    assert got.shape == (9, 12)


def test_scores_closed_forms():
    sp = oracle.SQRT_SOFTPLUS
    assert oracle.score(sp, 0.0) == pytest.approx(math.sqrt(LN2), abs=1e-15)
    assert oracle.score(sp, 0.0) == pytest.approx(0.8325546111576977, abs=1e-15)
    assert oracle.score(sp, 1.0) == pytest.approx(math.sqrt(math.log(1 + math.e)), abs=1e-15)
    assert oracle.score(sp, -1.0) == pytest.approx(math.sqrt(math.log(1 + 1 / math.e)), abs=1e-15)
    # softplus(l) -> l for large l, -> e^l for very negative l
    assert oracle.score(sp, 50.0) == pytest.approx(math.sqrt(50.0), rel=1e-15)
    assert oracle.score(sp, -40.0) == pytest.approx(math.sqrt(math.exp(-40.0)), rel=1e-12)
    sg = oracle.SIGMOID
    assert oracle.score(sg, 0.0) == 0.5
    assert oracle.score(sg, 1.0) == pytest.approx(0.7310585786300049, abs=1e-15)
    assert oracle.score(sg, -1.0) == pytest.approx(0.2689414213699951, abs=1e-15)


def test_softmax_hand_example_with_tie():
    # logits [1, 0, 1]: experts 0 and 2 tie; the lower index wins the first slot
    l = np.array([[1.0, 0.0, 1.0]])
    ids, w, _ = oracle.route(l, 1)
    assert ids.tolist() == [[0]] and w[0, 0] == 1.0
    ids, w, _ = oracle.route(l, 2)
    assert ids.tolist() == [[0, 2]] and np.allclose(w, [[0.5, 0.5]], atol=1e-15)
    ids, w, _ = oracle.route(l, 3)
    e = math.e
    assert ids.tolist() == [[0, 2, 1]]
    assert np.allclose(w, [[e / (2 * e + 1), e / (2 * e + 1), 1 / (2 * e + 1)]], atol=1e-15)
    assert np.allclose(w, [[0.4223187982515182, 0.4223187982515182, 0.1553624034969636]],
                       atol=1e-12)


def test_sqrt_softplus_hand_example_bias_selects_but_does_not_weigh():
    l = np.array([[0.0, 1.0, -1.0]])
    s0, s1 = math.sqrt(LN2), math.sqrt(math.log(1 + math.e))
    b = np.array([0.3, 0.0, 0.0], np.float32)
    ids, w, s = oracle.route(l, 1, oracle.SQRT_SOFTPLUS, True, 2.5, b)
    assert ids.tolist() == [[1]] and w[0, 0] == pytest.approx(2.5, abs=1e-15)
    ids, w, s = oracle.route(l, 2, oracle.SQRT_SOFTPLUS, True, 2.5, b)
    assert ids.tolist() == [[1, 0]]
    assert np.allclose(w, [[2.5 * s1 / (s0 + s1), 2.5 * s0 / (s0 + s1)]], atol=1e-15)
    assert np.allclose(w, [[1.44801415, 1.05198585]], atol=1e-8)
    # a larger bias on expert 0 flips the order, never the weights
    ids, w2, _ = oracle.route(l, 2, oracle.SQRT_SOFTPLUS, True, 2.5,
                              np.array([0.4, 0, 0], np.float32))
    assert ids.tolist() == [[0, 1]]
    assert np.allclose(w2[0], w[0][::-1], atol=1e-15)
    # sigma scores on the same logits
    ids, w, s = oracle.route(l, 3, oracle.SIGMOID, True, 1.0)
    assert ids.tolist() == [[1, 0, 2]]
    assert np.allclose(s, [[0.7310585786300049, 0.5, 0.2689414213699951]], atol=1e-15)


def _brute_topk(key, k):
    """Exhaustive: the k-subset whose every member outranks every non-member under
    (key desc, index asc), listed in that order."""
    E = len(key)
    rank = lambda e: (-key[e], e)  # noqa: E731
    for sub in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in sub]
        if all(rank(a) < rank(b) for a in sub for b in rest):
            return sorted(sub, key=rank)
    raise AssertionError("no subset")


@pytest.mark.parametrize("score", [oracle.SOFTMAX, oracle.SIGMOID, oracle.SQRT_SOFTPLUS])
def test_topk_brute_force_and_lexsort(score):
    rng = np.random.default_rng(11 + score)
    T, E, k = 40, 9, 3
    # coarse logits so that ties occur often
    l = np.round(rng.standard_normal((T, E)) * 2) / 2
    b = (np.round(rng.uniform(-0.1, 0.1, E) * 20) / 20).astype(np.float32)
    sb = None if score == oracle.SOFTMAX else b
    ids, w, s = oracle.route(l, k, score, True, 2.5 if score else 1.0, sb)
    for t in range(T):
        if score == oracle.SOFTMAX:
            key = l[t]
        else:
            key = np.array([np.float32(np.float32(oracle.score(score, v)) + b[e])
                            for e, v in enumerate(l[t])], dtype=np.float64)
        assert ids[t].tolist() == _brute_topk(list(key), k)
        assert ids[t].tolist() == list(np.lexsort((np.arange(E), -key))[:k])


def test_softmax_weights_equal_library_softmax_of_selected():
    rng = np.random.default_rng(5)
    l = rng.standard_normal((50, 32)) * 3
    ids, w, _ = oracle.route(l, 6)
    sel = np.take_along_axis(l, ids, 1)
    assert np.max(np.abs(w - softmax(sel, axis=1))) < 1e-14
    # not renormalised: the full softmax probability of each selected expert
    ids, w, _ = oracle.route(l, 6, oracle.SOFTMAX, False, 1.0)
    assert np.max(np.abs(w - np.take_along_axis(softmax(l, axis=1), ids, 1))) < 1e-14


@pytest.mark.parametrize("score,gamma", [(oracle.SOFTMAX, 1.0), (oracle.SIGMOID, 1.0),
                                         (oracle.SQRT_SOFTPLUS, 2.5)])
def test_route_invariants(score, gamma):
    rng = np.random.default_rng(21)
    T, E, k = 200, 64, 7
    l = rng.standard_normal((T, E))
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    ids, w, s = oracle.route(l, k, score, True, gamma, None if score == oracle.SOFTMAX else b)
    assert np.all((ids >= 0) & (ids < E))
    assert all(len(set(r)) == k for r in ids.tolist())
    assert np.allclose(w.sum(1), gamma, atol=1e-13)
    assert np.all(w > 0)
    if score != oracle.SOFTMAX:
        # weights are proportional to the unbiased scores of the selected experts
        sc = np.vectorize(lambda v: oracle.score(score, v))(np.take_along_axis(l, ids, 1))
        assert np.allclose(w, gamma * sc / sc.sum(1, keepdims=True), atol=1e-14)
    else:
        assert np.all(np.diff(w, axis=1) <= 0)


def test_zero_input_special_case():
    # x = 0 gives zero logits: softmax picks 0..k-1 with 1/k each; sqrt-softplus scores all
    # equal sqrt(ln 2), so the bias alone decides and each weight is 2.5/k.
    T, E, k = 3, 10, 4
    l = np.zeros((T, E))
    ids, w, _ = oracle.route(l, k)
    assert ids.tolist() == [[0, 1, 2, 3]] * T and np.allclose(w, 1.0 / k, atol=1e-15)
    b = np.linspace(-0.1, 0.1, E).astype(np.float32)
    ids, w, s = oracle.route(l, k, oracle.SQRT_SOFTPLUS, True, 2.5, b)
    assert ids.tolist() == [[9, 8, 7, 6]] * T
    assert np.allclose(w, 2.5 / k, atol=1e-15) and np.allclose(s, math.sqrt(LN2), atol=1e-15)


def test_k_equals_E_and_bad_k():
    l = np.array([[0.5, -1.0, 2.0, 2.0]])
    ids, w, _ = oracle.route(l, 4)
    assert ids.tolist() == [[2, 3, 0, 1]]
    assert np.allclose(w[0], softmax(l[0])[[2, 3, 0, 1]], atol=1e-15)
    with pytest.raises(ValueError):
        oracle.route(l, 5)
    with pytest.raises(ValueError):
        oracle.route(l, 0)


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (37, 3, 8), (300, 10, 512), (0, 2, 4), (64, 2, 16)])
def test_permute_matches_stable_argsort(T, k, E):
    rng = np.random.default_rng(T + k + E)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k))
    ids = ids.astype(np.int32)
    off, perm, inv = oracle.permute(ids, E)
    flat = ids.ravel()
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(perm, order // k)
    assert np.array_equal(inv[order], np.arange(T * k))
    counts = np.bincount(flat, minlength=E)
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(counts)]))
    assert off[-1] == T * k and np.all(np.diff(off) >= 0)
    # rows of each expert segment are in ascending token order
    for e in range(E):
        seg = perm[off[e]:off[e + 1]]
        assert np.all(np.diff(seg) > 0)


def test_permute_skewed_and_bad_id():
    ids = np.array([[3, 0], [3, 1], [3, 2], [0, 3]], np.int32)
    off, perm, inv = oracle.permute(ids, 5)
    assert off.tolist() == [0, 2, 3, 4, 8, 8]
    assert perm.tolist() == [0, 3, 1, 2, 0, 1, 2, 3]
    assert inv.tolist() == [4, 0, 5, 2, 6, 3, 1, 7]
    with pytest.raises(ValueError):
        oracle.permute(np.array([[5]], np.int32), 5)


# ---------------------------------------------------------------- weights without renormalising
# Router row of "Qwen3.5-397B-A17B vs DeepSeek-V4-Pro", DeepSeek-V4-Pro cell: the picked scores
# are normalised and then scaled.  With the normalisation switched off (renormalize = 0) each
# weight is gamma times the expert's own unbiased score: nothing is divided by the selected sum,
# gamma still applies, and the selection bias still only chooses.

SIG = [0.5, 0.7310585786300049, 0.2689414213699951]          # sigma(0), sigma(1), sigma(-1)
SQS = [0.8325546111576977, 1.145976303209723, 0.5596978537731075]  # sqrt(softplus(.)) of the same


def test_sigmoid_scores_without_renormalising_hand_example():
    l = np.array([[0.0, 1.0, -1.0]])
    ids, w, s = oracle.route(l, 3, oracle.SIGMOID, False, 2.5)
    assert ids.tolist() == [[1, 0, 2]]
    want = 2.5 * np.array([SIG[1], SIG[0], SIG[2]])
    assert np.allclose(w[0], want, rtol=0, atol=1e-15)
    assert np.allclose(w[0], [1.8276464465750123, 1.25, 0.6723535534249878], rtol=0, atol=1e-14)
    # not divided by the selected sum (that would give 2.5 in total) and gamma is applied
    assert abs(w.sum() - 2.5 * 1.5) < 1e-14
    assert np.allclose(s[0], [SIG[1], SIG[0], SIG[2]], rtol=0, atol=1e-15)


def test_sqrt_softplus_without_renormalising_hand_example():
    l = np.array([[0.0, 1.0, -1.0]])
    assert SQS[1] == pytest.approx(math.sqrt(math.log(1 + math.e)), abs=1e-15)
    assert SQS[2] == pytest.approx(math.sqrt(math.log(1 + 1 / math.e)), abs=1e-15)
    ids, w, _ = oracle.route(l, 2, oracle.SQRT_SOFTPLUS, False, 2.5)
    assert ids.tolist() == [[1, 0]]
    assert np.allclose(w[0], [2.5 * SQS[1], 2.5 * SQS[0]], rtol=0, atol=1e-15)
    # the bias flips the choice order; each weight stays gamma times its own score
    b = np.array([0.4, 0.0, 0.0], np.float32)
    ids, w, _ = oracle.route(l, 2, oracle.SQRT_SOFTPLUS, False, 2.5, b)
    assert ids.tolist() == [[0, 1]]
    assert np.allclose(w[0], [2.5 * SQS[0], 2.5 * SQS[1]], rtol=0, atol=1e-15)
    # k = 1: the weight is the score times gamma, not gamma
    ids, w, _ = oracle.route(l, 1, oracle.SQRT_SOFTPLUS, False, 1.0)
    assert ids.tolist() == [[1]] and w[0, 0] == pytest.approx(SQS[1], abs=1e-15)


@pytest.mark.parametrize("kind", [oracle.SIGMOID, oracle.SQRT_SOFTPLUS])
def test_sigma_family_without_renormalising_is_gamma_times_score(kind):
    # random logits and biases: w[t, j] = gamma * score(l[t, ids[t, j]]) for every slot, and the
    # renormalised weights are exactly these divided by their row sum times gamma
    rng = np.random.default_rng(21)
    T, E, k, gamma = 50, 33, 7, 1.75
    l = rng.standard_normal((T, E)) * 2
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    ids, w, _ = oracle.route(l, k, kind, False, gamma, b)
    ids_r, w_r, _ = oracle.route(l, k, kind, True, gamma, b)
    assert np.array_equal(ids, ids_r)   # renormalising never changes the choice
    f = (lambda v: 1 / (1 + np.exp(-v))) if kind == oracle.SIGMOID else \
        (lambda v: np.sqrt(np.logaddexp(0.0, v)))
    want = gamma * f(np.take_along_axis(l, ids, axis=1))
    assert np.allclose(w, want, rtol=1e-14, atol=0)
    assert np.allclose(w_r, gamma * w / w.sum(axis=1, keepdims=True), rtol=1e-14, atol=0)
