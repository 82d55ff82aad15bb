"""Pins of the sampled-walk oracle (oracle/sampling.py).

Temperature-sampling walk (DDTree notes §7.2-7.3; decoding page, "Gumbel Max技巧"):
* with zero noise and a power-of-two temperature the choice is the greedy argmax;
* a hand-computed row, ties to the lowest index;
* the Gumbel-max theorem: over many noise draws the choice frequencies match
  softmax(h / T) (the page's statement);
* losslessness (§7.3): the emitted tokens are distributed like plain
  autoregressive sampling from the target, whatever tokens the tree holds.

Stochastic min(1, p/q) walk ("02 · Token Tree 与 Tree Attention" §4):
* a hand-computed two-candidate case, residual included;
* q = p makes every first child accepted;
* losslessness of the rule when the children are draws from q: the first
  emitted token follows p at the root, the second follows the target's
  distribution after the first.
"""

import numpy as np
import pytest

from oracle import accept as A
from oracle import sampling as S


def test_zero_noise_is_greedy():
    rng = np.random.default_rng(1)
    rows = rng.standard_normal((50, 300)).astype(np.float32)
    rows[3, 7] = rows[3, 9] = rows[3].max() + 1  # a tie: lowest index
    zero = np.zeros_like(rows)
    greedy = A.row_argmax(rows.astype(np.float64))
    for T in (1.0, 0.5, 2.0, 0.125):  # powers of two scale exactly
        assert S.sampled_choice(rows, T, zero) == greedy
    assert greedy[3] == 7


def test_hand_computed_row():
    # x / T with T = 0.5 is 2x: [2, 4, 1, 4]; + g = [2.3, 3.0, 1.9, 4.0] -> index 3
    x = np.array([[1.0, 2.0, 0.5, 2.0]], np.float32)
    g = np.array([[0.3, -1.0, 0.9, 0.0]], np.float32)
    assert S.sampled_choice(x, 0.5, g) == [3]
    # equal perturbed values at 1 and 3 (4 + 0 = 3.5 + 0.5): the lower index wins
    g2 = np.array([[0.0, 0.0, 0.0, -0.5]], np.float32)
    x2 = np.array([[1.0, 2.0, 0.5, 2.25]], np.float32)
    assert S.sampled_choice(x2, 0.5, g2) == [1]
    # T = 4: x / T = 0.25 x exactly
    assert np.array_equal(S.perturbed_rows(np.array([[8.0, -4.0]], np.float32), 4.0, np.zeros((1, 2), np.float32)),
                          np.array([[2.0, -1.0]], np.float32))


def test_gumbel_max_frequencies_match_softmax():
    h = np.array([0.5, 1.0, -0.3, 2.0, 1.1], np.float32)
    T = 0.7
    n = 200_000
    rng = np.random.default_rng(11)
    g = rng.gumbel(size=(n, h.size)).astype(np.float32)
    ch = np.argmax(S.perturbed_rows(np.broadcast_to(h, (n, h.size)), T, g), axis=1)
    freq = np.bincount(ch, minlength=h.size) / n
    p = np.exp(h / T - (h / T).max())
    p /= p.sum()
    sigma = np.sqrt(p * (1 - p) / n)
    assert np.all(np.abs(freq - p) <= 5 * sigma), (freq, p)


def _ar_target(V, rng):
    """A target defined on prefixes: p0 at the root, P1[t] after token t."""
    p0 = rng.dirichlet(np.ones(V))
    P1 = rng.dirichlet(np.ones(V), size=V)
    return p0, P1


def test_temperature_walk_is_lossless():
    # tree: root children tokens [1, 3]; node 0 (token 1) has children tokens [0, 2]
    V, T = 4, 1.0
    parents = [-1, -1, 0, 0]
    tokens = [1, 3, 0, 2]
    rng = np.random.default_rng(5)
    p0, P1 = _ar_target(V, rng)
    # logits whose softmax is the target: log p (T = 1); row of node j = target after its token
    rows = np.log(np.stack([p0, P1[1], P1[3], P1[0], P1[2]])).astype(np.float32)
    n = 40_000
    first = np.zeros(V)
    second = np.zeros((V, V))
    for _ in range(n):
        g = rng.gumbel(size=rows.shape).astype(np.float32)
        ch = S.sampled_choice(rows, T, g)
        w = A.greedy_walk(ch, tokens, parents, 8)
        seq = w["accepted_tokens"] + [w["bonus"]]
        first[seq[0]] += 1
        if len(seq) > 1:
            second[seq[0], seq[1]] += 1
    f = first / n
    # float32 logits: the target is p0 up to float32 rounding of log p
    ps = np.exp(rows.astype(np.float64))
    ps /= ps.sum(axis=1, keepdims=True)
    assert np.all(np.abs(f - ps[0]) <= 5 * np.sqrt(ps[0] * (1 - ps[0]) / n) + 1e-6), (f, ps[0])
    # after token 1 (node 0 accepted) the next token follows the target's row after token 1
    c = second[1] / second[1].sum()
    m = second[1].sum()
    assert np.all(np.abs(c - ps[1]) <= 5 * np.sqrt(ps[1] * (1 - ps[1]) / m) + 1e-6), (c, ps[1])


def test_stochastic_hand_computed():
    # V = 3, T = 1, root with two children tokens [0, 1]; leaves
    logits = np.log(np.array([[0.5, 0.2, 0.3], [0.1, 0.1, 0.8], [0.6, 0.2, 0.2]])).astype(np.float32)
    q = np.array([[0.25, 0.5, 0.25], [1 / 3, 1 / 3, 1 / 3], [1 / 3, 1 / 3, 1 / 3]], np.float32)
    p = S.softmax_f64(logits[0], 1.0)
    # child 0 (token 0): p/q = 0.5/0.25 > 1: accepted for any u < 1
    w = S.stochastic_walk(logits, 1.0, q, np.array([0.99, 0.0], np.float32), np.zeros((3, 3), np.float32),
                          [0, 1], [-1, -1], 4)
    assert w["accepted"] == [0] and w["accepted_tokens"] == [0]
    # the bonus at leaf 0 is the Gumbel-max sample of its p with zero noise: the mode, token 2
    assert w["bonus"] == 2
    # child 1 (token 1) tried first as node 0 this time: p(1)/q(1) = 0.2/0.5 = 0.4
    w = S.stochastic_walk(logits, 1.0, q, np.array([0.45, 0.3], np.float32), np.zeros((3, 3), np.float32),
                          [1, 0], [-1, -1], 4)
    # u0 = 0.45 >= 0.4: rejected; residual max(0, p - q) = [0.25, 0, 0.05] / 0.3 = [5/6, 0, 1/6];
    # node 1 (token 0): r(0)/q(0) = (5/6)/0.25 > 1: accepted
    assert w["accepted"] == [1] and w["accepted_tokens"] == [0]
    w = S.stochastic_walk(logits, 1.0, q, np.array([0.35, 0.3], np.float32), np.zeros((3, 3), np.float32),
                          [1, 0], [-1, -1], 4)
    assert w["accepted"] == [0] and w["accepted_tokens"] == [1]  # u0 = 0.35 < 0.4
    # every child rejected: the correction comes from the residual; here token 2 only
    # has mass left after rejecting tokens 0 and 1 with q concentrated on them
    q2 = np.array([[0.5, 0.5, 0.0], [1, 0, 0], [1, 0, 0]], np.float32)
    w = S.stochastic_walk(logits, 1.0, q2, np.array([0.9999, 0.9999], np.float32), np.zeros((3, 3), np.float32),
                          [0, 1], [-1, -1], 4)
    # p(0)/q(0) = 1.0 > u: accepted -- so use a target below q on both tokens
    assert w["accepted"] == [0]
    logits3 = np.log(np.array([[0.2, 0.2, 0.6], [1, 1, 1], [1, 1, 1]])).astype(np.float32)
    w = S.stochastic_walk(logits3, 1.0, q2, np.array([0.9, 0.9], np.float32),
                          np.array([[5.0, 5.0, -5.0]] * 3, np.float32), [0, 1], [-1, -1], 4)
    # 0.9 * 0.5 = 0.45 >= 0.2 rejects token 0; residual max(0, p - q) = [0, 0, 0.6] / 0.6, so r(1) = 0 rejects token 1;
    # the correction is token 2 whatever the noise on the other tokens
    assert w["accepted"] == [] and w["bonus"] == 2
    assert abs(p[0] - 0.5) < 1e-6


def test_q_equal_p_accepts_first_children():
    rng = np.random.default_rng(2)
    V = 50
    parents = [-1, -1, 0, 0, 2, 1]
    tokens = [3, 4, 5, 6, 7, 8]
    logits = rng.standard_normal((7, V)).astype(np.float32)
    q = np.stack([S.softmax_f64(r, 1.0) for r in logits]).astype(np.float32)
    u = rng.random(6).astype(np.float32) * 0.999
    w = S.stochastic_walk(logits, 1.0, q, u, np.zeros((7, V), np.float32), tokens, parents, 8)
    assert w["accepted"] == [0, 2, 4]  # first child at every level down to a leaf


@pytest.mark.parametrize("seed", [3, 4])
def test_stochastic_walk_is_lossless(seed):
    """Children drawn i.i.d. from the draft q; the emitted tokens must follow the
    target: first ~ p0, second | first = t ~ P1[t] (the rule's guarantee)."""
    V, n = 4, 30_000
    rng = np.random.default_rng(seed)
    p0, P1 = _ar_target(V, rng)
    q0 = rng.dirichlet(np.ones(V))
    Q1 = rng.dirichlet(np.ones(V), size=V)
    first = np.zeros(V)
    second = np.zeros((V, V))
    for _ in range(n):
        # two root children drawn from q0; the first child has two children drawn from Q1[its token]
        a, b = rng.choice(V, 2, p=q0)
        c, d = rng.choice(V, 2, p=Q1[a])
        parents = [-1, -1, 0, 0]
        tokens = [a, b, c, d]
        rows = np.log(np.stack([p0, P1[a], P1[b], np.full(V, 1.0 / V), np.full(V, 1.0 / V)])).astype(np.float32)
        qr = np.stack([q0, Q1[a], Q1[b], np.full(V, 1.0 / V), np.full(V, 1.0 / V)]).astype(np.float32)
        u = rng.random(4).astype(np.float32)
        g = rng.gumbel(size=(5, V)).astype(np.float32)
        w = S.stochastic_walk(rows, 1.0, qr, u, g, tokens, parents, 8)
        seq = w["accepted_tokens"] + [w["bonus"]]
        first[seq[0]] += 1
        if len(seq) > 1:
            second[seq[0], seq[1]] += 1
    f = first / n
    tol = 5 * np.sqrt(p0 * (1 - p0) / n) + 2e-3
    assert np.all(np.abs(f - p0) <= tol), (f, p0)
    for t in range(V):
        m = second[t].sum()
        if m < 2000:
            continue
        c = second[t] / m
        assert np.all(np.abs(c - P1[t]) <= 5 * np.sqrt(P1[t] * (1 - P1[t]) / m) + 2e-3), (t, c, P1[t])
