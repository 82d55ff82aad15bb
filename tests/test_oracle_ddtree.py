"""Pins of the DDTree construction oracle (oracle/ddtree.py).

* the DDTree notes §6 worked example (vocab {A, B, C, D}, 3 positions,
  budget 6): its tree [A], [B], [A,B], [A,A], [B,B], [A,B,C] with flattened
  positions [0, 1, 1, 2, 2, 2, 3] (the page's marginals are lost in the
  extracted text; the ones below are chosen so that this is the top-6 set);
* brute force: the popped set is the B highest-scoring prefixes over every
  tuple of per-depth ranks (§4.2), popped in descending score (§5.3);
* prefix closure (Proposition 2): every node's parent comes before it;
* Lemma 1 (§4.3): the heap over each depth's top-min(B, V) ranks pops the
  same prefixes as over the whole vocab.
"""

import itertools

import numpy as np
import pytest

from oracle import ddtree as DD
from oracle import tree as T


def test_worked_example_tree():
    A, B, C, D = range(4)
    q = np.array([[0.6, 0.4, 1e-3, 1e-3],     # position 1
                  [0.45, 0.55, 1e-3, 1e-3],   # position 2
                  [1e-3, 1e-3, 0.75, 0.2]])   # position 3
    par, tok = DD.build_tree(np.log(q), 6)
    assert len(par) == 6
    paths = set()
    for i in range(6):
        paths.add(tuple(int(tok[j]) for j in T.ancestor_path(i, par)))
    assert paths == {(A,), (B,), (A, B), (A, A), (B, B), (A, B, C)}
    depths = sorted(T.depth_of(i, par) + 1 for i in range(6))
    assert [0] + depths == [0, 1, 1, 2, 2, 2, 3]


def _score(logq, ranks):
    return sum(logq[d][r] for d, r in enumerate(ranks))


@pytest.mark.parametrize("seed, V, L, budget", [(0, 5, 3, 8), (1, 4, 4, 20), (2, 6, 2, 30), (3, 3, 5, 50)])
def test_top_b_against_brute_force(seed, V, L, budget):
    rng = np.random.default_rng(seed)
    z = rng.standard_normal((L, V)) * 2
    K = min(budget, V)
    toks, logq = zip(*(DD.depth_topk(z[d], K) for d in range(L)))
    popped = DD.best_first(logq, budget)
    allp = [r for d in range(1, L + 1) for r in itertools.product(range(K), repeat=d)]
    allp.sort(key=lambda r: -_score(logq, r))
    assert set(popped) == set(allp[:len(popped)])
    sc = [_score(logq, r) for r in popped]
    assert all(sc[i] >= sc[i + 1] - 1e-12 for i in range(len(sc) - 1))
    par, tok = DD.build_tree(z, budget)
    assert T.parents_valid(par)
    for i, r in enumerate(popped):
        assert tok[i] == toks[len(r) - 1][r[-1]]


def test_depth_topk_order_and_normalisation():
    z = np.array([0.5, 2.0, 2.0, -1.0, 3.0, 2.0], np.float32)
    toks, logq = DD.depth_topk(z, 4)
    assert toks.tolist() == [4, 1, 2, 5]          # ties by token id
    assert abs(np.exp(logq).sum() - 1.0) < 1e-12  # renormalised over the kept four


def test_lemma1_topk_suffices():
    rng = np.random.default_rng(7)
    L, V, budget = 3, 40, 12
    logq_full = []
    for _ in range(L):
        p = rng.dirichlet(np.ones(V))
        logq_full.append(np.sort(np.log(p))[::-1])
    full = DD.best_first(logq_full, budget)
    trunc = DD.best_first([row[:min(budget, V)] for row in logq_full], budget)
    assert full == trunc
