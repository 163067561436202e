"""Pins of the oracle's offline lazy-layer selection (press-release page,
"LightTransfer method", steps 1-3: lazy ratio per layer measured on a set of
prompts; the 50% of layers with the highest ratio become streaming layers).

None of these retypes the oracle's loop: the selection is checked against its
definition by brute force over subsets with exact rational means, against the
queue (a different algorithm that reaches the same set on one prompt), and
against invariants of a mean.
"""
import itertools
import random
from fractions import Fraction

import pytest

import oracle


def brute_force_streaming(prompt_scores, C):
    """The unique set T of L - C layers such that every member ranks above
    every non-member under (exact mean score desc, layer index asc)."""
    P, L = len(prompt_scores), len(prompt_scores[0])
    mean = [sum(Fraction(row[l]) for row in prompt_scores) / P for l in range(L)]

    def above(a, b):
        return mean[a] > mean[b] or (mean[a] == mean[b] and a < b)

    found = []
    for T in itertools.combinations(range(L), L - C):
        rest = [x for x in range(L) if x not in T]
        if all(above(a, b) for a in T for b in rest):
            found.append(set(T))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("P", [1, 2, 3])
def test_offline_matches_brute_force_with_ties(P):
    rng = random.Random(100 + P)
    for _ in range(300):
        L = rng.randint(1, 7)
        C = rng.randint(0, L)
        scores = [[rng.choice([0.0, 0.25, 0.5, 0.75, 1.0]) for _ in range(L)] for _ in range(P)]
        mean, st = oracle.select_offline(scores, C)
        assert {l for l in range(L) if st[l]} == brute_force_streaming(scores, C)
        assert sum(st) == L - C
        for l in range(L):
            assert mean[l] == pytest.approx(sum(r[l] for r in scores) / P, abs=0, rel=1e-15)


def test_one_prompt_equals_the_queue():
    """On a single prompt the offline rule keeps the C lowest scores, which is
    also the set the push-then-pop queue keeps (two different algorithms)."""
    rng = random.Random(7)
    for _ in range(500):
        L = rng.randint(1, 40)
        C = rng.randint(0, L)
        scores = [rng.choice([rng.random(), 0.5]) for _ in range(L)]
        _, st_off = oracle.select_offline([scores], C)
        _, st_q = oracle.select_lazy_layers(scores, C, policy="after")
        assert st_off == st_q


def test_prompt_order_and_duplication_do_not_matter():
    """With scores that are exact in binary (multiples of 1/8) the mean, and so
    the selection, is the same for any prompt order and for every prompt
    counted twice."""
    rng = random.Random(11)
    for _ in range(200):
        P, L = rng.randint(1, 5), rng.randint(1, 24)
        C = rng.randint(0, L)
        scores = [[rng.randint(0, 8) / 8 for _ in range(L)] for _ in range(P)]
        ref = oracle.select_offline(scores, C)
        perm = scores[:]
        rng.shuffle(perm)
        assert oracle.select_offline(perm, C) == ref
        assert oracle.select_offline(scores + scores, C)[1] == ref[1]


def test_raising_a_score_never_takes_a_layer_out():
    rng = random.Random(13)
    for _ in range(300):
        P, L = rng.randint(1, 4), rng.randint(2, 20)
        C = rng.randint(0, L)
        scores = [[rng.random() for _ in range(L)] for _ in range(P)]
        _, st = oracle.select_offline(scores, C)
        l, p = rng.randrange(L), rng.randrange(P)
        bumped = [row[:] for row in scores]
        bumped[p][l] += 0.5
        _, st2 = oracle.select_offline(bumped, C)
        if st[l]:
            assert st2[l] == 1
        assert sum(st2) == L - C


def test_one_dominant_prompt_is_averaged_not_followed():
    """Two prompts that disagree: layer 0 laziest in prompt 0 only, layer 1
    moderately lazy in both.  The mean prefers layer 1."""
    scores = [[0.9, 0.6, 0.1, 0.1], [0.1, 0.6, 0.1, 0.2]]
    mean, st = oracle.select_offline(scores, 3)
    assert mean == pytest.approx([0.5, 0.6, 0.1, 0.15])
    assert st == [0, 1, 0, 0]


def test_offline_edges():
    assert oracle.select_offline([[0.3, 0.1, 0.2]], 0)[1] == [1, 1, 1]
    assert oracle.select_offline([[0.3, 0.1, 0.2]], 3)[1] == [0, 0, 0]
    assert oracle.select_offline([[0.5, 0.5, 0.5, 0.5]], 2)[1] == [1, 1, 0, 0]
    with pytest.raises(ValueError):
        oracle.select_offline([], 0)
    with pytest.raises(ValueError):
        oracle.select_offline([[0.1, 0.2], [0.3]], 1)
    with pytest.raises(ValueError):
        oracle.select_offline([[0.1, float("nan")]], 1)
    with pytest.raises(ValueError):
        oracle.select_offline([[0.1, 0.2]], 3)
