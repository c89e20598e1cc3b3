"""Pins of the oracle's greedy verification of a speculative round."""

import itertools
import os

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "verify_greedy_rounds.txt")


def _rounds():
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        idx, drafts, L, committed = (part.split() for part in line.split("|"))
        drafts = [] if drafts == ["-"] else drafts
        yield [int(v) for v in idx], [int(v) for v in drafts], int(L[0]), [int(v) for v in committed]


def test_worked_rounds():
    rounds = list(_rounds())
    assert len(rounds) == 10
    for idx, drafts, L, committed in rounds:
        assert oracle.verify_greedy(idx, drafts) == (L, committed), (idx, drafts)


def test_every_round_over_a_two_token_vocabulary():
    """Brute force over all rounds with up to 4 rows and tokens {0, 1}: the
    result is the unique L with the accepted drafts matching, the next one
    (if any) not, and the committed tokens the drafts then t_L."""
    for M in range(1, 5):
        for idx in itertools.product((0, 1), repeat=M):
            for drafts in itertools.product((0, 1), repeat=M - 1):
                L, committed = oracle.verify_greedy(idx, drafts)
                assert 0 <= L <= M - 1 and len(committed) == L + 1
                assert all(drafts[j] == idx[j] for j in range(L))
                assert L == M - 1 or drafts[L] != idx[L]
                assert committed == list(drafts[:L]) + [idx[L]]
