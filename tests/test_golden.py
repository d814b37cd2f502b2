"""The oracle's greedy acceptance against the hand-written cases in golden/."""
import os

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def load_accept_cases():
    cases = []
    with open(os.path.join(HERE, "golden", "accept_cases.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            d, t, n, e, src = [c.strip() for c in line.split(";")]
            cases.append(([int(x) for x in d.split()], [int(x) for x in t.split()], int(n),
                          [int(x) for x in e.split()], src))
    return cases


def test_accept_cases():
    cases = load_accept_cases()
    assert len(cases) >= 8
    for drafts, top1, n, emitted, src in cases:
        got_n, toks = oracle.accept_greedy(np.array(drafts), np.array(top1))
        assert got_n == n, (drafts, top1, src)
        assert list(toks[:n + 1]) == emitted, (drafts, top1, src)
        assert all(t == -1 for t in toks[n + 1:])
