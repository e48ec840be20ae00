"""Pins of the routing oracle (oracle/routing.py) against a hand-worked
example, brute-force loops on small inputs, and the invariants any grouping
of the routed rows must satisfy (a permutation of the valid choices, groups
contiguous and ascending, each group in (token, choice) order)."""
import numpy as np
import pytest

from oracle import routing as R


def test_hand_worked_top2():
    # 4 tokens, top-2 over 3 experts:
    #   token 0 -> (2, 0), token 1 -> (0, 1), token 2 -> (2, 1), token 3 -> (0, 2)
    # expert 0: tokens 0, 1, 3; expert 1: tokens 1, 2; expert 2: tokens 0, 2, 3
    ids = np.array([[2, 0], [0, 1], [2, 1], [0, 2]])
    r = R.route(ids, 3)
    assert r["group_ends"].tolist() == [3, 5, 8]
    assert r["row_index"].tolist() == [0, 1, 3, 1, 2, 0, 2, 3]
    # choice (t, j) -> row: (0,0)->5, (0,1)->0, (1,0)->1, (1,1)->3, (2,0)->6, (2,1)->4, (3,0)->2, (3,1)->7
    assert r["slot_row"].tolist() == [5, 0, 1, 3, 6, 4, 2, 7]


def _brute(ids, E):
    T, k = ids.shape
    rows, slot = [], {}
    ends = []
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if ids[t, j] == e:
                    slot[t * k + j] = len(rows)
                    rows.append(t)
        ends.append(len(rows))
    rows += [-1] * (T * k - len(rows))
    return ends, rows, [slot.get(i, -1) for i in range(T * k)]


@pytest.mark.parametrize("seed", range(6))
def test_brute_force(seed):
    rng = np.random.default_rng(seed)
    T, k, E = int(rng.integers(0, 40)), int(rng.integers(1, 5)), int(rng.integers(1, 9))
    ids = rng.integers(-1 if seed % 2 else 0, E + (1 if seed % 3 == 0 else 0), size=(T, k))
    r = R.route(ids, E)
    ends, rows, slot = _brute(ids, E)
    assert r["group_ends"].tolist() == ends
    assert r["row_index"].tolist() == rows
    assert r["slot_row"].tolist() == slot


def test_invariants_large():
    rng = np.random.default_rng(7)
    T, k, E = 5000, 6, 64
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :k]     # k distinct experts per token
    r = R.route(ids, E)
    ends = r["group_ends"]
    assert ends[-1] == T * k and np.all(np.diff(ends) >= 0)
    assert np.array_equal(np.diff(np.concatenate([[0], ends])), np.bincount(ids.reshape(-1), minlength=E))
    # the inverse map: choice -> row -> token and expert of that row
    rows_of = r["slot_row"]
    assert np.array_equal(np.sort(rows_of), np.arange(T * k))
    assert np.array_equal(r["row_index"][rows_of], np.repeat(np.arange(T), k))
    starts = np.concatenate([[0], ends[:-1]])
    expert_of_row = np.searchsorted(ends, np.arange(T * k), side="right")
    assert np.array_equal(expert_of_row[rows_of], ids.reshape(-1))
    # tokens ascend within each group
    for e in range(E):
        g = r["row_index"][starts[e]:ends[e]]
        assert np.all(np.diff(g) > 0)
