"""Pins for the oracle's greedy argmax (dasLLAMA-00 most_likely; the Go "llm"
package's Argmax, first index on ties).

* hand-worked cases (tests/golden/argmax_values.json): ties, infinities, signed
  zeros, NaN anywhere and at index 0;
* on random vectors without NaN: the first index of the maximum as numpy finds
  it (np.argmax returns the first occurrence);
* planted maxima: a unique maximum at every position of a vector is found.
"""
import numpy as np

import oracle
from tests import _golden as G


def test_argmax_golden():
    for c in G.load("argmax_values.json")["cases"]:
        v = np.array([G.num(x) for x in c["v"]], np.float32)
        assert oracle.argmax(v) == c["want"], c["working"]


def test_argmax_matches_first_max_on_random_vectors():
    rng = np.random.default_rng(41)
    for n in (1, 2, 31, 1000, 49152):
        v = rng.standard_normal(n).astype(np.float32)
        v[rng.integers(0, n, max(1, n // 10))] = v.max()   # ties with the maximum
        assert oracle.argmax(v) == int(np.argmax(v))


def test_argmax_planted_maximum_everywhere():
    v = np.zeros(257, np.float32)
    for i in range(257):
        w = v.copy()
        w[i] = 1.0
        assert oracle.argmax(w) == i
