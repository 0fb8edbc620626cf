"""Pins of the LRU neuron cache model (no GPU needed): a hand-worked sequence under
tests/golden (with its citation) and the invariants of the policy on long random sequences."""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_cache_golden_sequence():
    g = json.load(open(os.path.join(GOLD, "neuron_cache_tiny.json")))
    c = oracle.NeuronCache(g["ffn"], g["capacity"], g["n_pinned"])
    for tok in g["tokens"]:
        src, victim = c.step(tok["active"])
        assert src == tok["src"] and victim == tok["victim"], tok
        assert c.neuron_of.tolist() == tok["neuron_of"]
    assert c.last_use.tolist() == g["final_last_use"] and c.stamp == g["final_stamp"]


@pytest.mark.parametrize("capacity,n_pinned", [(64, 0), (64, 16), (200, 32), (16, 0)])
def test_cache_invariants(capacity, n_pinned):
    ffn = 256
    rng = np.random.default_rng(capacity + n_pinned)
    p = np.minimum(0.9, 3.0 / np.arange(1, ffn + 1))           # a power-law firing profile
    c = oracle.NeuronCache(ffn, capacity, n_pinned)
    for t in range(300):
        active = np.flatnonzero(rng.random(ffn) < p)
        before_last = c.last_use.copy()
        before_neuron = c.neuron_of.copy()
        src, victim = c.step(active)
        # slot_of and neuron_of stay inverse maps
        res = c.neuron_of[c.neuron_of >= 0]
        assert len(set(res.tolist())) == len(res)
        for s, n in enumerate(c.neuron_of):
            if n >= 0:
                assert c.slot_of[n] == s
        assert (c.slot_of >= 0).sum() == len(res) <= capacity
        # pinned head never moves
        assert np.array_equal(c.neuron_of[:n_pinned], np.arange(n_pinned))
        # a hit reads the slot its neuron held; a miss holds no slot before the token
        for j, n in enumerate(active):
            if src[j] >= 0:
                assert before_neuron[src[j]] == n and victim[j] == -1
            else:
                assert n not in before_neuron.tolist()
        # every admitted neuron is resident now, and evictions took least recently used slots:
        # any unpinned slot not touched by this token is at least as recent as every victim
        taken = [v for v in victim if v >= 0]
        untouched = [s for s in range(capacity) if before_last[s] != oracle.PINNED
                     and c.last_use[s] < c.stamp]
        for v in taken:
            assert c.neuron_of[v] in active.tolist() and c.last_use[v] == c.stamp
            for s in untouched:
                assert (before_last[v], v) < (before_last[s], s)
        # misses go unadmitted only when no evictable slot is left
        if any(s < 0 and v < 0 for s, v in zip(src, victim)):
            assert not untouched
