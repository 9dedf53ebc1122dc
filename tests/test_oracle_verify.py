"""Pins of the oracle's greedy verifier against the pages and brute force."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "new_york.json")


def _logits_for(argmaxes, V, rng=None, dtype=np.float64):
    """Target logits whose row argmaxes are the given tokens (strictly)."""
    rng = rng or np.random.default_rng(0)
    T = rng.standard_normal((len(argmaxes), V)).astype(dtype)
    for j, y in enumerate(argmaxes):
        T[j, y] = T[j].max() + 1.0
    return T


def test_new_york_cases():
    g = json.load(open(GOLDEN))
    voc = g["vocab"]
    V = len(voc)
    for case in g["cases"]:
        d = np.array([voc[w] for w in case["draft"]])
        T = _logits_for([voc[w] for w in case["target_argmax"]], V)
        n, emitted = oracle.verify(T, d)
        assert n == case["accept"], case
        assert emitted == [voc[w] for w in case["emitted"]], case


def test_brute_force_small_vocab():
    """Every draft of length 3 against every target argmax sequence of length 4
    over a 3-token vocabulary, compared with the definition written as a set:
    n = max{m : draft[:m] == y[:m]}."""
    V, K = 3, 3
    for d in itertools.product(range(V), repeat=K):
        for y in itertools.product(range(V), repeat=K + 1):
            T = np.zeros((K + 1, V))
            for j in range(K + 1):
                T[j, y[j]] = 1.0
            n, emitted = oracle.verify(T, np.array(d))
            n_def = max(m for m in range(K + 1) if list(d[:m]) == list(y[:m]))
            assert n == n_def
            assert emitted == list(d[:n_def]) + [y[n_def]]
            assert len(emitted) == n + 1


def test_argmax_tie_lowest_index_and_signed_zero():
    assert list(oracle.argmax_lowest(np.zeros((3, 7)))) == [0, 0, 0]
    row = np.array([1.0, 3.0, 2.0, 3.0, 3.0])
    assert oracle.argmax_lowest(row)[0] == 1
    z = np.array([-0.0, 0.0, -1.0])
    assert oracle.argmax_lowest(z)[0] == 0
    z = np.array([-5.0, -0.0, 0.0])
    assert oracle.argmax_lowest(z)[0] == 1
    # all-equal row of a verify: y = 0 for every position
    n, emitted = oracle.verify(np.zeros((17, 11)), np.zeros(16, dtype=int))
    assert n == 16 and emitted == [0] * 17


def test_lossless_against_plain_greedy_decoding():
    """Greedy speculative decoding emits exactly the target's greedy sequence
    whatever the drafts are (the lossless property the pages state)."""
    rng = np.random.default_rng(7)
    V, K, total = 50, 16, 300
    table = rng.standard_normal((V, V))          # toy bigram target: logits(next | prev)
    table[rng.integers(0, V, 20), rng.integers(0, V, 20)] += 5.0

    def target_next(prev):
        return int(np.flatnonzero(table[prev] == table[prev].max())[0])

    ref = [3]
    while len(ref) < total + 1:
        ref.append(target_next(ref[-1]))

    for policy in ("random", "oracle_prefix", "adversarial"):
        seq = [3]
        cycles = 0
        while len(seq) < total + 1:
            if policy == "random":
                d = rng.integers(0, V, K)
            elif policy == "adversarial":
                d = np.array([(target_next(seq[-1]) + 1) % V] * K)
            else:                                  # right for a random prefix length
                d, prev = [], seq[-1]
                good = rng.integers(0, K + 1)
                for j in range(K):
                    nxt = target_next(prev)
                    d.append(nxt if j < good else (nxt + 1) % V)
                    prev = d[-1]
                d = np.array(d)
            ctx = [seq[-1]] + list(d)
            T = np.stack([table[p] for p in ctx])  # row j scores draft slot j
            n, emitted = oracle.verify(T, d)
            seq.extend(emitted)
            cycles += 1
        assert seq[:total + 1] == ref[:total + 1], policy
        if policy == "adversarial":
            assert cycles >= total  # one target token per cycle
        if policy == "oracle_prefix":
            assert cycles < total


def test_verify_tree_best_branch():
    rng = np.random.default_rng(3)
    V, K = 40, 16
    drafts = rng.integers(0, V, (4, K))
    Ts = []
    for b, n in enumerate((7, 3, 9, 9)):
        y = list(drafts[b, :n]) + [(int(drafts[b, n]) + 1) % V] + list(rng.integers(0, V, K - n))
        Ts.append(_logits_for(y[:K + 1], V, rng))
    res, best = oracle.verify_tree(Ts, drafts)
    assert [r[0] for r in res] == [7, 3, 9, 9]
    assert best == 2        # lowest index among the longest


def test_planting_gives_requested_accept_length():
    cfg = synth.CONFIGS["tiny"]
    T = synth.make_target_logits(cfg, 1)[0]
    d = np.random.default_rng(1).integers(0, cfg.V, cfg.K)
    for n in range(cfg.K + 1):
        Tp = synth.plant(T, d, n)
        assert oracle.verify(Tp, d)[0] == n


def test_planting_bf16():
    cfg = synth.CONFIGS["tiny"].with_(dtype="bf16")
    T = synth.make_target_logits(cfg, 1)[0]
    assert T.dtype == np.uint16
    d = np.random.default_rng(2).integers(0, cfg.V, cfg.K)
    for n in (0, 5, 16):
        assert oracle.verify(synth.plant(T, d, n), d)[0] == n
