"""Pins of the temperature > 0 oracle (drafting by Gumbel-max sampling and the
speculative-sampling verifier) against closed forms, special cases that reduce
to the greedy verifier, and Monte-Carlo checks of the distributions the rule
guarantees.  The seeds are fixed, so every check is deterministic; the
Monte-Carlo tolerances are 4.5 binomial standard errors."""
import numpy as np
import pytest

import oracle

S = oracle.sampling
M32 = 1 << 32


def _inv32(a):
    return pow(a, -1, M32)


def _philox_inverse(out, seed):
    """Undo the ten rounds from the round's algebra: the low halves of the two
    products are stored as words 3 and 1, so the multiplied words come back by
    multiplying with the constants' inverses mod 2^32; the high halves then
    unmask words 0 and 2."""
    keys = []
    k0, k1 = seed & 0xFFFFFFFF, seed >> 32
    for r in range(10):
        if r:
            k0, k1 = (k0 + S.PHILOX_W0) % M32, (k1 + S.PHILOX_W1) % M32
        keys.append((k0, k1))
    o = [int(x) for x in out]
    for k0, k1 in reversed(keys):
        c0 = (o[3] * _inv32(S.PHILOX_M0)) % M32
        c2 = (o[1] * _inv32(S.PHILOX_M1)) % M32
        hi0 = (c0 * S.PHILOX_M0) >> 32
        hi1 = (c2 * S.PHILOX_M1) >> 32
        o = [c0, o[0] ^ hi1 ^ k0, c2, o[2] ^ hi0 ^ k1]
    return o


def test_philox_rounds_invert():
    rng = np.random.default_rng(5)
    for _ in range(20):
        ctr = rng.integers(0, M32, size=4, dtype=np.uint64)
        seed = int(rng.integers(0, 1 << 63))
        out = S.philox4x32_10(ctr[None, :], seed)[0]
        assert _philox_inverse(out, seed) == [int(x) for x in ctr]


def test_philox_known_answer_vectors():
    """The generator's published known-answer vectors (tests/golden/
    philox4x32_10_kat.json): zero counter and key, all-ones counter and key,
    and the hexadecimal digits of pi.  A wrong multiplier, Weyl constant,
    round count or word order changes every output word."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "philox4x32_10_kat.json")
    with open(path) as f:
        kat = json.load(f)
    assert len(kat["cases"]) == 3
    for case in kat["cases"]:
        ctr = np.array([int(x, 16) for x in case["counter"]], dtype=np.uint64)
        k0, k1 = (int(x, 16) for x in case["key"])
        out = S.philox4x32_10(ctr[None, :], k0 | (k1 << 32))[0]
        assert [int(x) for x in out] == [int(x, 16) for x in case["output"]], case


def test_philox_output_is_uniform_and_decorrelated():
    n = 1 << 17
    ctr = np.zeros((n, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(n)
    ctr[:, 1] = 3
    out = S.philox4x32_10(ctr, 12345).astype(np.float64)
    for w in range(4):
        hist = np.bincount((out[:, w] / 2 ** 24).astype(np.int64), minlength=256)
        chi2 = ((hist - n / 256) ** 2 / (n / 256)).sum()
        assert chi2 < 255 + 6 * np.sqrt(2 * 255), (w, chi2)   # ~6 sigma of chi2(255)
    u = (out + 0.5) / M32
    for a, b in [(0, 1), (0, 2), (1, 3), (2, 3)]:
        assert abs(np.corrcoef(u[:, a], u[:, b])[0, 1]) < 5 / np.sqrt(n)
    # neighbouring counters, and the same counter under neighbouring seeds
    assert abs(np.corrcoef(u[:-1, 0], u[1:, 0])[0, 1]) < 5 / np.sqrt(n)
    u2 = (S.philox4x32_10(ctr, 12346)[:, 0].astype(np.float64) + 0.5) / M32
    assert abs(np.corrcoef(u[:, 0], u2)[0, 1]) < 5 / np.sqrt(n)
    # counters that differ only in the row, branch or stream word differ
    base = S.uniforms(np.arange(1000), 0, 0, 0, 7)
    for kw in [(1, 0, 0), (0, 1, 0), (0, 0, 1)]:
        assert not np.any(S.uniforms(np.arange(1000), *kw, 7) == base)


def test_uniforms_stay_inside_the_open_interval():
    # extreme generator words map strictly inside (0, 1)
    assert (0.5 / M32) > 0 and ((M32 - 1) + 0.5) / M32 < 1
    u = S.uniforms(np.arange(1 << 16), 1, 2, 3, 99)
    assert u.min() > 0 and u.max() < 1


def _tol(p, n):
    return 4.5 * np.sqrt(np.maximum(p * (1 - p), 1e-4) / n) + 1e-9


def test_gumbel_max_draws_follow_the_tempered_softmax():
    logits = np.array([[0.3, -1.0, 2.0, 0.0, 1.1, 2.0]])
    tau = 0.7
    n = 20000
    counts = np.zeros(6)
    for seed in range(n):
        counts[S.sample_draft(logits, tau, seed)[0]] += 1
    p = np.exp(S.log_softmax_rows(logits, tau)[0])
    assert np.all(np.abs(counts / n - p) < _tol(p, n)), (counts / n, p)


def test_draft_sampling_at_small_temperature_is_the_argmax():
    rng = np.random.default_rng(1)
    logits = rng.standard_normal((16, 500))
    greedy = oracle.argmax_lowest(logits)
    for seed in range(5):
        assert np.array_equal(S.sample_draft(logits, 1e-4, seed), greedy)


def _toy(seed=0):
    """Two drafted positions over four tokens; drafter and target disagree."""
    T = np.array([[1.0, 0.2, -0.5, 0.8],
                  [-0.3, 1.5, 0.1, 0.0],
                  [0.4, 0.4, -1.0, 1.2]])
    Q = np.array([[0.1, 1.3, 0.0, -0.4],
                  [0.9, 0.2, 0.8, -1.0]])
    return T, Q


def test_lossless_marginals_and_acceptance_rate():
    """Drafts sampled from q and verified against p: the first emitted token is
    distributed as p_0, the token emitted at slot 1 (given slot 0 accepted) as
    p_1, and P(slot 0 accepted) = sum_v min(p_0(v), q_0(v))."""
    T, Q = _toy()
    tau = 0.8
    n = 20000
    first = np.zeros(4)
    second = np.zeros(4)
    acc0 = 0
    for seed in range(n):
        d = S.sample_draft(Q, tau, seed)
        r = S.verify_sample(T, Q, d, tau, seed)
        first[r["emitted"][0]] += 1
        if r["n"] >= 1:
            acc0 += 1
            second[r["emitted"][1]] += 1
    p = np.exp(S.log_softmax_rows(T, tau))
    q = np.exp(S.log_softmax_rows(Q, tau))
    assert np.all(np.abs(first / n - p[0]) < _tol(p[0], n)), (first / n, p[0])
    beta = np.minimum(p[0], q[0]).sum()
    assert abs(acc0 / n - beta) < _tol(beta, n), (acc0 / n, beta)
    assert np.all(np.abs(second / acc0 - p[1]) < _tol(p[1], acc0)), (second / acc0, p[1])


def test_acceptance_probability_of_a_fixed_draft():
    """P(accept d) = min(1, p(d) / q(d)) over the acceptance uniforms."""
    T, Q = _toy()
    tau = 1.0
    p = np.exp(S.log_softmax_rows(T, tau))
    q = np.exp(S.log_softmax_rows(Q, tau))
    n = 8000
    for d0 in range(4):
        d = np.array([d0, 0])
        acc = sum(S.verify_sample(T, Q, d, tau, seed)["n"] >= 1 for seed in range(n))
        a = min(1.0, p[0, d0] / q[0, d0])
        assert abs(acc / n - a) < _tol(a, n), (d0, acc / n, a)


def test_identical_distributions_accept_everything():
    T, Q = _toy()
    Tq = np.vstack([Q, T[2:]])
    for seed in range(50):
        d = S.sample_draft(Q, 0.9, seed)
        r = S.verify_sample(Tq, Q, d, 0.9, seed)
        assert r["n"] == 2 and r["emitted"][:2] == [int(x) for x in d]


def test_one_hot_target_rejects_other_drafts():
    """A target that puts all its mass on token 3 at slot 0 rejects any other
    draft there (p(d) = 0) and the residual is then exactly token 3."""
    T, Q = _toy()
    T = T.copy()
    T[0] = [-1e4, -1e4, -1e4, 0.0]
    for seed in range(50):
        r = S.verify_sample(T, Q, np.array([1, 0]), 1.0, seed)
        assert r["n"] == 0 and r["emitted"] == [3]


def test_small_temperature_reduces_to_the_greedy_verifier():
    rng = np.random.default_rng(2)
    V, K = 50, 6
    for case in range(20):
        T = rng.standard_normal((K + 1, V))
        Q = rng.standard_normal((K, V))
        d = oracle.argmax_lowest(Q)
        # plant agreement on a random prefix so that n varies
        m = case % (K + 1)
        for j in range(m):
            T[j, d[j]] = T[j].max() + 1.0
        n_g, emitted_g = oracle.verify(T, d)
        r = S.verify_sample(T, Q, d, 1e-4, case)
        assert (r["n"], r["emitted"]) == (n_g, emitted_g)
