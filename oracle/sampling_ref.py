"""CPU oracle of temperature > 0 drafting and probabilistic verification.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call this module; the HIP library never does, and
it shares no code with it.

Sources.  The pages require a separate "probabilistic" draft-sampling mode for
requests sampled at temperature above 0 and report results at temperatures 0
and 1 (feinterview.poetries.top, the deployment list of the last section;
wire.sakhanda.co, "Как развернуть FlashMap?").  By the alphasignal.ai page
("Why drafting still costs time"), verification is lossless when it leaves the
distribution of the target's samples unchanged.  The pages give no rule beyond
that.  READING: the standard speculative-sampling rule.
  - Drafts: at temperature tau every block row i is sampled independently from
    q_i = softmax(l_i / tau), where l_i are the drafter's float32 logits of the
    last jump.
  - Verify, with p_j = softmax(T_j / tau) for target rows j = 0..K: draft i is
    accepted while u_i * q_i(d_i) < p_i(d_i), i.e. u_i < p_i(d_i) / q_i(d_i),
    with u_i uniform on (0, 1).
  - The first rejected row n emits a sample of the residual max(0, p_n - q_n),
    normalised.  After K accepted drafts the bonus is a sample of p_K.
  - Emitted: d_0..d_{n-1}, y_n (n + 1 tokens).
With this rule every emitted token is distributed as the target's p given the
accepted prefix, whatever q is.

Randomness.  All random numbers come from Philox4x32-10 (Salmon, Moraes, Dror
and Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011), written here
from that definition: a 128-bit counter and a 64-bit key; each of ten rounds
multiplies two counter words by fixed odd constants, and the high halves are
XORed with the other two words and the round key.  The key advances by two
Weyl constants between rounds.
  - The key is the caller's 64-bit seed (low word, high word).
  - The counter is (v, row, branch, stream); output word 0 gives
    U = (x + 0.5) / 2^32 in (0, 1).
  - Stream 0: Gumbel noise of draft sampling.  Stream 1: Gumbel noise of the
    residual or bonus sample.  Stream 2: acceptance uniforms (v = 0).
Categorical samples use the Gumbel-max trick (the lowest index wins a tie):
  argmax_v (log w_v - log(-log U_v)) is distributed as w / sum(w).
Values are float64 here; the decisions are the same as the GPU's float32 ones
except where two candidates lie within rounding of each other (reported as
near-ties by the tests).
"""
from __future__ import annotations

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
MASK32 = 0xFFFFFFFF

STREAM_DRAFT = 0
STREAM_CORRECT = 1
STREAM_ACCEPT = 2


def philox4x32_10(ctr, seed):
    """Philox4x32 with 10 rounds.  ctr: uint32 array [..., 4]; seed: 64-bit int.
    Returns uint32 [..., 4]."""
    c = [np.asarray(ctr, dtype=np.uint64)[..., i] & MASK32 for i in range(4)]
    k0 = np.uint64(seed & MASK32)
    k1 = np.uint64((seed >> 32) & MASK32)
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    for r in range(10):
        if r:
            k0 = np.uint64((int(k0) + PHILOX_W0) & MASK32)
            k1 = np.uint64((int(k1) + PHILOX_W1) & MASK32)
        p0 = c[0] * m0            # < 2^64: exact in uint64
        p1 = c[2] * m1
        hi0, lo0 = p0 >> np.uint64(32), p0 & np.uint64(MASK32)
        hi1, lo1 = p1 >> np.uint64(32), p1 & np.uint64(MASK32)
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
    return np.stack(c, axis=-1).astype(np.uint32)


def uniforms(v, row, branch, stream, seed):
    """U in (0, 1) for counters (v, row, branch, stream); v may be an array."""
    v = np.asarray(v, dtype=np.uint64)
    ctr = np.zeros(v.shape + (4,), dtype=np.uint64)
    ctr[..., 0] = v
    ctr[..., 1] = row
    ctr[..., 2] = branch
    ctr[..., 3] = stream
    x = philox4x32_10(ctr, seed)[..., 0].astype(np.float64)
    return (x + 0.5) / 4294967296.0


def gumbel(v, row, branch, stream, seed):
    return -np.log(-np.log(uniforms(v, row, branch, stream, seed)))


def _argmax_lowest(x):
    """Lowest index of the maximum of a 1-D array (-inf entries never win
    unless all are -inf)."""
    return int(np.flatnonzero(x == x.max())[0])


def log_softmax_rows(logits, tau):
    x = np.asarray(logits, dtype=np.float64) / tau
    m = x.max(axis=-1, keepdims=True)
    return x - (m + np.log(np.exp(x - m).sum(axis=-1, keepdims=True)))


def logsumexp_rows(logits, tau):
    """log sum_v exp(l_v / tau) per row (the drafter's normaliser)."""
    x = np.asarray(logits, dtype=np.float64) / tau
    m = x.max(axis=-1)
    return m + np.log(np.exp(x - m[..., None]).sum(axis=-1))


def sample_draft(logits, tau, seed, branch=0):
    """Draft tokens at temperature tau: row i is argmax_v (l_iv / tau + G_iv)
    with G from stream 0, i.e. a sample of softmax(l_i / tau).
    logits: [K][V] float32 values (the drafter's last-jump logits)."""
    logits = np.asarray(logits, dtype=np.float64)
    K, V = logits.shape
    v = np.arange(V)
    return np.array([_argmax_lowest(logits[i] / tau + gumbel(v, i, branch, STREAM_DRAFT, seed))
                     for i in range(K)], dtype=np.int64)


def verify_sample(T, draft_logits, draft, tau, seed, branch=0):
    """Probabilistic verification of one branch.

    T            [K+1][V] target logits (values)
    draft_logits [K][V]   the drafter's float32 logits of the last jump
    draft        [K]      the drafted tokens
    Returns n (accepted drafts), the emitted tokens (n + 1), and the
    acceptance margins p(d) - u q(d) of the rows tested (for near-tie
    reports)."""
    T = np.asarray(T, dtype=np.float64)
    Q = np.asarray(draft_logits, dtype=np.float64)
    K = Q.shape[0]
    V = T.shape[1]
    logp = log_softmax_rows(T, tau)          # [K+1][V]
    logq = log_softmax_rows(Q, tau)          # [K][V]
    v = np.arange(V)

    margins = []
    n = K
    for i in range(K):
        d = int(draft[i])
        u = uniforms(0, i, branch, STREAM_ACCEPT, seed)
        p_d, q_d = np.exp(logp[i, d]), np.exp(logq[i, d])
        margins.append(float(p_d - u * q_d))
        if not u * q_d < p_d:
            n = i
            break

    # the emitted sample: row n's residual (n < K) or the bonus row (n = K)
    p = np.exp(logp[n])
    w = np.maximum(p - np.exp(logq[n]), 0.0) if n < K else p
    if not (w > 0).any():      # p == q on every token: fall back to p
        w = p
    with np.errstate(divide="ignore"):
        key = np.log(w) + gumbel(v, n, branch, STREAM_CORRECT, seed)
    emitted = [int(x) for x in draft[:n]] + [_argmax_lowest(key)]
    return {"n": n, "emitted": emitted, "margins": margins}
