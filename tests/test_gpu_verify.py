"""GPU parity of fm_verify against the oracle's verifier (bit-exact)."""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

fm = pytest.importorskip("step_flow_map_amd")
from gpu_util import to_dev  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "new_york.json")


def _gpu_verify(T: np.ndarray, drafts: np.ndarray):
    e, a, b = fm.verify(to_dev(T), torch.from_numpy(drafts.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    return e.cpu().numpy(), a.cpu().numpy(), int(b.cpu().numpy()[0])


def _ref(T, drafts):
    res, best = oracle.verify_tree([T[b] for b in range(T.shape[0])], drafts)
    K = drafts.shape[1]
    em = np.full((len(res), K + 1), -1, dtype=np.int64)
    for b, (n, emitted) in enumerate(res):
        em[b, :len(emitted)] = emitted
    return em, np.array([n for n, _ in res]), best


def _assert_same(T, drafts):
    e, a, b = _gpu_verify(T, drafts)
    re, ra, rb = _ref(T, drafts)
    assert np.array_equal(a, ra), (a, ra)
    assert np.array_equal(e, re)
    assert b == rb


def test_new_york_cases_on_gpu():
    g = json.load(open(GOLDEN))
    voc = g["vocab"]
    for case in g["cases"]:
        T = np.zeros((1, 3, 4), dtype=np.float32)
        for j, wd in enumerate(case["target_argmax"]):
            T[0, j, voc[wd]] = 1.0
        d = np.array([[voc[w] for w in case["draft"]]])
        e, a, b = _gpu_verify(T, d)
        assert a[0] == case["accept"]
        assert list(e[0, :a[0] + 1]) == [voc[w] for w in case["emitted"]]


def test_brute_force_small_vocab_on_gpu():
    V, K = 3, 3
    drafts = np.array(list(itertools.product(range(V), repeat=K)))
    ys = list(itertools.product(range(V), repeat=K + 1))
    for start in range(0, len(ys), 27):
        for y in ys[start:start + 27]:
            T = np.zeros((len(drafts), K + 1, V), dtype=np.float32)
            T[:, np.arange(K + 1), list(y)] = 1.0
            # B <= 64 per call
            for c in range(0, len(drafts), 27):
                _assert_same(T[c:c + 27], drafts[c:c + 27])


@pytest.mark.parametrize("V", [151936, 1000, 1001, 17])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_random_planted_and_ragged(V, dtype):
    cfg = synth.CONFIGS["tiny"].with_(V=V, dtype=dtype)
    rng = np.random.default_rng(V)
    B = 4
    T = synth.make_target_logits(cfg, B)
    drafts = rng.integers(0, V, (B, cfg.K))
    for b, n in enumerate((0, 7, 16, 3)):
        T[b] = synth.plant(T[b], drafts[b], n)
    _assert_same(T, drafts)


def test_ties_and_signed_zero():
    V, K = 64, 16
    T = np.zeros((2, K + 1, V), dtype=np.float32)
    T[1, :, :] = -0.0
    T[1, 3, 10] = 0.0                         # +0 ties -0: lowest index wins
    d = np.zeros((2, K), dtype=np.int64)
    _assert_same(T, d)
    # bf16 rows with many exact ties
    cfg = synth.CONFIGS["tiny"].with_(V=151936, dtype="bf16")
    T = synth.make_target_logits(cfg, 1)
    T[0, :, ::3] = T[0, :, 0:1]               # heavy ties at the row value of column 0
    _assert_same(T, np.zeros((1, 16), dtype=np.int64))
