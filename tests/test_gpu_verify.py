"""GPU parity of fm_verify and fm_verify_greedy against the oracle's verifier
(bit-exact)."""
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
from gpu_util import check_guards, guarded, make_drafter, to_dev  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "new_york.json")


def _gpu_verify(T: np.ndarray, drafts: np.ndarray):
    B, K1, _ = T.shape
    e = guarded(B, K1, dtype=torch.int32)
    a = guarded(B, dtype=torch.int32)
    b = guarded(1, dtype=torch.int32)
    fm.fm_verify(to_dev(T), torch.from_numpy(drafts.astype(np.int32)).cuda(), e, a, b)
    torch.cuda.synchronize()
    check_guards(e, a, b)
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


# ---------------------------------------------------------------- fm_verify_greedy
# The handle's sliced verifier (16 workgroups per target row) against the
# oracle and, bit for bit, against fm_verify on the same buffers.

def _greedy_drafter(V, dtype, B=4):
    cfg = synth.CONFIGS["tiny"].with_(V=V, dtype=dtype, B=B)
    return cfg, make_drafter(cfg, synth.make_weights(cfg), C_max=32, max_branches=B)


def _greedy_vs_both(dr, Td, drafts):
    B, K1, _ = Td.shape
    d = torch.from_numpy(drafts.astype(np.int32)).cuda()
    em = guarded(B, K1, dtype=torch.int32)
    acc = guarded(B, dtype=torch.int32)
    best = guarded(1, dtype=torch.int32)
    dr.verify(Td, d, em, acc, best)
    e1, a1, b1 = fm.verify(Td, d)
    torch.cuda.synchronize()
    check_guards(em, acc, best)
    assert torch.equal(em, e1) and torch.equal(acc, a1) and torch.equal(best, b1)
    re, ra, rb = _ref(Td.float().cpu().numpy(), drafts)
    assert np.array_equal(acc.cpu().numpy(), ra) and np.array_equal(em.cpu().numpy(), re)
    assert int(best.cpu()[0]) == rb


# 151936 bf16: 16 slices of 9496; 1000: slices of 64 with the last one
# short; 24 bf16 and 20 f32: slices of one vector, most of them empty
@pytest.mark.parametrize("V,dtype", [(151936, "bf16"), (151936, "f32"), (1000, "bf16"), (1000, "f32"),
                                     (24, "bf16"), (20, "f32")])
def test_greedy_sliced_matches_fm_verify(V, dtype):
    print(f"[verify_greedy] V={V} {dtype}", flush=True)
    cfg, dr = _greedy_drafter(V, dtype)
    rng = np.random.default_rng(V + 7)
    for B, accepts in ((4, (0, 16, 9, 16)), (1, (5,)), (3, (16, 2, 16))):
        T = synth.make_target_logits(cfg, B)
        drafts = rng.integers(0, V, (B, cfg.K))
        for b, n in enumerate(accepts):
            T[b] = synth.plant(T[b], drafts[b], n)
        _greedy_vs_both(dr, to_dev(T), drafts)


def test_greedy_sliced_ties_across_slices():
    cfg, dr = _greedy_drafter(151936, "bf16", B=2)
    T = synth.make_target_logits(cfg, 2)
    # every third column ties the row's column-0 value, and row maxima planted
    # at equal values in two slices: the lowest index must win across slices
    T[0, :, ::3] = T[0, :, 0:1]
    lo, hi = synth.to_bf16_bits(np.float32([-1.0, 4.0]))
    T[1, :, :] = lo
    T[1, :, 150000] = hi
    T[1, :, 9500] = hi
    T[1, 5, 3] = hi
    drafts = np.zeros((2, 16), dtype=np.int64)
    drafts[1, :] = 9500
    _greedy_vs_both(dr, to_dev(T), drafts)


def test_greedy_unaligned_view_takes_the_one_workgroup_path():
    cfg, dr = _greedy_drafter(1000, "bf16", B=2)
    T = synth.make_target_logits(cfg, 2)
    flat = torch.empty(2 * 17 * 1000 + 1, dtype=torch.bfloat16, device="cuda")
    view = flat[1:].view(2, 17, 1000)    # 2-byte aligned only
    view.copy_(to_dev(T))
    drafts = np.random.default_rng(3).integers(0, 1000, (2, 16))
    _greedy_vs_both(dr, view, drafts)


def test_greedy_rejects_more_branches_than_the_handle():
    cfg, dr = _greedy_drafter(1000, "bf16", B=2)
    T = to_dev(synth.make_target_logits(cfg, 3))
    d = torch.zeros(3, 16, dtype=torch.int32, device="cuda")
    out = torch.empty(3, 17, dtype=torch.int32, device="cuda")
    with pytest.raises(fm.FlashMapError) as e:
        dr.verify(T, d, out, out[:, 0].contiguous(), out[0, :1].contiguous())
    assert e.value.status == fm.FM_ECAPACITY
