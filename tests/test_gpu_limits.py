"""GPU parity at the limits the C ABI accepts: the widest drafter (d 4096,
32 heads, MLP 16384: unfused LayerNorm, a two-chunk-per-wave LM head, long-k
plans) with the most context rows a call may append (16), alone and as a
four-branch tree (80 rows in the QKV contraction); the smallest shapes
(d 128 or 64, V 16); and a context that fills the cache exactly."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

fm = pytest.importorskip("step_flow_map_amd")
from gpu_util import check_draft, exact_or_reseed, make_drafter, run_draft, to_dev  # noqa: E402

TINY = synth.CONFIGS["tiny"]
WIDEST = TINY.with_(name="widest_bf16", dtype="bf16", V=1000, d=4096, nh=32, H=520, L=1, c_prefill=24, n_new=16)
SMALLEST_BF16 = TINY.with_(name="smallest_bf16", dtype="bf16", V=16, d=128, nh=2, H=8, L=1, c_prefill=3, n_new=2)
SMALLEST_F32 = TINY.with_(name="smallest_f32", V=16, d=64, nh=1, H=4, L=1, c_prefill=3, n_new=2)


def _draft_parity(cfg, B=1, C_max=None):
    cfg = cfg.with_(B=B)
    print(f"[limits] {cfg.name} B={B}", flush=True)
    w = synth.make_weights(cfg)
    feats = synth.make_features(cfg)
    dr = make_drafter(cfg, w, C_max=C_max)
    dr.set_schedule(cfg.times)

    def case(draw):
        noise = synth.make_noise(cfg, B, draw)
        dr.truncate(0)
        tok, logits, _ = run_draft(dr, cfg, noise, feats, cfg.c_prefill)
        rel, ties = check_draft(cfg, w, noise, feats, cfg.c_prefill, tok, logits)
        print(f"  draw {draw}: logit error {rel:.2e}, near-ties {ties}", flush=True)
        return ties

    exact_or_reseed(case, f"{cfg.name} B={B}")
    return dr


@pytest.mark.parametrize("B", [1, 4])
def test_widest_drafter_with_most_new_rows(B):
    _draft_parity(WIDEST, B)


@pytest.mark.parametrize("cfg", [SMALLEST_BF16, SMALLEST_F32], ids=["smallest_bf16", "smallest_f32"])
def test_smallest_shapes(cfg):
    _draft_parity(cfg)
    _draft_parity(cfg, B=4)


@pytest.mark.parametrize("C", [64, 61])
def test_context_fills_the_cache(C):
    """C_max = C (a whole number of 32-key blocks, or not) and the draft
    appends the last rows: the cache is full, and one more row is refused."""
    cfg = TINY.with_(name=f"full_cache_{C}", dtype="bf16", V=1000, c_prefill=C - 8, n_new=8)
    dr = _draft_parity(cfg, C_max=C)
    assert dr.context_length == C
    with pytest.raises(fm.FlashMapError) as e:
        dr.append(to_dev(synth.make_features(cfg, rows=1)))
    assert e.value.status == fm.FM_ECAPACITY
