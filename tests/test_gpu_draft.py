"""GPU parity of fm_draft against the oracle on small workloads (several tiles
and ragged tails): tokens exact (near-ties reported), logits and the residual
stream within the stated norm-wise tolerance."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

fm = pytest.importorskip("step_flow_map_amd")
from gpu_util import check_draft, exact_or_reseed, make_drafter, run_draft, rowwise_rel_err, to_dev  # noqa: E402

TINY = synth.CONFIGS["tiny"]
# bf16 with ragged vocabulary (1000 = 62.5 column tiles, 31.25 row chunks) and
# a context width whose fused length 5*520 = 2600 is not a multiple of the chunk
SMALL_BF16 = TINY.with_(name="small_bf16", dtype="bf16", V=1000, H=520)
# width 384 = one and a half weight chunks (a ragged k range in every
# contraction and in the fused LayerNorm), head width 128, and a context of 308
# rows = 10 key blocks (the last one partial) spread over several ranges
MID_BF16 = TINY.with_(name="mid_bf16", dtype="bf16", V=2000, d=384, nh=3, H=520, c_prefill=300)
# float32 width 1152 = nine 128-column chunks: two chunks for the first wave of
# the k-split LM head and one for the rest, the LayerNorm left unfused, and a
# four-branch tree whose z no longer fits in registers (whole-tile LM head)
WIDE_F32 = TINY.with_(name="wide_f32", V=1000, d=1152, nh=9)
# bf16 at the drafter's real width (d 2048, 16 heads, MLP 8192) with a small
# vocabulary and two blocks: the persistent block tail (W_o, LN + W_1, W_2)
W2048_BF16 = TINY.with_(name="w2048_bf16", dtype="bf16", V=2000, d=2048, nh=16, H=520, c_prefill=40)


# context fusions long enough that a wave of the fusion contraction owns
# several chunks of its k split (the two-register-set pipeline): bf16 with
# 5*3304 = 16520 = 64.5 chunks (a ragged last chunk, a last split of two
# chunks), float32 with 5*2048 = 10240 = 80 chunks of 128
LONG_FUSE_BF16 = TINY.with_(name="long_fuse_bf16", dtype="bf16", V=1000, H=3304)
LONG_FUSE_F32 = TINY.with_(name="long_fuse_f32", H=2048)


def _case(cfg, variant="random", B=1, draw=0):
    w = synth.make_weights(cfg, variant)
    feats = synth.make_features(cfg)
    noise = synth.make_noise(cfg, B, draw)
    return w, feats, noise


@pytest.mark.parametrize("cfg", [TINY, SMALL_BF16, MID_BF16, WIDE_F32, W2048_BF16],
                         ids=["tiny_f32", "small_bf16", "mid_bf16", "wide_f32", "w2048_bf16"])
@pytest.mark.parametrize("variant", ["random", "unit_gate", "gate_zero"])
def test_draft_matches_oracle(cfg, variant):
    print(f"[draft parity] {cfg.name} {variant}", flush=True)
    w = synth.make_weights(cfg, variant)
    feats = synth.make_features(cfg)
    W = oracle.Weights.from_storage(w)
    dr = make_drafter(cfg, w)
    dr.set_schedule(cfg.times)

    def case(draw):
        noise = synth.make_noise(cfg, 1, draw)
        dr.truncate(0)
        tok, logits, hidden = run_draft(dr, cfg, noise, feats, cfg.c_prefill, want_hidden=True)
        rel, ties = check_draft(cfg, w, noise, feats, cfg.c_prefill, tok, logits, hidden)
        print(f"  draw {draw}: max row logit error {rel:.2e}, near-ties {ties}")
        # per-block residual stream
        ref = oracle.draft(W, cfg, noise[0], feats, trace=True)
        for l, blk in enumerate(ref["jumps"][0]["blocks"]):
            e = rowwise_rel_err(hidden[0, l + 1, 0], blk["h"])
            assert e.max() < 2e-2, (l, e.max())
        return ties

    exact_or_reseed(case, f"{cfg.name} {variant}")


@pytest.mark.parametrize("cfg", [LONG_FUSE_BF16, LONG_FUSE_F32], ids=["bf16", "f32"])
def test_long_context_fusion_matches_oracle(cfg):
    print(f"[draft parity] {cfg.name}", flush=True)
    w = synth.make_weights(cfg)
    feats = synth.make_features(cfg)
    dr = make_drafter(cfg, w)
    dr.set_schedule(cfg.times)

    def case(draw):
        noise = synth.make_noise(cfg, 1, draw)
        dr.truncate(0)
        tok, logits, hidden = run_draft(dr, cfg, noise, feats, cfg.c_prefill, want_hidden=True)
        rel, ties = check_draft(cfg, w, noise, feats, cfg.c_prefill, tok, logits, hidden)
        print(f"  draw {draw}: max row logit error {rel:.2e}, near-ties {ties}")
        return ties

    exact_or_reseed(case, cfg.name)


def test_context_paths_agree():
    """All context appended by fm_context_append, all appended inside fm_draft,
    or split between the two: the same draft.  Truncate + re-append reproduces
    a fresh build."""
    cfg = SMALL_BF16
    w, feats, noise = _case(cfg)
    dr = make_drafter(cfg, w)
    dr.set_schedule(cfg.times)
    t_split, l_split, _ = run_draft(dr, cfg, noise, feats, 24)
    dr.truncate(0)
    t_pre, l_pre, _ = run_draft(dr, cfg, noise, feats, 32)
    dr.truncate(16)
    dr.append(to_dev(feats[16:32]))                 # re-append rows 16..31
    t_tail, l_tail, _ = run_draft(dr, cfg, noise, feats[:0], 0)
    assert np.array_equal(t_split, t_pre) and np.array_equal(t_pre, t_tail)
    assert np.abs(l_split - l_pre).max() < 1e-2 * np.abs(l_pre).max()
    assert np.array_equal(l_pre, l_tail)
    assert dr.context_length == 32


def test_empty_context_and_no_new_rows():
    cfg = SMALL_BF16.with_(c_prefill=0, n_new=0)
    w = synth.make_weights(cfg)
    feats = np.zeros((0, 5, cfg.H), dtype=np.uint16)
    dr = make_drafter(cfg, w, C_max=8)
    dr.set_schedule(cfg.times)

    def case(draw):
        noise = synth.make_noise(cfg, 1, draw)
        tok, logits, _ = run_draft(dr, cfg, noise, feats, 0)
        return check_draft(cfg, w, noise, feats, 0, tok, logits)[1]

    exact_or_reseed(case, "empty context")


@pytest.mark.parametrize("cfg", [SMALL_BF16, W2048_BF16], ids=["small_bf16", "w2048_bf16"])
def test_bitwise_deterministic(cfg):
    w, feats, noise = _case(cfg)
    dr = make_drafter(cfg, w)
    dr.set_schedule(cfg.times)
    a = run_draft(dr, cfg, noise, feats, cfg.c_prefill)
    dr.truncate(cfg.c_prefill)
    x = to_dev(noise)
    new = to_dev(feats[cfg.c_prefill:])
    logits = torch.empty(1, cfg.K, cfg.V, device="cuda")
    tok = dr.draft(x, new_feats=new, logits=logits)
    torch.cuda.synchronize()
    assert np.array_equal(a[0], tok.cpu().numpy())
    assert np.array_equal(a[1], logits.cpu().numpy())


def test_errors_enqueue_nothing():
    cfg = SMALL_BF16
    w, feats, noise = _case(cfg)
    dr = make_drafter(cfg, w)
    x = to_dev(noise)
    with pytest.raises(fm.FlashMapError) as e:
        dr.draft(x)                                   # no schedule yet
    assert e.value.status == fm.FM_ESTATE
    dr.set_schedule(cfg.times)
    with pytest.raises(fm.FlashMapError) as e:
        dr.append(to_dev(synth.make_features(cfg, 40)))   # C_max = 32
    assert e.value.status == fm.FM_ECAPACITY
    assert dr.context_length == 0
    with pytest.raises(fm.FlashMapError):
        dr.set_schedule((0.0, 0.7, 0.5, 1.0))
    with pytest.raises(fm.FlashMapError) as e:
        dr.draft(to_dev(synth.make_noise(cfg, 2)))     # max_branches = 1
    assert e.value.status == fm.FM_ECAPACITY


def _parity(cfg, label, B=1, variant="random", after=None):
    """Draft B branches on each noise draw the re-seed rule asks for and check
    them against the oracle (residual stream after every block included);
    after(dr, noise, tok, logits), if given, adds checks of that draw."""
    w = synth.make_weights(cfg, variant)
    feats = synth.make_features(cfg)
    dr = make_drafter(cfg, w)
    dr.set_schedule(cfg.times)

    def case(draw):
        noise = synth.make_noise(cfg, B, draw)
        dr.truncate(0)
        tok, logits, hidden = run_draft(dr, cfg, noise, feats, cfg.c_prefill, want_hidden=True)
        rel, ties = check_draft(cfg, w, noise, feats, cfg.c_prefill, tok, logits, hidden)
        print(f"  {label} draw {draw}: logit error {rel:.2e}, near-ties {ties}", flush=True)
        if after is not None:
            after(w, feats, noise, tok, logits)
        return ties

    exact_or_reseed(case, label)


@pytest.mark.parametrize("cfg", [TINY, SMALL_BF16, MID_BF16, W2048_BF16],
                         ids=["tiny_f32", "small_bf16", "mid_bf16", "w2048_bf16"])
def test_two_step_schedule(cfg):
    _parity(cfg.with_(times=(0.0, 0.5, 1.0)), f"2-step {cfg.name}")


def test_draft_tree_of_three_at_width_2048():
    """Three bf16 branches at the drafter's real width: 48 block rows (plus 8
    appended context rows in QKV), so the contractions keep the rows' k slice
    in LDS (three and four row tiles) and sum the slices in a second pass."""
    _parity(W2048_BF16.with_(name="w2048_tree3", B=3), "tree of 3 at d 2048", B=3)


@pytest.mark.parametrize("prefill", [0, 24, 25, 142, 1500])
def test_tree_shared_context_lengths(prefill):
    """Four bf16 branches over one shared context at head width 128 (each key
    block read once per (head, range) and served to every branch): no context
    but the 8 appended rows, exactly one key block, one row past it, five
    blocks (three per range: a range whose second step has one stream idle),
    and 48 blocks over 12 ranges (merged by a separate pass)."""
    cfg = MID_BF16.with_(name=f"mid_tree_c{prefill}", B=4, c_prefill=prefill)
    _parity(cfg, f"tree C {cfg.C}", B=4)


@pytest.mark.parametrize("B", [2, 3])
@pytest.mark.parametrize("prefill", [0, 25, 1500])
def test_tree_of_two_or_three_shares_the_context(B, prefill):
    """Two or three bf16 branches through the shared-context kernel (the
    waves of the absent branches only load): no context, one key block plus
    one row, and 48 blocks over 12 ranges merged by the separate pass."""
    cfg = MID_BF16.with_(name=f"mid_tree{B}_c{prefill}", B=B, c_prefill=prefill)
    _parity(cfg, f"tree of {B}, C {cfg.C}", B=B)


@pytest.mark.parametrize("cfg", [TINY, SMALL_BF16, MID_BF16, WIDE_F32, W2048_BF16],
                         ids=["tiny_f32", "small_bf16", "mid_bf16", "wide_f32", "w2048_bf16"])
def test_draft_tree_of_four(cfg):
    cfg = cfg.with_(B=4)

    def branch_alone(w, feats, noise, tok, logits):
        # the branches are independent: branch 2 alone gives the same draft,
        # up to the rounding order of the two launch shapes; a branch seeing
        # another's rows would differ by far more
        one = cfg.with_(B=1)
        dr1 = make_drafter(one, w)
        dr1.set_schedule(one.times)
        t1, l1, _ = run_draft(dr1, one, noise[2:3], feats, one.c_prefill)
        assert np.array_equal(t1[0], tok[2])
        assert rowwise_rel_err(l1[0], logits[2]).max() <= 5e-3

    _parity(cfg, f"tree {cfg.name}", B=4, after=branch_alone)
