"""Pins of the oracle's drafter forward: an independent torch composition of the
block (library attention, layer norm and GELU), special weight variants that
reduce the model to two matrix products, invariances, the flow-map closed
forms, and the parameter count the pages report."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as Fn

import oracle
import synth

TINY = synth.CONFIGS["tiny"]


@pytest.fixture(scope="module")
def tiny():
    cfg = TINY
    w = synth.make_weights(cfg)
    return cfg, w, oracle.Weights.from_storage(w), synth.make_features(cfg), synth.make_noise(cfg)


def _torch_forward(cfg, W, noise, feats, s=0.0, t=1.0):
    """Independent float64 composition: nn.MultiheadAttention for the attention
    wiring (queries from the block, keys/values from [context; block] through the
    same in-projection), torch layer_norm / gelu / silu for the rest."""
    T = {k: torch.from_numpy(v) for k, v in W.items()}
    d = cfg.d

    def ln(x):
        return Fn.layer_norm(x, (x.shape[-1],), eps=1e-6)

    def temb(tau):
        half = 128
        fr = torch.exp(-math.log(10000.0) * torch.arange(half, dtype=torch.float64) / half)
        return torch.cat([torch.cos(tau * fr), torch.sin(tau * fr)])

    def te(p, tau):
        return T[p + ".W2"] @ Fn.silu(T[p + ".W1"] @ temb(tau) + T[p + ".b1"]) + T[p + ".b2"]

    c = Fn.silu(te("te_s", s) + te("te_t", t))
    half = d // 2
    fr = 10000.0 ** (-torch.arange(half, dtype=torch.float64) / half)
    ang = torch.arange(cfg.K, dtype=torch.float64)[:, None] * fr[None]
    P = torch.cat([torch.sin(ang), torch.cos(ang)], 1)
    x = torch.from_numpy(oracle.from_storage(noise))
    h = x @ T["E"] + P
    f = torch.from_numpy(oracle.from_storage(feats)).reshape(feats.shape[0], 5 * cfg.H)
    u = ln(f @ T["W_f"].T + T["b_f"])
    for l in range(cfg.L):
        p = f"blk{l}."
        mv = T[p + "W_ada"] @ c + T[p + "b_ada"]
        sh1, sc1, g1, sh2, sc2, g2 = mv.split(d)
        mha = torch.nn.MultiheadAttention(d, cfg.nh, bias=True, batch_first=True,
                                          dtype=torch.float64)
        with torch.no_grad():
            mha.in_proj_weight.copy_(T[p + "W_qkv"])
            mha.in_proj_bias.copy_(T[p + "b_qkv"])
            mha.out_proj.weight.copy_(T[p + "W_o"])
            mha.out_proj.bias.copy_(T[p + "b_o"])
            a = ln(h) * (1 + sc1) + sh1
            kv = torch.cat([u, a])[None]
            att, _ = mha(a[None], kv, kv, need_weights=False)
            h = h + g1 * att[0]
            m = ln(h) * (1 + sc2) + sh2
            mlp = Fn.gelu(m @ T[p + "W_1"].T + T[p + "b_1"], approximate="tanh") @ T[p + "W_2"].T + T[p + "b_2"]
            h = h + g2 * mlp
    fv = T["W_fa"] @ c + T["b_fa"]
    z = ln(h) * (1 + fv[d:]) + fv[:d]
    return (z @ T["W_lm"].T).numpy(), h.numpy()


@pytest.mark.parametrize("variant", ["random", "unit_gate"])
def test_forward_matches_independent_torch_composition(variant):
    cfg = TINY
    w = synth.make_weights(cfg, variant)
    W = oracle.Weights.from_storage(w)
    feats, noise = synth.make_features(cfg), synth.make_noise(cfg)[0]
    out = oracle.draft(W, cfg, noise, feats)
    ref_logits, ref_h = _torch_forward(cfg, W, noise, feats)
    assert np.allclose(out["jumps"][0]["h"], ref_h, rtol=0, atol=1e-9)
    # oracle logits are rounded to float32
    assert np.allclose(out["logits"], ref_logits, rtol=1e-6, atol=1e-6)
    if variant == "unit_gate":
        # blocks contribute at full strength: h moves far from h0
        assert np.abs(out["jumps"][0]["h"] - out["jumps"][0]["h0"]).max() > 0.5


def test_empty_context_is_attention_over_the_block_alone():
    """With no context rows the keys are the block's own rows only."""
    cfg = TINY
    w = synth.make_weights(cfg)
    W = oracle.Weights.from_storage(w)
    noise = synth.make_noise(cfg)[0]
    empty = np.zeros((0, 5, cfg.H), dtype=np.float32)
    out = oracle.draft(W, cfg, noise, empty)
    ref_logits, ref_h = _torch_forward(cfg, W, noise, empty)
    assert np.allclose(out["jumps"][0]["h"], ref_h, rtol=0, atol=1e-9)
    assert np.allclose(out["logits"], ref_logits, rtol=1e-6, atol=1e-6)


def test_gate_zero_reduces_to_two_matrix_products(tiny):
    cfg = TINY
    w = synth.make_weights(cfg, "gate_zero")
    W = oracle.Weights.from_storage(w)
    _, _, _, feats, noise = tiny
    out = oracle.draft(W, cfg, noise[0], feats)
    t = {k: torch.from_numpy(v) for k, v in W.items()}
    x = torch.from_numpy(oracle.from_storage(noise[0]))
    ref_h = x @ t["E"] + torch.from_numpy(oracle.positions(cfg.K, cfg.d))
    assert np.allclose(out["jumps"][0]["h"], ref_h.numpy(), atol=1e-12)
    sh, sc = out["jumps"][0]["mods"]["final"]
    z = Fn.layer_norm(ref_h, (cfg.d,), eps=1e-6) * (1 + torch.from_numpy(sc)) + torch.from_numpy(sh)
    logits = (z @ t["W_lm"].T).numpy().astype(np.float32)
    assert np.array_equal(out["tokens"], np.argmax(logits, axis=1))


def test_one_hot_noise_row_is_an_embedding_lookup(tiny):
    cfg, _, W, feats, noise = tiny
    x = np.zeros((cfg.K, cfg.V), dtype=np.float32)
    vocab_ids = [5, 0, 1023, 77] * 4
    for k, v in enumerate(vocab_ids):
        x[k, v] = 1.0
    out = oracle.draft(W, cfg, x, feats, use_pos=False)
    assert np.array_equal(out["jumps"][0]["h0"], W["E"][vocab_ids])
    out = oracle.draft(W, cfg, x, feats)
    assert np.allclose(out["jumps"][0]["h0"] - oracle.positions(cfg.K, cfg.d),
                       W["E"][vocab_ids], rtol=0, atol=1e-15)


def test_context_permutation_invariance(tiny):
    cfg, _, W, feats, noise = tiny
    a = oracle.draft(W, cfg, noise[0], feats)
    p = np.random.default_rng(5).permutation(feats.shape[0])
    b = oracle.draft(W, cfg, noise[0], feats[p])
    assert np.allclose(a["logits"], b["logits"], atol=1e-5)
    assert np.array_equal(a["tokens"], b["tokens"])


def test_block_row_equivariance_without_positions(tiny):
    cfg, _, W, feats, noise = tiny
    p = np.random.default_rng(6).permutation(cfg.K)
    a = oracle.draft(W, cfg, noise[0], feats, use_pos=False)
    b = oracle.draft(W, cfg, noise[0][p], feats, use_pos=False)
    assert np.allclose(a["logits"][p], b["logits"], atol=1e-5)
    # with positions the rows are not merely permuted
    c = oracle.draft(W, cfg, noise[0][p], feats)
    assert not np.allclose(oracle.draft(W, cfg, noise[0], feats)["logits"][p], c["logits"], atol=1e-3)


def test_flow_map_closed_forms():
    rng = np.random.default_rng(8)
    x, D = rng.standard_normal((4, 10)), oracle.softmax_rows(rng.standard_normal((4, 10)))
    for s in (0.0, 0.3, 0.5):
        assert np.array_equal(oracle.flow_map(x, D, s, s), x)
        assert np.allclose(oracle.flow_map(x, D, s, 1.0), D, atol=1e-15)
    # semigroup: jumping 0 -> 0.5 -> 1 with the same D equals one jump 0 -> 1
    mid = oracle.flow_map(x, D, 0.0, 0.5)
    assert np.allclose(oracle.flow_map(mid, D, 0.5, 1.0), oracle.flow_map(x, D, 0.0, 1.0))
    assert np.allclose(mid, 0.5 * x + 0.5 * D)


def test_zero_lm_head_gives_uniform_denoiser(tiny):
    """W_lm = 0: logits 0, D = 1/V, every token 0 (lowest index), and the
    two-step midpoint embedding is exactly (0.5 x0 + 0.5/V) E."""
    cfg, w, W, feats, noise = tiny
    W0 = oracle.Weights(W)
    W0["W_lm"] = np.zeros_like(W["W_lm"])
    out = oracle.draft(W0, cfg, noise[0], feats, times=(0.0, 0.5, 1.0))
    assert np.all(out["tokens"] == 0)
    x0 = oracle.from_storage(noise[0])
    mid = 0.5 * x0 + 0.5 / cfg.V
    P = oracle.positions(cfg.K, cfg.d)
    assert np.allclose(out["jumps"][1]["h0"] - P, mid @ W["E"], atol=1e-12)


def test_two_step_schedule_runs_two_jumps(tiny):
    cfg, _, W, feats, noise = tiny
    one = oracle.draft(W, cfg, noise[0], feats)
    two = oracle.draft(W, cfg, noise[0], feats, times=(0.0, 0.5, 1.0))
    assert len(two["jumps"]) == 2
    assert np.array_equal(two["jumps"][0]["h0"], one["jumps"][0]["h0"])
    # the first jump of the 2-step schedule uses the (0, 0.5) modulation
    assert not np.allclose(two["jumps"][0]["logits"], one["logits"])
    with pytest.raises(ValueError):
        oracle.draft(W, cfg, noise[0], feats, times=(0.0, 0.7, 0.5, 1.0))


def test_bf16_rounding_points_hold_bf16_values():
    cfg = TINY.with_(dtype="bf16")
    w = synth.make_weights(cfg)
    W = oracle.Weights.from_storage(w)
    out = oracle.draft(W, cfg, synth.make_noise(cfg)[0], synth.make_features(cfg), trace=True)
    for blk in out["jumps"][0]["blocks"]:
        for key in ("a", "q", "kb", "vb", "kc", "vc", "o", "m", "g"):
            assert np.array_equal(oracle.round_bf16(blk[key]), blk[key]), key
    assert np.array_equal(oracle.round_bf16(out["u"]), out["u"])
    # the residual stream is not rounded
    h = out["jumps"][0]["h"]
    assert not np.array_equal(oracle.round_bf16(h), h)


def test_tree_branches_are_independent_drafts(tiny):
    cfg, _, W, feats, _ = tiny
    noises = synth.make_noise(cfg, 3)
    tree = oracle.draft_tree(W, cfg, noises, feats)
    for b in range(3):
        assert np.array_equal(tree[b]["tokens"], oracle.draft(W, cfg, noises[b], feats)["tokens"])


def test_parameter_count_near_reported_drafter_sizes():
    """The pages report 500M (Qwen3-8B) and 475M (Qwen3-4B) drafter parameters;
    the reading of the architecture (frozen embedding and LM head excluded)
    lands within 5% of both."""
    n8 = oracle.trainable_params(synth.CONFIGS["qwen3_8b"])
    n4 = oracle.trainable_params(synth.CONFIGS["qwen3_4b"])
    assert abs(n8 / 500e6 - 1) < 0.05, n8
    assert abs(n4 / 475e6 - 1) < 0.05, n4
    assert n8 > n4
