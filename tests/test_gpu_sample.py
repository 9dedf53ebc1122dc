"""GPU parity of temperature > 0 drafting (fm_draft_sample) and probabilistic
verification (fm_verify_sample) against the oracle.

Sampled tokens are integers decided by floating point: every GPU token must be
the Gumbel-max winner of the GPU's own float32 logits under the oracle's noise
(up to float32 rounding of the key), and equal to the oracle's sample except
where the oracle's two best keys lie within the logit error / temperature
(near-ties, reported).  Verification outcomes (accepted prefix, emitted
tokens) are compared exactly except where an acceptance margin p - u q or the
emitted sample's key gap is within float32 rounding (near-ties, reported)."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

fm = pytest.importorskip("step_flow_map_amd")
from gpu_util import (check_guards, check_logits, check_sampled_tokens, exact_or_reseed, guarded,  # noqa: E402
                      is_near_tie, make_drafter, ref_verify_sample, to_dev)

S = oracle.sampling
TINY = synth.CONFIGS["tiny"]
SMALL_BF16 = TINY.with_(name="small_bf16", dtype="bf16", V=1000, H=520)
MID_BF16 = TINY.with_(name="mid_bf16", dtype="bf16", V=2000, d=384, nh=3, H=520, c_prefill=300)
WIDE_F32 = TINY.with_(name="wide_f32", V=1000, d=1152, nh=9)
# 10,625 vocabulary tiles over 512 LM-head workgroups: 20 or 21 tiles each, so
# the logits of one launch are written both ways (held in LDS up to 20 tiles,
# stored tile by tile beyond)
WIDEV_BF16 = TINY.with_(name="widev_bf16", dtype="bf16", V=170000, H=520)

def _run_sample(cfg, tau, seed, B=1, draw=0):
    cfg = cfg.with_(B=B)
    w = synth.make_weights(cfg)
    feats = synth.make_features(cfg)
    noise = synth.make_noise(cfg, B, draw)
    dr = make_drafter(cfg, w)
    dr.set_schedule(cfg.times)
    dr.append(to_dev(feats[:cfg.c_prefill]))
    new = to_dev(feats[cfg.c_prefill:]) if feats.shape[0] > cfg.c_prefill else None
    tok = guarded(B, cfg.K, dtype=torch.int32)
    logits = guarded(B, cfg.K, cfg.V)
    lse = guarded(B, cfg.K)
    fm.fm_draft_sample(dr.handle, to_dev(noise), tau, seed, tok, logits, lse, new_feats=new)
    torch.cuda.synchronize()
    check_guards(tok, logits, lse)
    return cfg, w, feats, noise, dr, tok, logits, lse


@pytest.mark.parametrize("cfg,B", [(TINY, 1), (SMALL_BF16, 1), (MID_BF16, 1), (WIDE_F32, 1), (WIDEV_BF16, 1),
                                   (TINY, 4), (MID_BF16, 4), (WIDE_F32, 4)],
                         ids=["tiny_f32", "small_bf16", "mid_bf16", "wide_f32", "widev_bf16", "tiny_tree",
                              "mid_tree", "wide_tree"])
@pytest.mark.parametrize("tau", [0.6, 1.0])
def test_draft_sample_matches_oracle(cfg, B, tau):
    seed = 1234 + B
    print(f"[draft sample] {cfg.name} B={B} tau={tau}", flush=True)

    def case(draw):
        c, w, feats, noise, dr, tok, logits, lse = _run_sample(cfg, tau, seed, B, draw)
        tok, logits, lse = tok.cpu().numpy(), logits.cpu().numpy(), lse.cpu().numpy()
        W = oracle.Weights.from_storage(w)
        refs = [oracle.draft(W, c, noise[b], feats)["logits"] for b in range(B)]
        for b in range(B):
            check_logits(logits[b], refs[b], c.dtype, f"branch {b}:")
        # the log-normaliser is that of the GPU's own logits (float32 online merge)
        own_lse = S.logsumexp_rows(logits.astype(np.float64), tau)
        assert np.abs(lse - own_lse).max() <= 1e-5 * (1 + np.abs(own_lse).max()), np.abs(lse - own_lse).max()
        ties = check_sampled_tokens(tok, logits, refs, tau, seed, c.dtype)
        print(f"  draw {draw}: near-ties {ties}", flush=True)
        # a different seed gives a different draft
        tok2, _, _ = dr.draft_sample(to_dev(noise), tau, seed + 1, new_feats=None)
        assert not np.array_equal(tok2.cpu().numpy(), tok)
        return ties

    exact_or_reseed(case, f"{cfg.name} B={B} tau={tau}")


def test_draft_sample_is_reproducible_and_small_tau_is_greedy():
    cfg = SMALL_BF16
    w = synth.make_weights(cfg)
    feats = synth.make_features(cfg)
    noise = to_dev(synth.make_noise(cfg, 1))
    dr = make_drafter(cfg, w)
    dr.set_schedule(cfg.times)
    dr.append(to_dev(feats))
    a = [dr.draft_sample(noise, 0.8, 77)[0].cpu().numpy() for _ in range(2)]
    assert np.array_equal(a[0], a[1])
    logits = torch.empty(1, cfg.K, cfg.V, device="cuda")
    greedy = dr.draft(noise, logits=logits).cpu().numpy()
    t, lg, _ = dr.draft_sample(noise, 1e-6, 5)
    assert np.array_equal(t.cpu().numpy(), greedy)
    assert torch.equal(lg, logits)


def _verify_handle(V, max_branches=4):
    """A handle with the vocabulary size but no weights: enough for
    fm_verify_sample, whose scratch lives in the handle's workspace."""
    c = fm.make_config(V=V, d=128, L=1, n_heads=1, H=8, C_max=0, dtype="bf16", max_branches=max_branches,
                       max_new=0, max_steps=1)
    n = fm.fm_workspace_bytes(c)
    raw = torch.empty(n + 256, dtype=torch.uint8, device="cuda")
    off = (-raw.data_ptr()) % 256
    ws = raw[off:off + n]
    return fm.fm_create(c, ws, n, 0), raw


def _gpu_verify_sample(h, T, Q, lseQ, d, tau, seed):
    B, K1, V = T.shape
    emitted = guarded(B, K1, dtype=torch.int32)
    accept = guarded(B, dtype=torch.int32)
    fm.fm_verify_sample(h, to_dev(T), to_dev(Q), to_dev(lseQ), torch.from_numpy(d.astype(np.int32)).cuda(),
                        tau, seed, emitted, accept)
    torch.cuda.synchronize()
    check_guards(emitted, accept)
    return emitted.cpu().numpy(), accept.cpu().numpy()


@pytest.mark.parametrize("V,dtype", [(1000, "f32"), (4104, "bf16"), (151936, "bf16")])
def test_verify_sample_matches_oracle(V, dtype):
    """Synthetic drafter logits Q, drafts sampled from them by the oracle, and
    target logits that agree with Q up to noise (so the accepted prefix
    varies); four branches, several seeds."""
    print(f"[verify sample] V={V} {dtype}", flush=True)
    h, ws = _verify_handle(V)
    rng = np.random.default_rng(V)
    B, K = 4, 16
    ties, lengths = [], []
    n_seeds = 8 if V > 10000 else 40
    for seed in range(n_seeds):
        tau = [1.0, 0.7, 1.3][seed % 3]
        Q = (rng.standard_normal((B, K, V)) * 1.5).astype(np.float32)
        noise_scale = [0.05, 0.3, 1.0][seed % 3]
        T = np.concatenate([Q + noise_scale * rng.standard_normal((B, K, V)),
                            rng.standard_normal((B, 1, V))], axis=1)
        if dtype == "bf16":
            T_vals = oracle.round_bf16(T)
            T_dev = _bf16_bits(T_vals)      # exact: the values are bf16 already
        else:
            T_vals = T.astype(np.float32).astype(np.float64)
            T_dev = T.astype(np.float32)
        lseQ = S.logsumexp_rows(Q.astype(np.float64), tau).astype(np.float32)
        d = np.stack([S.sample_draft(Q[b], tau, seed, b) for b in range(B)])
        e, a = _gpu_verify_sample(h, T_dev, Q, lseQ, d, tau, seed)
        re, ra, rs = ref_verify_sample(T_vals, Q, d, tau, seed)
        for b in range(B):
            if a[b] != ra[b] or not np.array_equal(e[b], re[b]):
                assert is_near_tie(T_vals, Q, d, tau, seed, b, int(a[b]), rs[b]), (seed, b, a[b], ra[b], e[b], re[b])
                ties.append((seed, b))
            else:
                lengths.append(int(a[b]))
    fm.fm_destroy(h)
    print(f"  accepted lengths {sorted(set(lengths))}, near-ties {ties}")
    assert len(ties) <= 2
    assert len(set(lengths)) >= 3        # the cases exercise several prefix lengths


def _bf16_bits(vals):
    f = np.asarray(vals, dtype=np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def test_verify_sample_of_drafter_output():
    """End to end at temperature 1: draft_sample, then verify_sample against
    target logits planted near the drafter's logits."""
    cfg = MID_BF16
    tau, seed = 1.0, 42
    cfg, w, feats, noise, dr, tok, logits, lse = _run_sample(cfg, tau, seed, B=1)
    rng = np.random.default_rng(3)
    Q = logits.cpu().numpy()
    T = np.concatenate([Q + 0.2 * rng.standard_normal(Q.shape), rng.standard_normal((1, 1, cfg.V))], axis=1)
    T_vals = oracle.round_bf16(T)
    e, a = dr.verify_sample(to_dev(_bf16_bits(T_vals)), logits, lse, tok, tau, seed)
    torch.cuda.synchronize()
    re, ra, rs = ref_verify_sample(T_vals, Q, tok.cpu().numpy(), tau, seed)
    if a.cpu().numpy()[0] != ra[0] or not np.array_equal(e.cpu().numpy()[0], re[0]):
        assert is_near_tie(T_vals, Q, tok.cpu().numpy(), tau, seed, 0, int(a.cpu()[0]), rs[0])
    print(f"  accepted {int(a.cpu()[0])}, emitted {e.cpu().numpy()[0].tolist()}")
