"""GPU parity at the full workload sizes (Qwen3-8B/4B-shaped, 2-step, 4-branch
tree), in the launch configuration bench.py times: tokens exact (near-ties
reported), logits within 2e-2 norm-wise, verify accept lengths bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

fm = pytest.importorskip("step_flow_map_amd")
from gpu_util import check_tokens, make_drafter, rowwise_rel_err, to_dev, LOGIT_RTOL  # noqa: E402


@pytest.mark.parametrize("name", ["qwen3_8b", "qwen3_4b", "qwen3_8b_2step", "qwen3_8b_tree4"])
def test_full_size_draft_and_verify(name):
    cfg = synth.CONFIGS[name]
    print(f"[full parity] {name}", flush=True)
    w = synth.make_weights(cfg)
    feats = synth.make_features(cfg)
    noise = synth.make_noise(cfg)
    dr = make_drafter(cfg, w, max_new=max(cfg.n_new, 1))
    dr.set_schedule(cfg.times)
    dr.append(to_dev(feats[:cfg.c_prefill]))
    logits = torch.empty(cfg.B, cfg.K, cfg.V, device="cuda")
    tok = dr.draft(to_dev(noise), new_feats=to_dev(feats[cfg.c_prefill:]), logits=logits)
    torch.cuda.synchronize()
    tok, logits = tok.cpu().numpy(), logits.cpu().numpy()
    del dr
    W = oracle.Weights.from_storage(w)
    ties, worst = [], 0.0
    refs = []
    for b in range(cfg.B):
        ref = oracle.draft(W, cfg, noise[b], feats)
        refs.append(ref["tokens"])
        rel = rowwise_rel_err(logits[b], ref["logits"])
        worst = max(worst, float(rel.max()))
        assert rel.max() <= LOGIT_RTOL, f"branch {b}: logit error {rel.max():.3e}"
        ties += check_tokens(tok[b], logits[b], ref["logits"], ref["tokens"])
    del W
    print(f"  max row logit error {worst:.2e}; near-ties {ties}", flush=True)
    # verify against target logits planted on the oracle's drafts
    T = synth.make_target_logits(cfg)
    planted = synth.PLANTED_ACCEPT_TREE if cfg.B > 1 else (7,)
    for b in range(cfg.B):
        T[b] = synth.plant(T[b], refs[b], planted[b])
    e, a, best = fm.verify(to_dev(T), torch.from_numpy(tok.astype(np.int32)).cuda())
    res, rbest = oracle.verify_tree([T[b] for b in range(cfg.B)], tok)
    assert a.cpu().numpy().tolist() == [n for n, _ in res]
    for b, (n, em) in enumerate(res):
        assert e.cpu().numpy()[b, :n + 1].tolist() == em
    assert int(best.cpu()[0]) == rbest
    if not ties:
        assert [n for n, _ in res] == list(planted)


def test_full_size_sampled_draft_and_verify():
    """Qwen3-8B-shaped step at temperature 1 in the launch configuration
    bench.py times (fm_draft_sample, then fm_verify_sample on the unplanted
    target logits): logits within 2e-2, sampled tokens and the verifier's
    outcome equal to the oracle's except reported near-ties."""
    from gpu_util import check_sampled_tokens, is_near_tie, ref_verify_sample
    cfg = synth.CONFIGS["qwen3_8b_t1"]
    tau = cfg.temperature
    print("[full parity] qwen3_8b_t1", flush=True)
    w = synth.make_weights(cfg)
    feats = synth.make_features(cfg)
    noise = synth.make_noise(cfg)
    dr = make_drafter(cfg, w, max_new=max(cfg.n_new, 1))
    dr.set_schedule(cfg.times)
    dr.append(to_dev(feats[:cfg.c_prefill]))
    T = synth.make_target_logits(cfg)
    T_dev = to_dev(T)
    outcomes = []
    for seed in synth.SAMPLE_SEEDS[:3]:
        dr.truncate(cfg.c_prefill)
        tok, logits, lse = dr.draft_sample(to_dev(noise), tau, seed, new_feats=to_dev(feats[cfg.c_prefill:]))
        e, a = dr.verify_sample(T_dev, logits, lse, tok, tau, seed)
        torch.cuda.synchronize()
        outcomes.append((seed, tok.cpu().numpy(), logits.cpu().numpy(), e.cpu().numpy(), a.cpu().numpy()))
    del dr
    W = oracle.Weights.from_storage(w)
    ref_logits = oracle.draft(W, cfg, noise[0], feats)["logits"]
    del W
    Tv = synth.values(T).astype(np.float64)
    for seed, tok, logits, e, a in outcomes:
        rel = rowwise_rel_err(logits[0], ref_logits)
        assert rel.max() <= LOGIT_RTOL, rel.max()
        ties = check_sampled_tokens(tok, logits, [ref_logits], tau, seed)
        re, ra, rs = ref_verify_sample(Tv, logits.astype(np.float64), tok, tau, seed)
        if a[0] != ra[0] or not np.array_equal(e[0], re[0]):
            assert is_near_tie(Tv, logits.astype(np.float64), tok, tau, seed, 0, int(a[0]), rs[0])
            ties.append(("verify", seed))
        print(f"  seed {seed}: logit error {rel.max():.2e}, accepted {int(a[0])}, near-ties {ties}", flush=True)
