"""GPU parity of fm_draft_batch: R independent requests, each with its own
context, drafted together as R*16 rows.  Every request's draft must match the
oracle's draft of that request alone (logits within 2e-2 norm-wise, tokens
exact except reported near-ties); a request's result must not depend on the
other requests' data (bitwise); greedy verification of the batch is per
request."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

fm = pytest.importorskip("step_flow_map_amd")
from gpu_util import (binding_weights, check_guards, check_logits, check_sampled_tokens, check_tokens,  # noqa: E402
                      exact_or_reseed, guarded, is_near_tie, ref_verify_sample, to_dev)

TINY = synth.CONFIGS["tiny"]
MID_BF16 = TINY.with_(name="mid_bf16", dtype="bf16", V=2000, d=384, nh=3, H=520, c_prefill=300)


def _handle(cfg, w, R, C_max, max_new=16):
    c = fm.make_config(K=cfg.K, V=cfg.V, d=cfg.d, L=cfg.L, n_heads=cfg.nh, H=cfg.H, C_max=C_max,
                       dtype=cfg.dtype, max_new=max_new, max_steps=max(cfg.num_steps, 1), max_requests=R)
    return fm.Drafter(c, binding_weights(w))


def _run(cfg, w, prefill, new, noise, feats, seed_dr=None):
    """prefill[r] rows appended per request, then new[r] rows inside the batch
    draft.  Returns tokens [R][K] and logits [R][K][V] (numpy)."""
    R = len(prefill)
    dr = _handle(cfg, w, R, C_max=max(p + n for p, n in zip(prefill, new)) + 8)
    dr.set_schedule(cfg.times)
    for r in range(R):
        if prefill[r]:
            dr.append_req(r, to_dev(feats[r][:prefill[r]]))
    rows = [feats[r][prefill[r]:prefill[r] + new[r]] for r in range(R)]
    cat = np.concatenate(rows) if sum(new) else None
    logits = guarded(R, cfg.K, cfg.V)
    tok = guarded(R, cfg.K, dtype=torch.int32)
    dr.draft_batch(to_dev(noise), new_feats=None if cat is None else to_dev(cat), n_new=new, logits=logits,
                   tokens=tok)
    torch.cuda.synchronize()
    check_guards(logits, tok)
    for r in range(R):
        assert dr.context_length_req(r) == prefill[r] + new[r]
    return tok.cpu().numpy(), logits.cpu().numpy(), dr


@pytest.mark.parametrize("cfg", [TINY, MID_BF16], ids=["tiny_f32", "mid_bf16"])
@pytest.mark.parametrize("variant", ["random", "unit_gate"])
def test_batch_matches_oracle_per_request(cfg, variant):
    """Three requests with different context lengths (one empty) and
    different numbers of appended rows (one none)."""
    print(f"[batch parity] {cfg.name} {variant}", flush=True)
    R = 3
    prefill = [cfg.c_prefill, 5, 0]
    new = [4, 0, 7]
    w = synth.make_weights(cfg, variant)
    feats = [synth.make_features(cfg, rows=prefill[r] + new[r], request=r) for r in range(R)]
    _batch_parity(cfg, w, prefill, new, feats, f"{cfg.name} {variant}")


def _batch_parity(cfg, w, prefill, new, feats, label):
    """Each request's draft against the oracle's draft of that request alone,
    on each noise draw the re-seed rule asks for."""
    R = len(prefill)
    W = oracle.Weights.from_storage(w)

    def case(draw):
        noise = synth.make_noise(cfg, R, draw)
        tok, logits, dr = _run(cfg, w, prefill, new, noise, feats)
        ties, worst = [], 0.0
        for r in range(R):
            ref = oracle.draft(W, cfg, noise[r], feats[r])
            worst = max(worst, check_logits(logits[r], ref["logits"], cfg.dtype, f"request {r}:"))
            ties += [(r,) + t for t in check_tokens(tok[r], logits[r], ref["logits"], ref["tokens"], cfg.dtype)]
        print(f"  {label} draw {draw}: max row logit error {worst:.2e}; near-ties {ties}", flush=True)
        return ties

    exact_or_reseed(case, label)


W2048_BF16 = TINY.with_(name="w2048_bf16", dtype="bf16", V=2000, d=2048, nh=16, H=520, c_prefill=40)


def test_batch_of_four_at_width_2048():
    """Four requests at the drafter's real width (64 block rows plus 13
    appended context rows in QKV): the contractions keep the rows' k slice in
    LDS, and the residual reduces apply the following LayerNorm.  Contexts of
    40, 33, 0 and 70 rows appending 4, 0, 7 and 2."""
    cfg = W2048_BF16
    print(f"[batch parity] {cfg.name} x4", flush=True)
    R = 4
    prefill = [40, 33, 0, 70]
    new = [4, 0, 7, 2]
    w = synth.make_weights(cfg)
    feats = [synth.make_features(cfg, rows=prefill[r] + new[r], request=r) for r in range(R)]
    _batch_parity(cfg, w, prefill, new, feats, f"{cfg.name} x4")


def test_requests_do_not_see_each_other():
    """Request 0's draft is bitwise the same whatever request 1 holds."""
    cfg = MID_BF16
    w = synth.make_weights(cfg)
    noise = synth.make_noise(cfg, 2)
    f0 = synth.make_features(cfg, rows=40, request=0)
    a = _run(cfg, w, [36, 20], [4, 3], noise, [f0, synth.make_features(cfg, rows=23, request=1)])
    b = _run(cfg, w, [36, 60], [4, 1], noise, [f0, synth.make_features(cfg, rows=61, request=2)])
    assert np.array_equal(a[0][0], b[0][0])
    assert np.array_equal(a[1][0], b[1][0])
    assert not np.array_equal(a[1][1], b[1][1])


def test_batch_contexts_advance_and_truncate_per_request():
    cfg = TINY
    w = synth.make_weights(cfg)
    noise = synth.make_noise(cfg, 2)
    feats = [synth.make_features(cfg, rows=30, request=r) for r in range(2)]
    tok1, lg1, dr = _run(cfg, w, [20, 10], [4, 8], noise, feats)
    # roll request 0 back and draft again with the same rows: same result
    dr.truncate_req(0, 20)
    dr.truncate_req(1, 10)
    cat = np.concatenate([feats[0][20:24], feats[1][10:18]])
    lg2 = torch.empty(2, cfg.K, cfg.V, dtype=torch.float32, device="cuda")
    tok2 = dr.draft_batch(to_dev(noise), new_feats=to_dev(cat), n_new=[4, 8], logits=lg2)
    torch.cuda.synchronize()
    assert np.array_equal(tok2.cpu().numpy(), tok1)
    assert np.array_equal(lg2.cpu().numpy(), lg1)
    with pytest.raises(fm.FlashMapError):
        dr.truncate_req(2, 0)                       # no request 2
    with pytest.raises(fm.FlashMapError) as e:
        dr.draft_batch(to_dev(synth.make_noise(cfg, 3)))   # R > max_requests
    assert e.value.status == fm.FM_ECAPACITY
    assert dr.context_length_req(0) == 24 and dr.context_length_req(1) == 18


def test_batch_verify_is_per_request():
    cfg = TINY
    w = synth.make_weights(cfg)
    R = 3
    noise = synth.make_noise(cfg, R)
    feats = [synth.make_features(cfg, rows=12, request=r) for r in range(R)]
    tok, logits, dr = _run(cfg, w, [8, 8, 8], [4, 4, 4], noise, feats)
    T = synth.make_target_logits(cfg, R)
    planted = [3, 16, 0]
    for r in range(R):
        T[r] = synth.plant(T[r], tok[r], planted[r])
    e, a, _ = fm.verify(to_dev(T), torch.from_numpy(tok.astype(np.int32)).cuda())
    torch.cuda.synchronize()
    assert a.cpu().numpy().tolist() == planted
    for r in range(R):
        n, em = oracle.verify(T[r], tok[r])
        assert e.cpu().numpy()[r, :n + 1].tolist() == em


@pytest.mark.parametrize("cfg", [TINY, MID_BF16], ids=["tiny_f32", "mid_bf16"])
def test_batch_sample_uses_each_requests_seed(cfg):
    """Three requests (different context lengths, one without appended rows)
    sampled together at temperature 0.8, each with its own seed: request r's
    logits match the oracle's draft of that request alone and its tokens are
    the oracle's sample under seeds[r] as branch 0 (near-ties excepted).
    fm_verify_sample_batch then verifies request r as the oracle verifies it
    alone with seeds[r], against target logits near the drafter's."""
    print(f"[batch sample] {cfg.name}", flush=True)
    tau, seeds = 0.8, [1001, 2002, 3003]
    R = 3
    prefill, new = [cfg.c_prefill, 5, 0], [4, 0, 7]
    w = synth.make_weights(cfg)
    W = oracle.Weights.from_storage(w)
    feats = [synth.make_features(cfg, rows=prefill[r] + new[r], request=r) for r in range(R)]
    S = oracle.sampling

    def case(draw):
        noise = synth.make_noise(cfg, R, draw)
        dr = _handle(cfg, w, R, C_max=max(p + n for p, n in zip(prefill, new)) + 8)
        dr.set_schedule(cfg.times)
        for r in range(R):
            if prefill[r]:
                dr.append_req(r, to_dev(feats[r][:prefill[r]]))
        cat = np.concatenate([feats[r][prefill[r]:] for r in range(R)])
        tok = guarded(R, cfg.K, dtype=torch.int32)
        logits = guarded(R, cfg.K, cfg.V)
        lse = guarded(R, cfg.K)
        fm.fm_draft_batch_sample(dr.handle, to_dev(noise), tau, seeds, tok, logits, lse, new_feats=to_dev(cat),
                                 n_new=new)
        torch.cuda.synchronize()
        check_guards(tok, logits, lse)
        tk, lg, ls = tok.cpu().numpy(), logits.cpu().numpy(), lse.cpu().numpy()
        ties = []
        for r in range(R):
            ref = oracle.draft(W, cfg, noise[r], feats[r])["logits"]
            check_logits(lg[r], ref, cfg.dtype, f"request {r}:")
            own = S.logsumexp_rows(lg[r].astype(np.float64), tau)
            assert np.abs(ls[r] - own).max() <= 1e-5 * (1 + np.abs(own).max())
            ties += [(r,) + t for t in check_sampled_tokens(tk[r:r + 1], lg[r:r + 1], [ref], tau, seeds[r],
                                                            cfg.dtype)]
        # probabilistic verification of every request with its own seed
        rng = np.random.default_rng(11 + draw)
        T = np.concatenate([lg + 0.2 * rng.standard_normal(lg.shape), rng.standard_normal((R, 1, cfg.V))], axis=1)
        if cfg.dtype == "bf16":
            T_vals = oracle.round_bf16(T)
            T_dev = to_dev(synth.to_bf16_bits(T_vals.astype(np.float32)))
        else:
            T_vals = T.astype(np.float32).astype(np.float64)
            T_dev = to_dev(T.astype(np.float32))
        em = guarded(R, cfg.K + 1, dtype=torch.int32)
        acc = guarded(R, dtype=torch.int32)
        fm.fm_verify_sample_batch(dr.handle, T_dev, logits, lse, tok, tau, seeds, em, acc)
        torch.cuda.synchronize()
        check_guards(em, acc)
        e, a = em.cpu().numpy(), acc.cpu().numpy()
        for r in range(R):
            re, ra, rs = ref_verify_sample(T_vals[r:r + 1], lg[r:r + 1], tk[r:r + 1], tau, seeds[r])
            if a[r] != ra[0] or not np.array_equal(e[r], re[0]):
                assert is_near_tie(T_vals[r:r + 1], lg[r:r + 1], tk[r:r + 1], tau, seeds[r], 0, int(a[r]), rs[0]), (
                    r, a[r], ra[0])
                ties.append((r, "verify"))
        print(f"  draw {draw}: accepted {a.tolist()}, near-ties {ties}", flush=True)
        dr.close()
        return ties

    exact_or_reseed(case, f"batch sample {cfg.name}")
