"""Helpers for the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI, compare with the oracle under the stated tolerances."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import step_flow_map_amd as fm
import synth

S = oracle.sampling

# logits: per row, max |gpu - ref| <= LOGIT_RTOL * max |ref|   (norm-wise relative)
LOGIT_RTOL = 2e-2
# residual stream after every block, same norm-wise measure
HIDDEN_RTOL = 2e-2
# a draft token may differ from the oracle's only where the oracle's gap between
# the two candidates is within NEAR_TIE_FACTOR x the row's measured logit error
NEAR_TIE_FACTOR = 4.0


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def binding_weights(w: dict, device="cuda") -> dict:
    out = {}
    for k, v in w.items():
        name = k.replace("te_s.", "te_s_").replace("te_t.", "te_t_")
        out[name] = to_dev(v, device)
    return out


def make_drafter(cfg, w, C_max=None, max_steps=None, max_new=16, max_branches=None):
    c = fm.make_config(K=cfg.K, V=cfg.V, d=cfg.d, L=cfg.L, n_heads=cfg.nh, H=cfg.H,
                       C_max=cfg.capacity if C_max is None else C_max, dtype=cfg.dtype,
                       max_branches=cfg.B if max_branches is None else max_branches,
                       max_new=max_new, max_steps=max(cfg.num_steps, 1) if max_steps is None else max_steps)
    return fm.Drafter(c, binding_weights(w))


def run_draft(dr: fm.Drafter, cfg, noise: np.ndarray, feats: np.ndarray, prefill: int, want_hidden=False):
    """Prefill `prefill` context rows, then draft with the remaining rows as
    n_new.  Returns numpy (tokens [B][K], logits [B][K][V], hidden or None)."""
    dev = dr.device
    if prefill:
        dr.append(to_dev(feats[:prefill]))
    new = to_dev(feats[prefill:]) if feats.shape[0] > prefill else None
    x = to_dev(noise)
    B = noise.shape[0]
    logits = torch.empty(B, cfg.K, cfg.V, dtype=torch.float32, device=dev)
    hidden = None
    if want_hidden:
        hidden = torch.empty(cfg.num_steps, cfg.L + 1, B, cfg.K, cfg.d, dtype=torch.float32, device=dev)
    tok = dr.draft(x, new_feats=new, logits=logits, hidden=hidden)
    torch.cuda.synchronize()
    return (tok.cpu().numpy(), logits.cpu().numpy(),
            None if hidden is None else hidden.cpu().numpy())


def rowwise_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    got = got.reshape(-1, got.shape[-1]).astype(np.float64)
    ref = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    return np.abs(got - ref).max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-30)


def check_tokens(tok_gpu, logits_gpu, ref_logits, ref_tok):
    """Exact token parity, except near-ties (reported).  Also: each GPU token is
    the lowest-index argmax of the GPU's own float32 logits, always."""
    tok_gpu = tok_gpu.reshape(-1)
    lg = logits_gpu.reshape(-1, logits_gpu.shape[-1])
    lr = ref_logits.reshape(-1, ref_logits.shape[-1])
    rt = np.asarray(ref_tok).reshape(-1)
    own = oracle.argmax_lowest(lg)
    assert np.array_equal(tok_gpu, own), "fused argmax differs from argmax of the dumped logits"
    ties = []
    for r in range(tok_gpu.shape[0]):
        if tok_gpu[r] != rt[r]:
            err = np.abs(lg[r].astype(np.float64) - lr[r]).max()
            gap = lr[r][rt[r]] - lr[r][tok_gpu[r]]
            assert gap <= NEAR_TIE_FACTOR * err, (
                f"row {r}: token {tok_gpu[r]} vs oracle {rt[r]}, oracle gap {gap:.3e} > "
                f"{NEAR_TIE_FACTOR} x logit error {err:.3e}")
            ties.append((r, float(gap), float(err)))
    return ties


def check_draft(cfg, w, noise, feats, prefill, tok, logits, hidden=None, times=None):
    W = oracle.Weights.from_storage(w)
    rel_max = 0.0
    all_ties = []
    for b in range(noise.shape[0]):
        ref = oracle.draft(W, cfg, noise[b], feats, times=times)
        rel = rowwise_rel_err(logits[b], ref["logits"])
        assert rel.max() <= LOGIT_RTOL, f"branch {b}: logit error {rel.max():.3e}"
        rel_max = max(rel_max, float(rel.max()))
        all_ties += check_tokens(tok[b], logits[b], ref["logits"], ref["tokens"])
        if hidden is not None:
            for j, jt in enumerate(ref["jumps"]):
                e = rowwise_rel_err(hidden[j, 0, b], jt["h0"])
                assert e.max() <= HIDDEN_RTOL, f"jump {j} embedding error {e.max():.3e}"
    return rel_max, all_ties


# ------------------------------------------------------------ temperature > 0

# float32 evaluation of a key l / tau + G (division, two logarithms): relative
KEY_EPS = 2e-6
# acceptance u q < p in float32 with a 24-bit uniform
ACCEPT_EPS = 2e-6


def _sample_keys(logits_row, tau, seed, row, branch):
    V = logits_row.shape[0]
    return logits_row.astype(np.float64) / tau + S.gumbel(np.arange(V), row, branch, S.STREAM_DRAFT, seed)


def check_sampled_tokens(tok, logits_gpu, ref_logits, tau, seed):
    """tok [B][K]; logits [B][K][V]; returns the near-ties."""
    ties = []
    B, K, _ = logits_gpu.shape
    for b in range(B):
        for i in range(K):
            own = _sample_keys(logits_gpu[b, i], tau, seed, i, b)
            t = int(tok[b, i])
            eps = KEY_EPS * (1.0 + np.abs(own).max())
            assert own[t] >= own.max() - eps, (b, i, t, int(own.argmax()), own.max() - own[t])
            ref = _sample_keys(ref_logits[b][i], tau, seed, i, b)
            r = int(np.flatnonzero(ref == ref.max())[0])
            if t != r:
                err = np.abs(logits_gpu[b, i].astype(np.float64) - ref_logits[b][i]).max() / tau
                gap = ref[r] - ref[t]
                assert gap <= NEAR_TIE_FACTOR * err + eps, (b, i, t, r, gap, err)
                ties.append((b, i, float(gap)))
    return ties


def ref_verify_sample(T, Q, d, tau, seed):
    B, K = d.shape
    em = np.full((B, K + 1), -1, dtype=np.int64)
    acc = np.zeros(B, dtype=np.int64)
    rs = []
    for b in range(B):
        r = S.verify_sample(T[b], Q[b], d[b], tau, seed, b)
        em[b, :r["n"] + 1] = r["emitted"]
        acc[b] = r["n"]
        rs.append(r)
    return em, acc, rs


def is_near_tie(T, Q, d, tau, seed, b, n_gpu, r):
    """A disagreement is a near-tie when an acceptance margin up to the
    earlier stop is within rounding, or the emitted row's two best keys are."""
    logq = S.log_softmax_rows(Q[b], tau)
    logp = S.log_softmax_rows(T[b], tau)
    stop = min(n_gpu, r["n"])
    for i, m in enumerate(r["margins"][:stop + 1]):
        q = np.exp(logq[i, int(d[b, i])])
        if abs(m) <= ACCEPT_EPS * max(q, 1e-30):
            return True
    if n_gpu == r["n"]:
        n = r["n"]
        K = Q.shape[1]
        p = np.exp(logp[n])
        wgt = np.maximum(p - np.exp(logq[n]), 0.0) if n < K else p
        with np.errstate(divide="ignore"):
            key = np.log(wgt) + S.gumbel(np.arange(T.shape[2]), n, b, S.STREAM_CORRECT, seed)
        top = np.sort(key[np.isfinite(key)])[-2:]
        return len(top) == 2 and top[1] - top[0] <= 1e-4 * (1 + abs(top[1]))
    return False
