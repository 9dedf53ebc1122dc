"""fm_verify_sample_noalloc, the probabilistic verifier for callers that cannot
allocate (its scratch is a static device array of the library, no handle),
against fm_verify_sample (scratch in a handle's workspace) on the same inputs:
accepted prefixes and emitted tokens bit-identical, on two calls in a row, the
second with a smaller input (fewer branches, a shorter vocabulary, the other
storage type), so it runs over what the first left in the shared array."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

fm = pytest.importorskip("step_flow_map_amd")

S = oracle.sampling
K = 16


def _handle(V):
    c = fm.make_config(V=V, d=128, L=1, n_heads=1, H=8, C_max=0, dtype="bf16", max_branches=4, max_new=0,
                       max_steps=1)
    n = fm.fm_workspace_bytes(c)
    raw = torch.empty(n + 256, dtype=torch.uint8, device="cuda")
    off = (-raw.data_ptr()) % 256
    return fm.fm_create(c, raw[off:off + n], n, 0), raw


def _inputs(B, V, dtype, tau, seed):
    """Drafter logits, their normalisers, drafts sampled from them (oracle),
    and target logits that agree with the drafter up to noise."""
    rng = np.random.default_rng(seed)
    Q = (rng.standard_normal((B, K, V)) * 1.5).astype(np.float32)
    T = np.concatenate([Q + 0.3 * rng.standard_normal((B, K, V)), rng.standard_normal((B, 1, V))],
                       axis=1).astype(np.float32)
    lseQ = S.logsumexp_rows(Q.astype(np.float64), tau).astype(np.float32)
    d = np.stack([S.sample_draft(Q[b], tau, seed, b) for b in range(B)]).astype(np.int32)
    Td = torch.from_numpy(T).cuda()
    if dtype == "bf16":
        Td = Td.to(torch.bfloat16)
    return Td, torch.from_numpy(Q).cuda(), torch.from_numpy(lseQ).cuda(), torch.from_numpy(d).cuda()


def test_noalloc_verifier_matches_the_handle_verifier():
    cases = [(4, 151936, "bf16", 1.0, 11), (2, 4104, "f32", 0.7, 12)]   # the second call is smaller
    for B, V, dtype, tau, seed in cases:
        print(f"[no-alloc verify] B={B} V={V} {dtype}", flush=True)
        T, Q, lseQ, d = _inputs(B, V, dtype, tau, seed)
        h, ws = _handle(V)
        e_ref = torch.empty(B, K + 1, dtype=torch.int32, device="cuda")
        a_ref = torch.empty(B, dtype=torch.int32, device="cuda")
        fm.fm_verify_sample(h, T, Q, lseQ, d, tau, seed, e_ref, a_ref)
        e = torch.full((B, K + 1), -7, dtype=torch.int32, device="cuda")
        a = torch.full((B,), -7, dtype=torch.int32, device="cuda")
        fm.fm_verify_sample_noalloc(T, Q, lseQ, d, tau, seed, e, a)
        torch.cuda.synchronize()
        fm.fm_destroy(h)
        assert torch.equal(a, a_ref), (a.tolist(), a_ref.tolist())
        assert torch.equal(e, e_ref)
        print(f"  accepted {a.tolist()}", flush=True)


def test_noalloc_verifier_rejects_sizes_beyond_its_scratch():
    T, Q, lseQ, d = _inputs(5, 1000, "f32", 1.0, 3)
    e = torch.empty(5, K + 1, dtype=torch.int32, device="cuda")
    a = torch.empty(5, dtype=torch.int32, device="cuda")
    with pytest.raises(fm.FlashMapError) as err:
        fm.fm_verify_sample_noalloc(T, Q, lseQ, d, 1.0, 3, e, a)
    assert err.value.status == fm.FM_ECAPACITY
    assert "static scratch" in str(err.value)
