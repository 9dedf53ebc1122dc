"""One captured HIP graph of draft -> verify replayed over several cycles of
the speculative loop (alphasignal.ai, "Why drafting still costs time": propose
a block, score it in parallel, keep the longest matching prefix, resume from a
target token).  The context length lives on the device, so every replay writes
its new context rows after the previous ones and attends over the grown
context; each cycle is matched against the oracle drafting over every row so
far.  Each cycle appends n + 1 rows for the n = 7 tokens its target logits
accept, plus the target's own token.

Every replay is one draft: its logits are held to the contract and the
regression bound, and its tokens must match the oracle's except at near-ties
inside the fixed window, at most one per draft.  (The single-draft parity
tests also re-run a case with a near-tie on the next noise draw; four chained
drafts would make that re-run itself a coin toss at the bf16 error level.)"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

fm = pytest.importorskip("step_flow_map_amd")
from gpu_util import check_logits, check_tokens, make_drafter, to_dev  # noqa: E402

TINY = synth.CONFIGS["tiny"]
ACCEPT = 7            # planted accepted prefix of every cycle
ROWS = ACCEPT + 1     # context rows each cycle appends
CYCLES = 4


def _copy(dst: torch.Tensor, a: np.ndarray):
    dst.copy_(to_dev(a).view(dst.shape))


@pytest.mark.parametrize("cfg", [
    # context 300 -> 332 rows: the attention's key ranges, planned on the device
    # from the current length, change between replays (10 -> 11 blocks)
    TINY.with_(name="mid_bf16", dtype="bf16", V=2000, d=384, nh=3, H=520, c_prefill=300, n_new=ROWS),
    # the drafter's real width (fused LayerNorm path)
    TINY.with_(name="w2048_bf16", dtype="bf16", V=2000, d=2048, nh=16, H=520, c_prefill=40, n_new=ROWS),
    # float32 storage
    TINY.with_(name="tiny_f32", c_prefill=24, n_new=ROWS),
], ids=["mid_bf16", "w2048_bf16", "tiny_f32"])
def test_one_graph_serves_a_growing_context(cfg):
    print(f"[cycle] {cfg.name}", flush=True)
    total = cfg.c_prefill + CYCLES * ROWS
    w = synth.make_weights(cfg)
    feats = synth.make_features(cfg, rows=total)
    W = oracle.Weights.from_storage(w)
    # room for the cycles and half of one more: the fifth replay overflows
    C_max = total + ROWS // 2
    dr = make_drafter(cfg, w, C_max=C_max, max_new=ROWS)
    dr.set_schedule(cfg.times)
    dev = dr.device
    noise_buf = torch.empty(1, cfg.K, cfg.V, dtype=torch.bfloat16 if cfg.dtype == "bf16" else torch.float32,
                            device=dev)
    feat_buf = torch.empty(ROWS, 5, cfg.H, dtype=noise_buf.dtype, device=dev)
    T_buf = torch.empty(1, cfg.K + 1, cfg.V, dtype=noise_buf.dtype, device=dev)
    tok = torch.empty(1, cfg.K, dtype=torch.int32, device=dev)
    logits = torch.empty(1, cfg.K, cfg.V, dtype=torch.float32, device=dev)
    emitted = torch.empty(1, cfg.K + 1, dtype=torch.int32, device=dev)
    accept = torch.empty(1, dtype=torch.int32, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)

    def run(draw):
        dr.truncate(0)
        dr.append(to_dev(feats[:cfg.c_prefill]))
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            dr.draft(noise_buf, new_feats=feat_buf, logits=logits, tokens=tok)
            fm.fm_verify(T_buf, tok, emitted, accept, best)
        # the capture ran nothing: reload the host mirror from the device
        dr.sync_context()
        assert dr.context_length == cfg.c_prefill
        for k in range(CYCLES):
            C = cfg.c_prefill + (k + 1) * ROWS
            noise = synth.make_noise(cfg, 1, 1 + CYCLES * draw + k)
            ref = oracle.draft(W, cfg, noise[0], feats[:C])
            T = synth.plant(synth.make_target_logits(cfg)[0], ref["tokens"], ACCEPT)
            _copy(noise_buf, noise)
            _copy(feat_buf, feats[C - ROWS:C])
            _copy(T_buf, T[None])
            g.replay()
            torch.cuda.synchronize()
            lg, tk = logits.cpu().numpy()[0], tok.cpu().numpy()[0]
            rel = check_logits(lg, ref["logits"], cfg.dtype, f"cycle {k}:")
            cyc = check_tokens(tk, lg, ref["logits"], ref["tokens"], cfg.dtype)
            assert len(cyc) <= 1, f"cycle {k}: {len(cyc)} near-ties in one draft: {cyc}"
            # the verifier on the same replay: the oracle's outcome for the GPU's draft
            n, em = oracle.verify(T, tk)
            assert int(accept.cpu()[0]) == n and emitted.cpu().numpy()[0, :n + 1].tolist() == em
            if not cyc:
                assert n == ACCEPT
            dr.sync_context()
            assert dr.context_length == C
            print(f"  draw {draw} cycle {k}: context {C}, logit error {rel:.2e}, accepted {n}, "
                  f"near-ties {cyc}", flush=True)
        # one more replay passes the capacity: the length stops at C_max, the rows
        # past it are dropped, and the sync reports it
        g.replay()
        with pytest.raises(fm.FlashMapError) as e:
            dr.sync_context()
        assert e.value.status == fm.FM_ECAPACITY
        assert dr.context_length == C_max
        dr.sync_context()   # the flag was cleared

    run(0)
