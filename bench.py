#!/usr/bin/env python3
"""Benchmark one FlashMap drafting step + greedy verify on one MI355X.

A step is fm_draft (one flow-map jump from a 16 x V Gaussian noise block to a
16-token draft, with 8 new context rows fused in) followed by greedy
verification (fm_verify_greedy) against target logits [17][V].  Inputs are seeded synthetic tensors of the
Qwen3-8B-shaped drafter, resident in HBM before the timed region.  Steps are
replayed from HIP graphs (one per planted target-logit set) and timed with HIP
events; the dominant kernel is timed live with events recorded around its
launch (fm_set_probe).  The CPU oracle is timed on the host beside it.

    python bench.py [--gpus 1] [--steps 500] [--warmup 50] [--config qwen3_8b]

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
METRIC = "draft+verify steps/sec at K=16, batch 1 (Qwen3-8B-shaped); % of HBM peak"
KERNEL_SOURCES = {"lmhead_kernel": ["lmhead.hpp", "common.hpp", "philox.hpp", "stream.hpp"],
                  "lmhead_ks_kernel": ["lmhead.hpp", "common.hpp", "philox.hpp", "stream.hpp"],
                  "embed_kernel": ["embed.hpp", "common.hpp", "stream.hpp"]}


def lm_kernel_name(cfg) -> str:
    """The LM head kernel the library plans for this shape: k split over the
    8 waves when z fits in registers (row tiles x chunks per wave <= 4)."""
    ve = 8 if cfg.dtype == "bf16" else 4
    mt = -(-cfg.B * cfg.requests * cfg.K // 16)
    cpw = -(-(-(-cfg.d // (32 * ve))) // 8)
    return "lmhead_ks_kernel" if mt * cpw <= 4 else "lmhead_kernel"


def alg_bytes(cfg) -> dict:
    """Algorithmic bytes of one step: every weight read once, the context K/V
    read once, inputs and outputs once (adaLN vectors are precomputed)."""
    es = 2 if cfg.dtype == "bf16" else 4
    d, F, V, L, K = cfg.d, cfg.F, cfg.V, cfg.L, cfg.K
    B = cfg.B * cfg.requests   # row blocks: branches of one request or requests of a batch
    R = cfg.requests           # contexts
    n = cfg.num_steps
    Mb = B * K
    parts = {
        "E": n * V * d * es,
        "W_lm": n * V * d * es,
        "blocks": n * L * ((3 * d * d + d * d + F * d + d * F) + (3 * d + d + F + d)) * es,
        "fusion": (d * 5 * cfg.H + d) * es,
        "ctx_kv_read": n * L * R * cfg.C * 2 * d * es,
        "ctx_kv_write": L * R * cfg.n_new * 2 * d * es,
        "noise": Mb * V * es,
        "feats": R * cfg.n_new * 5 * cfg.H * es,
        "target_logits": B * (K + 1) * V * es,
        "mod_vectors": n * (6 * L + 2) * d * 4,
        "softmax_round_trip": (n - 1) * Mb * V * (4 + 4 + es + es),
    }
    if cfg.temperature > 0:   # sampled: the draft's float32 logits out, read back by verify
        parts["draft_logits_write"] = Mb * V * 4
        parts["draft_logits_read"] = Mb * V * 4
    parts["total"] = sum(parts.values())
    return parts


def kernel_alg_bytes(cfg, kernel: str) -> int:
    es = 2 if cfg.dtype == "bf16" else 4
    Mb = cfg.B * cfg.requests * cfg.K
    if kernel.startswith("lmhead"):    # W_lm, z in, tokens out (sampled: float32 logits out)
        return cfg.V * cfg.d * es + Mb * cfg.d * es + Mb * 4 + (Mb * cfg.V * 4 if cfg.temperature > 0 else 0)
    if kernel == "embed_kernel":       # E, x in, e and h out (float32)
        return cfg.V * cfg.d * es + Mb * cfg.V * es + 2 * Mb * cfg.d * 4
    raise KeyError(kernel)


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "step_flow_map_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("source_hash") != source_hash(kernel):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(cfg, w, noise, feats, T):
    """Time the oracle (one full draft + verify of the same workload)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    W = oracle.Weights.from_storage(w)
    steps = 0
    t0 = time.perf_counter()
    while True:   # whole steps until about 10 s of CPU work
        for r in range(1, cfg.requests):   # the other requests of a batch (own contexts)
            oracle.draft(W, cfg, noise[r], synth.make_features(cfg, request=r))
        ref = oracle.draft(W, cfg, noise[0], feats)
        if cfg.temperature > 0:
            d = oracle.sampling.sample_draft(ref["logits"], cfg.temperature, synth.SAMPLE_SEEDS[0])
            oracle.sampling.verify_sample(synth.values(T[0]), ref["logits"], d, cfg.temperature,
                                          synth.SAMPLE_SEEDS[0])
        else:
            oracle.verify(T[0], ref["tokens"])
        steps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or steps >= 1000:
            break
    del W
    return ref["tokens"], {
        "value": steps / dt, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
        "sample": f"{steps} full {cfg.name} draft+verify steps (the oracle recomputes the "
                  f"{cfg.C}-row context each step) in {dt:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", default="qwen3_8b", choices=sorted(synth.CONFIGS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time eager calls instead of graph replays")
    ap.add_argument("--cycle", action="store_true",
                    help="replay one graph of draft + verify without resetting the context, which then grows "
                         "by the appended rows every step (the speculative loop) from the workload's prefill; "
                         "the capacity covers every replay")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="only copy this many bytes device to device five times and exit (the plain copy "
                         "kernel that calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the drafting step runs on the GPU that holds the "
              "target (single-GPU build); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_bytes:
        src = torch.full((args.copy_bytes,), 1, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.copy_bytes, "launches": 5}))
        return
    import step_flow_map_amd as fm

    def to_dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()

    def binding_weights(w):
        return {k.replace("te_s.", "te_s_").replace("te_t.", "te_t_"): to_dev(v) for k, v in w.items()}

    cfg = synth.CONFIGS[args.config]
    t_gen = time.perf_counter()
    w = synth.make_weights(cfg)
    feats = synth.make_features(cfg)
    noise = synth.make_noise(cfg, cfg.B * cfg.requests)
    T_raw = synth.make_target_logits(cfg, cfg.B * cfg.requests)
    print(f"[bench] inputs generated in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)

    baseline = None
    ref_tokens = None
    if not args.no_cpu_baseline:
        ref_tokens, baseline = cpu_baseline(cfg, w, noise, feats, T_raw)
        print(f"[bench] oracle {baseline['sample']}", file=sys.stderr, flush=True)

    dev = torch.device("cuda", 0)
    R = cfg.requests
    NB = cfg.B * R   # row blocks
    n_replays = len(synth.PLANTED_ACCEPT) + args.warmup + args.steps + 1
    C_max = cfg.c_prefill + n_replays * cfg.n_new + cfg.n_new if args.cycle else cfg.capacity
    c = fm.make_config(K=cfg.K, V=cfg.V, d=cfg.d, L=cfg.L, n_heads=cfg.nh, H=cfg.H, C_max=C_max,
                       dtype=cfg.dtype, max_branches=cfg.B, max_new=max(R * cfg.n_new, 1),
                       max_steps=cfg.num_steps, max_requests=R)
    dr = fm.Drafter(c, binding_weights(w))
    dr.set_schedule(cfg.times)
    req_feats = [feats] + [synth.make_features(cfg, request=r) for r in range(1, R)]
    if cfg.c_prefill:
        for r in range(R):
            dr.append_req(r, to_dev(req_feats[r][:cfg.c_prefill]))
    x = to_dev(noise)
    new = to_dev(np.concatenate([f[cfg.c_prefill:] for f in req_feats])) if cfg.n_new else None
    tokens = torch.empty(NB, cfg.K, dtype=torch.int32, device=dev)
    emitted = torch.empty(NB, cfg.K + 1, dtype=torch.int32, device=dev)
    accept = torch.empty(NB, dtype=torch.int32, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()

    temp = cfg.temperature
    logits_q = lse_q = None
    if temp > 0:
        logits_q = torch.empty(cfg.B, cfg.K, cfg.V, dtype=torch.float32, device=dev)
        lse_q = torch.empty(cfg.B, cfg.K, dtype=torch.float32, device=dev)

    def draft_and_verify(T, seed):
        if R > 1:
            dr.draft_batch(x, new_feats=new, n_new=[cfg.n_new] * R, tokens=tokens)
            dr.verify(T, tokens, emitted, accept, best)
        elif temp > 0:
            fm.fm_draft_sample(dr.handle, x, temp, seed, tokens, logits_q, lse_q, new_feats=new)
            fm.fm_verify_sample(dr.handle, T, logits_q, lse_q, tokens, temp, seed, emitted, accept)
        else:
            dr.draft(x, new_feats=new, tokens=tokens)
            dr.verify(T, tokens, emitted, accept, best)

    sets = []   # (target logits, seed, planted accept lengths or None)
    if temp > 0:
        # sampled steps: the unplanted target logits, one seed per replayed step
        T_dev = to_dev(T_raw)
        sets = [(T_dev, s, None) for s in synth.SAMPLE_SEEDS]
    else:
        # draft once to learn the tokens when the oracle did not run
        for r in range(R):
            dr.truncate_req(r, cfg.c_prefill)
        draft_and_verify(to_dev(T_raw), 0)
        gpu_tokens = tokens.cpu().numpy()
        plant_from = ref_tokens[None] if ref_tokens is not None else gpu_tokens
        planted = synth.PLANTED_ACCEPT_TREE if cfg.B > 1 else synth.PLANTED_ACCEPT
        if R > 1:   # every request planted with the same accept length, one set per length
            plant_from = gpu_tokens
            if ref_tokens is not None:
                plant_from = np.concatenate([ref_tokens[None], gpu_tokens[1:]])
            for n in planted:
                src = np.stack([synth.plant(T_raw[r], plant_from[r], n) for r in range(R)])
                sets.append((to_dev(src), 0, [n] * R))
        elif cfg.B > 1:
            src = np.stack([synth.plant(T_raw[b], gpu_tokens[b], planted[b]) for b in range(cfg.B)])
            sets.append((to_dev(src), 0, list(planted)))
        else:
            for n in planted:
                sets.append((to_dev(synth.plant(T_raw[0], plant_from[0], n)[None]), 0, [n]))

    def step(T, seed):
        for r in range(R):
            dr.truncate_req(r, cfg.c_prefill)
        draft_and_verify(T, seed)

    stream = torch.cuda.current_stream()
    graphs = []
    if args.cycle:
        # one graph, no reset: every replay appends n_new rows to each context
        T, seed, _ = sets[0]
        step(T, seed)   # warm the path outside capture
        torch.cuda.synchronize()
        for r in range(R):
            dr.truncate_req(r, cfg.c_prefill)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            draft_and_verify(T, seed)
        dr.sync_context()
        graphs = [g] * len(sets)
    elif not args.eager:
        # a graph per target set; each replay first resets the device-resident
        # context length (a captured write), so every step appends the same rows
        # and attends over the same context
        for T, seed, _ in sets:
            step(T, seed)   # warm the path outside capture
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(T, seed)
            graphs.append(g)
        torch.cuda.synchronize()

    def run(i):
        if graphs:
            graphs[i % len(graphs)].replay()
        else:
            step(*sets[i % len(sets)][:2])

    # accept lengths of every planted set (checks the planted workload)
    accepts = []
    for i in range(len(sets)):
        run(i)
        torch.cuda.synchronize()
        accepts.append(accept.cpu().numpy().tolist())

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        run(i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    ctx_range = None
    if args.cycle:
        dr.sync_context()
        ctx_end = dr.context_length_req(0)
        ctx_range = [ctx_end - (args.steps - 1) * cfg.n_new, ctx_end]   # rows seen by the first and last timed step
        for r in range(R):
            dr.truncate_req(r, cfg.c_prefill)

    # Spread of single-step times: an event between consecutive replays on the
    # replay stream (the timed loop above stays one bracket of K steps).
    n_dist = min(args.steps, 200)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n_dist + 1)]
    evs[0].record(stream)
    for i in range(n_dist):
        run(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_us = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(n_dist)])
    step_us = {"median": float(np.median(per_us)), "p10": float(np.percentile(per_us, 10)),
               "p90": float(np.percentile(per_us, 90)), "steps": n_dist}
    if args.cycle:
        for r in range(R):
            dr.truncate_req(r, cfg.c_prefill)

    # The loop as a host would drive it: after every step the accept lengths
    # come back to pinned host memory and the host waits for them (wall clock).
    acc_host = torch.empty(accept.shape, dtype=accept.dtype, pin_memory=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(n_dist):
        run(i)
        acc_host.copy_(accept, non_blocking=True)
        stream.synchronize()
    ms_sync = (time.perf_counter() - t0) * 1e3 / n_dist
    host_sync = {"ms_per_step": ms_sync, "steps_per_s": 1000.0 / ms_sync, "steps": n_dist}
    if args.cycle:
        for r in range(R):
            dr.truncate_req(r, cfg.c_prefill)

    # practical streaming ceiling: a plain 1 GiB device-to-device copy (bytes
    # read + bytes written per copy)
    cp_src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cp_dst = torch.empty_like(cp_src)
    cp_dst.copy_(cp_src)
    c0 = torch.cuda.Event(enable_timing=True)
    c1 = torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(5):
        cp_dst.copy_(cp_src)
    c1.record(stream)
    torch.cuda.synchronize()
    cp_gbs = 5 * 2 * (1 << 30) / (c0.elapsed_time(c1) * 1e-3) / 1e9
    copy_ceiling = {"bytes_per_copy": 2 * (1 << 30), "gbs": cp_gbs, "frac_of_peak": cp_gbs / HBM_PEAK_GBS}
    del cp_src, cp_dst

    # live per-kernel durations: events around the kernel's launch, eager calls
    kernels = {}
    for name, probe in ((lm_kernel_name(cfg), fm.FM_PROBE_LM_HEAD), ("embed_kernel", fm.FM_PROBE_EMBED)):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)   # torch creates the HIP events on first record
        b.record(stream)
        torch.cuda.synchronize()
        fm.fm_set_probe(dr.handle, probe, a, b)
        durs = []
        for i in range(20):
            step(*sets[i % len(sets)][:2])
            torch.cuda.synchronize()
            durs.append(a.elapsed_time(b))
        fm.fm_set_probe(dr.handle, fm.FM_PROBE_NONE)
        us = float(np.mean(durs[5:])) * 1e3
        ab = kernel_alg_bytes(cfg, name)
        kernels[name] = {"us": us, "alg_bytes": ab, "gbs": ab / us / 1e3}
    # several jumps: the same step with the one-jump schedule, same context and
    # inputs, so the cost of each further jump is the difference
    one_jump = None
    if cfg.num_steps > 1 and not args.cycle and not args.eager:
        dr.set_schedule((0.0, 1.0))
        g1 = []
        for T, seed, _ in sets:
            step(T, seed)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(T, seed)
            g1.append(g)
        for i in range(args.warmup):
            g1[i % len(g1)].replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            g1[i % len(g1)].replay()
        e1.record(stream)
        torch.cuda.synchronize()
        ms1 = e0.elapsed_time(e1) / args.steps
        one_jump = {"ms_per_step": ms1, "ms_per_further_jump": (ms - ms1) / (cfg.num_steps - 1),
                    "ratio": ms / ms1}
        dr.set_schedule(cfg.times)
    dom = max(kernels, key=lambda k: kernels[k]["us"])
    kd = kernels[dom]
    traffic = measured_traffic(dom, cfg.name)
    ab = alg_bytes(cfg)
    out = {
        "metric": METRIC,
        "value": 1000.0 / ms,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded random weights ~N(0,0.02), features/noise/target logits ~N(0,1); " + (
                f"sampled at temperature {cfg.temperature} with seeds {list(synth.SAMPLE_SEEDS)}, target "
                "logits not planted)" if cfg.temperature > 0 else
                "target logits planted for accept lengths 7,7,7,7,7,7,7,6,6,6)"),
        "config": {"workload": cfg.name, "K": cfg.K, "V": cfg.V, "d": cfg.d, "L": cfg.L,
                   "heads": cfg.nh, "H": cfg.H, "context": cfg.C, "new_rows_per_step": cfg.n_new,
                   "branches": cfg.B, "requests": R, "schedule": list(cfg.times),
                   "temperature": cfg.temperature,
                   "replay": "eager" if args.eager else "hipgraph"}
                  | ({"context_grows": True, "context_timed": ctx_range} if args.cycle else {}),
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": kd["gbs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": kd["gbs"] / HBM_PEAK_GBS, "traffic": traffic,
                     "alg_bytes_per_launch": kd["alg_bytes"], "us_per_launch": kd["us"]},
        "step_roofline": {"alg_bytes": ab["total"], "achieved_gbs": ab["total"] / ms / 1e6,
                          "frac": ab["total"] / ms / 1e6 / HBM_PEAK_GBS},
        "step_us": step_us,
        "host_sync": host_sync,
        "copy_ceiling": copy_ceiling,
        "kernels": kernels,
        "accept": accepts,
        "tau": float(np.mean([np.mean(a) for a in accepts]) + 1.0),
        "cpu_baseline": baseline,
    }
    if one_jump is not None:
        out["one_jump_same_context"] = one_jump
    print(json.dumps(out))


if __name__ == "__main__":
    main()
