"""CPU oracle for one FlashMap drafting step and its greedy verifier.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call this module; the HIP library never does, and
it shares no code with it (the only common import is the seeded input module
``synth``, which holds no arithmetic of the method).

Sources.  The method is described on five news pages about FlashMap:
  [zh]  "FlashMap并行草拟加速大模型解码" (feinterview.poetries.top)
  [ru]  "Polymathic AI и исследователи из Princeton выпустили FlashMap ..."
        (wire.sakhanda.co)
  [fa]  eskul.ir, "flashmap-16-token-drafter-6x-faster-qwen3"
  [it]  the-ai.news, "polymathic-ai-princeton-flashmap-acceleratore-decoding-llm"
  [en]  "FlashMap Drafts 16 Dependent Tokens at Once, Hitting 6.1x Faster
        Decoding" (alphasignal.ai)
They fix: K=16 drafted tokens verified in one target pass, longest matching
prefix kept, decoding resumes from a target token ([zh] first section, [ru]
"Что такое FlashMap?", [en] "Why drafting still costs time"); Gaussian noise
mapped to the whole block in one jump ([zh] first section, [ru] "Почему
diffusion-драфтеры..."); a 6-block DiT of width 2048 with 16 heads reading
target layers 1, 9, 17, 25, 33, with frozen embedding and LM head copied from the
target ([zh] second section, [ru] "Как работает FlashMap?"); a flow teacher over
one-hot token blocks trained with cross-entropy and distilled into a two-time
flow map that goes from noise to data in one step (same sections).

Everything else (interpolant, time embedding, adaLN layout, attention wiring,
norms, positions, tie-breaks) is not on the pages.  Each such choice below is
marked READING and takes the plainest form the rest supports: a DiT with adaLN
time modulation, non-causal attention of the block over [context; block] keys,
LayerNorm without affine, tanh-GELU MLP of width 4d, the linear interpolant
x_tau = (1 - tau) x_0 + tau * onehot, and lowest-index argmax.

Precision.  Everything is computed in float64.  For bf16 workloads the values the
GPU path stores in bfloat16 are rounded here at the same points:
  R0 weights, noise, context features and target logits are bf16 inputs;
  R1 every activation operand of a contraction is rounded to bf16 just before
     use (u, a, attention output O, m, GELU output, z, and D in the 2-step map);
  R2 Q, K, V (block and context rows) are rounded to bf16 after the bias add;
  the residual stream h, LN statistics, modulation vectors, the time embedding,
  attention scores/probabilities and logits are not rounded (float64 here).
Draft tokens are the argmax of the logits rounded to float32 (the precision the
GPU decides them in).  The f32 workload has no bf16 rounding points.
"""
from __future__ import annotations

import math

import numpy as np

EPS = 1e-6


# --------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------

def round_f32(x):
    """float64 -> nearest float32 value (returned as float64)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(x):
    """float64 -> nearest bfloat16 value via the float32 the GPU holds:
    float32 bits + 0x7FFF + lsb(bit 16), low 16 bits cleared (ties to even)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def from_storage(a):
    """Input array (uint16 bfloat16 bits or float32) -> float64 values."""
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


class Precision:
    """Rounding points of a workload: 'bf16' emulates R1/R2, 'f32' is identity."""

    def __init__(self, dtype: str):
        self.bf16 = dtype == "bf16"

    def act(self, x):
        return round_bf16(x) if self.bf16 else np.asarray(x, dtype=np.float64)


# --------------------------------------------------------------------------
# scalar / row functions (READINGS: the pages name none of them)
# --------------------------------------------------------------------------

def layer_norm(x, eps=EPS):
    """Per-row LayerNorm without affine: (x - mean) / sqrt(biased var + eps)."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps)


def modulate(x, shift, scale):
    """adaLN modulation x * (1 + scale) + shift."""
    return x * (1.0 + scale) + shift


def gelu_tanh(x):
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def silu(x):
    return x / (1.0 + np.exp(-x))


def softmax_rows(x):
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return e / e.sum(axis=-1, keepdims=True)


def argmax_lowest(rows):
    """Index of the maximum of each row; among equal maxima the lowest index
    (IEEE equality, so -0 and +0 tie).  NaN inputs are out of scope."""
    rows = np.atleast_2d(np.asarray(rows))
    out = np.empty(rows.shape[0], dtype=np.int64)
    for r in range(rows.shape[0]):
        m = rows[r].max()
        out[r] = int(np.flatnonzero(rows[r] == m)[0])
    return out


# --------------------------------------------------------------------------
# time conditioning: the two times of the flow map ([ru] "Как работает
# FlashMap?": the student is a denoiser with two time points)
# --------------------------------------------------------------------------

def timestep_features(tau, dim=256):
    """READING: sinusoidal features [cos(tau w_i), sin(tau w_i)], i < dim/2,
    w_i = exp(-ln(1e4) i / (dim/2)); tau in [0, 1] is used as is."""
    half = dim // 2
    w = np.exp(-math.log(10000.0) * np.arange(half, dtype=np.float64) / half)
    a = float(tau) * w
    return np.concatenate([np.cos(a), np.sin(a)])


def time_embed(W, prefix, tau):
    """READING: TE(tau) = W2 silu(W1 feat(tau) + b1) + b2, all float64."""
    W1, b1 = W[prefix + ".W1"], W[prefix + ".b1"]
    W2, b2 = W[prefix + ".W2"], W[prefix + ".b2"]
    hid = silu(W1 @ timestep_features(tau, W1.shape[1]) + b1)
    return W2 @ hid + b2


def modulation(W, L, d, s, t):
    """adaLN vectors of the jump s -> t.

    READING: c = TE_s(s) + TE_t(t); per block l
    [shift1, scale1, gate1, shift2, scale2, gate2] = W_ada^l silu(c) + b_ada^l,
    final layer [shift_f, scale_f] = W_fa silu(c) + b_fa.  Depends on (s, t)
    and the weights only, never on the noise or the context."""
    c = time_embed(W, "te_s", s) + time_embed(W, "te_t", t)
    sc = silu(c)
    blocks = []
    for l in range(L):
        v = W[f"blk{l}.W_ada"] @ sc + W[f"blk{l}.b_ada"]
        blocks.append(tuple(v[i * d:(i + 1) * d] for i in range(6)))
    f = W["W_fa"] @ sc + W["b_fa"]
    return {"blocks": blocks, "final": (f[:d], f[d:])}


def positions(K, d):
    """READING: fixed sinusoidal table P[k] = [sin(k w'_i), cos(k w'_i)],
    i < d/2, w'_i = 10000^(-i/(d/2)); added to the block rows only."""
    half = d // 2
    w = 10000.0 ** (-np.arange(half, dtype=np.float64) / half)
    a = np.arange(K, dtype=np.float64)[:, None] * w[None, :]
    return np.concatenate([np.sin(a), np.cos(a)], axis=1)


# --------------------------------------------------------------------------
# context: hidden states of target layers 1, 9, 17, 25, 33 ([zh] second
# section; [ru] "Как работает FlashMap?"; [en] the flow map is conditioned on
# target hidden states)
# --------------------------------------------------------------------------

def fuse_context(W, feats, prec):
    """u_p = LN(W_f concat_l F[p, l] + b_f), rounded to bf16 (R1).

    feats: [C][5][H] values in layer order 1, 9, 17, 25, 33."""
    C = feats.shape[0]
    f = feats.reshape(C, feats.shape[1] * feats.shape[2])  # C may be 0
    return prec.act(layer_norm(f @ W["W_f"].T + W["b_f"]))


def attention(q, k, v, nh):
    """Multi-head attention, no mask (every query sees every key).

    q [M][d], k/v [N][d]; head j uses columns j*hd:(j+1)*hd; scale 1/sqrt(hd)."""
    M, d = q.shape
    hd = d // nh
    out = np.empty((M, d), dtype=np.float64)
    for j in range(nh):
        sl = slice(j * hd, (j + 1) * hd)
        s = (q[:, sl] @ k[:, sl].T) / math.sqrt(hd)
        out[:, sl] = softmax_rows(s) @ v[:, sl]
    return out


def dit_block(W, l, h, u, mods, nh, prec, trace=None):
    """One DiT block on the block rows h [K][d] with context rows u [C][d].

    READING (the pages give only the block count, width and heads):
      a = mod(LN(h), shift1, scale1)                       -> bf16 (R1)
      Q, Kb, Vb = a W_qkv^T + b_qkv                        -> bf16 (R2)
      Kc, Vc from u with the same W_k, W_v (context rows)  -> bf16 (R2)
      O = attention(Q, [Kc; Kb], [Vc; Vb])                 -> bf16 (R1)
      h = h + gate1 * (O W_o^T + b_o)
      m = mod(LN(h), shift2, scale2)                       -> bf16 (R1)
      g = GELU(m W_1^T + b_1)                              -> bf16 (R1)
      h = h + gate2 * (g W_2^T + b_2)
    The context rows are not updated by the blocks, so their K/V depend only on
    the context and the block weights."""
    sh1, sc1, g1, sh2, sc2, g2 = mods
    d = h.shape[1]
    Wqkv, bqkv = W[f"blk{l}.W_qkv"], W[f"blk{l}.b_qkv"]
    a = prec.act(modulate(layer_norm(h), sh1, sc1))
    qkv = prec.act(a @ Wqkv.T + bqkv)
    q, kb, vb = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
    kc = prec.act(u @ Wqkv[d:2 * d].T + bqkv[d:2 * d])
    vc = prec.act(u @ Wqkv[2 * d:].T + bqkv[2 * d:])
    o = prec.act(attention(q, np.concatenate([kc, kb]), np.concatenate([vc, vb]), nh))
    h = h + g1 * (o @ W[f"blk{l}.W_o"].T + W[f"blk{l}.b_o"])
    m = prec.act(modulate(layer_norm(h), sh2, sc2))
    g = prec.act(gelu_tanh(m @ W[f"blk{l}.W_1"].T + W[f"blk{l}.b_1"]))
    h = h + g2 * (g @ W[f"blk{l}.W_2"].T + W[f"blk{l}.b_2"])
    if trace is not None:
        trace.append({"a": a, "q": q, "kb": kb, "vb": vb, "kc": kc, "vc": vc,
                      "o": o, "m": m, "g": g, "h": h})
    return h


def head_logits(W, h, mods_final, prec):
    """z = mod(LN(h), shift_f, scale_f) -> bf16 (R1); logits = z W_lm^T (no bias)."""
    z = prec.act(modulate(layer_norm(h), *mods_final))
    return z @ W["W_lm"].T


# --------------------------------------------------------------------------
# the flow map (READING: linear interpolant, noise at tau=0, data at tau=1)
# --------------------------------------------------------------------------

def flow_map(x_s, D, s, t):
    """X_{s,t}(x_s) = ((1-t)/(1-s)) x_s + ((t-s)/(1-s)) D, where D is the
    two-time denoiser's clean-block estimate (softmax of the logits, the
    expectation of the one-hot block under the cross-entropy-trained model).
    X_{s,s} is the identity and X_{s,1} = D: one jump from noise to data."""
    if s == 1.0:
        raise ValueError("flow map starts before data time 1")
    return ((1.0 - t) / (1.0 - s)) * x_s + ((t - s) / (1.0 - s)) * D


class Weights(dict):
    """Name -> float64 array, converted once from storage arrays."""

    @classmethod
    def from_storage(cls, w):
        return cls({k: from_storage(v) for k, v in w.items()})


def draft(W, cfg, noise, feats, times=None, use_pos=True, trace=False):
    """One FlashMap drafting step for one noise branch.

    W      Weights (float64 values)
    cfg    synth.Config-like object (K, V, d, L, nh, dtype)
    noise  [K][V] noise block (storage array or values)
    feats  [C][5][H] target hidden states of every context row (no cache)
    times  schedule 0 = s_0 < ... < s_n = 1 (default: cfg.times)

    Each jump s -> t: h = x_s E + P, the L blocks with the (s, t) modulation,
    final LN/mod, logits = z W_lm^T.  At t = 1 the draft is the row argmax of
    the float32 logits (softmax is monotone, so D is never needed).  Before
    t = 1 the state moves by the flow map; it is carried in embedding space:
    e_t = ((1-t)/(1-s)) e_s + ((t-s)/(1-s)) bf16(D) E (linear in x, so equal to
    X_{s,t}(x_s) E up to the rounding of D).  Returns a dict with 'tokens' [K],
    'logits' (float32 values, last jump) and, per jump, h0, h, logits, the
    modulation vectors and (trace=True) every block's intermediates.
    use_pos=False drops the positional table (for permutation tests)."""
    prec = Precision(cfg.dtype)
    times = tuple(cfg.times if times is None else times)
    if times[0] != 0.0 or times[-1] != 1.0 or any(b <= a for a, b in zip(times, times[1:])):
        raise ValueError("schedule must rise strictly from 0 to 1")
    x = from_storage(noise)
    E = W["E"]
    e = x @ E
    P = positions(cfg.K, cfg.d) if use_pos else 0.0
    u = fuse_context(W, from_storage(feats), prec)
    out = {"jumps": []}
    for s, t in zip(times, times[1:]):
        mods = modulation(W, cfg.L, cfg.d, s, t)
        h = e + P
        jt = {"h0": h, "blocks": [] if trace else None}
        for l in range(cfg.L):
            h = dit_block(W, l, h, u, mods["blocks"][l], cfg.nh, prec, jt["blocks"])
        logits = round_f32(head_logits(W, h, mods["final"], prec))
        jt.update(h=h, logits=logits, mods=mods)
        out["jumps"].append(jt)
        if t == 1.0:
            out["tokens"] = argmax_lowest(logits)
            out["logits"] = logits
        else:
            D = softmax_rows(logits)
            e = ((1.0 - t) / (1.0 - s)) * e + ((t - s) / (1.0 - s)) * (prec.act(D) @ E)
    out["u"] = u
    return out


def draft_tree(W, cfg, noises, feats, times=None, use_pos=True):
    """Independent branches sharing one context (READING: branch b attends to
    the context and its own K rows only).  noises [B][K][V]."""
    return [draft(W, cfg, noises[b], feats, times, use_pos) for b in range(len(noises))]


# --------------------------------------------------------------------------
# greedy verifier ([zh] first section; [ru] "Что такое FlashMap?"; [en] "Why
# drafting still costs time": keep the longest prefix of the draft that the
# target agrees with, then continue from the target's own token)
# --------------------------------------------------------------------------

def verify(T, draft_tokens):
    """Greedy verification of one branch.

    T [K+1][V]: target logits; row j is the target's prediction for draft slot j
    given the prefix and draft[0..j-1]; row K predicts the token after a fully
    accepted block.  y_j = argmax_lowest(T[j]).
    Returns (n, emitted): n = the largest m <= K with draft[i] == y_i for all
    i < m; emitted = draft[0..n-1] followed by y_n (n + 1 tokens)."""
    y = argmax_lowest(from_storage(T))
    K = len(draft_tokens)
    n = 0
    while n < K and int(draft_tokens[n]) == int(y[n]):
        n += 1
    emitted = [int(v) for v in draft_tokens[:n]] + [int(y[n])]
    return n, emitted


def verify_tree(Ts, drafts):
    """Verify each branch; best = the lowest branch index among the longest."""
    res = [verify(Ts[b], drafts[b]) for b in range(len(drafts))]
    ns = [n for n, _ in res]
    best = ns.index(max(ns))
    return res, best


# --------------------------------------------------------------------------
# architecture size, for comparison with the parameter counts on the pages
# --------------------------------------------------------------------------

def trainable_params(cfg):
    """Parameters outside the frozen embedding and LM head."""
    d, F, H = cfg.d, cfg.F, cfg.H
    blocks = cfg.L * (6 * d * d + 6 * d + 3 * d * d + 3 * d + d * d + d
                      + F * d + F + d * F + d)
    fusion = d * 5 * H + d
    te = 2 * (d * 256 + d + d * d + d)
    final = 2 * d * d + 2 * d
    return blocks + fusion + te + final
