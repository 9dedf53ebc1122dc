"""ctypes binding of libflashmap.so (declarations in include/flashmap.h).

Argument marshalling only: every function below forwards torch tensors' device
pointers and the current HIP stream to the C entry point of the same name and
raises FlashMapError on a non-zero status.  All compute runs in the library's
HIP kernels; there is no fallback, and loading fails loudly when the library
has not been built (python -m step_flow_map_amd.build).
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflashmap.so")

FM_OK, FM_EINVAL, FM_ECAPACITY, FM_EHIP, FM_ESTATE = range(5)
FM_BF16, FM_F32 = 0, 1
FM_PROBE_NONE, FM_PROBE_EMBED, FM_PROBE_LM_HEAD, FM_PROBE_FC1, FM_PROBE_VERIFY = range(5)
STATUS_NAMES = {0: "FM_OK", 1: "FM_EINVAL", 2: "FM_ECAPACITY", 3: "FM_EHIP", 4: "FM_ESTATE"}

BLOCK_FIELDS = ("W_ada", "b_ada", "W_qkv", "b_qkv", "W_o", "b_o", "W_1", "b_1", "W_2", "b_2")
TOP_FIELDS = ("E", "W_lm", "W_f", "b_f", "te_s_W1", "te_s_b1", "te_s_W2", "te_s_b2",
              "te_t_W1", "te_t_b1", "te_t_W2", "te_t_b2", "W_fa", "b_fa")


class fm_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in
                ("K", "V", "d", "L", "n_heads", "mlp_mult", "H", "n_ctx_layers", "C_max",
                 "max_branches", "max_new", "max_steps", "dtype", "max_requests")]


class fm_block_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in BLOCK_FIELDS]


class fm_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in TOP_FIELDS] + [
        ("blocks", ctypes.POINTER(fm_block_weights))]


class FlashMapError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libflashmap.so once; raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m step_flow_map_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i, st = ctypes.c_void_p, ctypes.c_int, ctypes.c_int
    L.fm_workspace_bytes.argtypes = [ctypes.POINTER(fm_config)]
    L.fm_workspace_bytes.restype = ctypes.c_size_t
    L.fm_create.argtypes = [ctypes.POINTER(fm_config), vp, ctypes.c_size_t, i, ctypes.POINTER(vp)]
    L.fm_create.restype = st
    L.fm_destroy.argtypes = [vp]
    L.fm_destroy.restype = None
    L.fm_set_weights.argtypes = [vp, ctypes.POINTER(fm_weights)]
    L.fm_set_weights.restype = st
    L.fm_set_schedule.argtypes = [vp, ctypes.POINTER(ctypes.c_float), i, vp]
    L.fm_set_schedule.restype = st
    L.fm_context_append.argtypes = [vp, vp, i, vp]
    L.fm_context_append.restype = st
    L.fm_context_truncate.argtypes = [vp, i, vp]
    L.fm_context_truncate.restype = st
    L.fm_context_sync.argtypes = [vp, vp]
    L.fm_context_sync.restype = st
    L.fm_context_length.argtypes = [vp]
    L.fm_context_length.restype = i
    L.fm_context_append_req.argtypes = [vp, i, vp, i, vp]
    L.fm_context_append_req.restype = st
    L.fm_context_truncate_req.argtypes = [vp, i, i, vp]
    L.fm_context_truncate_req.restype = st
    L.fm_context_length_req.argtypes = [vp, i]
    L.fm_context_length_req.restype = i
    L.fm_draft_batch.argtypes = [vp, vp, i, vp, ctypes.POINTER(ctypes.c_int), vp, vp, vp]
    L.fm_draft_batch.restype = st
    L.fm_draft.argtypes = [vp, vp, i, vp, i, vp, vp, vp, vp]
    L.fm_draft.restype = st
    L.fm_verify.argtypes = [vp, i, i, i, i, vp, vp, vp, vp, vp]
    L.fm_verify.restype = st
    L.fm_verify_greedy.argtypes = [vp, vp, i, i, vp, vp, vp, vp, vp]
    L.fm_verify_greedy.restype = st
    f32, u64 = ctypes.c_float, ctypes.c_uint64
    L.fm_draft_sample.argtypes = [vp, vp, i, vp, i, f32, u64, vp, vp, vp, vp]
    L.fm_draft_sample.restype = st
    L.fm_verify_sample.argtypes = [vp, vp, i, i, vp, vp, vp, f32, u64, vp, vp, vp]
    L.fm_verify_sample.restype = st
    u64p = ctypes.POINTER(ctypes.c_uint64)
    L.fm_draft_batch_sample.argtypes = [vp, vp, i, vp, ctypes.POINTER(ctypes.c_int), f32, u64p, vp, vp, vp, vp]
    L.fm_draft_batch_sample.restype = st
    L.fm_verify_sample_batch.argtypes = [vp, vp, i, i, vp, vp, vp, f32, u64p, vp, vp, vp]
    L.fm_verify_sample_batch.restype = st
    L.fm_verify_sample_noalloc.argtypes = [vp, i, i, i, i, vp, vp, vp, f32, u64, vp, vp, vp]
    L.fm_verify_sample_noalloc.restype = st
    L.fm_set_probe.argtypes = [vp, i, vp, vp]
    L.fm_set_probe.restype = st
    L.fm_last_error.argtypes = []
    L.fm_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def fm_last_error() -> str:
    return lib().fm_last_error().decode()


def _check(status: int):
    if status != FM_OK:
        raise FlashMapError(status, fm_last_error())


def _ptr(t) -> ctypes.c_void_p:
    if t is None:
        return ctypes.c_void_p(None)
    if isinstance(t, int):
        return ctypes.c_void_p(t)
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return FM_BF16
    if t == torch.float32:
        return FM_F32
    raise ValueError(f"unsupported storage dtype {t}")


def make_config(*, K=16, V, d, L, n_heads, H, C_max, dtype="bf16", mlp_mult=4, n_ctx_layers=5,
                max_branches=1, max_new=16, max_steps=2, max_requests=1) -> fm_config:
    return fm_config(K=K, V=V, d=d, L=L, n_heads=n_heads, mlp_mult=mlp_mult, H=H,
                     n_ctx_layers=n_ctx_layers, C_max=C_max, max_branches=max_branches,
                     max_new=max_new, max_steps=max_steps,
                     dtype=FM_BF16 if dtype in ("bf16", FM_BF16) else FM_F32, max_requests=max_requests)


# ----------------------------------------------------------------- C entry points

def fm_workspace_bytes(cfg: fm_config) -> int:
    return int(lib().fm_workspace_bytes(ctypes.byref(cfg)))


def fm_create(cfg: fm_config, workspace, ws_bytes: int | None = None, device: int = 0) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    n = workspace.numel() * workspace.element_size() if ws_bytes is None else ws_bytes
    _check(lib().fm_create(ctypes.byref(cfg), _ptr(workspace), n, device, ctypes.byref(h)))
    return h


def fm_destroy(h) -> None:
    lib().fm_destroy(h)


def fm_set_weights(h, weights: dict, L: int):
    """weights: name -> device tensor, names as in fm_weights ('E', 'W_lm',
    'te_s_W1', ..., 'blk{l}.W_qkv', ...).  The tensors must outlive the handle."""
    blocks = (fm_block_weights * L)()
    for l in range(L):
        for f in BLOCK_FIELDS:
            setattr(blocks[l], f, _ptr(weights[f"blk{l}.{f}"]).value)
    w = fm_weights()
    for f in TOP_FIELDS:
        setattr(w, f, _ptr(weights[f]).value)
    w.blocks = blocks
    _check(lib().fm_set_weights(h, ctypes.byref(w)))


def fm_set_schedule(h, times, stream=None):
    arr = (ctypes.c_float * len(times))(*[float(t) for t in times])
    _check(lib().fm_set_schedule(h, arr, len(times) - 1, _stream(stream)))


def fm_context_append(h, feats, stream=None):
    n = 0 if feats is None else int(feats.shape[0])
    _check(lib().fm_context_append(h, _ptr(feats), n, _stream(stream)))


def fm_context_truncate(h, new_len: int, stream=None):
    _check(lib().fm_context_truncate(h, int(new_len), _stream(stream)))


def fm_context_sync(h, stream=None):
    _check(lib().fm_context_sync(h, _stream(stream)))


def fm_context_length(h) -> int:
    return int(lib().fm_context_length(h))


def fm_context_append_req(h, req: int, feats, stream=None):
    n = 0 if feats is None else int(feats.shape[0])
    _check(lib().fm_context_append_req(h, int(req), _ptr(feats), n, _stream(stream)))


def fm_context_truncate_req(h, req: int, new_len: int, stream=None):
    _check(lib().fm_context_truncate_req(h, int(req), int(new_len), _stream(stream)))


def fm_context_length_req(h, req: int) -> int:
    return int(lib().fm_context_length_req(h, int(req)))


def fm_draft_batch(h, noise, tokens, new_feats=None, n_new=None, logits=None, stream=None):
    """noise [R][K][V]; tokens [R][K] int32 out; new_feats [sum n_new][5][H] or
    None; n_new: R counts (host) or None; logits [R][K][V] float32 or None."""
    R = int(noise.shape[0])
    counts = None
    if n_new is not None:
        counts = (ctypes.c_int * R)(*[int(x) for x in n_new])
    _check(lib().fm_draft_batch(h, _ptr(noise), R, _ptr(new_feats), counts, _ptr(tokens), _ptr(logits),
                                _stream(stream)))


def fm_draft(h, noise, tokens, new_feats=None, logits=None, hidden=None, stream=None):
    """noise [B][K][V]; tokens [B][K] int32 out; new_feats [n_new][5][H] or None;
    logits [B][K][V] float32 out or None; hidden [steps][L+1][B][K][d] or None."""
    n_new = 0 if new_feats is None else int(new_feats.shape[0])
    _check(lib().fm_draft(h, _ptr(noise), int(noise.shape[0]), _ptr(new_feats), n_new,
                          _ptr(tokens), _ptr(logits), _ptr(hidden), _stream(stream)))


def fm_draft_sample(h, noise, temperature, seed, tokens, logits, lse, new_feats=None, stream=None):
    """Temperature > 0 draft: tokens [B][K] int32, logits [B][K][V] float32
    and lse [B][K] float32 outputs."""
    n_new = 0 if new_feats is None else int(new_feats.shape[0])
    _check(lib().fm_draft_sample(h, _ptr(noise), int(noise.shape[0]), _ptr(new_feats), n_new,
                                 float(temperature), int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(tokens),
                                 _ptr(logits), _ptr(lse), _stream(stream)))


def fm_verify_sample(h, target_logits, draft_logits, draft_lse, draft, temperature, seed, emitted, accept,
                     stream=None):
    """Probabilistic verify: target_logits [B][K+1][V] (bf16 or float32),
    draft_logits [B][K][V] and draft_lse [B][K] float32, draft [B][K] int32;
    outputs emitted [B][K+1] and accept [B] int32."""
    B = int(target_logits.shape[0])
    _check(lib().fm_verify_sample(h, _ptr(target_logits), dtype_code(target_logits.dtype), B,
                                  _ptr(draft_logits), _ptr(draft_lse), _ptr(draft), float(temperature),
                                  int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(emitted), _ptr(accept),
                                  _stream(stream)))


def _seeds(seeds):
    arr = (ctypes.c_uint64 * len(seeds))(*[int(x) & 0xFFFFFFFFFFFFFFFF for x in seeds])
    return arr


def fm_draft_batch_sample(h, noise, temperature, seeds, tokens, logits, lse, new_feats=None, n_new=None,
                          stream=None):
    """Temperature > 0 batch draft: request r samples with seeds[r]; tokens
    [R][K] int32, logits [R][K][V] and lse [R][K] float32 outputs."""
    R = int(noise.shape[0])
    if len(seeds) != R:
        raise ValueError("one seed per request")
    nn = (ctypes.c_int * R)(*([0] * R if n_new is None else [int(x) for x in n_new]))
    _check(lib().fm_draft_batch_sample(h, _ptr(noise), R, _ptr(new_feats), nn, float(temperature), _seeds(seeds),
                                       _ptr(tokens), _ptr(logits), _ptr(lse), _stream(stream)))


def fm_verify_sample_batch(h, target_logits, draft_logits, draft_lse, draft, temperature, seeds, emitted, accept,
                           stream=None):
    """Probabilistic verify of the requests of a batch, request r with
    seeds[r]: shapes as for fm_verify_sample with B = R."""
    R = int(target_logits.shape[0])
    if len(seeds) != R:
        raise ValueError("one seed per request")
    _check(lib().fm_verify_sample_batch(h, _ptr(target_logits), dtype_code(target_logits.dtype), R,
                                        _ptr(draft_logits), _ptr(draft_lse), _ptr(draft), float(temperature),
                                        _seeds(seeds), _ptr(emitted), _ptr(accept), _stream(stream)))


def fm_verify_sample_noalloc(target_logits, draft_logits, draft_lse, draft, temperature, seed, emitted, accept,
                             stream=None):
    """fm_verify_sample with the library's static scratch (no handle):
    target_logits [B][K+1][V], draft_logits [B][K][V], draft_lse [B][K],
    draft [B][K]; outputs emitted [B][K+1] and accept [B] int32."""
    B, K1, V = (int(s) for s in target_logits.shape)
    _check(lib().fm_verify_sample_noalloc(_ptr(target_logits), dtype_code(target_logits.dtype), B, K1 - 1, V,
                                          _ptr(draft_logits), _ptr(draft_lse), _ptr(draft), float(temperature),
                                          int(seed) & 0xFFFFFFFFFFFFFFFF, _ptr(emitted), _ptr(accept),
                                          _stream(stream)))


def fm_verify(target_logits, draft, emitted, accept, best, stream=None):
    """target_logits [B][K+1][V] (bf16 or float32); draft [B][K] int32; outputs
    emitted [B][K+1], accept [B], best [1] int32."""
    B, K1, V = (int(s) for s in target_logits.shape)
    _check(lib().fm_verify(_ptr(target_logits), dtype_code(target_logits.dtype), B, K1 - 1, V,
                           _ptr(draft), _ptr(emitted), _ptr(accept), _ptr(best), _stream(stream)))


def fm_verify_greedy(h, target_logits, draft, emitted, accept, best, stream=None):
    """fm_verify for a handle's drafts, each target row read by several
    workgroups: target_logits [B][17][V]; draft [B][16] int32; outputs
    emitted [B][17], accept [B], best [1] int32."""
    B = int(target_logits.shape[0])
    _check(lib().fm_verify_greedy(h, _ptr(target_logits), dtype_code(target_logits.dtype), B, _ptr(draft),
                                  _ptr(emitted), _ptr(accept), _ptr(best), _stream(stream)))


def fm_set_probe(h, kernel: int, ev_start=None, ev_stop=None):
    """ev_start/ev_stop: torch.cuda.Event(enable_timing=True) objects or raw
    hipEvent_t integers."""
    def raw(e):
        if e is None:
            return ctypes.c_void_p(None)
        return ctypes.c_void_p(e.cuda_event if hasattr(e, "cuda_event") else int(e))
    _check(lib().fm_set_probe(h, int(kernel), raw(ev_start), raw(ev_stop)))


# ----------------------------------------------------------------- convenience

class Drafter:
    """Owns a handle, its workspace tensor and references to the weights."""

    def __init__(self, cfg: fm_config, weights: dict, device: int = 0):
        self.cfg = cfg
        self.device = torch.device("cuda", device)
        n = fm_workspace_bytes(cfg)
        if n == 0:
            raise FlashMapError(FM_EINVAL, fm_last_error())
        # 256 bytes of slack so the workspace can start 256-byte aligned
        self._ws_raw = torch.empty(n + 256, dtype=torch.uint8, device=self.device)
        off = (-self._ws_raw.data_ptr()) % 256
        self.workspace = self._ws_raw[off:off + n]
        self.weights = weights
        self.handle = fm_create(cfg, self.workspace, n, device)
        fm_set_weights(self.handle, weights, cfg.L)
        self.times = None

    def set_schedule(self, times, stream=None):
        fm_set_schedule(self.handle, times, stream)
        self.times = tuple(times)

    def append(self, feats, stream=None):
        fm_context_append(self.handle, feats, stream)

    def truncate(self, n, stream=None):
        fm_context_truncate(self.handle, n, stream)

    def sync_context(self, stream=None):
        fm_context_sync(self.handle, stream)

    def append_req(self, req, feats, stream=None):
        fm_context_append_req(self.handle, req, feats, stream)

    def truncate_req(self, req, n, stream=None):
        fm_context_truncate_req(self.handle, req, n, stream)

    def context_length_req(self, req):
        return fm_context_length_req(self.handle, req)

    def draft_batch(self, noise, new_feats=None, n_new=None, logits=None, tokens=None, stream=None):
        if tokens is None:
            tokens = torch.empty(noise.shape[0], noise.shape[1], dtype=torch.int32, device=self.device)
        fm_draft_batch(self.handle, noise, tokens, new_feats, n_new, logits, stream)
        return tokens

    @property
    def context_length(self):
        return fm_context_length(self.handle)

    def draft(self, noise, new_feats=None, logits=None, hidden=None, tokens=None, stream=None):
        if tokens is None:
            tokens = torch.empty(noise.shape[0], noise.shape[1], dtype=torch.int32, device=self.device)
        fm_draft(self.handle, noise, tokens, new_feats, logits, hidden, stream)
        return tokens

    def draft_sample(self, noise, temperature, seed, new_feats=None, stream=None):
        """Returns (tokens, logits, lse) of a temperature > 0 draft."""
        B, K, V = (int(x) for x in noise.shape)
        tokens = torch.empty(B, K, dtype=torch.int32, device=self.device)
        logits = torch.empty(B, K, V, dtype=torch.float32, device=self.device)
        lse = torch.empty(B, K, dtype=torch.float32, device=self.device)
        fm_draft_sample(self.handle, noise, temperature, seed, tokens, logits, lse, new_feats, stream)
        return tokens, logits, lse

    def verify(self, target_logits, draft, emitted, accept, best, stream=None):
        """Greedy verification through the handle (fm_verify_greedy)."""
        fm_verify_greedy(self.handle, target_logits, draft, emitted, accept, best, stream)

    def verify_sample(self, target_logits, draft_logits, draft_lse, draft, temperature, seed, stream=None):
        """Returns (emitted, accept) of probabilistic verification."""
        B, K1, _ = target_logits.shape
        emitted = torch.empty(B, K1, dtype=torch.int32, device=self.device)
        accept = torch.empty(B, dtype=torch.int32, device=self.device)
        fm_verify_sample(self.handle, target_logits, draft_logits, draft_lse, draft, temperature, seed,
                         emitted, accept, stream)
        return emitted, accept

    def close(self):
        if self.handle is not None:
            fm_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def verify(target_logits, draft, stream=None):
    """Allocate outputs and run fm_verify; returns (emitted, accept, best)."""
    B, K1, _ = target_logits.shape
    dev = target_logits.device
    emitted = torch.empty(B, K1, dtype=torch.int32, device=dev)
    accept = torch.empty(B, dtype=torch.int32, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    fm_verify(target_logits, draft, emitted, accept, best, stream)
    return emitted, accept, best
