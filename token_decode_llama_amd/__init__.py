"""Python binding of liblmdecode.so: the MI355X (gfx950) quantized Llama decode step.

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI (include/lmdecode.h).  PyTorch is used for device
memory and streams (``decode_step_dev`` takes torch CUDA tensors).  There is
no CPU fallback: if the library is not built, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblmdecode.so")

LM_OK, LM_E_ARG, LM_E_STATE, LM_E_OOM, LM_E_HIP, LM_E_CTX = range(6)
LM_Q4_0, LM_Q8_0, LM_Q4_K, LM_Q5_K, LM_Q6_K = 2, 8, 12, 13, 14
KERNEL_KINDS = ("embed", "qkv", "attn", "wo", "gateup", "down", "lmhead", "copy")

# every symbol include/lmdecode.h declares
EXPORTS = (
    "lm_model_create", "lm_model_destroy", "lm_load_layer_weights", "lm_load_global_weights",
    "lm_load_kv", "lm_get_kv", "lm_set_position", "lm_get_position", "lm_stream_mode",
    "lm_set_residency", "lm_tier_sizes", "lm_plan_residency", "lm_set_layer_skip",
    "lm_layer_similarity", "lm_get_layer_similarity", "lm_skip_similar_layers", "lm_speculative_step",
    "lm_decode_step", "lm_decode_step_dev", "lm_decode_step_dev_noalloc", "lm_set_graph", "lm_stream", "lm_last_error",
    "lm_kernel_timing", "lm_kernel_stats", "lm_time_kind", "lm_kernel_bytes", "lm_debug_dequant",
    "lm_debug_read_bw", "lm_debug_gemv", "lm_debug_fail_alloc", "lm_debug_alloc_count",
)


class LMError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


class Config(ctypes.Structure):
    _fields_ = [("vocab", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("rms_eps", ctypes.c_double),
                ("rope_theta", ctypes.c_double), ("max_ctx", ctypes.c_int32),
                ("max_seqs", ctypes.c_int32), ("qtype", ctypes.c_int32)]


class LayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "ffn_norm", "wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")]


_lib = None


def load():
    """Loads the built library (no build here: __graft_entry__.build() compiles it)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: the HIP library must be built "
                           "(python -c 'import __graft_entry__ as g; g.build()')")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    st = ctypes.c_int
    sig = {
        "lm_model_create": ([ctypes.POINTER(Config), vp, ctypes.POINTER(vp)], st),
        "lm_model_destroy": ([vp], None),
        "lm_load_layer_weights": ([vp, i32, ctypes.POINTER(LayerWeights)], st),
        "lm_load_global_weights": ([vp, vp, vp, vp], st),
        "lm_load_kv": ([vp, i32, i32, vp, vp, i32], st),
        "lm_get_kv": ([vp, i32, i32, vp, vp, i32], st),
        "lm_set_position": ([vp, i32, i32], st),
        "lm_get_position": ([vp, i32, ctypes.POINTER(i32)], st),
        "lm_stream_mode": ([vp, i32], st),
        "lm_set_residency": ([vp, i32], st),
        "lm_tier_sizes": ([i32, i64, i64, i64, ctypes.POINTER(i32), ctypes.POINTER(i32)], st),
        "lm_plan_residency": ([vp, i64, i64, ctypes.POINTER(i32)], st),
        "lm_set_layer_skip": ([vp, vp], st),
        "lm_layer_similarity": ([vp, i32], st),
        "lm_get_layer_similarity": ([vp, vp, vp], st),
        "lm_skip_similar_layers": ([vp, dbl, ctypes.POINTER(i32)], st),
        "lm_speculative_step": ([vp, i32, i32, i32, vp, ctypes.POINTER(i32)], st),
        "lm_decode_step": ([vp, vp, i32, vp, vp], st),
        "lm_decode_step_dev": ([vp, vp, i32, vp, vp], st),
        "lm_decode_step_dev_noalloc": ([vp, vp, i32, vp, vp], st),
        "lm_set_graph": ([vp, i32], st),
        "lm_stream": ([vp], vp),
        "lm_last_error": ([vp], ctypes.c_char_p),
        "lm_kernel_timing": ([vp, i32], st),
        "lm_kernel_stats": ([vp, i32, ctypes.POINTER(i64), ctypes.POINTER(dbl)], st),
        "lm_kernel_bytes": ([vp, i32, i32, ctypes.POINTER(dbl)], st),
        "lm_time_kind": ([vp, i32, i32, i32, ctypes.POINTER(dbl)], st),
        "lm_debug_dequant": ([vp, i32, i32, i32, i32, vp], st),
        "lm_debug_read_bw": ([vp, i64, i32, ctypes.POINTER(dbl)], st),
        "lm_debug_gemv": ([vp, i32, i32, i32, vp, vp], st),
        "lm_debug_fail_alloc": ([i64], None),
        "lm_debug_alloc_count": ([], i64),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def tier_sizes(n_layers: int, layer_bytes: int, hbm_bytes: int, host_bytes: int):
    """(tier_a, tier_b, all_fit) by the tier sizing rule (host arithmetic in the library)."""
    a, b = ctypes.c_int32(), ctypes.c_int32()
    st = load().lm_tier_sizes(n_layers, layer_bytes, hbm_bytes, host_bytes, ctypes.byref(a), ctypes.byref(b))
    if st not in (LM_OK, LM_E_OOM):
        raise LMError(f"lm_tier_sizes: status {st}")
    return a.value, b.value, st == LM_OK


def make_config(cfg, max_seqs: int | None = None, max_ctx: int | None = None) -> Config:
    """lm_config from a synth.ModelConfig-like object."""
    return Config(cfg.vocab, cfg.hidden, cfg.n_layers, cfg.n_heads, cfg.n_kv_heads, cfg.head_dim,
                  cfg.ffn, float(cfg.rms_eps), float(cfg.rope_theta),
                  int(max_ctx or cfg.max_ctx), int(max_seqs or cfg.batch), int(cfg.qtype))


class Model:
    """One lm_model.  All methods raise LMError on a non-OK status."""

    def __init__(self, cfg, max_seqs: int | None = None, max_ctx: int | None = None,
                 stream: int | None = None):
        L = load()
        self._lib = L
        self.cfg = cfg
        self.c = make_config(cfg, max_seqs, max_ctx)
        h = ctypes.c_void_p()
        st = L.lm_model_create(ctypes.byref(self.c), ctypes.c_void_p(stream or 0), ctypes.byref(h))
        if st != LM_OK:
            raise LMError(st, L.lm_last_error(None).decode())
        self._h = h

    # -- lifetime ------------------------------------------------------------
    def close(self):
        if getattr(self, "_h", None):
            self._lib.lm_model_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *a):
        self.close()

    def _check(self, st: int):
        if st != LM_OK:
            raise LMError(st, self._lib.lm_last_error(self._h).decode())

    @property
    def handle(self):
        return self._h

    @property
    def stream(self) -> int:
        return int(self._lib.lm_stream(self._h) or 0)

    # -- loading -------------------------------------------------------------
    def load_layer(self, layer: int, w):
        arrs = [np.ascontiguousarray(a) for a in
                (w.attn_norm, w.ffn_norm, w.wq, w.wk, w.wv, w.wo, w.w_gate, w.w_up, w.w_down)]
        lw = LayerWeights(*[_p(a) for a in arrs])
        self._check(self._lib.lm_load_layer_weights(self._h, layer, ctypes.byref(lw)))

    def load_global(self, tok_embd: np.ndarray, out_norm: np.ndarray, lm_head: np.ndarray):
        e = np.ascontiguousarray(tok_embd, dtype=np.uint16)
        g = np.ascontiguousarray(out_norm, dtype=np.float32)
        h = np.ascontiguousarray(lm_head, dtype=np.uint8)
        self._check(self._lib.lm_load_global_weights(self._h, _p(e), _p(g), _p(h)))

    def load_model(self, model):
        for l, w in enumerate(model.layers):
            self.load_layer(l, w)
        self.load_global(model.tok_embd, model.out_norm, model.lm_head)

    def load_kv(self, seq: int, layer: int, k: np.ndarray, v: np.ndarray):
        k = np.ascontiguousarray(k, dtype=np.uint16)
        v = np.ascontiguousarray(v, dtype=np.uint16)
        self._check(self._lib.lm_load_kv(self._h, seq, layer, _p(k), _p(v), k.shape[1]))

    def get_kv(self, seq: int, layer: int, n_pos: int):
        shape = (self.cfg.n_kv_heads, n_pos, self.cfg.head_dim)
        k = np.empty(shape, np.uint16)
        v = np.empty(shape, np.uint16)
        self._check(self._lib.lm_get_kv(self._h, seq, layer, _p(k), _p(v), n_pos))
        return k, v

    def set_position(self, seq: int, pos: int):
        self._check(self._lib.lm_set_position(self._h, seq, pos))

    def position(self, seq: int) -> int:
        p = ctypes.c_int32()
        self._check(self._lib.lm_get_position(self._h, seq, ctypes.byref(p)))
        return p.value

    # -- decoding ------------------------------------------------------------
    def step(self, tokens, want_logits: bool = True):
        """One decode step from host tokens; returns (fp32 logits [n, vocab] or None, argmax [n])."""
        t = np.ascontiguousarray(tokens, dtype=np.int32).ravel()
        n = t.size
        am = np.empty(n, np.int32)
        lg = np.empty((n, self.cfg.vocab), np.float32) if want_logits else None
        self._check(self._lib.lm_decode_step(self._h, _p(t), n, _p(lg) if lg is not None else None,
                                             _p(am)))
        return lg, am

    def step_dev(self, d_tokens, n_seq: int, d_argmax, d_logits=None):
        """Asynchronous step on device buffers (torch tensors or raw pointers)."""
        ptr = lambda x: x if isinstance(x, int) or x is None else x.data_ptr()
        self._check(self._lib.lm_decode_step_dev(self._h, ptr(d_tokens), n_seq, ptr(d_logits),
                                                 ptr(d_argmax)))

    def step_dev_noalloc(self, d_tokens, n_seq: int, d_argmax, d_logits=None):
        """step_dev without any device allocation (working memory in the library's fixed scratch array)."""
        ptr = lambda x: x if isinstance(x, int) or x is None else x.data_ptr()
        self._check(self._lib.lm_decode_step_dev_noalloc(self._h, ptr(d_tokens), n_seq, ptr(d_logits),
                                                         ptr(d_argmax)))

    def stream_mode(self, enable):
        """False / 0: resident; True / 1: streamed (pipelined); 2: streamed, copy then compute per layer."""
        self._check(self._lib.lm_stream_mode(self._h, int(enable)))

    def set_residency(self, n_resident: int):
        """Layers 0..n_resident-1 in HBM, the rest streamed from pinned host memory."""
        self._check(self._lib.lm_set_residency(self._h, n_resident))

    def set_layer_skip(self, mask=None):
        """mask: [n_layers] of 0/1 (1 = skip), or None to compute every layer."""
        if mask is None:
            self._check(self._lib.lm_set_layer_skip(self._h, None))
            return
        m = np.ascontiguousarray(mask, dtype=np.uint8)
        if m.size != self.cfg.n_layers:
            raise ValueError(f"skip mask has {m.size} entries; expected {self.cfg.n_layers}")
        self._check(self._lib.lm_set_layer_skip(self._h, _p(m)))

    def layer_similarity(self, enable: bool):
        self._check(self._lib.lm_layer_similarity(self._h, 1 if enable else 0))

    def get_layer_similarity(self):
        """(mean cosine per layer, records per layer)."""
        mean = np.empty(self.cfg.n_layers, np.float64)
        cnt = np.empty(self.cfg.n_layers, np.int32)
        self._check(self._lib.lm_get_layer_similarity(self._h, _p(mean), _p(cnt)))
        return mean, cnt

    def skip_similar_layers(self, threshold: float = 0.98) -> int:
        n = ctypes.c_int32()
        self._check(self._lib.lm_skip_similar_layers(self._h, float(threshold), ctypes.byref(n)))
        return n.value

    def speculative_step(self, token: int, draft_layers: int, k: int) -> np.ndarray:
        """One self-speculative round for sequence 0: the accepted tokens (1..k+1)."""
        out = np.zeros(k + 1, np.int32)
        n = ctypes.c_int32()
        self._check(self._lib.lm_speculative_step(self._h, int(token), int(draft_layers), int(k), _p(out),
                                                  ctypes.byref(n)))
        return out[:n.value].copy()

    def plan_residency(self, hbm_bytes: int = 0, host_bytes: int = 0) -> int:
        """Tier-A layer count by the tier sizing rule (0: query the device / host)."""
        n = ctypes.c_int32()
        self._check(self._lib.lm_plan_residency(self._h, hbm_bytes, host_bytes, ctypes.byref(n)))
        return n.value

    def set_graph(self, enable: bool):
        self._check(self._lib.lm_set_graph(self._h, 1 if enable else 0))

    # -- measurement ---------------------------------------------------------
    def kernel_timing(self, mode):
        """0/False off; 1/True eager steps with events; 2 events inside the replayed graph."""
        self._check(self._lib.lm_kernel_timing(self._h, int(mode)))

    def time_kind(self, kind: str, n_seq: int = 1, reps: int = 20) -> float:
        """Microseconds per launch of one kernel family, replayed as the step graph runs it."""
        us = ctypes.c_double()
        self._check(self._lib.lm_time_kind(self._h, KERNEL_KINDS.index(kind), n_seq, reps, ctypes.byref(us)))
        return us.value

    def kernel_stats(self, kind: str):
        c = ctypes.c_int64()
        ms = ctypes.c_double()
        self._check(self._lib.lm_kernel_stats(self._h, KERNEL_KINDS.index(kind), ctypes.byref(c),
                                              ctypes.byref(ms)))
        return c.value, ms.value

    def kernel_bytes(self, kind: str, n_seq: int = 1) -> float:
        b = ctypes.c_double()
        self._check(self._lib.lm_kernel_bytes(self._h, KERNEL_KINDS.index(kind), n_seq, ctypes.byref(b)))
        return b.value

    def debug_dequant(self, layer: int, which: int, row0: int, n_rows: int, cols: int) -> np.ndarray:
        out = np.empty((n_rows, cols), np.float32)
        self._check(self._lib.lm_debug_dequant(self._h, layer, which, row0, n_rows, _p(out)))
        return out

    def debug_gemv(self, layer: int, which: int, x: np.ndarray) -> np.ndarray:
        """y = W x through the step's GEMV kernel (which: 0 QKV, 1 Wo, 2 gate/up
        interleaved, 3 down, 4 LM head); x fp32 [n_seq, K] -> y fp32 [n_seq, N]."""
        x = np.ascontiguousarray(x, dtype=np.float32)
        if x.ndim == 1:
            x = x[None]
        n = {0: self.cfg.n_heads * self.cfg.head_dim + 2 * self.cfg.n_kv_heads * self.cfg.head_dim,
             1: self.cfg.hidden, 2: 2 * self.cfg.ffn, 3: self.cfg.hidden, 4: self.cfg.vocab}[which]
        y = np.empty((x.shape[0], n), np.float32)
        self._check(self._lib.lm_debug_gemv(self._h, layer, which, x.shape[0], _p(x), _p(y)))
        return y

    def debug_read_bw(self, n_bytes: int, iters: int = 10) -> float:
        ms = ctypes.c_double()
        self._check(self._lib.lm_debug_read_bw(self._h, n_bytes, iters, ctypes.byref(ms)))
        return ms.value


def fail_alloc(n: int):
    """The n-th library allocation from now on fails (LM_E_OOM); 0 disarms."""
    load().lm_debug_fail_alloc(int(n))


def alloc_count() -> int:
    return int(load().lm_debug_alloc_count())


def open_model(model, kv_fn, max_seqs: int | None = None, kv_seqs: int | None = None,
               stream: int | None = None, max_ctx: int | None = None) -> Model:
    """Creates an lm_model for a model object (cfg, layers, tok_embd, out_norm,
    lm_head), loads its weights, and installs the cache that kv_fn(seq, layer)
    returns (fp16 bits [n_kv, n_pos, hd] for K and V) for sequences
    0..kv_seqs-1 (default max_seqs).  max_ctx: cache positions (default the
    config's ctx + steps)."""
    cfg = model.cfg
    m = Model(cfg, max_seqs=max_seqs, max_ctx=max_ctx, stream=stream)
    m.load_model(model)
    n = kv_seqs if kv_seqs is not None else m.c.max_seqs
    for s in range(n):
        for l in range(cfg.n_layers):
            k, v = kv_fn(s, l)
            m.load_kv(s, l, k, v)
    return m
