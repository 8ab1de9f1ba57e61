"""fp64 CPU oracle of the quantized Llama decode step (ctypes over oracle.c).

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg use this package.  It imports nothing from the HIP library
package and the library imports nothing from here.  The only code both sides
share is the input generator in ``synth``.

Each wrapper names the passage of the pages it follows (see oracle.c's
header for the full list and for the readings taken where the pages are
silent).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
# another build of the same source (the sanitizer test loads one)
LOAD_PATH = os.environ.get("LM_ORACLE_LIB") or LIB_PATH

Q4_0 = 2
Q8_0 = 8
Q4_K = 12
Q5_K = 13
Q6_K = 14


def build() -> str:
    """Compile oracle.c (plain C, OpenMP over output rows, no FMA contraction)."""
    import subprocess
    src = os.path.join(_HERE, "oracle.c")
    tmp = LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                           "-fPIC", "-shared", "-o", tmp, src, "-lm"])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


class _Config(ctypes.Structure):
    _fields_ = [("vocab", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_layers", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("rms_eps", ctypes.c_double),
                ("rope_theta", ctypes.c_double), ("max_ctx", ctypes.c_int32),
                ("max_seqs", ctypes.c_int32), ("qtype", ctypes.c_int32)]


class _Layer(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "ffn_norm", "wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down")]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LOAD_PATH):
            raise RuntimeError(f"{LOAD_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LOAD_PATH)
        vp, i64, i32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        sig = {
            "orc_f16_to_f64": ([ctypes.c_uint16], f64),
            "orc_f64_to_f16": ([f64], ctypes.c_uint16),
            "orc_block_bytes": ([i32], i32),
            "orc_block_weights": ([i32], i32),
            "orc_row_bytes": ([i32, i64], i64),
            "orc_dequant_row": ([i32, vp, i64, vp], i32),
            "orc_gemv": ([i32, vp, i64, i64, vp, vp], i32),
            "orc_rmsnorm": ([vp, vp, i64, f64, vp], None),
            "orc_rope": ([vp, i32, i32, i64, f64], None),
            "orc_silu": ([f64], f64),
            "orc_attention": ([vp, vp, vp, i32, i32, i32, i64, i64, vp], None),
            "orc_argmax_f32": ([vp, i64], ctypes.c_int32),
            "orc_model_create": ([ctypes.POINTER(_Config)], vp),
            "orc_model_destroy": ([vp], None),
            "orc_model_set_layer": ([vp, i32, ctypes.POINTER(_Layer)], None),
            "orc_model_set_global": ([vp, vp, vp, vp], None),
            "orc_model_load_kv": ([vp, i32, i32, vp, vp, i64], i32),
            "orc_model_get_kv": ([vp, i32, i32, vp, vp, i64], i32),
            "orc_model_set_position": ([vp, i32, i64], i32),
            "orc_model_position": ([vp, i32], i64),
            "orc_decode_step": ([vp, vp, i32, vp, vp], i32),
            "orc_decode_step_ex": ([vp, vp, i32, vp, vp, vp, vp], i32),
            "orc_cosine": ([vp, vp, i64], f64),
            "orc_skip_list": ([vp, i32, f64, vp], i32),
            "orc_spec_accept": ([vp, vp, i32, vp], i32),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def _c64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# single operations
# ---------------------------------------------------------------------------

def f16_to_f64(bits: int) -> float:
    """Exact value of a binary16 bit pattern."""
    return lib().orc_f16_to_f64(int(bits))


def f64_to_f16(v: float) -> int:
    """binary16 bits nearest to v (ties to even)."""
    return int(lib().orc_f64_to_f16(float(v)))


def dequant(qtype: int, blocks: np.ndarray, rows: int, cols: int) -> np.ndarray:
    """GGUF blocks [rows, row bytes] -> fp64 [rows, cols]: Q8_0/Q4_0 as the
    workload defines them, Q4_K/Q5_K/Q6_K as the GGUF format publishes them (all
    four named on the C/CUDA Llama engine page, section 1)."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(rows, -1)
    out = np.empty((rows, cols), np.float64)
    for r in range(rows):
        if lib().orc_dequant_row(qtype, _p(b[r]), cols, _p(out[r])) != 0:
            raise ValueError("bad dequant arguments")
    return out


def gemv(qtype: int, blocks: np.ndarray, rows: int, cols: int, x) -> np.ndarray:
    """y = W x over quantised rows (C/CUDA Llama engine page, section 4.4, GEMV)."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    x = _c64(x)
    y = np.empty(rows, np.float64)
    if lib().orc_gemv(qtype, _p(b), rows, cols, _p(x), _p(y)) != 0:
        raise ValueError("bad gemv arguments")
    return y


def rmsnorm(x, g, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g (C/CUDA Llama engine page, sections 1, 4.4)."""
    x = _c64(x)
    g = np.ascontiguousarray(g, dtype=np.float32)
    out = np.empty_like(x)
    lib().orc_rmsnorm(_p(x), _p(g), x.size, eps, _p(out))
    return out


def rope(v, n_heads: int, head_dim: int, pos: int, theta: float) -> np.ndarray:
    """Rotate adjacent pairs of each head by pos*theta^(-2i/hd) (C/CUDA Llama
    engine page, section 4.4; positions as on the SwarmKV page, section 4)."""
    out = _c64(v).copy()
    lib().orc_rope(_p(out), n_heads, head_dim, pos, theta)
    return out


def silu(a: float) -> float:
    return lib().orc_silu(float(a))


def attention(q, K: np.ndarray, V: np.ndarray, n_heads: int, n_kv: int, head_dim: int,
              n_ctx: int) -> np.ndarray:
    """GQA decode attention with causal softmax over keys 0..n_ctx-1.
    K, V: fp16 bits [n_kv, kv_stride, hd] (C/CUDA Llama engine page, sections 1, 4.4)."""
    q = _c64(q)
    K = np.ascontiguousarray(K, dtype=np.uint16)
    V = np.ascontiguousarray(V, dtype=np.uint16)
    stride = K.shape[1]
    out = np.empty(n_heads * head_dim, np.float64)
    lib().orc_attention(_p(q), _p(K), _p(V), n_heads, n_kv, head_dim, stride, n_ctx, _p(out))
    return out


def cosine(a, b) -> float:
    a, b = _c64(a), _c64(b)
    return float(lib().orc_cosine(_p(a), _p(b), a.size))


def skip_list(mean_cos, threshold: float) -> np.ndarray:
    m = _c64(mean_cos)
    mask = np.zeros(m.size, np.uint8)
    lib().orc_skip_list(_p(m), m.size, float(threshold), _p(mask))
    return mask


def spec_accept(draft, verify):
    """Accepted tokens of one self-speculative round (len(verify) == len(draft) + 1)."""
    d = np.ascontiguousarray(draft, dtype=np.int32)
    v = np.ascontiguousarray(verify, dtype=np.int32)
    if v.size != d.size + 1:
        raise ValueError("verify holds one token more than draft")
    out = np.empty(v.size, np.int32)
    n = lib().orc_spec_accept(_p(d) if d.size else None, _p(v), d.size, _p(out))
    return out[:n]


def argmax_f32(v) -> int:
    v = _c64(v)
    return int(lib().orc_argmax_f32(_p(v), v.size))


# ---------------------------------------------------------------------------
# whole model
# ---------------------------------------------------------------------------

class OracleModel:
    """fp64 reference model over the generator's bytes.  Weight arrays are
    borrowed (kept alive by holding the synth.Model)."""

    def __init__(self, model, max_seqs: int | None = None, max_ctx: int | None = None):
        cfg = model.cfg
        self.cfg = cfg
        self._model = model
        self.max_seqs = max_seqs or cfg.batch
        self.max_ctx = max_ctx or cfg.max_ctx
        c = _Config(cfg.vocab, cfg.hidden, cfg.n_layers, cfg.n_heads, cfg.n_kv_heads,
                    cfg.head_dim, cfg.ffn, cfg.rms_eps, cfg.rope_theta, self.max_ctx,
                    self.max_seqs, cfg.qtype)
        self._h = lib().orc_model_create(ctypes.byref(c))
        if not self._h:
            raise MemoryError("oracle model allocation failed")
        self._keep = []
        for l, w in enumerate(model.layers):
            arrs = [np.ascontiguousarray(a) for a in
                    (w.attn_norm, w.ffn_norm, w.wq, w.wk, w.wv, w.wo, w.w_gate, w.w_up, w.w_down)]
            self._keep.append(arrs)
            lw = _Layer(*[_p(a) for a in arrs])
            lib().orc_model_set_layer(self._h, l, ctypes.byref(lw))
        g = [np.ascontiguousarray(model.tok_embd), np.ascontiguousarray(model.out_norm),
             np.ascontiguousarray(model.lm_head)]
        self._keep.append(g)
        lib().orc_model_set_global(self._h, _p(g[0]), _p(g[1]), _p(g[2]))

    def close(self):
        if self._h:
            lib().orc_model_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def load_kv(self, seq: int, layer: int, k: np.ndarray, v: np.ndarray):
        k = np.ascontiguousarray(k, dtype=np.uint16)
        v = np.ascontiguousarray(v, dtype=np.uint16)
        if lib().orc_model_load_kv(self._h, seq, layer, _p(k), _p(v), k.shape[1]) != 0:
            raise ValueError("bad load_kv arguments")

    def get_kv(self, seq: int, layer: int, n_pos: int):
        shape = (self.cfg.n_kv_heads, n_pos, self.cfg.head_dim)
        k = np.empty(shape, np.uint16)
        v = np.empty(shape, np.uint16)
        if lib().orc_model_get_kv(self._h, seq, layer, _p(k), _p(v), n_pos) != 0:
            raise ValueError("bad get_kv arguments")
        return k, v

    def set_position(self, seq: int, pos: int):
        if lib().orc_model_set_position(self._h, seq, pos) != 0:
            raise ValueError("bad position")

    def position(self, seq: int) -> int:
        return int(lib().orc_model_position(self._h, seq))

    def step(self, tokens, skip=None, with_cos: bool = False):
        """One decode step; returns (fp64 logits [n_seq, vocab], argmax [n_seq]),
        plus the per-layer input/output cosine similarities [n_seq, n_layers]
        with with_cos.  skip: [n_layers] mask of skipped layers."""
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        n = t.size
        logits = np.empty((n, self.cfg.vocab), np.float64)
        am = np.empty(n, np.int32)
        sk = None if skip is None else np.ascontiguousarray(skip, dtype=np.uint8)
        cos = np.empty((n, self.cfg.n_layers), np.float64) if with_cos else None
        if lib().orc_decode_step_ex(self._h, _p(t), n, _p(logits), _p(am),
                                    None if sk is None else _p(sk), None if cos is None else _p(cos)) != 0:
            raise ValueError("oracle decode step rejected its arguments")
        return (logits, am, cos) if with_cos else (logits, am)
