"""Seeded synthetic inputs shared by the oracle and the HIP library.

Only input generation lives here (random numbers, random models already in
the GGUF Q8_0/Q4_0/Q4_K/Q5_K/Q6_K block formats, fp16 tables, token ids); none of the decode
step's arithmetic does.  The C core is ``synth.c``; ``build()`` compiles it.

Workloads (the decode-step configurations this project is measured on):

* tiny: vocab 512, hidden 256, 2 layers, 4/2 heads, hd 64, ffn 704, Q8_0,
  16 cached positions, 4 greedy steps, seed 0
* llama8b_q8: Llama-3.1-8B shape, Q8_0, ctx 512 (+64 steps), batch 1, seed 1
* llama8b_q4: Llama-3.1-8B shape, Q4_0, ctx 4096 (+32 steps), batch 4, seed 2
* multi_*: Llama-3.2-1B / Qwen2-0.5B / SmolLM2-360M shapes, Q8_0, ctx 2048,
  32 steps each, seed 3, tensor-id namespaces 0/1/2
* llama70b_q4: Llama-3.1-70B shape, Q4_0, ctx 1024, 16 steps, seed 4
* llama8b_q4k / llama8b_q6k: the 8B shape in Q4_K / Q6_K, ctx 512 (+64 steps),
  batch 1, seeds 5 / 6
* llama70b_q4k / llama70b_q6k: the 70B shape in Q4_K / Q6_K, ctx 1024,
  16 steps, seeds 7 / 8
* llama8b_q5k: the 8B shape in Q5_K, ctx 512 (+64 steps), batch 1, seed 9

Distributions: weights N(0, 0.02) quantised block by block; fp16 token
embeddings N(0, 0.02); fp32 norm gains N(1, 0.1); fp16 KV N(0, 1) for every
(sequence, layer, KV head, position); start tokens uniform over the vocab.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field, asdict

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
# another build of the same source (the sanitizer test loads one)
LOAD_PATH = os.environ.get("LM_SYNTH_LIB") or LIB_PATH

Q4_0 = 2
Q8_0 = 8
Q4_K = 12
Q5_K = 13
Q6_K = 14
BLOCK_BYTES = {Q8_0: 34, Q4_0: 18, Q4_K: 144, Q5_K: 176, Q6_K: 210}     # bytes per block
BLOCK_WEIGHTS = {Q8_0: 32, Q4_0: 32, Q4_K: 256, Q5_K: 256, Q6_K: 256}   # weights per block
QTYPE_NAMES = {Q8_0: "Q8_0", Q4_0: "Q4_0", Q4_K: "Q4_K", Q5_K: "Q5_K", Q6_K: "Q6_K"}


def row_bytes(qtype: int, cols: int) -> int:
    """Bytes of one row of `cols` weights in GGUF blocks."""
    if cols % BLOCK_WEIGHTS[qtype]:
        raise ValueError(f"{cols} columns is not a multiple of the {QTYPE_NAMES[qtype]} block")
    return cols // BLOCK_WEIGHTS[qtype] * BLOCK_BYTES[qtype]


def build() -> str:
    """Compile synth.c into libsynth.so (gcc, OpenMP)."""
    import subprocess
    src = os.path.join(_HERE, "synth.c")
    tmp = LIB_PATH + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                           "-o", tmp, src, "-lm"])
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LOAD_PATH):
            raise RuntimeError(f"{LOAD_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LOAD_PATH)
        u64, i64, f64, i32, u32 = (ctypes.c_uint64, ctypes.c_int64, ctypes.c_double,
                                   ctypes.c_int32, ctypes.c_uint32)
        vp = ctypes.c_void_p
        L.synth_philox4x32_10.argtypes = [vp, vp, vp]
        L.synth_philox4x32_10.restype = None
        L.synth_f64_to_f16.argtypes = [f64]
        L.synth_f64_to_f16.restype = ctypes.c_uint16
        L.synth_quantize.argtypes = [vp, i64, ctypes.c_int, vp]
        L.synth_quantize.restype = ctypes.c_int
        L.synth_normal_f32.argtypes = [u64, u64, i64, i64, f64, f64, vp]
        L.synth_normal_f32.restype = None
        L.synth_normal_f16.argtypes = [u64, u64, i64, i64, f64, f64, vp]
        L.synth_normal_f16.restype = None
        L.synth_uniform_int.argtypes = [u64, u64, i64, u32, vp]
        L.synth_uniform_int.restype = None
        L.synth_quant_matrix.argtypes = [u64, u64, i64, i64, f64, ctypes.c_int, vp]
        L.synth_quant_matrix.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ---------------------------------------------------------------------------
# primitives
# ---------------------------------------------------------------------------

def philox4x32_10(ctr, key) -> np.ndarray:
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    lib().synth_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def f64_to_f16_bits(v: float) -> int:
    return int(lib().synth_f64_to_f16(float(v)))


def quantize(w: np.ndarray, qtype: int) -> np.ndarray:
    """Quantise fp32 values (length a multiple of the block size) into GGUF blocks."""
    w = np.ascontiguousarray(w, dtype=np.float32).ravel()
    out = np.zeros(row_bytes(qtype, w.size), np.uint8)
    if lib().synth_quantize(_ptr(w), w.size, qtype, _ptr(out)) != 0:
        raise ValueError("bad quantize arguments")
    return out


def normal_f32(seed, tid, n, mean=0.0, std=1.0, offset=0) -> np.ndarray:
    out = np.empty(n, np.float32)
    lib().synth_normal_f32(seed, tid, offset, n, mean, std, _ptr(out))
    return out


def normal_f16_bits(seed, tid, n, mean=0.0, std=1.0, offset=0) -> np.ndarray:
    out = np.empty(n, np.uint16)
    lib().synth_normal_f16(seed, tid, offset, n, mean, std, _ptr(out))
    return out


def uniform_int(seed, tid, n, bound) -> np.ndarray:
    out = np.empty(n, np.int32)
    lib().synth_uniform_int(seed, tid, n, bound, _ptr(out))
    return out


def quant_matrix(seed, tid, rows, cols, std, qtype) -> np.ndarray:
    """rows x cols matrix of (float)(std*z), quantised: uint8 [rows, row_bytes(qtype, cols)]."""
    out = np.empty((rows, row_bytes(qtype, cols)), np.uint8)
    if lib().synth_quant_matrix(seed, tid, rows, cols, std, qtype, _ptr(out)) != 0:
        raise ValueError("bad quant_matrix arguments")
    return out


# ---------------------------------------------------------------------------
# model configurations
# ---------------------------------------------------------------------------

@dataclass
class ModelConfig:
    name: str
    vocab: int
    hidden: int
    n_layers: int
    n_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    qtype: int = Q8_0
    rms_eps: float = 1e-5
    rope_theta: float = 500000.0
    ctx: int = 16            # prefilled KV positions
    steps: int = 4           # greedy decode steps
    batch: int = 1           # sequences decoded together
    seed: int = 0
    ns: int = 0              # tensor-id namespace (several models under one seed)

    @property
    def max_ctx(self) -> int:
        return self.ctx + self.steps

    def as_dict(self):
        return asdict(self)

    def weight_bytes(self) -> int:
        """Quantised weight bytes read per token (all layers + LM head)."""
        qt = self.qtype
        H, F = self.hidden, self.ffn
        qkv = (self.n_heads + 2 * self.n_kv_heads) * self.head_dim
        per_layer = (qkv * row_bytes(qt, H) + H * row_bytes(qt, self.n_heads * self.head_dim)
                     + 2 * F * row_bytes(qt, H) + H * row_bytes(qt, F))
        return per_layer * self.n_layers + self.vocab * row_bytes(qt, H)


def _cfg(**kw) -> ModelConfig:
    return ModelConfig(**kw)


CONFIGS = {
    "tiny": _cfg(name="tiny", vocab=512, hidden=256, n_layers=2, n_heads=4, n_kv_heads=2,
                 head_dim=64, ffn=704, qtype=Q8_0, ctx=16, steps=4, batch=1, seed=0),
    "llama8b_q8": _cfg(name="llama8b_q8", vocab=128256, hidden=4096, n_layers=32, n_heads=32,
                       n_kv_heads=8, head_dim=128, ffn=14336, qtype=Q8_0, ctx=512, steps=64,
                       batch=1, seed=1),
    "llama8b_q4": _cfg(name="llama8b_q4", vocab=128256, hidden=4096, n_layers=32, n_heads=32,
                       n_kv_heads=8, head_dim=128, ffn=14336, qtype=Q4_0, ctx=4096, steps=32,
                       batch=4, seed=2),
    "multi_llama1b": _cfg(name="multi_llama1b", vocab=128256, hidden=2048, n_layers=16,
                          n_heads=32, n_kv_heads=8, head_dim=64, ffn=8192, qtype=Q8_0,
                          ctx=2048, steps=32, batch=1, seed=3, ns=0),
    "multi_qwen05b": _cfg(name="multi_qwen05b", vocab=151936, hidden=896, n_layers=24,
                          n_heads=14, n_kv_heads=2, head_dim=64, ffn=4864, qtype=Q8_0,
                          ctx=2048, steps=32, batch=1, seed=3, ns=1),
    "multi_smol360m": _cfg(name="multi_smol360m", vocab=49152, hidden=960, n_layers=32,
                           n_heads=15, n_kv_heads=5, head_dim=64, ffn=2560, qtype=Q8_0,
                           ctx=2048, steps=32, batch=1, seed=3, ns=2),
    "llama70b_q4": _cfg(name="llama70b_q4", vocab=128256, hidden=8192, n_layers=80,
                        n_heads=64, n_kv_heads=8, head_dim=128, ffn=28672, qtype=Q4_0,
                        ctx=1024, steps=16, batch=1, seed=4),
    # the GGUF K formats of the engine page's 70B figures, on the 8B and 70B shapes
    "llama8b_q4k": _cfg(name="llama8b_q4k", vocab=128256, hidden=4096, n_layers=32, n_heads=32,
                        n_kv_heads=8, head_dim=128, ffn=14336, qtype=Q4_K, ctx=512, steps=64,
                        batch=1, seed=5),
    "llama8b_q6k": _cfg(name="llama8b_q6k", vocab=128256, hidden=4096, n_layers=32, n_heads=32,
                        n_kv_heads=8, head_dim=128, ffn=14336, qtype=Q6_K, ctx=512, steps=64,
                        batch=1, seed=6),
    "llama8b_q5k": _cfg(name="llama8b_q5k", vocab=128256, hidden=4096, n_layers=32, n_heads=32,
                        n_kv_heads=8, head_dim=128, ffn=14336, qtype=Q5_K, ctx=512, steps=64,
                        batch=1, seed=9),
    "llama70b_q4k": _cfg(name="llama70b_q4k", vocab=128256, hidden=8192, n_layers=80,
                         n_heads=64, n_kv_heads=8, head_dim=128, ffn=28672, qtype=Q4_K,
                         ctx=1024, steps=16, batch=1, seed=7),
    "llama70b_q6k": _cfg(name="llama70b_q6k", vocab=128256, hidden=8192, n_layers=80,
                         n_heads=64, n_kv_heads=8, head_dim=128, ffn=28672, qtype=Q6_K,
                         ctx=1024, steps=16, batch=1, seed=8),
}


def variant(name: str, **changes) -> ModelConfig:
    d = CONFIGS[name].as_dict()
    d.update(changes)
    return ModelConfig(**d)


# tensor ids ---------------------------------------------------------------
T_EMBD, T_OUT_NORM, T_LM_HEAD, T_TOKENS = 1, 2, 3, 4
K_ATTN_NORM, K_FFN_NORM, K_WQ, K_WK, K_WV, K_WO, K_GATE, K_UP, K_DOWN = range(9)


def tensor_id(cfg: ModelConfig, local: int) -> int:
    return (cfg.ns << 28) | local


def layer_tid(cfg: ModelConfig, layer: int, kind: int) -> int:
    return tensor_id(cfg, 1024 + layer * 16 + kind)


def kv_tid(cfg: ModelConfig, seq: int, layer: int, which: int) -> int:
    return tensor_id(cfg, (1 << 20) | (seq << 12) | (layer * 2 + which))


@dataclass
class LayerWeights:
    attn_norm: np.ndarray
    ffn_norm: np.ndarray
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray
    w_gate: np.ndarray
    w_up: np.ndarray
    w_down: np.ndarray


@dataclass
class Model:
    cfg: ModelConfig
    tok_embd: np.ndarray      # uint16 fp16 bits [vocab, hidden]
    out_norm: np.ndarray      # float32 [hidden]
    lm_head: np.ndarray       # uint8 blocks [vocab, hidden/32*bb]
    layers: list = field(default_factory=list)


def make_layer(cfg: ModelConfig, l: int) -> LayerWeights:
    s, H, F, hd = cfg.seed, cfg.hidden, cfg.ffn, cfg.head_dim
    qt = cfg.qtype
    return LayerWeights(
        attn_norm=normal_f32(s, layer_tid(cfg, l, K_ATTN_NORM), H, 1.0, 0.1),
        ffn_norm=normal_f32(s, layer_tid(cfg, l, K_FFN_NORM), H, 1.0, 0.1),
        wq=quant_matrix(s, layer_tid(cfg, l, K_WQ), cfg.n_heads * hd, H, 0.02, qt),
        wk=quant_matrix(s, layer_tid(cfg, l, K_WK), cfg.n_kv_heads * hd, H, 0.02, qt),
        wv=quant_matrix(s, layer_tid(cfg, l, K_WV), cfg.n_kv_heads * hd, H, 0.02, qt),
        wo=quant_matrix(s, layer_tid(cfg, l, K_WO), H, cfg.n_heads * hd, 0.02, qt),
        w_gate=quant_matrix(s, layer_tid(cfg, l, K_GATE), F, H, 0.02, qt),
        w_up=quant_matrix(s, layer_tid(cfg, l, K_UP), F, H, 0.02, qt),
        w_down=quant_matrix(s, layer_tid(cfg, l, K_DOWN), H, F, 0.02, qt),
    )


def make_model(cfg: ModelConfig) -> Model:
    s, H, V = cfg.seed, cfg.hidden, cfg.vocab
    m = Model(
        cfg=cfg,
        tok_embd=normal_f16_bits(s, tensor_id(cfg, T_EMBD), V * H, 0.0, 0.02).reshape(V, H),
        out_norm=normal_f32(s, tensor_id(cfg, T_OUT_NORM), H, 1.0, 0.1),
        lm_head=quant_matrix(s, tensor_id(cfg, T_LM_HEAD), V, H, 0.02, cfg.qtype),
    )
    m.layers = [make_layer(cfg, l) for l in range(cfg.n_layers)]
    return m


def make_kv(cfg: ModelConfig, seq: int, layer: int, n_pos: int | None = None):
    """Prefilled (already rotated) fp16 K and V: uint16 [n_kv, n_pos, hd] each."""
    n_pos = cfg.ctx if n_pos is None else n_pos
    n = cfg.n_kv_heads * n_pos * cfg.head_dim
    shape = (cfg.n_kv_heads, n_pos, cfg.head_dim)
    k = normal_f16_bits(cfg.seed, kv_tid(cfg, seq, layer, 0), n, 0.0, 1.0).reshape(shape)
    v = normal_f16_bits(cfg.seed, kv_tid(cfg, seq, layer, 1), n, 0.0, 1.0).reshape(shape)
    return k, v


def start_tokens(cfg: ModelConfig, n_seq: int | None = None) -> np.ndarray:
    n = cfg.batch if n_seq is None else n_seq
    return uniform_int(cfg.seed, tensor_id(cfg, T_TOKENS), n, cfg.vocab)
