"""GGUF K formats (Q4_K, Q5_K, Q6_K) on the batch-1 path against the fp64 oracle.

The C/CUDA Llama engine page, section 1, lists them among the formats it reads
and quotes its 70B figures in them.  Same bar as the Q8_0 / Q4_0 parity tests:
dequantisation bit-exact, logits within 1e-3 max|logit| per step, the argmax
equal, appended K/V rows within one fp16 ulp plus the fp32 error.
"""
import numpy as np
import pytest

import oracle
import synth
from synth import Q4_K, Q5_K, Q6_K
from tests.helpers import log, open_gpu
from tests.test_gpu_parity import run_parity

pytestmark = pytest.mark.gpu

CASES = {
    # one super-block per hidden row (8 blocks: a lane group of 8, one block each)
    "tiny_q4k": synth.variant("tiny", qtype=Q4_K, ffn=768),
    "tiny_q6k": synth.variant("tiny", qtype=Q6_K, ffn=768),
    "tiny_q5k": synth.variant("tiny", qtype=Q5_K, ffn=768),
    # an empty prefilled cache (first token at position 0)
    "tiny_q4k_ctx0": synth.variant("tiny", qtype=Q4_K, ffn=768, ctx=0, steps=3),
    # 64 blocks per row: half of every lane's second pipeline slot is past the row end
    "llama1b_q4k_2layers": synth.variant("multi_llama1b", n_layers=2, qtype=Q4_K, ctx=64, steps=3),
    "llama1b_q6k_2layers": synth.variant("multi_llama1b", n_layers=2, qtype=Q6_K, ctx=64, steps=3),
    "llama1b_q5k_2layers": synth.variant("multi_llama1b", n_layers=2, qtype=Q5_K, ctx=64, steps=3),
    # 8B layer shapes (down: 448 blocks per row, a ragged last chunk), context crossing a chunk
    "llama8b_q4k_2layers_ctx127": synth.variant("llama8b_q8", n_layers=2, qtype=Q4_K, ctx=127, steps=3),
    "llama8b_q6k_2layers_ctx127": synth.variant("llama8b_q8", n_layers=2, qtype=Q6_K, ctx=127, steps=3),
    "llama8b_q5k_2layers_ctx127": synth.variant("llama8b_q8", n_layers=2, qtype=Q5_K, ctx=127, steps=3),
    # the 70B shape's layers (hidden 8192, ffn 28672, 64/8 heads) at its context length
    "llama70b_q4k_2layers": synth.variant("llama70b_q4", n_layers=2, qtype=Q4_K, steps=2),
    "llama70b_q6k_2layers": synth.variant("llama70b_q4", n_layers=2, qtype=Q6_K, steps=2),
    "llama70b_q5k_2layers": synth.variant("llama70b_q4", n_layers=2, qtype=Q5_K, steps=2),
}

_models = {}


def get_model(name):
    if name not in _models:
        log("generate", name)
        _models[name] = synth.make_model(CASES[name])
    return _models[name]


@pytest.mark.parametrize("name", list(CASES))
def test_kquant_decode_parity(name):
    run_parity(get_model(name), n_seq=1)


@pytest.mark.parametrize("name", ["tiny_q4k", "tiny_q6k", "tiny_q5k", "llama1b_q4k_2layers",
                                  "llama1b_q6k_2layers", "llama1b_q5k_2layers"])
def test_kquant_dequant_bit_exact_all_rows(name):
    model = get_model(name)
    cfg = model.cfg
    g = open_gpu(model, max_seqs=1)
    try:
        H, F, Q, KV = cfg.hidden, cfg.ffn, cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
        for l, w in enumerate(model.layers):
            for which, (arr, rows, cols) in enumerate([(w.wq, Q, H), (w.wk, KV, H), (w.wv, KV, H),
                                                       (w.wo, H, Q), (w.w_gate, F, H),
                                                       (w.w_up, F, H), (w.w_down, H, F)]):
                log(f"{name}: dequant layer {l} matrix {which}")
                got = g.debug_dequant(l, which, 0, rows, cols)
                ref = oracle.dequant(cfg.qtype, arr, rows, cols)
                # fp32 result of the exact fp64 value (Q4_K: one rounding of d*sc*q - dmin*m)
                assert np.array_equal(got, ref.astype(np.float32)), (l, which)
        got = g.debug_dequant(0, 7, 0, cfg.vocab, H)
        assert np.array_equal(got, oracle.dequant(cfg.qtype, model.lm_head, cfg.vocab, H).astype(np.float32))
    finally:
        g.close()


@pytest.mark.parametrize("name", ["tiny_q4k", "llama1b_q6k_2layers"])
def test_kquant_streaming_and_hybrid_bit_identical(name):
    """Layer streaming and every resident prefix give the resident outputs bit for bit."""
    model = get_model(name)
    cfg = model.cfg
    g = open_gpu(model, max_seqs=1)
    try:
        toks = synth.start_tokens(cfg, 1)

        def run():
            g.set_position(0, cfg.ctx)
            res, t = [], toks
            for _ in range(cfg.steps):
                lg, am = g.step(t)
                res.append((lg.copy(), am.copy()))
                t = am
            return res

        ref = run()
        g.stream_mode(True)
        runs = [run()]
        g.stream_mode(False)
        for k in range(cfg.n_layers + 1):
            g.set_residency(k)
            runs.append(run())
        for other in runs:
            for (a, b), (c, d) in zip(ref, other):
                assert np.array_equal(a, c) and np.array_equal(b, d)
    finally:
        g.close()


def test_kquant_speculative_rejected():
    """The speculative verify pass runs on the several-sequence path, built for
    Q8_0 / Q4_0 only: asking for it on a K-format model is an error, and the
    model keeps decoding."""
    import token_decode_llama_amd as lm
    model = get_model("tiny_q4k")
    g = open_gpu(model, max_seqs=1)
    try:
        with pytest.raises(lm.LMError) as e:           # the verify pass needs the several-sequence path
            g.speculative_step(1, 1, 1)
        assert e.value.status == lm.LM_E_STATE
        lg, am = g.step(synth.start_tokens(model.cfg, 1))
        assert np.all(np.isfinite(lg))
    finally:
        g.close()


@pytest.mark.parametrize("name,mask", [("tiny_q6k", [1, 0]), ("llama1b_q4k_2layers", [0, 1])])
def test_kquant_layer_skip_parity(name, mask):
    """Layer skip on K-format models: the oracle with the same mask."""
    from tests.helpers import compare_step, open_oracle
    model = get_model(name)
    cfg = model.cfg
    g = open_gpu(model, max_seqs=1)
    om = open_oracle(model, 1)
    skip = np.array(mask, np.uint8)
    g.set_layer_skip(skip)
    toks = synth.start_tokens(cfg, 1)
    try:
        for st in range(cfg.steps):
            lg_o, am_o = om.step(toks, skip=skip)
            lg_g, am_g = g.step(toks)
            compare_step(lg_g, am_g, lg_o, am_o, f"{name} skip {mask} step {st}")
            toks = am_o
    finally:
        g.close()
        om.close()


@pytest.mark.parametrize("name", ["llama8b_q4k", "llama8b_q5k", "llama8b_q6k"])
def test_kquant_full_size_parity(name):
    """The full 8B-shape K-format models at context 512, the launch
    configuration the benchmark times: two teacher-forced steps against the
    oracle, plus sampled rows of every matrix dequantised bit-exactly."""
    cfg = synth.CONFIGS[name]
    log(f"generate {name}")
    model = synth.make_model(cfg)
    log("run parity")
    run_parity(model, n_seq=1, steps=2)
    g = open_gpu(model, max_seqs=1)
    try:
        H, F, Q, KV = cfg.hidden, cfg.ffn, cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
        rng = np.random.default_rng(0)
        for l in (0, cfg.n_layers - 1):
            w = model.layers[l]
            for which, (arr, rows, cols) in enumerate([(w.wq, Q, H), (w.wk, KV, H), (w.wv, KV, H),
                                                       (w.wo, H, Q), (w.w_gate, F, H),
                                                       (w.w_up, F, H), (w.w_down, H, F)]):
                for r in (0, rows - 1, int(rng.integers(rows))):
                    got = g.debug_dequant(l, which, r, 1, cols)
                    ref = oracle.dequant(cfg.qtype, arr[r:r + 1], 1, cols).astype(np.float32)
                    assert np.array_equal(got, ref), (l, which, r)
        for r in (0, cfg.vocab - 1, 77777):
            got = g.debug_dequant(0, 7, r, 1, H)
            assert np.array_equal(got, oracle.dequant(cfg.qtype, model.lm_head[r:r + 1], 1, H).astype(np.float32))
    finally:
        g.close()


def test_kquant_algorithmic_bytes_follow_the_format():
    """The benchmark's algorithmic bytes (lm_kernel_bytes) differ between two
    formats of the same shape by exactly the weight-byte difference of the
    GGUF rows (the activation terms are the same)."""
    base_cfg = synth.variant("tiny", ffn=768)
    H, F, V = base_cfg.hidden, base_cfg.ffn, base_cfg.vocab
    Q, KV, L = base_cfg.n_heads * base_cfg.head_dim, base_cfg.n_kv_heads * base_cfg.head_dim, base_cfg.n_layers
    shapes = {"qkv": (L * (Q + 2 * KV), H), "wo": (L * H, Q), "gateup": (L * 2 * F, H),
              "down": (L * H, F), "lmhead": (V, H)}
    got = {}
    for qt in (synth.Q8_0, Q4_K, Q5_K, Q6_K):
        model = synth.make_model(synth.variant("tiny", ffn=768, qtype=qt))
        g = open_gpu(model, max_seqs=1)
        try:
            got[qt] = {k: g.kernel_bytes(k, 1) for k in shapes}
        finally:
            g.close()
    for qt in (Q4_K, Q5_K, Q6_K):
        for k, (rows, cols) in shapes.items():
            want = rows * (synth.row_bytes(qt, cols) - synth.row_bytes(synth.Q8_0, cols))
            assert got[qt][k] - got[synth.Q8_0][k] == want, (qt, k)
