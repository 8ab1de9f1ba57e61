"""GPU parity of the multi-sequence step (2..4 sequences per step: the
activation-fragment kernel plus the MFMA dequant-GEMV) through the C ABI.

Bars as for one sequence: argmax identical to the oracle, per step and
sequence max|d logit| <= 1e-3 * max|logit|, appended K/V within one fp16 ulp
plus 2e-5 * max|row|.  In addition each sequence of a batched step must agree
with the one-sequence path run on that sequence alone (same tolerance,
identical argmax), and a model built for several sequences must give the
one-sequence kernel's bit-identical result when stepped with one.
"""
import numpy as np
import pytest

import synth
from synth import Q4_0, Q8_0
from tests.helpers import LOGIT_RTOL, log, open_gpu
from tests.test_gpu_parity import run_parity

pytestmark = pytest.mark.gpu

BATCH_CASES = {
    "tiny_q8_b2": (synth.variant("tiny", batch=2), 2),
    "tiny_q8_b3": (synth.variant("tiny", batch=3), 3),
    "tiny_q4_b4": (synth.variant("tiny", qtype=Q4_0, batch=4), 4),
    # down projection of 5120 columns: the digits staged by each workgroup in
    # two batches (the first requested before the weights, the second after)
    "tiny_ffn5120_q8_b2": (synth.variant("tiny", ffn=5120, batch=2), 2),
    "tiny_ffn5120_q4_b3": (synth.variant("tiny", ffn=5120, qtype=Q4_0, batch=3), 3),
    # down projection of 6400 columns, wider than a workgroup's prologue digits:
    # the gate/up kernel writes h's digits in its epilogue, four consecutive
    # tiles (one 32-column block of h) per round, 200 blocks (fewer than the
    # CUs); an empty sequence slot at three sequences
    "tiny_ffn6400_q8_b3": (synth.variant("tiny", ffn=6400, batch=3), 3),
    "tiny_ffn6400_q4_b2": (synth.variant("tiny", ffn=6400, qtype=Q4_0, batch=2), 2),
    # vocabulary that ends inside a 16-row tile (498 = 31 * 16 + 2)
    "tiny_q8_vocab498_b2": (synth.variant("tiny", vocab=498, batch=2), 2),
    # ragged block counts (28 and 30 blocks/row), GQA groups of 7 and 3
    "qwen05b_2layers_b2": (synth.variant("multi_qwen05b", n_layers=2, ctx=130, steps=3, batch=2), 2),
    "smol360m_2layers_b3": (synth.variant("multi_smol360m", n_layers=2, ctx=70, steps=3, batch=3), 3),
    # the 8B Q4_0 four-sequence workload's layer shapes at its context length
    # (attention: several 64-position tiles per workgroup, partial states merged)
    "llama8b_q4_2layers_b4": (synth.variant("llama8b_q4", n_layers=2, steps=2), 4),
    # 4 x 8 KV heads x 128 chunks: four tiles per attention workgroup (head_dim 64, the
    # resident-grid choice);
    # 127 tiles (the last span has a tile past the context), then a lone key in tile 128
    "llama1b_2layers_b4_ctx8k": (synth.variant("multi_llama1b", n_layers=2, ctx=8127, steps=2, batch=4), 4),
}


@pytest.mark.parametrize("name", list(BATCH_CASES))
def test_batch_parity(name):
    cfg, n_seq = BATCH_CASES[name]
    log("generate", name)
    run_parity(synth.make_model(cfg), n_seq=n_seq)


def _steps(g, toks, n):
    out = []
    t = toks
    for _ in range(n):
        lg, am = g.step(t)
        out.append((lg.copy(), am.copy()))
        t = am
    return out


@pytest.mark.parametrize("name,qtype", [("llama1b_b4_q8", Q8_0), ("llama1b_b4_q4", Q4_0)])
def test_batch_matches_single_sequence(name, qtype):
    """Each sequence of a four-sequence step against the one-sequence path on
    that sequence alone (own model handle with only that sequence's cache)."""
    import token_decode_llama_amd as lm
    cfg = synth.variant("multi_llama1b", n_layers=2, ctx=64, steps=3, batch=4, qtype=qtype)
    model = synth.make_model(cfg)
    toks = synth.start_tokens(cfg, 4)
    g = open_gpu(model, max_seqs=4)
    try:
        batched = _steps(g, toks, cfg.steps)
    finally:
        g.close()
    for s in range(4):
        gs = lm.open_model(model, lambda _s, l, s=s: synth.make_kv(cfg, s, l), max_seqs=1)
        try:
            t = toks[s:s + 1]
            for st in range(cfg.steps):
                lg, am = gs.step(t)
                ref = lg[0].astype(np.float64)
                got = batched[st][0][s].astype(np.float64)
                rel = float(np.max(np.abs(got - ref))) / float(np.max(np.abs(ref)))
                log(f"{name} seq {s} step {st}: batched vs single rel {rel:.2e}")
                assert rel <= LOGIT_RTOL, (s, st, rel)
                assert am[0] == batched[st][1][s], (s, st)
                t = batched[st][1][s:s + 1]
        finally:
            gs.close()


def test_batched_model_single_sequence_bit_identical():
    """A model created for four sequences, stepped with one, runs the
    one-sequence kernels on the same data: identical to a one-sequence model."""
    cfg = synth.variant("tiny", batch=1)
    model = synth.make_model(cfg)
    toks = synth.start_tokens(cfg, 1)
    g1 = open_gpu(model, max_seqs=1)
    g4 = open_gpu(model, max_seqs=4, kv_seqs=1)
    try:
        a = _steps(g1, toks, cfg.steps)
        b = _steps(g4, toks, cfg.steps)
        for (x, y), (u, v) in zip(a, b):
            assert np.array_equal(x, u) and np.array_equal(y, v)
    finally:
        g1.close()
        g4.close()


def test_batch_graph_replay_equals_eager():
    cfg = synth.variant("multi_smol360m", n_layers=2, ctx=70, steps=3, batch=3)
    model = synth.make_model(cfg)
    g = open_gpu(model, max_seqs=3)
    try:
        toks = synth.start_tokens(cfg, 3)
        runs = []
        for mode in (False, True, True, False, True):
            g.set_graph(mode)
            for s in range(3):
                g.set_position(s, cfg.ctx)
            runs.append(_steps(g, toks, 3))
        for other in runs[1:]:
            for (a, b), (c, d) in zip(runs[0], other):
                assert np.array_equal(a, c) and np.array_equal(b, d)
    finally:
        g.close()
