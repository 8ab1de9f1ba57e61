"""GPU parity: the HIP decode step (through the C ABI) against the fp64 oracle
on identical seeded inputs.

Bars: dequantised weights bit-exact; argmax identical; per step and
sequence max|d logit| <= 1e-3 * max|logit|; appended fp16 K/V within one
fp16 ulp plus 2e-5 * max|K or V row| (the GPU rounds an fp32 value carrying
the fp32 GEMV's absolute error, the oracle an fp64 one).
Steps are teacher-forced with the oracle's token so one near-tie cannot
cascade; a mismatch reports the oracle's top-2 gap.
"""
import numpy as np
import pytest

import oracle
import synth
from synth import Q4_0, Q8_0
from tests.helpers import compare_step, f16_close, log, open_gpu, open_oracle

pytestmark = pytest.mark.gpu

CASES = {
    "tiny_q8": synth.CONFIGS["tiny"],
    "tiny_q4": synth.variant("tiny", qtype=Q4_0),
    # the multi-model shapes: ragged block counts (28, 30 blocks/row), GQA groups 7 and 3
    "qwen05b_2layers": synth.variant("multi_qwen05b", n_layers=2, ctx=130, steps=3),
    "smol360m_2layers": synth.variant("multi_smol360m", n_layers=2, ctx=70, steps=3),
    "llama1b_2layers": synth.variant("multi_llama1b", n_layers=2, ctx=64, steps=3),
    # the attention context crosses a 256-position chunk: one chunk, then a
    # second chunk holding a single key (wavefronts with no valid key)
    "llama1b_2layers_ctx255": synth.variant("multi_llama1b", n_layers=2, ctx=255, steps=3),
    # 8B layer shapes in Q4_0 with a long context (65 attention chunks)
    "llama8b_q4_2layers_ctx4k": synth.variant("llama8b_q8", n_layers=2, qtype=Q4_0, ctx=4090,
                                              steps=3, batch=1),
    # the 70B shape's layers (hidden 8192, ffn 28672, 64/8 heads) in Q4_0 at its context length
    "llama70b_q4_2layers": synth.variant("llama70b_q4", n_layers=2, steps=2),
    # 8B layer shapes in Q8_0; positions 127, 128, 129: the new key ends a
    # 64-position attention chunk, then is alone in a fresh chunk, then second
    "llama8b_q8_2layers_ctx127": synth.variant("llama8b_q8", n_layers=2, ctx=127, steps=3, batch=1),
    # five layers: resident prefixes of every length, both streaming buffers in turn
    "tiny_5layers": synth.variant("tiny", n_layers=5, steps=3),
    # an empty prefilled cache: the first token sits at position 0 and attends to itself only
    "tiny_ctx0": synth.variant("tiny", ctx=0, steps=3),
    # down projection of 48 blocks per row: 32-lane groups per row (every other
    # lane-group width, 8, 16 and 64, is in the shapes above), Q8_0 and Q4_0
    "tiny_ffn1536_q8": synth.variant("tiny", ffn=1536, steps=3),
    "tiny_ffn1536_q4": synth.variant("tiny", ffn=1536, qtype=Q4_0, steps=3),
    # down projection of 9216 columns on 256 rows: four-wavefront workgroups,
    # whose input batch holds 8192 columns, so its prologue takes two batches
    "tiny_ffn9216_q8": synth.variant("tiny", ffn=9216, steps=3),
    "tiny_ffn9216_q4": synth.variant("tiny", ffn=9216, qtype=Q4_0, steps=3),
}

_models = {}


def get_model(name):
    if name not in _models:
        log("generate", name)
        _models[name] = synth.make_model(CASES[name])
    return _models[name]


def run_parity(model, n_seq, steps=None, setup=None):
    """setup(g): puts the GPU model in the mode under test (residency) first."""
    cfg = model.cfg
    steps = steps or cfg.steps
    g = open_gpu(model, max_seqs=n_seq)
    if setup:
        setup(g)
    om = open_oracle(model, n_seq)
    toks = synth.start_tokens(cfg, n_seq)
    worst = 0.0
    try:
        for st in range(steps):
            p = cfg.ctx + st
            log(f"{cfg.name}: step {st} pos {p} n_seq {n_seq}")
            lg_o, am_o = om.step(toks)
            lg_g, am_g = g.step(toks)
            worst = max(worst, compare_step(lg_g, am_g, lg_o, am_o, f"{cfg.name} step {st}"))
            for s in range(n_seq):
                for l in range(cfg.n_layers):
                    kg, vg = g.get_kv(s, l, p + 1)
                    ko, vo = om.get_kv(s, l, p + 1)
                    c0 = cfg.ctx
                    assert np.array_equal(kg[:, :c0], ko[:, :c0]), "prefilled K rows changed"
                    assert np.array_equal(vg[:, :c0], vo[:, :c0]), "prefilled V rows changed"
                    # rows appended by this and earlier steps: fp16 of fp32 vs of fp64
                    assert f16_close(kg[:, c0:p + 1], ko[:, c0:p + 1]), (s, l, "K append")
                    assert f16_close(vg[:, c0:p + 1], vo[:, c0:p + 1]), (s, l, "V append")
            toks = am_o
            assert g.position(0) == p + 1
    finally:
        g.close()
        om.close()
    log(f"{cfg.name}: worst max|dlogit|/max|logit| = {worst:.3e}")
    return worst


@pytest.mark.parametrize("name", list(CASES))
def test_decode_parity(name):
    run_parity(get_model(name), n_seq=1)


@pytest.mark.parametrize("name,k", [("llama70b_q4_2layers", 0), ("llama70b_q4_2layers", 1),
                                    ("tiny_5layers", 0), ("tiny_5layers", 2)])
def test_decode_parity_streamed(name, k):
    """Layers k..L-1 streamed from pinned host memory through the two HBM layer
    buffers (k = 0: every layer; the engine page's double-buffered streaming and
    tier split), checked against the oracle itself, not only against resident
    runs."""
    run_parity(get_model(name), n_seq=1, setup=lambda g: g.set_residency(k))


def _steps(g, cfg, n):
    g.set_position(0, cfg.ctx)
    t = synth.start_tokens(cfg, 1)
    out = []
    for _ in range(n):
        lg, am = g.step(t)
        out.append((lg.copy(), am.copy()))
        t = am
    return out


@pytest.mark.parametrize("mode", [1, 2])
def test_kernel_timing_modes(mode):
    """Per-kernel timing, eager (1) or with events captured inside the step
    graph (2): the outputs are those of untimed steps, and every launch of the
    step is counted once per step."""
    model = get_model("llama1b_2layers")
    cfg = model.cfg
    g = open_gpu(model, max_seqs=1)
    try:
        ref = _steps(g, cfg, 3)
        g.kernel_timing(mode)
        got = _steps(g, cfg, 3)
        counts = {k: g.kernel_stats(k) for k in ("embed", "qkv", "attn", "wo", "gateup", "down", "lmhead")}
        g.kernel_timing(0)
        again = _steps(g, cfg, 3)
        for other in (got, again):
            for (a, b), (c, d) in zip(ref, other):
                assert np.array_equal(a, c) and np.array_equal(b, d)
        for k, (n, ms) in counts.items():
            per_step = 1 if k in ("embed", "lmhead") else cfg.n_layers
            assert n == 3 * per_step, (k, n)
            assert ms > 0.0, k
    finally:
        g.close()


def test_time_kind_graph_replay():
    """lm_time_kind: every family's launches replayed alone as a graph give a
    positive per-launch time, leave the position where it was, and the steps
    after it equal those before."""
    model = get_model("llama1b_2layers")
    cfg = model.cfg
    g = open_gpu(model, max_seqs=1)
    try:
        ref = _steps(g, cfg, 2)
        g.set_position(0, cfg.ctx)
        for k in ("embed", "qkv", "attn", "wo", "gateup", "down", "lmhead"):
            us = g.time_kind(k, 1, 3)
            assert us > 0.0, k
            assert g.position(0) == cfg.ctx, k
        again = _steps(g, cfg, 2)
        for (a, b), (c, d) in zip(ref, again):
            assert np.array_equal(a, c) and np.array_equal(b, d)
    finally:
        g.close()


@pytest.mark.parametrize("name,n_seq", [("tiny_q8", 3), ("tiny_q4", 4)])
def test_decode_parity_batch(name, n_seq):
    cfg = synth.variant(CASES[name].name, qtype=CASES[name].qtype, batch=n_seq)
    run_parity(synth.make_model(cfg), n_seq=n_seq)


def _bb(qt):
    return synth.BLOCK_BYTES[qt]


@pytest.mark.parametrize("name", ["tiny_q8", "tiny_q4", "qwen05b_2layers"])
def test_dequant_bit_exact_all_rows(name):
    model = get_model(name)
    cfg = model.cfg
    g = open_gpu(model, max_seqs=1)
    try:
        H, F, Q, KV = cfg.hidden, cfg.ffn, cfg.n_heads * cfg.head_dim, cfg.n_kv_heads * cfg.head_dim
        for l, w in enumerate(model.layers):
            for which, (arr, rows, cols) in enumerate([(w.wq, Q, H), (w.wk, KV, H), (w.wv, KV, H),
                                                       (w.wo, H, Q), (w.w_gate, F, H),
                                                       (w.w_up, F, H), (w.w_down, H, F)]):
                got = g.debug_dequant(l, which, 0, rows, cols)
                ref = oracle.dequant(cfg.qtype, arr, rows, cols)
                assert np.array_equal(got.astype(np.float64), ref), (l, which)
        got = g.debug_dequant(0, 7, 0, cfg.vocab, H)
        assert np.array_equal(got.astype(np.float64), oracle.dequant(cfg.qtype, model.lm_head, cfg.vocab, H))
    finally:
        g.close()


def test_graph_replay_equals_eager():
    model = get_model("llama1b_2layers")
    cfg = model.cfg
    g = open_gpu(model, max_seqs=1)
    try:
        toks = synth.start_tokens(cfg, 1)
        outs = {}
        for mode in (True, False, True):
            g.set_graph(mode)
            g.set_position(0, cfg.ctx)
            seq = []
            t = toks
            for _ in range(3):
                lg, am = g.step(t)
                seq.append((lg.copy(), am.copy()))
                t = am
            outs.setdefault(mode, []).append(seq)
        ref = outs[True][0]
        for runs in outs.values():
            for seq in runs:
                for (a, b), (c, d) in zip(seq, ref):
                    assert np.array_equal(a, c) and np.array_equal(b, d)
    finally:
        g.close()


@pytest.mark.parametrize("name", ["tiny_q8", "llama1b_2layers", "llama70b_q4_2layers"])
def test_stream_mode_bit_identical(name):
    model = get_model(name)
    cfg = model.cfg
    g = open_gpu(model, max_seqs=1)
    try:
        toks = synth.start_tokens(cfg, 1)

        def run():
            g.set_position(0, cfg.ctx)
            res = []
            t = toks
            for _ in range(cfg.steps):
                lg, am = g.step(t)
                res.append((lg.copy(), am.copy()))
                t = am
            return res

        resident = run()
        g.stream_mode(True)
        streamed = run()
        streamed2 = run()
        g.stream_mode(2)                       # serial: copy, then compute, per layer
        serial = run()
        g.stream_mode(True)
        streamed3 = run()
        g.stream_mode(False)
        back = run()
        for other in (streamed, streamed2, serial, streamed3, back):
            for (a, b), (c, d) in zip(resident, other):
                assert np.array_equal(a, c) and np.array_equal(b, d)
    finally:
        g.close()


@pytest.mark.parametrize("name,plan", [("tiny_5layers", [3, 1, 0, 4, 2, 5]),
                                       ("llama70b_q4_2layers", [1, 0, 1, 2])])
def test_hybrid_residency_bit_identical(name, plan):
    """The first k layers resident and the rest streamed: every k gives the
    fully resident outputs bit for bit, through any sequence of moves."""
    model = get_model(name)
    cfg = model.cfg
    g = open_gpu(model, max_seqs=1)
    try:
        toks = synth.start_tokens(cfg, 1)

        def run():
            g.set_position(0, cfg.ctx)
            res = []
            t = toks
            for _ in range(cfg.steps):
                lg, am = g.step(t)
                res.append((lg.copy(), am.copy()))
                t = am
            return res

        resident = run()
        for k in plan:
            log(f"{name}: {k} of {cfg.n_layers} layers resident")
            g.set_residency(k)
            for _ in range(2):       # twice: the second starts from the previous step's prefetch
                for (a, b), (c, d) in zip(resident, run()):
                    assert np.array_equal(a, c) and np.array_equal(b, d), k
        import token_decode_llama_amd as lm
        with pytest.raises(lm.LMError):
            g.set_residency(cfg.n_layers + 1)
        assert g.plan_residency(hbm_bytes=1, host_bytes=1 << 40) == 0
        assert g.plan_residency(hbm_bytes=1 << 50, host_bytes=1) == cfg.n_layers
        assert g.plan_residency() == cfg.n_layers      # a small model fits the device
    finally:
        g.close()


@pytest.mark.parametrize("name", ["llama1b_2layers", "llama8b_q8_2layers_ctx127"])
def test_long_cache_short_context_bit_identical(name):
    """A cache far longer than the context: the attention grid follows the
    context (64-position chunks up to the next power of two), so the outputs
    equal those of a model whose cache ends at the context, bit for bit."""
    import token_decode_llama_amd as lm
    model = get_model(name)
    cfg = model.cfg
    toks = synth.start_tokens(cfg, 1)
    outs = []
    for max_ctx in (cfg.max_ctx, 8192):
        g = lm.open_model(model, lambda s, l: synth.make_kv(cfg, s, l), max_seqs=1, max_ctx=max_ctx)
        try:
            res, t = [], toks
            for _ in range(cfg.steps):
                lg, am = g.step(t)
                res.append((lg.copy(), am.copy()))
                t = am
            outs.append(res)
        finally:
            g.close()
    for (a, b), (c, d) in zip(*outs):
        assert np.array_equal(a, c) and np.array_equal(b, d)


@pytest.mark.parametrize("name,n_seq,mask", [("tiny_5layers", 1, [0, 1, 0, 1, 0]),
                                              ("tiny_5layers", 1, [1, 1, 1, 1, 1]),
                                              ("llama1b_2layers", 1, [0, 1])])
def test_layer_skip_parity(name, n_seq, mask):
    """Skipped layers (the engine page's layer skip) against the oracle with the
    same mask: logits, argmax, appended rows of computed layers; a skipped
    layer's cache rows stay as they were."""
    model = get_model(name)
    cfg = model.cfg
    g = open_gpu(model, max_seqs=n_seq)
    om = open_oracle(model, n_seq)
    skip = np.array(mask, np.uint8)
    g.set_layer_skip(skip)
    toks = synth.start_tokens(cfg, n_seq)
    try:
        for st in range(cfg.steps):
            p = cfg.ctx + st
            lg_o, am_o = om.step(toks, skip=skip)
            lg_g, am_g = g.step(toks)
            compare_step(lg_g, am_g, lg_o, am_o, f"{name} skip {mask} step {st}")
            for s in range(n_seq):
                for l in range(cfg.n_layers):
                    kg, vg = g.get_kv(s, l, p + 1)
                    ko, vo = om.get_kv(s, l, p + 1)
                    if skip[l]:
                        assert np.array_equal(kg[:, cfg.ctx:], np.zeros_like(kg[:, cfg.ctx:])), (l, "skipped K row")
                    else:
                        assert f16_close(kg[:, cfg.ctx:p + 1], ko[:, cfg.ctx:p + 1]), (s, l, "K append")
                        assert f16_close(vg[:, cfg.ctx:p + 1], vo[:, cfg.ctx:p + 1]), (s, l, "V append")
            toks = am_o
    finally:
        g.close()
        om.close()


@pytest.mark.parametrize("name", ["tiny_5layers", "llama70b_q4_2layers"])
def test_layer_skip_streaming_bit_identical(name):
    """Skipped layers are not copied in streaming mode; every residency gives the
    resident outputs bit for bit with the same mask."""
    model = get_model(name)
    cfg = model.cfg
    mask = np.zeros(cfg.n_layers, np.uint8)
    mask[1] = 1
    if cfg.n_layers >= 5:
        mask[3] = 1
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

        g.set_layer_skip(mask)
        resident = run()
        for k in (0, 1, cfg.n_layers - 1):
            g.set_residency(k)
            for _ in range(2):
                for (a, b), (c, d) in zip(resident, run()):
                    assert np.array_equal(a, c) and np.array_equal(b, d), k
        g.set_residency(cfg.n_layers)
        g.set_layer_skip(None)
        full = run()
        g.set_layer_skip(mask)
        again = run()
        for (a, b), (c, d) in zip(resident, again):
            assert np.array_equal(a, c) and np.array_equal(b, d)
        assert not all(np.array_equal(a, c) for (a, _), (c, _) in zip(resident, full))
    finally:
        g.close()


@pytest.mark.parametrize("name,n_seq", [("tiny_5layers", 1), ("tiny_q4", 1)])
def test_layer_similarity_and_calibrated_skip(name, n_seq):
    """Recorded per-layer input/output cosine similarities against the oracle's,
    and the calibrated list (mean above the threshold) equal to the oracle's."""
    import oracle
    model = get_model(name)
    cfg = model.cfg
    g = open_gpu(model, max_seqs=n_seq)
    om = open_oracle(model, n_seq)
    toks = synth.start_tokens(cfg, n_seq)
    try:
        g.layer_similarity(True)
        sums = np.zeros(cfg.n_layers)
        for st in range(cfg.steps):
            lg_o, am_o, cos = om.step(toks, with_cos=True)
            g.step(toks)
            sums += cos.sum(axis=0)
            toks = am_o
        g.layer_similarity(False)
        mean, cnt = g.get_layer_similarity()
        ref = sums / (cfg.steps * n_seq)
        assert np.all(cnt == cfg.steps * n_seq)
        assert np.allclose(mean, ref, rtol=0, atol=2e-6), (mean, ref)
        # a threshold between two recorded means: the same list on both sides
        srt = np.sort(ref)
        thr = float((srt[len(srt) // 2 - 1] + srt[len(srt) // 2]) / 2) if len(srt) > 1 else float(srt[0] - 1e-3)
        n = g.skip_similar_layers(thr)
        expect = oracle.skip_list(ref, thr)
        assert n == int(expect.sum())
        # the model now skips exactly those layers: compare a step with the oracle's
        toks = synth.start_tokens(cfg, n_seq)
        for s in range(n_seq):
            om.set_position(s, cfg.ctx)
            g.set_position(s, cfg.ctx)
        lg_o, am_o = om.step(toks, skip=expect)
        lg_g, am_g = g.step(toks)
        compare_step(lg_g, am_g, lg_o, am_o, f"{name} calibrated skip")
    finally:
        g.close()
        om.close()


def test_state_and_context_errors():
    import token_decode_llama_amd as lm
    cfg = CASES["tiny_q8"]
    model = get_model("tiny_q8")
    m = lm.Model(cfg, max_seqs=1)
    try:
        with pytest.raises(lm.LMError) as e:
            m.step([1])
        assert e.value.status == lm.LM_E_STATE
        m.load_model(model)
        for l in range(cfg.n_layers):
            k, v = synth.make_kv(cfg, 0, l)
            m.load_kv(0, l, k, v)
        with pytest.raises(lm.LMError) as e:
            m.step([cfg.vocab])
        assert e.value.status == lm.LM_E_ARG
        with pytest.raises(lm.LMError) as e:
            m.step([1, 2])
        assert e.value.status == lm.LM_E_ARG
        with pytest.raises(lm.LMError) as e:      # an empty batch
            m.step([])
        assert e.value.status == lm.LM_E_ARG
        first = m.step([5])
        for _ in range(cfg.steps - 1):
            m.step([5])
        assert m.position(0) == cfg.max_ctx
        with pytest.raises(lm.LMError) as e:
            m.step([5])
        assert e.value.status == lm.LM_E_CTX and "max_ctx" in str(e.value)
        m.set_position(0, cfg.ctx)
        again = m.step([5])
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])
        with pytest.raises(lm.LMError) as e:
            m.set_position(0, cfg.max_ctx + 1)
        assert e.value.status == lm.LM_E_ARG
    finally:
        m.close()


@pytest.mark.slow
def test_llama8b_q8_full_size_parity():
    """The full 8B-shape Q8_0 model at context 512, the launch configuration
    the benchmark times: two teacher-forced steps against the oracle, plus
    sampled rows of every matrix dequantised bit-exactly."""
    cfg = synth.CONFIGS["llama8b_q8"]
    log("generate llama8b_q8 (~8 GB)")
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
                    ref = oracle.dequant(cfg.qtype, arr[r:r + 1], 1, cols)
                    assert np.array_equal(got.astype(np.float64), ref), (l, which, r)
        for r in (0, cfg.vocab - 1, 77777):
            got = g.debug_dequant(0, 7, r, 1, H)
            assert np.array_equal(got.astype(np.float64), oracle.dequant(cfg.qtype, model.lm_head[r:r + 1], 1, H))
    finally:
        g.close()
