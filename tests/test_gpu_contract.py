"""GPU checks of what the parity steps do not reach on their own:

* the argmax rule on exact ties (lowest index wins) across the LM head's
  workgroups, on the one-sequence and the matrix-core paths;
* the GEMV's integer-digit activations on inputs whose 32-column blocks each
  hold one outlier channel 10^3 times the rest, against the oracle's GEMV
  within a bound derived from the digit rounding;
* the all-or-nothing contract of lm_model_create and lm_set_residency under
  injected allocation failures: the error is LM_E_OOM, device memory is
  what it was, and the model decodes as before.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.helpers import compare_step, log, open_gpu, open_oracle

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# argmax ties
# ---------------------------------------------------------------------------
def _tied_model(cfg, tok):
    """The model with the LM-head row of the oracle's argmax r (for sequence 0's
    first step) copied into rows in other workgroups, one of them the last row,
    one below r when r > 0: the largest logit is then reached exactly at every
    copy, and the lowest index must win.  Returns (model, the copies' rows)."""
    model = synth.make_model(cfg)
    om = open_oracle(model, 1)
    try:
        _, am = om.step(tok[:1])
    finally:
        om.close()
    r = int(am[0])
    V = cfg.vocab
    rows = {V - 1, (r + 3 * 64) % V, r ^ 1}
    if r > 0:
        rows.add(r // 2)
    rows.discard(r)
    for i in rows:
        model.lm_head[i] = model.lm_head[r]
    return model, sorted(rows | {r}), r


@pytest.mark.parametrize("n_seq", [1, 4])
def test_argmax_exact_ties_take_the_lowest_index(n_seq):
    cfg = synth.variant("tiny", batch=n_seq, steps=2)
    tok = synth.start_tokens(cfg, n_seq)
    model, tied, r = _tied_model(cfg, tok)
    log(f"argmax row {r}; identical LM-head rows {tied}")
    g = open_gpu(model, max_seqs=n_seq)
    om = open_oracle(model, n_seq)
    try:
        lg_o, am_o = om.step(tok)
        lg_g, am_g = g.step(tok)
        ref = lg_o[0].astype(np.float32)
        assert all(ref[i] == ref[r] for i in tied), "the copies must tie exactly in fp32"
        assert int(am_o[0]) == min(tied)
        assert all(lg_g[0][i] == lg_g[0][r] for i in tied), "identical rows must give identical GPU logits"
        compare_step(lg_g, am_g, lg_o, am_o, f"ties n_seq {n_seq}")
        assert int(am_g[0]) == min(tied)
    finally:
        g.close()
        om.close()


def test_argmax_all_rows_tied():
    """Every LM-head row identical: every logit ties and row 0 wins."""
    cfg = synth.variant("tiny", steps=1)
    model = synth.make_model(cfg)
    model.lm_head[:] = model.lm_head[7]
    tok = synth.start_tokens(cfg, 1)
    g = open_gpu(model, max_seqs=1)
    try:
        lg, am = g.step(tok)
        assert np.all(lg[0] == lg[0][0])
        assert int(am[0]) == 0
    finally:
        g.close()


# ---------------------------------------------------------------------------
# GEMV with one outlier channel per block
# ---------------------------------------------------------------------------
# The GEMV feeds each 32-column block b of the input to the integer dot
# products as X_i = rint(x_i / s_b), s_b = max|x_b| / (127 * 2^16), so each
# input carries an absolute error of at most s_b / 2.  For row r with block
# scales d_rb and quants q_ri:
#   |y_gpu - y| <= sum_b |d_rb| (s_b / 2) sum_{i in b} |q_ri|      (digits)
#                + 2^-22 (nb + 16) sum_i |w_ri| |x_i|              (fp32 sums)
# The second term is four times the unit roundoff per term of a summation
# nb + 16 deep (blocks per row plus the cross-lane and cross-wavefront
# reduction levels), a deliberately loose bound on fp32 accumulation.
OUTLIER = 1e3


def _outlier_input(K, n_seq, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n_seq, K))
    for s in range(n_seq):
        for b in range(K // 32):
            x[s, 32 * b + rng.integers(32)] = OUTLIER * rng.choice([-1.0, 1.0])
    return x.astype(np.float32)


def _matrix(model, layer, which):
    cfg = model.cfg
    if which == 4:
        return model.lm_head, cfg.vocab, cfg.hidden
    w = model.layers[layer]
    if which == 0:
        m = np.concatenate([w.wq, w.wk, w.wv])
        return m, m.shape[0], cfg.hidden
    if which == 1:
        return w.wo, cfg.hidden, cfg.n_heads * cfg.head_dim
    if which == 2:
        m = np.empty((2 * cfg.ffn, w.w_gate.shape[1]), np.uint8)
        m[0::2] = w.w_gate
        m[1::2] = w.w_up
        return m, 2 * cfg.ffn, cfg.hidden
    return w.w_down, cfg.hidden, cfg.ffn


def _bound(qt, blocks, rows, K, x):
    """Per-row error bound above.  w_i = d_rb q_i exactly (Q8_0: q the int8;
    Q4_0: q = nibble - 8, the 8 removed through exact digit sums), so
    |d_rb| sum_{i in b} |q_ri| = sum_{i in b} |w_ri|."""
    absw = np.abs(oracle.dequant(qt, blocks, rows, K))            # [rows, K], exact
    x64 = x.astype(np.float64)
    nb = K // 32
    s = np.abs(x64.reshape(nb, 32)).max(axis=1) / (127 * 65536.0)
    e_dig = absw @ np.repeat(s / 2, 32)
    e_fp = 2.0 ** -22 * (nb + 16) * (absw @ np.abs(x64))
    return e_dig + e_fp


_gemv_models = {}


def _gemv_model(name):
    if name not in _gemv_models:
        cfgs = {"tiny_q8": synth.CONFIGS["tiny"],
                "tiny_q4": synth.variant("tiny", qtype=synth.Q4_0),
                "llama8b_q8_1layer": synth.variant("llama8b_q8", n_layers=1, ctx=16, steps=1),
                "llama8b_q4_1layer": synth.variant("llama8b_q8", n_layers=1, qtype=synth.Q4_0, ctx=16, steps=1)}
        log("generate", name)
        _gemv_models[name] = synth.make_model(cfgs[name])
    return _gemv_models[name]


@pytest.mark.parametrize("name", ["tiny_q8", "tiny_q4", "llama8b_q8_1layer", "llama8b_q4_1layer"])
@pytest.mark.parametrize("n_seq", [1, 4])
def test_gemv_outlier_channels_within_digit_bound(name, n_seq):
    import token_decode_llama_amd as lm
    model = _gemv_model(name)
    cfg = model.cfg
    qt = cfg.qtype
    g = lm.Model(cfg, max_seqs=n_seq)
    try:
        g.load_model(model)
        for which in range(5):
            blocks, rows, K = _matrix(model, 0, which)
            x = _outlier_input(K, n_seq, seed=which)
            y = g.debug_gemv(0, which, x)
            worst = 0.0
            for s in range(n_seq):
                ref = oracle.gemv(qt, blocks, rows, K, x[s].astype(np.float64))
                bound = _bound(qt, blocks, rows, K, x[s])
                err = np.abs(y[s].astype(np.float64) - ref)
                bad = np.nonzero(err > bound)[0]
                assert bad.size == 0, (f"{name} which {which} seq {s}: row {bad[0]} error {err[bad[0]]:.3e} "
                                       f"> bound {bound[bad[0]]:.3e}")
                worst = max(worst, float(np.max(err / bound)))
            log(f"{name} n_seq {n_seq} which {which}: worst error / bound = {worst:.3f}")
    finally:
        g.close()


# ---------------------------------------------------------------------------
# all-or-nothing under allocation failures
# ---------------------------------------------------------------------------
def _free_device_bytes():
    import torch
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


@pytest.mark.parametrize("n_seq", [1, 4])
def test_create_failure_at_every_allocation_leaks_nothing(n_seq):
    import token_decode_llama_amd as lm
    cfg = synth.CONFIGS["tiny"]
    lm.Model(cfg, max_seqs=n_seq).close()               # the runtime's own first-use allocations
    c0 = lm.alloc_count()
    lm.Model(cfg, max_seqs=n_seq).close()
    n_alloc = lm.alloc_count() - c0
    assert n_alloc >= 20
    try:
        for n in range(1, n_alloc + 1):
            free0 = _free_device_bytes()
            lm.fail_alloc(n)
            with pytest.raises(lm.LMError) as e:
                lm.Model(cfg, max_seqs=n_seq)
            assert e.value.status == lm.LM_E_OOM, (n, str(e.value))
            assert "injected" in str(e.value), (n, str(e.value))
            assert _free_device_bytes() == free0, f"allocation {n} of {n_alloc}: device memory changed"
    finally:
        lm.fail_alloc(0)
    g = lm.Model(cfg, max_seqs=n_seq)                    # and creation works again
    g.close()


def test_residency_move_failure_leaves_the_model_as_it_was():
    import token_decode_llama_amd as lm
    cfg = synth.variant("tiny", n_layers=5, steps=3)
    model = synth.make_model(cfg)
    g = open_gpu(model, max_seqs=1)
    tok = synth.start_tokens(cfg, 1)

    def run():
        g.set_position(0, cfg.ctx)
        out, t = [], tok
        for _ in range(cfg.steps):
            lg, am = g.step(t)
            out.append((lg.copy(), am.copy()))
            t = am
        return out

    try:
        ref = run()
        for start, target in ((5, 0), (5, 2), (2, 0), (0, 5), (2, 4), (0, 3)):
            g.set_residency(start)
            # fail the move's first, second, ... allocation until one attempt makes
            # fewer allocations than that (it then succeeds)
            for n in range(1, 16):
                free0 = _free_device_bytes()
                c0 = lm.alloc_count()
                lm.fail_alloc(n)
                try:
                    g.set_residency(target)
                    moved = True
                except lm.LMError as e:
                    moved = False
                    assert e.status == lm.LM_E_OOM, (start, target, n, str(e))
                lm.fail_alloc(0)
                if moved:
                    assert lm.alloc_count() - c0 < n, (start, target, n)
                    log(f"residency {start} -> {target}: {n - 1} allocations, each failure rolled back")
                    break
                assert _free_device_bytes() == free0, (start, target, n)
                for (a, b), (c, d) in zip(ref, run()):
                    assert np.array_equal(a, c) and np.array_equal(b, d), (start, target, n)
            assert moved, (start, target)
            for (a, b), (c, d) in zip(ref, run()):
                assert np.array_equal(a, c) and np.array_equal(b, d), (start, target)
    finally:
        lm.fail_alloc(0)
        g.close()
