"""Self-speculative decoding (the C/CUDA Llama engine page, sections 3.5 and
5.3: draft with the bottom layers, verify with the full model) through the C
ABI.  The accepted tokens must be the oracle's greedy tokens, and the cache
rows below the final position must be the full model's (the verify pass is
k+1 plain steps over sequence 0's cache)."""
import numpy as np
import pytest

import synth
from synth import Q4_0
from tests.helpers import f16_close, log, open_gpu, open_oracle

pytestmark = pytest.mark.gpu

N_TOKENS = 10

SPEC_CASES = {
    "tiny_5layers_q8": synth.variant("tiny", n_layers=5, steps=N_TOKENS + 6, batch=4),
    "tiny_3layers_q4": synth.variant("tiny", n_layers=3, qtype=Q4_0, steps=N_TOKENS + 6, batch=4),
    "llama1b_2layers": synth.variant("multi_llama1b", n_layers=2, ctx=64, steps=N_TOKENS + 6, batch=4),
}
_models = {}


def _model(name):
    if name not in _models:
        _models[name] = synth.make_model(SPEC_CASES[name])
    return _models[name]


def _oracle_greedy(model, n):
    cfg = model.cfg
    om = open_oracle(model, 1)
    t = int(synth.start_tokens(cfg, 1)[0])
    out = []
    for _ in range(n):
        _, am = om.step([t])
        t = int(am[0])
        out.append(t)
    return out, om


@pytest.mark.parametrize("name,draft_layers,k", [
    ("tiny_5layers_q8", 2, 3), ("tiny_5layers_q8", 5, 3), ("tiny_5layers_q8", 0, 2),
    ("tiny_3layers_q4", 1, 3), ("llama1b_2layers", 1, 3), ("llama1b_2layers", 2, 1),
])
def test_speculative_rounds_equal_greedy(name, draft_layers, k):
    model = _model(name)
    cfg = model.cfg
    greedy, om = _oracle_greedy(model, N_TOKENS)
    g = open_gpu(model, max_seqs=4)
    try:
        t = int(synth.start_tokens(cfg, 1)[0])
        out, rounds = [], 0
        while len(out) < N_TOKENS:
            acc = g.speculative_step(t, draft_layers, k)
            assert 1 <= len(acc) <= k + 1
            if draft_layers == cfg.n_layers:         # drafts by the full model: all accepted
                assert len(acc) == k + 1
            out += acc.tolist()
            t = int(acc[-1])
            rounds += 1
        log(f"{name} draft {draft_layers} k {k}: {len(out)} tokens in {rounds} rounds")
        assert out[:N_TOKENS] == greedy
        pos = g.position(0)
        assert pos == cfg.ctx + len(out)
        # every cache row below the final position is the full model's
        n = min(pos, cfg.ctx + N_TOKENS)
        for l in range(cfg.n_layers):
            kg, vg = g.get_kv(0, l, n)
            ko, vo = om.get_kv(0, l, n)
            assert np.array_equal(kg[:, :cfg.ctx], ko[:, :cfg.ctx])
            assert f16_close(kg[:, cfg.ctx:n], ko[:, cfg.ctx:n]), (l, "K rows")
            assert f16_close(vg[:, cfg.ctx:n], vo[:, cfg.ctx:n]), (l, "V rows")
    finally:
        g.close()
        om.close()


def test_speculative_errors():
    import token_decode_llama_amd as lm
    model = _model("tiny_5layers_q8")
    cfg = model.cfg
    g = open_gpu(model, max_seqs=4)
    try:
        with pytest.raises(lm.LMError) as e:
            g.speculative_step(1, 2, 4)                     # k + 1 > max_seqs
        assert e.value.status == lm.LM_E_ARG
        with pytest.raises(lm.LMError) as e:
            g.speculative_step(1, cfg.n_layers + 1, 2)      # draft_layers out of range
        assert e.value.status == lm.LM_E_ARG
        g.set_position(0, cfg.max_ctx - 2)
        with pytest.raises(lm.LMError) as e:
            g.speculative_step(1, 2, 2)                     # p + k + 1 > max_ctx
        assert e.value.status == lm.LM_E_CTX
        g.set_position(0, cfg.ctx)
        g.stream_mode(True)
        with pytest.raises(lm.LMError) as e:
            g.speculative_step(1, 2, 2)
        assert e.value.status == lm.LM_E_STATE
    finally:
        g.close()
