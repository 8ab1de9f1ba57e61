"""Whole-step pins of the fp64 oracle and determinism pins of the generator.

* special case: with W_o = W_down = 0 the residual stream stays E[tok], so
  logits = W_lm * rmsnorm(E[tok]) * g_out in closed form;
* composition: the oracle's step against Hugging Face transformers'
  LlamaForCausalLM run in fp64 on the same dequantised weights and the same
  prefilled cache (an independent implementation of the architecture; its
  rotate-half RoPE is matched by the standard per-head row permutation of
  W_q / W_k, and it keeps the new token's k/v in fp64 where the oracle rounds
  them to fp16, hence the 1e-4 relative bound instead of exact agreement);
* generator: Philox4x32-10 known-answer vectors and identical bytes for any
  thread count.
"""
import hashlib
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import oracle
import synth
from synth import Q4_0, Q4_K, Q5_K, Q6_K, Q8_0
from tests.test_oracle_pins import _numpy_dequant

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load_oracle(model, n_seq=1, ctx=None):
    cfg = model.cfg
    om = oracle.OracleModel(model, max_seqs=n_seq)
    for s in range(n_seq):
        for l in range(cfg.n_layers):
            k, v = synth.make_kv(cfg, s, l, ctx)
            om.load_kv(s, l, k, v)
    return om


def test_zero_wo_wdown_closed_form():
    cfg = synth.variant("tiny", qtype=Q8_0)
    model = synth.make_model(cfg)
    for w in model.layers:
        w.wo[:] = 0
        w.w_down[:] = 0
    om = _load_oracle(model)
    tok = int(synth.start_tokens(cfg)[0])
    logits, am = om.step([tok])
    e = model.tok_embd[tok].view(np.float16).astype(np.float64)
    xf = torch.nn.functional.rms_norm(torch.from_numpy(e), (cfg.hidden,),
                                      weight=torch.from_numpy(model.out_norm.astype(np.float64)),
                                      eps=cfg.rms_eps).numpy()
    W = _numpy_dequant(cfg.qtype, model.lm_head, cfg.vocab, cfg.hidden)
    expect = W @ xf
    assert np.allclose(logits[0], expect, rtol=1e-12, atol=1e-14)
    assert am[0] == int(np.argmax(expect.astype(np.float32)))


def _hf_model(model):
    from transformers import LlamaConfig, LlamaForCausalLM
    cfg = model.cfg
    hc = LlamaConfig(vocab_size=cfg.vocab, hidden_size=cfg.hidden, intermediate_size=cfg.ffn,
                     num_hidden_layers=cfg.n_layers, num_attention_heads=cfg.n_heads,
                     num_key_value_heads=cfg.n_kv_heads, head_dim=cfg.head_dim,
                     rms_norm_eps=cfg.rms_eps, rope_theta=cfg.rope_theta,
                     tie_word_embeddings=False, attention_bias=False, mlp_bias=False,
                     max_position_embeddings=8192)
    hc._attn_implementation = "eager"
    hf = LlamaForCausalLM(hc).double().eval()
    hd = cfg.head_dim
    # adjacent pairs (2i, 2i+1) <-> rotate-half pairs (i, i + hd/2)
    perm = np.concatenate([np.arange(0, hd, 2), np.arange(1, hd, 2)])

    def rows_perm(W, n_heads):
        return W.reshape(n_heads, hd, -1)[:, perm, :].reshape(n_heads * hd, -1)

    def T(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))

    H, F = cfg.hidden, cfg.ffn
    qt = cfg.qtype
    with torch.no_grad():
        hf.model.embed_tokens.weight.copy_(T(model.tok_embd.view(np.float16)))
        hf.model.norm.weight.copy_(T(model.out_norm))
        hf.lm_head.weight.copy_(T(_numpy_dequant(qt, model.lm_head, cfg.vocab, H)))
        for l, w in enumerate(model.layers):
            L = hf.model.layers[l]
            L.input_layernorm.weight.copy_(T(w.attn_norm))
            L.post_attention_layernorm.weight.copy_(T(w.ffn_norm))
            L.self_attn.q_proj.weight.copy_(T(rows_perm(_numpy_dequant(qt, w.wq, cfg.n_heads * hd, H), cfg.n_heads)))
            L.self_attn.k_proj.weight.copy_(T(rows_perm(_numpy_dequant(qt, w.wk, cfg.n_kv_heads * hd, H), cfg.n_kv_heads)))
            L.self_attn.v_proj.weight.copy_(T(_numpy_dequant(qt, w.wv, cfg.n_kv_heads * hd, H)))
            L.self_attn.o_proj.weight.copy_(T(_numpy_dequant(qt, w.wo, H, cfg.n_heads * hd)))
            L.mlp.gate_proj.weight.copy_(T(_numpy_dequant(qt, w.w_gate, F, H)))
            L.mlp.up_proj.weight.copy_(T(_numpy_dequant(qt, w.w_up, F, H)))
            L.mlp.down_proj.weight.copy_(T(_numpy_dequant(qt, w.w_down, H, F)))
    return hf, perm, hc


# the K formats' 256-weight super-blocks need every input width a multiple of 256
@pytest.mark.parametrize("name,qtype,ffn", [("tiny", Q8_0, 704), ("tiny", Q4_0, 704),
                                            ("tiny", Q4_K, 768), ("tiny", Q5_K, 768), ("tiny", Q6_K, 768)])
def test_oracle_matches_transformers_llama(name, qtype, ffn):
    from transformers.cache_utils import DynamicCache
    cfg = synth.variant(name, qtype=qtype, ffn=ffn)
    model = synth.make_model(cfg)
    om = _load_oracle(model)
    hf, perm, hc = _hf_model(model)
    cache = DynamicCache(config=hc)
    for l in range(cfg.n_layers):
        k, v = synth.make_kv(cfg, 0, l)
        kf = k.view(np.float16).astype(np.float64)[:, :, perm]
        vf = v.view(np.float16).astype(np.float64)
        cache.update(torch.from_numpy(kf[None].copy()), torch.from_numpy(vf[None].copy()), l)
    tok = int(synth.start_tokens(cfg)[0])
    for step in range(cfg.steps):
        p = cfg.ctx + step
        logits, am = om.step([tok])
        with torch.no_grad():
            out = hf(input_ids=torch.tensor([[tok]]), position_ids=torch.tensor([[p]]),
                     cache_position=torch.tensor([p]), past_key_values=cache, use_cache=True)
        ref = out.logits[0, -1].numpy()
        err = np.max(np.abs(logits[0] - ref))
        assert err <= 1e-4 * np.max(np.abs(ref)), (step, err)
        # the token the oracle appended at p equals the library's k (fp16-rounded, <= 1 ulp)
        for l in range(cfg.n_layers):
            ko, vo = om.get_kv(0, l, p + 1)
            kh = cache.layers[l].keys[0, :, p, :].numpy()[:, np.argsort(perm)]
            vh = cache.layers[l].values[0, :, p, :].numpy()
            for got, want in ((ko[:, p], kh), (vo[:, p], vh)):
                g = got.view(np.float16).astype(np.float64)
                if l == 0:
                    # same inputs on both sides: fp16 rounding is the only difference
                    ulp = np.abs(np.spacing(want.astype(np.float16)).astype(np.float64))
                    assert np.all(np.abs(g - want) <= ulp), (step, l)
                else:
                    # deeper layers also carry layer 0's fp16-vs-fp64 new-token difference
                    assert np.max(np.abs(g - want)) <= 2e-3 * np.max(np.abs(want)), (step, l)
        tok = int(am[0])


def test_oracle_positions_and_context_limit():
    cfg = synth.variant("tiny", steps=2)
    model = synth.make_model(cfg)
    om = _load_oracle(model)
    assert om.position(0) == cfg.ctx
    om.step([1])
    om.step([2])
    assert om.position(0) == cfg.ctx + 2
    with pytest.raises(ValueError):
        om.step([3])                      # max_ctx = ctx + steps reached
    om.set_position(0, cfg.ctx)
    om.step([1])


def test_oracle_step_is_repeatable_after_rewind():
    cfg = synth.CONFIGS["tiny"]
    model = synth.make_model(cfg)
    om = _load_oracle(model)
    a, _ = om.step([7])
    om.set_position(0, cfg.ctx)
    b, _ = om.step([7])
    assert np.array_equal(a, b)


def test_batch_sequences_are_independent():
    cfg = synth.variant("tiny", batch=2)
    model = synth.make_model(cfg)
    om2 = _load_oracle(model, n_seq=2)
    lg2, am2 = om2.step([11, 300])
    for s, t in ((0, 11), (1, 300)):
        om1 = oracle.OracleModel(model, max_seqs=1)
        for l in range(cfg.n_layers):
            k, v = synth.make_kv(cfg, s, l)
            om1.load_kv(0, l, k, v)
        lg1, am1 = om1.step([t])
        assert np.array_equal(lg1[0], lg2[s]) and am1[0] == am2[s]


# ---------------------------------------------------------------------------
# generator
# ---------------------------------------------------------------------------

def test_philox_known_answer_vectors():
    # known-answer vectors published with Philox4x32-10 (Salmon et al., SC'11)
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, out in kat:
        assert list(synth.philox4x32_10(ctr, key)) == out


_DIGEST_SNIPPET = r"""
import hashlib, sys
sys.path.insert(0, {root!r})
import synth
h = hashlib.sha256()
h.update(synth.quant_matrix(1, 77, 96, 512, 0.02, 8).tobytes())
h.update(synth.quant_matrix(1, 78, 40, 256, 0.02, 2).tobytes())
h.update(synth.normal_f16_bits(1, 79, 10001, 0.0, 1.0).tobytes())
h.update(synth.normal_f32(1, 80, 999, 1.0, 0.1).tobytes())
print(h.hexdigest())
"""


def test_generator_bytes_independent_of_thread_count():
    code = _DIGEST_SNIPPET.format(root=ROOT)
    digests = []
    for n in ("1", "3", "8"):
        env = dict(os.environ, OMP_NUM_THREADS=n)
        digests.append(subprocess.check_output([sys.executable, "-c", code], env=env).strip())
    assert len(set(digests)) == 1


def test_generator_distributions():
    w = synth.normal_f32(9, 1, 200000, 0.0, 1.0).astype(np.float64)
    assert abs(w.mean()) < 0.01 and abs(w.std() - 1.0) < 0.01
    g = synth.normal_f32(9, 2, 100000, 1.0, 0.1).astype(np.float64)
    assert abs(g.mean() - 1.0) < 0.002 and abs(g.std() - 0.1) < 0.002
    t = synth.uniform_int(9, 3, 50000, 512)
    assert t.min() >= 0 and t.max() < 512 and abs(t.mean() - 255.5) < 5
    cfg = synth.CONFIGS["tiny"]
    blocks = synth.quant_matrix(0, 5, 64, 256, 0.02, Q8_0)
    W = _numpy_dequant(Q8_0, blocks, 64, 256)
    assert abs(W.std() - 0.02) < 0.001
    assert cfg.max_ctx == 20


# ---------------------------------------------------------------------------
# layer skip (the C/CUDA Llama engine page, sections 2.5, 3.5 and 4.5)
# ---------------------------------------------------------------------------

def test_oracle_cosine_properties():
    rng = np.random.default_rng(7)
    a = rng.standard_normal(97)
    b = rng.standard_normal(97)
    assert oracle.cosine(a, a) == pytest.approx(1.0, abs=1e-15)
    assert oracle.cosine(a, -a) == pytest.approx(-1.0, abs=1e-15)
    assert oracle.cosine(a, 3.0 * a) == pytest.approx(1.0, abs=1e-15)          # scale invariance
    assert oracle.cosine(a, b) == pytest.approx(oracle.cosine(b, a), abs=0)       # symmetry
    assert abs(oracle.cosine(a, b)) <= 1.0                                       # Cauchy-Schwarz
    assert oracle.cosine([1.0, 0.0], [0.0, 2.0]) == 0.0                          # orthogonal
    assert oracle.cosine([1.0, 0.0], [1.0, 3.0 ** 0.5]) == pytest.approx(0.5, abs=1e-15)   # 60 degrees
    assert oracle.cosine([0.0, 0.0], [1.0, 2.0]) == 0.0                          # zero vector: 0


def test_oracle_skip_list_is_strictly_above():
    mask = oracle.skip_list([0.5, 0.98, 0.99, 0.981, float("nan")], 0.98)
    assert mask.tolist() == [0, 0, 1, 1, 0]


def test_skip_all_layers_closed_form():
    """Every layer skipped: the residual stream stays E[tok], so the logits are
    W_lm * rmsnorm(E[tok]) * g_out (the same closed form as zero W_o, W_down)."""
    cfg = synth.variant("tiny", qtype=Q4_0)
    model = synth.make_model(cfg)
    om = _load_oracle(model)
    tok = int(synth.start_tokens(cfg)[0])
    logits, am, cos = om.step([tok], skip=np.ones(cfg.n_layers, np.uint8), with_cos=True)
    e = model.tok_embd[tok].view(np.float16).astype(np.float64)
    xf = torch.nn.functional.rms_norm(torch.from_numpy(e), (cfg.hidden,),
                                      weight=torch.from_numpy(model.out_norm.astype(np.float64)),
                                      eps=cfg.rms_eps).numpy()
    expect = _numpy_dequant(cfg.qtype, model.lm_head, cfg.vocab, cfg.hidden) @ xf
    assert np.allclose(logits[0], expect, rtol=1e-12, atol=1e-14)
    assert np.all(cos == 0.0)
    # no cache row written by a skipped layer
    k, v = om.get_kv(0, 0, cfg.ctx + 1)
    assert np.all(k[:, cfg.ctx] == 0) and np.all(v[:, cfg.ctx] == 0)


def test_skip_equals_model_without_that_layer():
    """Skipping layer 1 of three is the two-layer model made of layers 0 and 2
    (with their caches), exactly; each computed layer's similarity is the same
    number in both."""
    cfg3 = synth.variant("tiny", n_layers=3)
    m3 = synth.make_model(cfg3)
    cfg2 = synth.variant("tiny", n_layers=2)
    m2 = synth.Model(cfg=cfg2, tok_embd=m3.tok_embd, out_norm=m3.out_norm, lm_head=m3.lm_head,
                     layers=[m3.layers[0], m3.layers[2]])
    o3 = oracle.OracleModel(m3, max_seqs=2)
    o2 = oracle.OracleModel(m2, max_seqs=2)
    for s in range(2):
        for l in range(3):
            o3.load_kv(s, l, *synth.make_kv(cfg3, s, l))
        o2.load_kv(s, 0, *synth.make_kv(cfg3, s, 0))
        o2.load_kv(s, 1, *synth.make_kv(cfg3, s, 2))
    toks = synth.start_tokens(cfg3, 2)
    skip = np.array([0, 1, 0], np.uint8)
    for _ in range(3):
        l3, a3, c3 = o3.step(toks, skip=skip, with_cos=True)
        l2, a2, c2 = o2.step(toks, with_cos=True)
        assert np.array_equal(l3, l2) and np.array_equal(a3, a2)
        assert np.array_equal(c3[:, [0, 2]], c2) and np.all(c3[:, 1] == 0.0)
        assert np.all(np.abs(c2) <= 1.0)
        toks = a3


def test_zero_update_layer_similarity_is_one():
    """A layer with W_o = W_down = 0 passes its input through: similarity 1."""
    cfg = synth.variant("tiny")
    model = synth.make_model(cfg)
    model.layers[1].wo[:] = 0
    model.layers[1].w_down[:] = 0
    om = _load_oracle(model)
    _, _, cos = om.step(synth.start_tokens(cfg, 1), with_cos=True)
    assert cos[0, 1] == pytest.approx(1.0, abs=1e-15)
    assert cos[0, 0] < 1.0


# ---------------------------------------------------------------------------
# self-speculative decoding (the C/CUDA Llama engine page, sections 3.5 and 5.3)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("draft,verify,expect", [
    ([5, 6, 7], [5, 6, 7, 9], [5, 6, 7, 9]),     # every draft accepted, plus the bonus token
    ([5, 6, 7], [5, 8, 7, 9], [5, 8]),           # first mismatch at 2: d1 then the model's own token
    ([5, 6, 7], [4, 6, 7, 9], [4]),              # nothing accepted: one token, the model's
    ([], [3], [3]),                              # k = 0: a plain step
    ([1, 1], [1, 1, 1], [1, 1, 1]),
])
def test_spec_accept_hand_cases(draft, verify, expect):
    assert oracle.spec_accept(draft, verify).tolist() == expect


def test_speculative_round_equals_greedy():
    """A round drafted with the bottom layers (the other layers skipped) and
    verified by k+1 full steps yields exactly the greedy tokens; with every
    layer drafting, all k drafts are accepted."""
    cfg = synth.variant("tiny", n_layers=3, steps=12)
    model = synth.make_model(cfg)
    tok = int(synth.start_tokens(cfg)[0])
    greedy = _load_oracle(model)
    g_toks, t = [], tok
    for _ in range(8):
        _, am = greedy.step([t])
        t = int(am[0])
        g_toks.append(t)
    for d_layers, k in ((1, 3), (3, 3), (0, 2)):
        om = _load_oracle(model)
        p0 = om.position(0)
        out, t = [], tok
        while len(out) < 8:
            p = om.position(0)
            skip = np.array([l >= d_layers for l in range(cfg.n_layers)], np.uint8)
            draft, dt = [], t
            for _ in range(k):                   # draft: bottom layers only
                _, am = om.step([dt], skip=skip)
                dt = int(am[0])
                draft.append(dt)
            om.set_position(0, p)                # verify: k+1 full steps over [t, d1..dk]
            verify = []
            for x in [t] + draft:
                _, am = om.step([x])
                verify.append(int(am[0]))
            acc = oracle.spec_accept(draft, verify).tolist()
            if d_layers == cfg.n_layers:
                assert len(acc) == k + 1
            out += acc
            t = acc[-1]
            om.set_position(0, p + len(acc))
        assert out[:8] == g_toks, (d_layers, k)
        assert om.position(0) == p0 + len(out)
