"""lm_decode_step_dev_noalloc, the step for callers that cannot allocate,
against lm_decode_step_dev on the same model, inputs and positions: two
calls in a row, the second with fewer sequences at shorter contexts, on a
one-sequence model and on 8B-shaped Q8_0 / Q4_0 layers (the matrix-core
path).  Logits, argmax and the appended K/V rows must be identical (the same
kernels on the same inputs), which is within the decode bar of 1e-3 of the
largest logit and exact argmax.  Also: no library allocation and no change
in free device memory across the calls, and the clear error when the
working memory exceeds the fixed array."""
import numpy as np
import pytest

import synth
from tests.helpers import compare_step, log, open_gpu

pytestmark = pytest.mark.gpu


def _buffers(g, tokens):
    import torch
    n = len(tokens)
    return (torch.tensor(np.asarray(tokens, np.int32), device="cuda"),
            torch.empty(n, dtype=torch.int32, device="cuda"),
            torch.empty((n, g.cfg.vocab), dtype=torch.float32, device="cuda"))


def _run(g, fn, bufs, pos):
    """Sets the positions, runs one step through fn on the device buffers
    (tokens, argmax, logits) and returns (logits, argmax, positions after,
    K/V rows written)."""
    import torch
    d_tok, d_am, d_lg = bufs
    n = d_tok.numel()
    for s in range(n):
        g.set_position(s, int(pos[s]))
    d_am.fill_(-1)
    d_lg.fill_(float("nan"))
    torch.cuda.synchronize()                  # the model runs on a stream of its own
    fn(d_tok, n, d_am, d_lg)
    torch.cuda.synchronize()
    kv = []
    for s in range(n):
        for l in range(g.cfg.n_layers):
            k, v = g.get_kv(s, l, int(pos[s]) + 1)
            kv.append((k[:, -1].copy(), v[:, -1].copy()))
    return d_lg.cpu().numpy(), d_am.cpu().numpy(), [g.position(s) for s in range(n)], kv


def _free_device_bytes():
    import torch
    torch.cuda.synchronize()
    return torch.cuda.mem_get_info()[0]


CASES = {
    "tiny_q8": dict(name="tiny", changes=dict(ctx=40, steps=4)),
    "llama8b_q8_2layer": dict(name="llama8b_q8", changes=dict(n_layers=2, ctx=300, steps=4)),
    "llama8b_q4_2layer": dict(name="llama8b_q4", changes=dict(n_layers=2, ctx=300, steps=4)),
}


@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_step_matches_the_step(case):
    import token_decode_llama_amd as lm
    spec = CASES[case]
    cfg = synth.variant(spec["name"], **spec["changes"])
    log("generate", case)
    model = synth.make_model(cfg)
    g = open_gpu(model, max_seqs=4)
    try:
        tok4 = synth.start_tokens(cfg, 4)
        # call 1: four sequences at different positions; call 2: two sequences,
        # shorter contexts (a smaller input in the same array)
        calls = [(tok4, np.array([cfg.ctx, cfg.ctx + 1, cfg.ctx - 3, cfg.ctx // 2])),
                 (tok4[:2][::-1].copy(), np.array([cfg.ctx - 5, 7]))]
        for i, (tok, pos) in enumerate(calls):
            bufs = _buffers(g, tok)
            ref = _run(g, g.step_dev, bufs, pos)
            c0, f0 = lm.alloc_count(), _free_device_bytes()
            got = _run(g, g.step_dev_noalloc, bufs, pos)
            assert lm.alloc_count() == c0, f"{case} call {i}: the library allocated"
            assert _free_device_bytes() == f0, f"{case} call {i}: free device memory changed"
            lg_r, am_r, pos_r, kv_r = ref
            lg_g, am_g, pos_g, kv_g = got
            log(f"{case} call {i}: n_seq {len(tok)} positions {list(pos)} argmax {list(am_g)}")
            compare_step(lg_g, am_g, lg_r.astype(np.float64), am_r, f"{case} call {i}")
            assert np.array_equal(lg_g, lg_r), f"{case} call {i}: logits differ"
            assert np.array_equal(am_g, am_r), f"{case} call {i}: argmax differs"
            assert pos_g == pos_r == [int(p) + 1 for p in pos]
            for (ka, va), (kb, vb) in zip(kv_g, kv_r):
                assert np.array_equal(ka, kb) and np.array_equal(va, vb), f"{case} call {i}: K/V rows differ"
    finally:
        g.close()


def test_noalloc_step_rejects_working_memory_beyond_the_array():
    import token_decode_llama_amd as lm
    import torch
    # 32 query heads of 64 over 65536 positions: the attention partial states
    # alone take 4 * 32 * 1024 * 66 * 4 bytes > 32 MiB for four sequences,
    # 8.6 MB for one
    cfg = synth.variant("tiny", hidden=2048, n_heads=32, n_kv_heads=4, head_dim=64, ffn=512, n_layers=1,
                        ctx=16, steps=2)
    model = synth.make_model(cfg)
    g = lm.open_model(model, lambda s, l: synth.make_kv(cfg, s, l), max_seqs=4, max_ctx=65536)
    try:
        tok = synth.start_tokens(cfg, 4)
        d_tok = torch.tensor(np.asarray(tok, np.int32), device="cuda")
        d_am = torch.empty(4, dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        for s in range(4):
            g.set_position(s, cfg.ctx)
        with pytest.raises(lm.LMError) as e:
            g.step_dev_noalloc(d_tok, 4, d_am)
        assert e.value.status == lm.LM_E_ARG and "scratch" in str(e.value), str(e.value)
        assert [g.position(s) for s in range(4)] == [cfg.ctx] * 4
        g.step_dev_noalloc(d_tok, 1, d_am)             # one sequence fits
        torch.cuda.synchronize()
        assert g.position(0) == cfg.ctx + 1
        am1 = int(d_am[0].item())
        g.set_position(0, cfg.ctx)
        g.step_dev(d_tok, 1, d_am)
        torch.cuda.synchronize()
        assert int(d_am[0].item()) == am1
    finally:
        g.close()
