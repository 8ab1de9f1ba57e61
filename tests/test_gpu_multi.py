"""Several models resident at once, each on its own HIP stream, decoded
round-robin through the C ABI's device entry point (graph replay): every
model's logits and tokens must be bit-identical to the same model decoded
alone.  The three shapes are the 1B / 0.5B / 360M workload's, at two layers.
"""
import numpy as np
import pytest

import synth
from tests.helpers import log

pytestmark = pytest.mark.gpu

NAMES = ["multi_llama1b", "multi_qwen05b", "multi_smol360m"]


def _cfgs():
    return [synth.variant(n, n_layers=2, ctx=96, steps=4) for n in NAMES]


def _open(model, stream):
    import token_decode_llama_amd as lm
    return lm.open_model(model, lambda s, l: synth.make_kv(model.cfg, s, l), max_seqs=1, kv_seqs=1,
                         stream=stream)


def test_round_robin_on_streams_bit_identical_to_solo():
    import torch
    cfgs = _cfgs()
    models = [synth.make_model(c) for c in cfgs]
    streams = [torch.cuda.Stream() for _ in cfgs]
    gs = [_open(m, s.cuda_stream) for m, s in zip(models, streams)]
    dev = torch.device("cuda:0")
    try:
        def fresh():
            toks, lgs = [], []
            for g, c, s in zip(gs, cfgs, streams):
                g.set_position(0, c.ctx)
                with torch.cuda.stream(s):
                    toks.append(torch.from_numpy(synth.start_tokens(c, 1)).to(dev))
                    lgs.append(torch.empty((c.steps, c.vocab), dtype=torch.float32, device=dev))
            torch.cuda.synchronize()
            return toks, lgs

        # each model alone (the others idle)
        solo = []
        toks, lgs = fresh()
        for i, (g, c) in enumerate(zip(gs, cfgs)):
            for st in range(c.steps):
                g.step_dev(toks[i], 1, toks[i], lgs[i][st])
            torch.cuda.synchronize()
            solo.append(lgs[i].cpu().numpy().copy())
        # round-robin, all three in flight on their own streams
        for rep in range(2):
            toks, lgs = fresh()
            for st in range(max(c.steps for c in cfgs)):
                for i, (g, c) in enumerate(zip(gs, cfgs)):
                    if st < c.steps:
                        g.step_dev(toks[i], 1, toks[i], lgs[i][st])
            torch.cuda.synchronize()
            for i, c in enumerate(cfgs):
                got = lgs[i].cpu().numpy()
                log(f"{c.name} rep {rep}: round-robin vs solo max|d| = {np.max(np.abs(got - solo[i])):.3e}")
                assert np.array_equal(got, solo[i]), c.name
                assert np.array_equal(np.argmax(got, axis=1), np.argmax(solo[i], axis=1))
    finally:
        for g in gs:
            g.close()
