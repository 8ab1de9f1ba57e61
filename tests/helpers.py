"""Shared test plumbing: build a generator model, open it on the GPU library
and on the oracle with the same prefilled cache, compare steps."""
from __future__ import annotations

import sys
import time

import numpy as np

import oracle
import synth

LOGIT_RTOL = 1e-3     # max|d logit| <= 1e-3 * max|logit| per step and sequence


def log(*a):
    print(time.strftime("%H:%M:%S"), *a, flush=True)
    sys.stdout.flush()


def kv_fn(cfg):
    return lambda s, l: synth.make_kv(cfg, s, l)


def open_gpu(model, max_seqs=None, kv_seqs=None):
    import token_decode_llama_amd as lm
    return lm.open_model(model, kv_fn(model.cfg), max_seqs=max_seqs, kv_seqs=kv_seqs)


def open_oracle(model, n_seq):
    om = oracle.OracleModel(model, max_seqs=n_seq)
    for s in range(n_seq):
        for l in range(model.cfg.n_layers):
            k, v = synth.make_kv(model.cfg, s, l)
            om.load_kv(s, l, k, v)
    return om


def f16_ulp_diff(a_bits: np.ndarray, b_bits: np.ndarray) -> int:
    """Largest distance in fp16 ulps between two arrays of fp16 bit patterns."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + (x & 0x7FFF))
    return int(np.max(np.abs(ordered(a_bits) - ordered(b_bits)))) if a_bits.size else 0


def f16_close(got_bits: np.ndarray, ref_bits: np.ndarray, rel_abs: float = 2e-5) -> bool:
    """fp16 values from an fp32 computation against fp16 values from an fp64
    one: each may sit one fp16 ulp off (different rounding inputs), plus the
    fp32 computation's absolute error, bounded by rel_abs * max|ref|."""
    g = got_bits.view(np.float16).astype(np.float64)
    r = ref_bits.view(np.float16).astype(np.float64)
    if r.size == 0:
        return True
    ulp = np.spacing(np.maximum(np.abs(g), np.abs(r)).astype(np.float16)).astype(np.float64)
    tol = ulp + rel_abs * float(np.max(np.abs(r)))
    return bool(np.all(np.abs(g - r) <= tol))


def compare_step(lg_gpu, am_gpu, lg_orc, am_orc, tag=""):
    """Per-sequence logit bound and argmax equality; returns the worst relative error."""
    worst = 0.0
    for s in range(lg_orc.shape[0]):
        ref = lg_orc[s]
        err = float(np.max(np.abs(lg_gpu[s].astype(np.float64) - ref)))
        scale = float(np.max(np.abs(ref)))
        rel = err / scale
        worst = max(worst, rel)
        assert rel <= LOGIT_RTOL, f"{tag} seq {s}: max|dlogit| = {err:.3e} > 1e-3 * {scale:.3e}"
        if am_gpu[s] != am_orc[s]:
            top = np.sort(ref.astype(np.float32))[-2:]
            raise AssertionError(f"{tag} seq {s}: argmax {am_gpu[s]} != oracle {am_orc[s]} "
                                 f"(oracle top-2 gap {float(top[1] - top[0]):.3e}, "
                                 f"max|dlogit| {err:.3e})")
    return worst
