"""bench.py's profile summaries attribute every kernel of a trace or counter run
to a step operator by parsing the kernel's name and template arguments.  Every
kernel the library instantiates must be attributed, to the operator its
epilogue argument names; a changed template signature otherwise drops a
kernel from the tables (and the traffic figure) without an error.  Reads the
kernel names from the built library's symbol table (no GPU)."""
import importlib.util
import os
import re
import subprocess
import sys

import token_decode_llama_amd as lm

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EPI_KIND = {0: "qkv", 2: "gateup", 3: "lmhead"}          # epilogue argument -> operator
RESIDUAL_KINDS = {"wo", "down"}                          # epilogue 1: the two residual GEMVs


def _bench():
    spec = importlib.util.spec_from_file_location("bench_for_tests", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    argv = sys.argv
    sys.argv = ["bench.py"]
    try:
        spec.loader.exec_module(mod)
    finally:
        sys.argv = argv
    return mod


def _kernel_names():
    lm.load()
    out = subprocess.check_output(["nm", "-C", "--defined-only", lm.LIB_PATH], text=True)
    names = set()
    for line in out.splitlines():
        parts = line.split(" ", 2)
        if len(parts) == 3 and "lmk::k_" in parts[2] and "__device_stub" not in parts[2]:
            names.add(parts[2])
    return sorted(names)


def test_every_kernel_is_attributed_to_its_operator():
    kind_of = _bench().kind_of
    names = _kernel_names()
    gemv = [n for n in names if "lmk::k_gemv<" in n]
    gemv_mb = [n for n in names if "lmk::k_gemv_mb<" in n]
    assert gemv and gemv_mb and any("lmk::k_attn<" in n for n in names), names[:10]
    for n in gemv:
        epi = int(re.search(r"k_gemv<\d+, \d+, (\d+),", n).group(1))
        got = kind_of(n)
        assert got in RESIDUAL_KINDS if epi == 1 else got == EPI_KIND[epi], (n, got)
    for n in gemv_mb:
        epi = int(re.search(r"k_gemv_mb<\d+, (\d+),", n).group(1))
        got = kind_of(n)
        assert got in RESIDUAL_KINDS if epi == 1 else got == EPI_KIND[epi], (n, got)
    for key, kind in (("lmk::k_attn<", "attn"), ("lmk::k_embed(", "embed"), ("lmk::k_xdigits(", "digits"),
                      ("lmk::k_read_bw(", "read_bw"), ("lmk::k_dequant(", "dequant")):
        hits = [n for n in names if key in n]
        assert hits, key
        for n in hits:
            assert kind_of(n) == kind, (n, kind_of(n))
    # both load flavours of the one-sequence GEMV and the digit-writing gate/up are built
    assert any(n.endswith(", false>(lmk::GemvArgs)") for n in gemv)
    assert any(re.search(r"k_gemv_mb<\d+, 2, 4, true, true>", n) for n in gemv_mb)
