"""Pins of the fp64 oracle against things other than itself.

Each test ties one oracle function to a closed form, an invariant, a library
routine, brute force or a hand-worked block, chosen so that a plausible slip
(a dropped term, a wrong sign or index, a transposed operand) fails one of
them.  None of these tests touches the GPU.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import synth
from synth import Q4_0, Q4_K, Q5_K, Q6_K, Q8_0

RNG = np.random.default_rng(1234)


# ---------------------------------------------------------------------------
# fp16 codec (IEEE binary16; numpy's float16 is the library routine)
# ---------------------------------------------------------------------------

def test_f16_decode_all_bit_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # the two scale values the hand-worked blocks below rely on
    assert oracle.f16_to_f64(0x1419) == 0.0010004043579101562
    assert oracle.f16_to_f64(0x211F) == 0.01000213623046875


def _f16_cases():
    v = np.concatenate([
        RNG.standard_normal(20000) * 3.0,
        RNG.standard_normal(5000) * 1e-5,                    # subnormal range
        RNG.standard_normal(2000) * 3e4,                     # near overflow
        np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 1e9, -1e9, 2.0 ** -24,
                  2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -14, 1.0 + 2.0 ** -11,
                  1.0 + 3 * 2.0 ** -11, 2049.0, 2051.0, -2051.0, 5e-324]),
    ])
    # exact ties between neighbouring fp16 values
    h = RNG.integers(1, 0x7BFF, 3000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    return np.concatenate([v, (lo + hi) / 2, -(lo + hi) / 2])


def test_oracle_f64_to_f16_round_nearest_even():
    v = _f16_cases()
    ref = v.astype(np.float16).view(np.uint16)
    got = np.array([oracle.f64_to_f16(x) for x in v], dtype=np.uint16)
    assert np.array_equal(got, ref)


def test_generator_f64_to_f16_round_nearest_even():
    v = _f16_cases()
    ref = v.astype(np.float16).view(np.uint16)
    got = np.array([synth.f64_to_f16_bits(x) for x in v], dtype=np.uint16)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------
# hand-worked blocks (formats as the workload defines them)
# ---------------------------------------------------------------------------

def test_q8_0_hand_worked_block():
    w = np.zeros(32, np.float32)
    w[0], w[1], w[2], w[3] = 0.127, -0.127, 0.05, 0.0
    blk = synth.quantize(w, Q8_0)
    assert blk.size == 34
    assert int(blk[0]) | (int(blk[1]) << 8) == 0x1419          # d = fp16(0.127/127)
    q = blk[2:].view(np.int8)
    assert (q[0], q[1], q[2], q[3]) == (127, -127, 50, 0)
    deq = oracle.dequant(Q8_0, blk, 1, 32)[0]
    assert deq[0] == 0.12705135345458984
    assert deq[1] == -0.12705135345458984
    assert deq[2] == 0.05002021789550781
    assert deq[3] == 0.0 and np.all(deq[4:] == 0.0)


def test_q8_0_round_half_away_from_zero():
    w = np.zeros(32, np.float32)
    w[0], w[1], w[2] = 127.0, 2.5, -2.5                          # d = 1 exactly
    blk = synth.quantize(w, Q8_0)
    assert int(blk[0]) | (int(blk[1]) << 8) == 0x3C00
    q = blk[2:].view(np.int8)
    assert (q[0], q[1], q[2]) == (127, 3, -3)
    assert list(oracle.dequant(Q8_0, blk, 1, 32)[0][:3]) == [127.0, 3.0, -3.0]


def test_q4_0_hand_worked_block():
    w = np.zeros(32, np.float32)
    w[0], w[1], w[2], w[3] = 0.07, -0.07, 0.034, -0.016
    w[17] = 0.07
    blk = synth.quantize(w, Q4_0)
    assert blk.size == 18
    assert int(blk[0]) | (int(blk[1]) << 8) == 0x211F          # d = fp16(0.07/7)
    nib_lo = blk[2:] & 0xF
    nib_hi = blk[2:] >> 4
    assert list(nib_lo[:4]) == [15, 1, 11, 6]
    assert nib_lo[4] == 8 and nib_hi[0] == 8 and nib_hi[1] == 15   # element 17 -> byte 1 high
    deq = oracle.dequant(Q4_0, blk, 1, 32)[0]
    assert deq[0] == 0.07001495361328125
    assert deq[1] == -0.07001495361328125
    assert deq[2] == 0.03000640869140625
    assert deq[3] == -0.0200042724609375
    assert deq[17] == 0.07001495361328125
    assert deq[16] == 0.0 and deq[4] == 0.0


def test_q4_0_nibble_order():
    blk = np.zeros(18, np.uint8)
    blk[0], blk[1] = 0x00, 0x3C                                  # d = 1.0
    blk[2] = 0x80                                                # byte 0: lo 0 (elem 0), hi 8 (elem 16)
    blk[3] = 0xF1                                                # byte 1: lo 1 (elem 1), hi 15 (elem 17)
    blk[2 + 15] = 0x2E                                           # byte 15: lo 14 (elem 15), hi 2 (elem 31)
    deq = oracle.dequant(Q4_0, blk, 1, 32)[0]
    assert deq[0] == -8.0 and deq[16] == 0.0
    assert deq[1] == -7.0 and deq[17] == 7.0
    assert deq[15] == 6.0 and deq[31] == -6.0


def test_all_zero_blocks():
    z = np.zeros(64, np.float32)
    b8 = synth.quantize(z, Q8_0)
    b4 = synth.quantize(z, Q4_0)
    assert np.all(b8 == 0)
    assert np.all(b4[:2] == 0) and np.all(b4[2:18] == 0x88)
    assert np.all(oracle.dequant(Q8_0, b8, 1, 64) == 0)
    assert np.all(oracle.dequant(Q4_0, b4, 1, 64) == 0)


# ---------------------------------------------------------------------------
# GGUF K formats (named on the C/CUDA Llama engine page, section 1, as the
# formats of its 70B figures; byte layout as GGUF publishes it)
# ---------------------------------------------------------------------------

def test_q4_k_hand_worked_superblock():
    # d = 1.0, dmin = 0.25; (scale, min) per sub-block:
    #   (1, 0) (2, 4) (63, 1) (0, 63) (17, 40) (33, 21) (48, 63) (5, 16)
    # packed by hand: bytes 0-3 = low 6 bits of scales 0-3 with the top 2 bits
    # of scales 4-7 above them; bytes 4-7 = the same for the mins; bytes 8-11 =
    # low nibble: scale 4-7 & 15, high nibble: min 4-7 & 15
    blk = np.zeros(144, np.uint8)
    blk[0:4] = [0x00, 0x3C, 0x00, 0x34]
    blk[4:16] = [65, 130, 255, 0, 128, 68, 193, 127, 129, 81, 240, 5]
    qs = blk[16:]
    qs[0] = 0x07      # element 0   (sub-block 0, low nibble):  q = 7
    qs[1] = 0x90      # element 33  (sub-block 1, high nibble): q = 9
    qs[37] = 0x0F     # element 69  (sub-block 2, low):  q = 15
    qs[63] = 0x40     # element 127 (sub-block 3, high): q = 4
    qs[66] = 0x03     # element 130 (sub-block 4, low):  q = 3
    qs[74] = 0x10     # element 170 (sub-block 5, high): q = 1
    qs[96] = 0x02     # element 192 (sub-block 6, low):  q = 2
    qs[127] = 0xF0    # element 255 (sub-block 7, high): q = 15
    expect = np.repeat([0.0, -1.0, -0.25, -15.75, -10.0, -5.25, -15.75, -4.0], 32)  # q = 0: -dmin * min
    expect[0] = 7.0          # 1 * 7 - 0
    expect[33] = 17.0        # 2 * 9 - 0.25 * 4
    expect[69] = 944.75      # 63 * 15 - 0.25 * 1
    expect[127] = -15.75     # 0 * 4 - 0.25 * 63
    expect[130] = 41.0       # 17 * 3 - 0.25 * 40
    expect[170] = 27.75      # 33 * 1 - 0.25 * 21
    expect[192] = 80.25      # 48 * 2 - 0.25 * 63
    expect[255] = 71.0       # 5 * 15 - 0.25 * 16
    got = oracle.dequant(Q4_K, blk, 1, 256)[0]
    assert np.array_equal(got, expect), np.nonzero(got != expect)


def test_q6_k_hand_worked_superblock():
    # d = 0.5, scales[k] = k - 8 (negative, zero and positive); every q is 0
    # (value 0.5 * (k - 8) * -32) except the elements set below
    blk = np.zeros(210, np.uint8)
    blk[192:208] = (np.arange(16) - 8).astype(np.int8).view(np.uint8)
    blk[208:210] = [0x00, 0x38]
    ql, qh = blk[0:128], blk[128:192]
    ql[0] = 0x0F; qh[0] = 0x03           # element 0:   q = 63 (scale -8)
    ql[40] = 0x01; qh[8] = 0x08          # element 40:  q = 33 (low nibble of byte 32+8, bits 2-3)
    ql[17] = 0x40; qh[17] = 0x10         # element 81:  q = 20 (high nibble of byte 17, bits 4-5)
    qh[31] = 0xC0                        # element 127: q = 48 (bits 6-7 of high-bit byte 31)
    ql[69] = 0x0D; qh[37] = 0x02         # element 133: q = 45 (second half: bytes 64+5, 32+5)
    ql[96] = 0xF0; qh[32] = 0x40         # element 224: q = 31 (high nibble of byte 64+32)
    ql[127] = 0xE0; qh[63] = 0xC0        # element 255: q = 62
    expect = np.repeat(-16.0 * (np.arange(16) - 8), 16)
    expect[0] = -124.0       # 0.5 * -8 * 31
    expect[40] = -3.0        # 0.5 * -6 * 1
    expect[81] = 18.0        # 0.5 * -3 * -12
    expect[127] = -8.0       # 0.5 * -1 * 16
    expect[133] = 0.0        # scale 0
    expect[224] = -3.0       # 0.5 * 6 * -1
    expect[255] = 105.0      # 0.5 * 7 * 30
    got = oracle.dequant(Q6_K, blk, 1, 256)[0]
    assert np.array_equal(got, expect), np.nonzero(got != expect)


def _encode_q4_k(d_bits, dmin_bits, sc, mn, q):
    """Field-by-field encoder (the opposite direction of the dequantiser)."""
    blk = np.zeros(144, np.uint8)
    blk[0], blk[1] = d_bits & 255, d_bits >> 8
    blk[2], blk[3] = dmin_bits & 255, dmin_bits >> 8
    for j in range(8):
        if j < 4:
            blk[4 + j] |= sc[j] & 63
            blk[8 + j] |= mn[j] & 63
        else:
            blk[12 + j - 4] |= (sc[j] & 15) | ((mn[j] & 15) << 4)
            blk[4 + j - 4] |= (sc[j] >> 4) << 6
            blk[8 + j - 4] |= (mn[j] >> 4) << 6
    for e in range(256):
        j, i = divmod(e, 32)
        blk[16 + 32 * (j // 2) + i] |= q[e] << (4 * (j % 2))
    return blk


def _encode_q5_k(d_bits, dmin_bits, sc, mn, q):
    """Q4_K's encoding of the low four bits, then the fifth bits after the header."""
    b4 = _encode_q4_k(d_bits, dmin_bits, sc, mn, np.asarray(q) & 15)
    blk = np.zeros(176, np.uint8)
    blk[0:16] = b4[0:16]
    blk[48:176] = b4[16:144]
    for e in range(256):
        blk[16 + e % 32] |= ((q[e] >> 4) & 1) << (e // 32)
    return blk


def test_q5_k_hand_worked_superblock():
    # the Q4_K header of the hand-worked Q4_K case (d 1.0, dmin 0.25, the same
    # eight (scale, min) pairs); fifth bits set for elements 33 (byte 1, bit 1),
    # 130 (byte 2, bit 4) and 255 (byte 31, bit 7)
    blk = np.zeros(176, np.uint8)
    blk[0:4] = [0x00, 0x3C, 0x00, 0x34]
    blk[4:16] = [65, 130, 255, 0, 128, 68, 193, 127, 129, 81, 240, 5]
    qh, qs = blk[16:48], blk[48:]
    qh[1] = 0x02
    qh[2] = 0x10
    qh[31] = 0x80
    qs[1] = 0x90      # element 33 (sub-block 1, high nibble): q = 9 + 16 = 25
    qs[66] = 0x03     # element 130 (sub-block 4, low nibble): q = 3 + 16 = 19
    qs[0] = 0x07      # element 0 (sub-block 0): q = 7, no fifth bit
    expect = np.repeat([0.0, -1.0, -0.25, -15.75, -10.0, -5.25, -15.75, -4.0], 32)
    expect[0] = 7.0          # 1 * 7
    expect[33] = 49.0        # 2 * 25 - 0.25 * 4
    expect[130] = 313.0      # 17 * 19 - 0.25 * 40
    expect[255] = 76.0       # 5 * 16 - 0.25 * 16 (nibble 0, fifth bit set)
    got = oracle.dequant(Q5_K, blk, 1, 256)[0]
    assert np.array_equal(got, expect), np.nonzero(got != expect)


def _encode_q6_k(d_bits, sc, q):
    blk = np.zeros(210, np.uint8)
    for e in range(256):
        h, r = divmod(e, 128)
        t, l = divmod(r, 32)
        blk[64 * h + 32 * (t % 2) + l] |= (q[e] & 15) << (4 * (t // 2))
        blk[128 + 32 * h + l] |= (q[e] >> 4) << (2 * t)
    blk[192:208] = np.asarray(sc, np.int8).view(np.uint8)
    blk[208], blk[209] = d_bits & 255, d_bits >> 8
    return blk


def _f16_bits(v):
    return int(np.float16(v).view(np.uint16))


@pytest.mark.parametrize("seed", range(6))
def test_k_formats_decode_random_fields(seed):
    r = np.random.default_rng(seed)
    d, dmin = np.float16(r.uniform(-2, 2)), np.float16(r.uniform(0, 1))
    sc, mn, q = r.integers(0, 64, 8), r.integers(0, 64, 8), r.integers(0, 16, 256)
    blk = _encode_q4_k(_f16_bits(d), _f16_bits(dmin), sc, mn, q)
    want = float(d) * np.repeat(sc, 32) * q - float(dmin) * np.repeat(mn, 32)
    assert np.array_equal(oracle.dequant(Q4_K, blk, 1, 256)[0], want)
    q5 = r.integers(0, 32, 256)
    blk5 = _encode_q5_k(_f16_bits(d), _f16_bits(dmin), sc, mn, q5)
    want5 = float(d) * np.repeat(sc, 32) * q5 - float(dmin) * np.repeat(mn, 32)
    assert np.array_equal(oracle.dequant(Q5_K, blk5, 1, 256)[0], want5)
    d6, sc6, q6 = np.float16(r.uniform(-1, 1)), r.integers(-128, 128, 16), r.integers(0, 64, 256)
    blk6 = _encode_q6_k(_f16_bits(d6), sc6, q6)
    want6 = float(d6) * np.repeat(sc6, 16) * (q6 - 32)
    assert np.array_equal(oracle.dequant(Q6_K, blk6, 1, 256)[0], want6)


@pytest.mark.parametrize("qtype,step_bound", [(Q4_K, 0.55), (Q5_K, 0.55), (Q6_K, 0.55)])
def test_k_quantizer_round_trip(qtype, step_bound):
    # the generator's K blocks dequantise to within about half a quantisation
    # step of the drawn values (clamping can only widen the extreme bins)
    w = synth.normal_f32(11, 3, 256 * 16, std=0.02)
    blk = synth.quantize(w, qtype)
    assert blk.size == 16 * synth.BLOCK_BYTES[qtype]
    got = oracle.dequant(qtype, blk, 1, w.size)[0]
    span = {Q4_K: 15, Q5_K: 31, Q6_K: 62}[qtype]
    sub = 16 if qtype == Q6_K else 32
    ws = w.reshape(-1, sub).astype(np.float64)
    step = (ws.max(1) - np.minimum(ws.min(1), 0)) / span if qtype != Q6_K else np.abs(ws).max(1) * 2 / span
    err = np.abs(got.reshape(-1, sub) - ws)
    assert np.all(err <= step_bound * step[:, None] * 1.2 + 1e-9)
    assert np.corrcoef(got, w)[0, 1] > {Q4_K: 0.99, Q5_K: 0.998, Q6_K: 0.999}[qtype]
    z = synth.quantize(np.zeros(512, np.float32), qtype)
    assert np.all(oracle.dequant(qtype, z, 1, 512) == 0)


def _numpy_dequant(qtype, blocks, rows, cols):
    """Independent dequantiser written from the format definition (vectorised
    over whole planes, where the oracle walks element by element)."""
    if qtype in (Q4_K, Q5_K, Q6_K):
        return _numpy_dequant_k(qtype, blocks, rows, cols)
    bb = synth.BLOCK_BYTES[qtype]
    b = np.ascontiguousarray(blocks, np.uint8).reshape(rows, cols // 32, bb)
    d = b[:, :, :2].copy().view(np.float16)[:, :, 0].astype(np.float64)
    if qtype == Q8_0:
        q = b[:, :, 2:].view(np.int8).astype(np.float64)
    else:
        lo = (b[:, :, 2:] & 0xF).astype(np.float64) - 8
        hi = (b[:, :, 2:] >> 4).astype(np.float64) - 8
        q = np.concatenate([lo, hi], axis=2)
    return (q * d[:, :, None]).reshape(rows, cols)


def _numpy_dequant_k(qtype, blocks, rows, cols):
    """GGUF K formats, 256-weight super-blocks, from the published layout."""
    nsb = cols // 256
    b = np.ascontiguousarray(blocks, np.uint8).reshape(rows, nsb, synth.BLOCK_BYTES[qtype])
    if qtype in (Q4_K, Q5_K):
        d = b[..., 0:2].copy().view(np.float16)[..., 0].astype(np.float64)
        dmin = b[..., 2:4].copy().view(np.float16)[..., 0].astype(np.float64)
        s = b[..., 4:16].astype(np.int64)
        sc = np.concatenate([s[..., 0:4] & 63, (s[..., 8:12] & 15) | ((s[..., 0:4] >> 6) << 4)], axis=-1)
        mn = np.concatenate([s[..., 4:8] & 63, (s[..., 8:12] >> 4) | ((s[..., 4:8] >> 6) << 4)], axis=-1)
        off = 16 if qtype == Q4_K else 48
        qs = b[..., off:off + 128].reshape(rows, nsb, 4, 32).astype(np.int64)
        q = np.stack([qs & 15, qs >> 4], axis=3).reshape(rows, nsb, 8, 32)   # sub-blocks 2g, 2g+1
        if qtype == Q5_K:
            qh = b[..., 16:48].astype(np.int64)                               # [l], bit j: sub-block j
            q = q | (((qh[:, :, None, :] >> np.arange(8)[None, None, :, None]) & 1) << 4)
        w = d[..., None, None] * sc[..., None] * q - dmin[..., None, None] * mn[..., None]
        return w.reshape(rows, cols)
    ql = b[..., 0:128].reshape(rows, nsb, 2, 2, 32).astype(np.int64)   # [half][which 32 bytes][l]
    qh = b[..., 128:192].reshape(rows, nsb, 2, 32).astype(np.int64)
    sc = b[..., 192:208].view(np.int8).astype(np.float64)
    d = b[..., 208:210].copy().view(np.float16)[..., 0].astype(np.float64)
    quarters = []
    for t in range(4):              # element 128h + 32t + l
        lo = (ql[:, :, :, t % 2, :] >> (4 * (t // 2))) & 15
        hi = (qh >> (2 * t)) & 3
        quarters.append(lo | (hi << 4))
    q = np.stack(quarters, axis=3).reshape(rows, nsb, 256)
    w = d[..., None] * np.repeat(sc, 16, axis=-1) * (q - 32)
    return w.reshape(rows, cols)


@pytest.mark.parametrize("qtype,cols", [(Q8_0, 32 * 13), (Q4_0, 32 * 13), (Q4_K, 256 * 3), (Q5_K, 256 * 3),
                                        (Q6_K, 256 * 3)])
def test_dequant_matches_format_definition(qtype, cols):
    rows = 37
    blocks = synth.quant_matrix(7, 99, rows, cols, 0.02, qtype)
    assert np.array_equal(oracle.dequant(qtype, blocks, rows, cols),
                          _numpy_dequant(qtype, blocks, rows, cols))


# ---------------------------------------------------------------------------
# GEMV: brute force in exact rationals
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("qtype,rows,cols", [(Q8_0, 8, 64), (Q4_0, 6, 96), (Q8_0, 3, 32),
                                             (Q4_K, 3, 512), (Q5_K, 2, 512), (Q6_K, 3, 256)])
def test_gemv_brute_force_fraction(qtype, rows, cols):
    blocks = synth.quant_matrix(5, 17 + rows, rows, cols, 0.02, qtype)
    x = RNG.standard_normal(cols)
    y = oracle.gemv(qtype, blocks, rows, cols, x)
    W = _numpy_dequant(qtype, blocks, rows, cols)
    for r in range(rows):
        exact = sum(Fraction(float(W[r, c])) * Fraction(float(x[c])) for c in range(cols))
        bound = cols * 2.0 ** -53 * float(np.sum(np.abs(W[r] * x))) + 1e-300
        assert abs(Fraction(float(y[r])) - exact) <= Fraction(bound), (r, float(exact), y[r])


def test_gemv_row_order_not_transposed():
    # a one-hot input picks column c of W; a one-hot row picks row r
    rows, cols = 5, 64
    blocks = synth.quant_matrix(3, 5, rows, cols, 0.02, Q8_0)
    W = _numpy_dequant(Q8_0, blocks, rows, cols)
    for c in (0, 31, 32, 63):
        e = np.zeros(cols)
        e[c] = 1.0
        assert np.array_equal(oracle.gemv(Q8_0, blocks, rows, cols, e), W[:, c])


# ---------------------------------------------------------------------------
# RMSNorm
# ---------------------------------------------------------------------------

def test_rmsnorm_constant_vector_closed_form():
    n, c, eps = 256, 0.37, 1e-5
    g = np.random.default_rng(355).standard_normal(n).astype(np.float32)
    out = oracle.rmsnorm(np.full(n, c), g, eps)
    expect = g.astype(np.float64) * c / math.sqrt(c * c + eps)
    # the sequential sum of n squares carries a relative error of up to n * 2^-53
    # (standard summation bound); the root halves it, a few roundings add to it
    assert np.allclose(out, expect, rtol=n * 2.0 ** -53, atol=0)


def test_rmsnorm_matches_torch():
    n, eps = 4096, 1e-5
    x = RNG.standard_normal(n) * 0.3
    g = (1 + 0.1 * RNG.standard_normal(n)).astype(np.float32)
    ref = F.rms_norm(torch.from_numpy(x), (n,), weight=torch.from_numpy(g.astype(np.float64)), eps=eps)
    assert np.allclose(oracle.rmsnorm(x, g, eps), ref.numpy(), rtol=1e-14, atol=0)


def test_rmsnorm_scale_invariance_small_eps():
    n = 64
    x = RNG.standard_normal(n)
    g = np.ones(n, np.float32)
    a = oracle.rmsnorm(x, g, 0.0)
    b = oracle.rmsnorm(x * 1000.0, g, 0.0)
    assert np.allclose(a, b, rtol=1e-14)
    assert abs(np.mean(a * a) - 1.0) < 1e-14


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------

def test_rope_position_zero_is_identity():
    v = RNG.standard_normal(4 * 64)
    assert np.array_equal(oracle.rope(v, 4, 64, 0, 5e5), v)


def test_rope_preserves_pair_norms():
    hd, nh = 128, 3
    v = RNG.standard_normal(nh * hd)
    out = oracle.rope(v, nh, hd, 4093, 5e5)
    n0 = v.reshape(-1, 2)
    n1 = out.reshape(-1, 2)
    assert np.allclose(np.hypot(n1[:, 0], n1[:, 1]), np.hypot(n0[:, 0], n0[:, 1]), rtol=1e-15, atol=0)


def test_rope_pair_zero_turns_by_position_radians():
    hd = 64
    for p in (1, 7, 511, 4095):
        e0 = np.zeros(hd)
        e0[0] = 1.0
        out = oracle.rope(e0, 1, hd, p, 5e5)
        assert out[0] == pytest.approx(math.cos(p), abs=1e-15)
        assert out[1] == pytest.approx(math.sin(p), abs=1e-15)
        assert np.all(out[2:] == 0.0)          # adjacent pairing: nothing leaks past (0, 1)


def test_rope_frequencies_match_transformers():
    from transformers import LlamaConfig
    from transformers.models.llama.modeling_llama import LlamaRotaryEmbedding
    hd, theta = 128, 500000.0
    cfg = LlamaConfig(hidden_size=hd * 4, num_attention_heads=4, head_dim=hd, rope_theta=theta)
    inv_freq, _ = LlamaRotaryEmbedding.compute_default_rope_parameters(cfg, device="cpu")
    inv_freq = inv_freq.double().numpy()
    p = 3
    for i in range(hd // 2):
        e = np.zeros(hd)
        e[2 * i] = 1.0
        out = oracle.rope(e, 1, hd, p, theta)
        ang = math.atan2(out[2 * i + 1], out[2 * i])
        # the library computes its frequencies in fp32: compare at that precision
        assert ang == pytest.approx(p * inv_freq[i], rel=1e-6, abs=1e-9), i


def test_rope_scores_depend_only_on_offset():
    hd = 64
    q = RNG.standard_normal(hd)
    k = RNG.standard_normal(hd)
    a = np.dot(oracle.rope(q, 1, hd, 100, 5e5), oracle.rope(k, 1, hd, 90, 5e5))
    b = np.dot(oracle.rope(q, 1, hd, 1010, 5e5), oracle.rope(k, 1, hd, 1000, 5e5))
    assert a == pytest.approx(b, rel=1e-11, abs=1e-11)


def test_rope_matches_complex_rotation():
    # (x_2i + i x_2i+1) * exp(i * p * f_i): the complex-number form of the rotation
    hd, nh, p, th = 64, 2, 37, 5e5
    v = RNG.standard_normal(nh * hd)
    out = oracle.rope(v, nh, hd, p, th)
    z = v.reshape(nh, hd // 2, 2)
    z = z[..., 0] + 1j * z[..., 1]
    f = th ** (-np.arange(0, hd, 2) / hd)
    r = z * np.exp(1j * p * f)[None, :]
    ref = np.stack([r.real, r.imag], axis=-1).reshape(-1)
    assert np.allclose(out, ref, rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------
# SiLU / SwiGLU pieces
# ---------------------------------------------------------------------------

def test_silu_matches_scipy_expit():
    from scipy.special import expit
    assert oracle.silu(0.0) == 0.0
    for a in (-30.0, -3.5, -1e-3, 0.25, 1.0, 7.0, 40.0):
        assert oracle.silu(a) == pytest.approx(a * expit(a), rel=1e-15, abs=1e-300)


# ---------------------------------------------------------------------------
# attention (causal softmax, GQA)
# ---------------------------------------------------------------------------

def _f16(a):
    return np.asarray(a, np.float64).astype(np.float16).view(np.uint16)


def _f16v(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


def test_attention_context_one_returns_v0():
    nq, nkv, hd, stride = 4, 2, 64, 8
    q = RNG.standard_normal(nq * hd)
    K = _f16(RNG.standard_normal((nkv, stride, hd)))
    V = _f16(RNG.standard_normal((nkv, stride, hd)))
    out = oracle.attention(q, K, V, nq, nkv, hd, 1).reshape(nq, hd)
    for h in range(nq):
        assert np.array_equal(out[h], _f16v(V[h // 2, 0]))


def test_attention_identical_keys_give_mean_of_values():
    nq, nkv, hd, n = 2, 1, 32, 9
    q = RNG.standard_normal(nq * hd)
    k1 = RNG.standard_normal(hd)
    K = _f16(np.broadcast_to(k1, (nkv, n, hd)))
    V = _f16(RNG.standard_normal((nkv, n, hd)))
    out = oracle.attention(q, K, V, nq, nkv, hd, n).reshape(nq, hd)
    mean = _f16v(V[0]).mean(axis=0)
    for h in range(nq):
        assert np.allclose(out[h], mean, rtol=1e-14, atol=1e-15)


def test_attention_causal_keys_beyond_context_ignored():
    nq, nkv, hd, stride, n = 2, 1, 16, 12, 5
    q = RNG.standard_normal(nq * hd)
    K = _f16(RNG.standard_normal((nkv, stride, hd)))
    V = _f16(RNG.standard_normal((nkv, stride, hd)))
    a = oracle.attention(q, K, V, nq, nkv, hd, n)
    K2, V2 = K.copy(), V.copy()
    K2[:, n:] = _f16(np.full((nkv, stride - n, hd), 50.0))
    V2[:, n:] = _f16(np.full((nkv, stride - n, hd), 9.0))
    assert np.array_equal(a, oracle.attention(q, K2, V2, nq, nkv, hd, n))


def test_attention_dominant_score_is_one_hot():
    hd, n = 16, 6
    K = np.zeros((1, n, hd))
    K[0, 3, 0] = 60.0
    q = np.zeros(hd)
    q[0] = 60.0                                  # score 60*60/4 = 900 at t = 3, 0 elsewhere
    V = RNG.standard_normal((1, n, hd))
    out = oracle.attention(q, _f16(K), _f16(V), 1, 1, hd, n)
    assert np.allclose(out, _f16v(_f16(V))[0, 3], rtol=0, atol=1e-300)


@pytest.mark.parametrize("nq,nkv,hd,n", [(4, 2, 64, 17), (14, 2, 64, 33), (15, 5, 64, 40), (32, 8, 128, 70)])
def test_attention_matches_torch_sdpa_gqa(nq, nkv, hd, n):
    q = RNG.standard_normal(nq * hd)
    K = _f16(RNG.standard_normal((nkv, n + 3, hd)))
    V = _f16(RNG.standard_normal((nkv, n + 3, hd)))
    out = oracle.attention(q, K, V, nq, nkv, hd, n)
    tq = torch.from_numpy(q.reshape(1, nq, 1, hd))
    tk = torch.from_numpy(_f16v(K)[:, :n].reshape(1, nkv, n, hd).copy())
    tv = torch.from_numpy(_f16v(V)[:, :n].reshape(1, nkv, n, hd).copy())
    ref = F.scaled_dot_product_attention(tq, tk, tv, enable_gqa=True).reshape(-1).numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_attention_gqa_equals_mha_with_replicated_heads():
    nq, nkv, hd, n = 6, 2, 32, 11
    q = RNG.standard_normal(nq * hd)
    K = _f16(RNG.standard_normal((nkv, n, hd)))
    V = _f16(RNG.standard_normal((nkv, n, hd)))
    gqa = oracle.attention(q, K, V, nq, nkv, hd, n)
    rep = np.repeat(np.arange(nkv), nq // nkv)     # head h -> kv head h // 3
    mha = oracle.attention(q, K[rep], V[rep], nq, nq, hd, n)
    assert np.array_equal(gqa, mha)


def test_softmax_weights_sum_to_one_via_constant_values():
    # with every value vector equal to 1, the output is the softmax row sum
    nq, nkv, hd, n = 4, 1, 8, 300
    q = RNG.standard_normal(nq * hd) * 3
    K = _f16(RNG.standard_normal((nkv, n, hd)))
    V = _f16(np.ones((nkv, n, hd)))
    out = oracle.attention(q, K, V, nq, nkv, hd, n)
    assert np.allclose(out, 1.0, rtol=0, atol=1e-14)


def test_softmax_shift_invariance():
    # adding the same vector c to every key shifts all scores by q.c/sqrt(hd)
    nq, nkv, hd, n = 1, 1, 16, 7
    q = np.zeros(hd)
    q[0] = 1.0
    base = np.round(RNG.standard_normal((nkv, n, hd)) * 8) / 8   # exact in fp16
    shifted = base.copy()
    shifted[:, :, 0] += 4.0
    V = _f16(RNG.standard_normal((nkv, n, hd)))
    a = oracle.attention(q, _f16(base), V, nq, nkv, hd, n)
    b = oracle.attention(q, _f16(shifted), V, nq, nkv, hd, n)
    assert np.allclose(a, b, rtol=1e-14, atol=1e-15)


# ---------------------------------------------------------------------------
# argmax
# ---------------------------------------------------------------------------

def test_argmax_first_of_fp32_max():
    v = RNG.standard_normal(5000)
    assert oracle.argmax_f32(v) == int(np.argmax(v.astype(np.float32)))
    w = np.zeros(10)
    w[3] = w[7] = 2.0
    assert oracle.argmax_f32(w) == 3
    # values that differ in fp64 but tie in fp32: the first one wins
    t = np.zeros(8)
    t[2] = 1.0 + 2.0 ** -40
    t[5] = 1.0 + 2.0 ** -30
    assert oracle.argmax_f32(t) == 2
