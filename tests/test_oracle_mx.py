"""Pins for the oracle's MXFP8 E4M3 conversion (blog post "What it is selling":
MXFP8 E4M3 with prepared weights; the OCP MX v1.0 conversion rule).

* E4M3 code points fixed by the format: 448 is 0x7E, 2^-6 is the smallest
  normal (0x08), 2^-9 the smallest subnormal (0x01), ties to even in both
  ranges, saturation to +-448, signed zero.
* Every code round-trips through decode/encode.
* Every finite BF16 value, clamped to +-448, encodes exactly as torch's own
  float8_e4m3fn cast (a library routine, round to nearest even).
* The shared exponent of a block is floor(log2(amax)) - 8 as a biased E8M0
  byte, clamped to [0, 254]; the dequantized block is within half an E4M3
  step of the input (or saturates at the top).
"""
import math

import numpy as np
import torch


def test_code_points(orc):
    enc, dec = orc.e4m3_encode, orc.e4m3_decode
    assert enc(448.0) == 0x7E and dec(0x7E) == 448.0
    assert enc(-448.0) == 0xFE
    assert enc(2.0 ** -6) == 0x08 and dec(0x08) == 2.0 ** -6
    assert enc(2.0 ** -9) == 0x01 and dec(0x01) == 2.0 ** -9
    assert dec(0x07) == 7 * 2.0 ** -9                      # largest subnormal
    assert enc(1.0) == 0x38 and dec(0x38) == 1.0
    assert enc(0.0) == 0x00 and enc(-0.0) == 0x80
    assert enc(2.0 ** -10) == 0x00                          # tie between 0 and 2^-9 -> even (0)
    assert enc(3 * 2.0 ** -10) == 0x02                      # tie between 1 and 2 steps -> 2
    assert enc(1.0 + 1 / 16) == 0x38                        # tie between 1.0 and 1.125 -> 1.0
    assert enc(1.0 + 3 / 16) == 0x3A                        # tie between 1.125 and 1.25 -> 1.25
    assert enc(464.0) == 0x7E and enc(1e30) == 0x7E         # saturate, never NaN
    assert enc(15 * 2.0 ** -10) == 0x08                     # 7.5 steps rounds up into the normals
    assert math.isnan(dec(0x7F)) and math.isnan(dec(0xFF))


def test_all_codes_round_trip(orc):
    for c in range(256):
        if c in (0x7F, 0xFF):
            continue
        assert orc.e4m3_encode(orc.e4m3_decode(c)) == c


def test_all_bf16_values_match_torch_cast(orc):
    bits = np.arange(65536, dtype=np.uint32)
    vals = ((bits << 16).view(np.float32))
    finite = np.isfinite(vals)
    vals = np.clip(vals[finite], -448.0, 448.0)
    ref = torch.from_numpy(vals.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = np.array([orc.e4m3_encode(float(v)) for v in vals], np.uint8)
    # torch keeps the sign of values that round to zero as we do
    assert np.array_equal(ours, ref)


def test_scale_byte_rule(orc):
    sb = orc.mx_scale_byte
    assert sb(np.r_[448.0, np.zeros(31)]) == 127            # floor(log2 448) = 8 -> 2^0
    assert sb(np.r_[1.0, np.zeros(31)]) == 119              # 2^-8
    assert sb(np.r_[511.9, np.zeros(31)]) == 127
    assert sb(np.r_[512.0, np.zeros(31)]) == 128
    assert sb(np.zeros(32)) == 0
    assert sb(np.r_[2.0 ** -130, np.zeros(31)]) == 0        # clamped at the bottom
    assert sb(np.r_[-3.0, 0.5, np.zeros(30)]) == 120        # amax uses |v|


def test_block_quantize_error_bound(orc):
    rng = np.random.default_rng(0)
    v = (rng.standard_normal((64, 256)) * np.exp(rng.normal(0, 3, (64, 1)))).astype(np.float32)
    codes, scales = orc.mx_quantize(v)
    back = orc.mx_dequantize(codes, scales).astype(np.float64)
    X = np.repeat(np.exp2(scales.astype(np.float64) - 127), 32, axis=1)
    q = v.astype(np.float64) / X                           # value on the element grid
    # half a step of the E4M3 grid at |q| (step 2^(floor(log2|q|)-3), at least 2^-9)
    step = np.exp2(np.maximum(np.floor(np.log2(np.maximum(np.abs(q), 2.0 ** -6))) - 3, -9))
    err = np.abs(back / X - np.clip(q, -448, 448))
    assert np.all(err <= step / 2 + 1e-12)
    # elements above 448 after scaling saturate to +-448 (the floor rule lets |q| reach 512)
    sat = np.abs(q) > 448.0
    assert np.all(np.abs(back[sat] / X[sat]) == 448.0)
    # grid values survive exactly
    on_grid = np.array([orc.e4m3_decode(c) for c in range(0x00, 0x7F)])
    blk = np.r_[on_grid[-32:]].astype(np.float32)           # amax 448 -> scale byte 127
    c2, s2 = orc.mx_quantize(blk[None, :])
    assert s2[0, 0] == 127
    assert np.array_equal(orc.mx_dequantize(c2, s2)[0], blk)


def test_mx_forward_reduces_to_plain_on_grid_values(orc):
    # When x and every SwiGLU output already sit on their MX grids the quantized
    # forward equals the plain one; with I = 32 and a single token we can force
    # that by making W2 and everything downstream irrelevant: zero scores give +0.
    from mixture_experts_routed_dispatch_amd import inputs
    inp = inputs.generate(T=4, d=64, I=32, E=2, k=1, seed=9)
    y = orc.forward_tokens_mx(inp.x, inp.ids, np.zeros_like(inp.scores), inp.w13, inp.w2)
    assert np.all(y == 0.0)
    yq = orc.forward_tokens_mx(inp.x, inp.ids, inp.scores, inp.w13, inp.w2)
    yp = orc.forward_tokens(inp.x, inp.ids, inp.scores, inp.w13, inp.w2)
    rel = np.linalg.norm(yq - yp) / np.linalg.norm(yp)
    assert 1e-3 < rel < 0.1                                  # quantization noise, not a bug
