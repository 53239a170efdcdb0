"""Pins of the oracle's E4M3 activation quantisation (encoder, per-row
quantiser, mirror mode) against what the OCP E4M3 definition and the
quantisation rule fix: round trips over every code, the tie cases, saturation,
the scale of each row group, the format's error bound and the exact result on
values the format represents."""
import numpy as np
import pytest

import oracle


def test_encode_inverts_decode_on_every_finite_code():
    codes = np.arange(256, dtype=np.uint8)
    finite = (codes & 0x7F) != 0x7F
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes[finite])), codes[finite])


@pytest.mark.parametrize("x,code", [
    (1.0625, 0x38),        # halfway between 1.0 (mantissa 0) and 1.125 (mantissa 1): even -> 1.0
    (1.1875, 0x3A),        # halfway between 1.125 (m 1) and 1.25 (m 2): even -> 1.25
    (2.0 ** -10, 0x00),    # halfway between 0 and the smallest subnormal 2^-9: even -> 0
    (3 * 2.0 ** -10, 0x02),  # halfway between 2^-9 (code 1) and 2^-8 (code 2): even -> 2^-8
    (-1.0625, 0xB8),
    (432.0, 0x7E),         # halfway between 416 (m 5) and 448 (m 6): even -> 448
    (448.0, 0x7E),
    (1000.0, 0x7E),        # saturates
    (-1e6, 0xFE),
    (-0.0, 0x80),
    (0.0, 0x00),
])
def test_encode_ties_and_saturation(x, code):
    assert int(oracle.e4m3_encode(np.float64(x))) == code


def test_encode_is_nearest():
    # every representable magnitude is within half a spacing of the input
    rng = np.random.default_rng(3)
    x = rng.uniform(-448, 448, 20000) * rng.choice([1.0, 1e-2, 1e-3], 20000)
    v = oracle.e4m3_decode(oracle.e4m3_encode(x))
    table = np.sort(np.unique(np.abs(oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8)))))
    best = np.min(np.abs(np.abs(x)[:, None] - table[None, :]), axis=1)
    assert np.array_equal(np.abs(np.abs(x) - np.abs(v)), best)
    assert np.all(np.sign(v[v != 0]) == np.sign(x[v != 0]))


def test_quantize_rows_scales_and_exact_groups():
    # each (row, group) gets its own scale amax/448; a group whose values are
    # E4M3 values times a power of two with amax 448*s comes back exactly
    rng = np.random.default_rng(4)
    R, C = 3, 512
    codes = rng.integers(0, 0x7E, size=(R, C)).astype(np.uint8)
    base = oracle.e4m3_decode(codes)
    base[:, ::128] = 448.0  # every group's amax is 448 before scaling
    pw = 2.0 ** rng.integers(-6, 4, size=(R, C // 128))
    x = (base.reshape(R, C // 128, 128) * pw[:, :, None]).reshape(R, C).astype(np.float32)
    q, s = oracle.quantize_rows_e4m3(x)
    assert s.dtype == np.float32 and s.shape == (R, C // 128)
    assert np.array_equal(s.astype(np.float64), pw)
    assert np.array_equal(oracle.dequant_rows(q, s), x.astype(np.float64))


def test_quantize_rows_zero_group_and_error_bound():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 384)).astype(np.float32)
    x[1, 128:256] = 0.0
    q, s = oracle.quantize_rows_e4m3(x)
    assert s[1, 1] == 1.0 and not q[1, 128:256].any()
    # normal-range values: relative error at most half the 3-bit mantissa spacing
    xd = oracle.dequant_rows(q, s)
    sc = np.repeat(s.astype(np.float64), 128, axis=1)
    normal = np.abs(x) / sc >= 2.0 ** -6
    rel = np.abs(xd - x)[normal] / np.abs(x)[normal]
    assert rel.max() <= 2.0 ** -4 * (1 + 1e-6)
    # the largest magnitude of each group maps to 448 exactly
    for r in range(4):
        for g in range(3):
            blk = np.abs(x[r, 128 * g:128 * (g + 1)])
            if blk.max() > 0:
                assert np.abs(oracle.e4m3_decode(q[r, 128 * g:128 * (g + 1)])).max() == 448.0


def test_mirror_mode_is_the_exact_ffn_on_representable_activations():
    # activations that the quantiser reproduces exactly (E4M3 values, group
    # amax 448) and weights that keep h representable leave the FFN unchanged
    rng = np.random.default_rng(6)
    x = oracle.e4m3_decode(rng.integers(0, 0x7E, size=(5, 128)).astype(np.uint8))
    x[:, 0] = 448.0
    W1 = np.zeros((128, 128)); W3 = np.zeros((128, 128)); W2 = rng.standard_normal((128, 64))
    y_exact = oracle.swiglu_ffn(x, W1, W3, W2)
    y_mirror = oracle.swiglu_ffn(x, W1, W3, W2, act_quant=True)
    assert np.array_equal(y_exact, y_mirror)  # h = 0 quantises exactly
    W1 = rng.standard_normal((128, 128)) * 0.02
    W3 = rng.standard_normal((128, 128)) * 0.02
    y_exact = oracle.swiglu_ffn(x, W1, W3, W2)
    y_mirror = oracle.swiglu_ffn(x, W1, W3, W2, act_quant=True)
    # only h is rounded here (x is exact): bf16 storage (relative 2^-8 at
    # most) then E4M3 (2^-4 relative, or half the subnormal spacing), through W2
    h = oracle.silu(x @ W1) * (x @ W3)
    bound = (2.0 ** -4 + 2.0 ** -7) * np.abs(h) @ np.abs(W2) + 2.0 ** -9 * np.abs(h).max() * np.abs(W2).sum(axis=0)
    assert np.all(np.abs(y_mirror - y_exact) <= bound + 1e-12)


def test_round_bf16_matches_torch_and_ties():
    import torch
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-8, 8, 5000),
                        [0.0, -0.0, 1.0, 3.0e38, -1e-40]])
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(oracle.round_bf16(x), ref)
    # ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 (bf16 has 7 stored bits): even -> 1
    assert oracle.round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert oracle.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6


def test_mirror_quantises_only_fp8_shared_experts():
    # activation quantisation is part of the W8A8 form of E4M3 experts: the
    # mirror applies it to an E4M3 shared expert and leaves a bf16 one exact
    rng = np.random.default_rng(9)
    T, H, F, E = 3, 128, 128, 2
    X = rng.standard_normal((T, H)).astype(np.float32)
    ones = np.ones((E, 1, 1), dtype=np.float32)
    codes = [rng.integers(0x20, 0x38, size=(E, H, F)).astype(np.uint8) for _ in range(3)]
    routed = dict(X=X, Wg=(rng.standard_normal((H, E)) * 0.02).astype(np.float32), gate_bias=None,
                  W1=codes[0], W3=codes[1], W2=codes[2], S1=ones, S3=ones, S2=ones)
    shared_codes = [rng.integers(0x20, 0x38, size=(H, F)).astype(np.uint8) for _ in range(3)]
    one = np.ones((1, 1), dtype=np.float32)
    shared_vals = [oracle.dequant_blocks(c, one) for c in shared_codes]
    d_bf16 = dict(routed, Ws1=shared_vals[0].astype(np.float32), Ws3=shared_vals[1].astype(np.float32),
                  Ws2=shared_vals[2].astype(np.float32), Ss1=None, Ss3=None, Ss2=None)
    d_fp8 = dict(routed, Ws1=shared_codes[0], Ws3=shared_codes[1], Ws2=shared_codes[2], Ss1=one, Ss3=one, Ss2=one)
    x64 = X.astype(np.float64)
    exact = oracle.swiglu_ffn(x64, *shared_vals)
    mirrored = oracle.swiglu_ffn(x64, *shared_vals, act_quant=True)
    assert not np.array_equal(exact, mirrored)  # the two readings differ on these inputs
    out_bf16 = oracle.forward_tokens(oracle.Layer(d_bf16, 1), np.arange(T), act_quant=True)
    out_fp8 = oracle.forward_tokens(oracle.Layer(d_fp8, 1), np.arange(T), act_quant=True)
    assert np.array_equal(out_bf16["S"], exact)
    assert np.array_equal(out_fp8["S"], mirrored)
    # the routed part is mirrored the same way in both
    assert np.array_equal(out_bf16["y"], out_fp8["y"])
