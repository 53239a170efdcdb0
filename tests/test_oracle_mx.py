"""Pins of the oracle's MXFP4 decoding (E2M1 elements, E8M0 scales, the
packed layout) and of the generator's MXFP4 quantiser, against what the OCP
microscaling format definition fixes: the representable E2M1 values, torch's
own E8M0 decode, hand-built layouts, exact round trips and the nearest-value
rule."""
import numpy as np
import pytest
import torch

import oracle
from synth import quantize_mxfp4

# E2M1 from its definition (sign bit 3, exponent bits 2-1 with bias 1, one
# mantissa bit; exponent 0 is subnormal): codes 0..7 are the non-negative
# values in increasing order, codes 8..15 their negatives
E2M1_VALUES = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_every_code():
    got = oracle.e2m1_decode(np.arange(16, dtype=np.uint8))
    want = np.array(E2M1_VALUES + [-v for v in E2M1_VALUES])
    assert np.array_equal(got, want)
    assert np.signbit(got[8])  # code 8 is -0
    # the high nibble of a byte is ignored
    assert np.array_equal(oracle.e2m1_decode(np.arange(16, dtype=np.uint8) | 0xA0), got)


def test_e8m0_every_code_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = oracle.e8m0_decode(codes.numpy())
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_dequant_layout_nibbles_and_blocks():
    K, N = 64, 3
    packed = np.zeros((K // 2, N), dtype=np.uint8)
    packed[0, 0] = 0x21            # row 0 <- code 1 (0.5), row 1 <- code 2 (1.0)
    packed[16, 1] = 0x9F           # row 32 <- code 15 (-6), row 33 <- code 9 (-0.5)
    packed[31, 2] = 0x70           # row 62 <- 0, row 63 <- code 7 (6)
    scales = np.full((K // 32, N), 127, dtype=np.uint8)
    scales[0, 0] = 128             # 2.0 for rows 0..31 of column 0
    scales[1, 1] = 125             # 0.25 for rows 32..63 of column 1
    W = oracle.dequant_mxfp4(packed, scales)
    assert W.shape == (K, N)
    assert W[0, 0] == 1.0 and W[1, 0] == 2.0
    assert W[32, 1] == -1.5 and W[33, 1] == -0.125
    assert W[62, 2] == 0.0 and W[63, 2] == 6.0
    assert np.count_nonzero(W) == 5


def _block_of(values, k):
    """One column of 32 values times 2^k, as a float32 [32, 1] matrix."""
    return torch.tensor(np.asarray(values, dtype=np.float64) * 2.0 ** k, dtype=torch.float32)[:, None]


@pytest.mark.parametrize("k", [-8, 0, 3])
def test_quantiser_round_trips_representable_blocks(k):
    rng = np.random.default_rng(k + 20)
    vals = rng.choice(E2M1_VALUES, size=32) * rng.choice([-1.0, 1.0], size=32)
    vals[5] = 6.0  # the block's amax is 6 * 2^k, so its scale is 2^k
    w = _block_of(vals, k)
    q, s = quantize_mxfp4(w)
    assert int(s[0, 0]) == 127 + k
    assert np.array_equal(oracle.dequant_mxfp4(q, s), w.double().numpy())


@pytest.mark.parametrize("x,expect", [
    (0.25, 0.0), (0.75, 1.0), (1.25, 1.0), (1.75, 2.0), (2.5, 2.0), (3.5, 4.0), (5.0, 4.0),  # ties to even
    (0.3, 0.5), (2.6, 3.0), (7.5, 6.0),                                                     # nearest, saturation
])
def test_quantiser_ties_and_saturation(x, expect):
    vals = np.zeros(32)
    vals[0] = 4.0   # amax 4..7.99 keeps the scale at 1
    vals[1] = x
    if x > 4.0:
        vals[0] = x
    q, s = quantize_mxfp4(_block_of(vals, 0))
    assert int(s[0, 0]) == 127
    assert oracle.dequant_mxfp4(q, s)[1, 0] == expect


def test_quantiser_zero_block_and_nearest():
    w = torch.zeros(64, 2)
    w[32:, 1] = torch.randn(32) * 0.02
    q, s = quantize_mxfp4(w)
    assert int(s[0, 0]) == 127 and int(s[1, 0]) == 127 and not q[:, 0].any()
    # every stored value is the representable value nearest to w / scale,
    # unless w / scale lies beyond the largest magnitude 6
    rng = torch.Generator().manual_seed(3)
    w = torch.randn(256, 16, generator=rng) * 0.02
    q, s = quantize_mxfp4(w)
    sc = np.repeat(oracle.e8m0_decode(s), 32, axis=0)
    x = w.double().numpy() / sc
    got = oracle.dequant_mxfp4(q, s) / sc
    grid = np.array(E2M1_VALUES)
    best = np.min(np.abs(np.abs(x)[..., None] - grid), axis=-1)
    inside = np.abs(x) <= 6.0
    assert np.array_equal(np.abs(np.abs(x) - np.abs(got))[inside], best[inside])
    assert np.all(got[~inside] == np.sign(x[~inside]) * 6.0)


def test_layer_reads_mxfp4_experts_by_their_byte_scales():
    # E8M0 byte scales select the MXFP4 decode, fp32 scales the E4M3 one
    E, H, F = 2, 64, 32
    W1 = [quantize_mxfp4(torch.randn(H, F) * 0.02) for _ in range(E)]
    d = {"X": torch.zeros(1, H), "Wg": torch.zeros(H, E), "gate_bias": None,
         "W1": torch.stack([q for q, _ in W1]), "S1": torch.stack([s for _, s in W1]),
         "W3": torch.stack([q for q, _ in W1]), "S3": torch.stack([s for _, s in W1]),
         "W2": torch.zeros(E, F, H), "S2": None}
    L = oracle.Layer(d, 1)
    for e in range(E):
        assert np.array_equal(L.expert(e)[0], oracle.dequant_mxfp4(*W1[e]))
    from synth import quantize_e4m3_blocks
    c, s = quantize_e4m3_blocks(torch.randn(128, 128) * 0.02)
    d8 = dict(d, W1=c[None], S1=s[None], W3=c[None], S3=s[None], W2=torch.zeros(1, 128, 128))
    d8["X"], d8["Wg"] = torch.zeros(1, 128), torch.zeros(128, 1)
    assert np.array_equal(oracle.Layer(d8, 1).expert(0)[0], oracle.dequant_blocks(c, s))
