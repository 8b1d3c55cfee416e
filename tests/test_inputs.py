"""The seeded input recipe and the bf16 rounding it uses (CPU only)."""
import numpy as np
import torch

from exact_attention_48_amd import inputs as I


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-39).astype(np.float32),          # subnormals
        np.array([0.0, -0.0, np.inf, -np.inf, 3.0e38, -3.0e38, 1.0 + 2**-8, 1.0 + 3 * 2**-8,
                  1.0 + 2**-8 + 2**-20], dtype=np.float32),             # ties to even and just above
    ])
    ours = I.f32_to_bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    back = I.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_nan_stays_nan():
    b = I.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(I.bf16_bits_to_f32(b)[0])


def test_uniform_inputs_are_seeded_and_shaped():
    a = I.make_inputs(2, 5, 4, 2, 8, True, seed=7, with_do=True)
    b = I.make_inputs(2, 5, 4, 2, 8, True, seed=7, with_do=True)
    assert a.q.shape == (2, 5, 4, 8) and a.k.shape == (2, 5, 2, 8) and a.do.shape == (2, 5, 4, 8)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v), (a.do, b.do)):
        assert x.dtype == np.uint16 and np.array_equal(x, y)
    # the draw order is Q, K, V, dO from one generator
    rng = np.random.default_rng(7)
    q = I.f32_to_bf16_bits(rng.standard_normal((2, 5, 4, 8), dtype=np.float32))
    assert np.array_equal(q, a.q)


def test_packed_lengths_drawn_first():
    w = I.WORKLOADS["fwd_causal_varlen16_hq32_hkv8_d128"]
    rng = np.random.default_rng(w.seed)
    lens = I.draw_lengths(rng, w.B, w.len_lo, w.len_hi)
    assert len(lens) == 16 and lens.min() >= 512 and lens.max() <= 16384
    small = I.make_inputs(0, 0, 2, 1, 8, True, seed=w.seed, len_range=(3, 9), n_seqs=5)
    rng = np.random.default_rng(w.seed)
    l2 = I.draw_lengths(rng, 5, 3, 9)
    assert np.array_equal(np.diff(small.cu_seqlens), l2)
    assert small.cu_seqlens.dtype == np.int32 and small.cu_seqlens[0] == 0
    assert small.q.shape == (int(l2.sum()), 2, 8) and small.N == int(l2.max())


def test_counted_flops():
    assert I.counted_flops([4096] * 4, 16, 128, False) == 4 * 4 * 16 * 4096**2 * 128
    assert abs(I.counted_flops([4096] * 4, 16, 128, False) - 5.498e11) / 5.498e11 < 1e-3
    assert abs(I.counted_flops([16384] * 2, 16, 128, True) - 2.199e12) / 2.199e12 < 1e-3
    assert abs(I.counted_flops([8192] * 2, 16, 128, True, backward=True) - 1.3744e12) / 1.3744e12 < 1e-3


def test_scale_is_float32_rounded():
    assert I.WORKLOADS["fwd_b1_h2_n256_d64"].scale == 0.125
    s = I.WORKLOADS["fwd_b4_h16_n4096_d128"].scale
    assert s == float(np.float32(1 / np.sqrt(128)))


def test_e4m3_encoder_round_trips_and_rounds_to_even():
    import oracle
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_to_float(codes)
    keep = ~np.isnan(vals) & (codes != 0x80)                # -0 encodes as +0
    assert np.array_equal(I.f32_to_e4m3_bits(vals[keep]), codes[keep])
    # halfway cases go to the even code; beyond 448 saturates
    got = I.f32_to_e4m3_bits(np.array([1.0625, 1.1875, 2.0 ** -10, 3 * 2.0 ** -10, 500.0, -1e9, np.nan]))
    assert got.tolist() == [0x38, 0x3A, 0x00, 0x02, 0x7E, 0xFE, 0x7F]


def test_bf16_ulp_is_the_spacing_of_bf16_values():
    """The O gate's ulp (tests/gpu_helpers.py) against the bf16 grid itself: the
    distance from a bf16 value to the next one up."""
    from tests import gpu_helpers as H
    rng = np.random.default_rng(5)
    x = rng.standard_normal(4000) * np.exp2(rng.integers(-6, 6, 4000))
    bits = I.f32_to_bf16_bits(x.astype(np.float32))
    v = I.bf16_bits_to_f64(bits)
    up = I.bf16_bits_to_f64((bits.astype(np.uint32) + 1).astype(np.uint16))
    np.testing.assert_array_equal(np.abs(up - v), H.bf16_ulp(v))
    assert H.o_bound(np.array([0.5, 1.99, 2.0, 3.9, 4.0]))[[0, 1, 2, 4]].tolist() == [1e-2, 1e-2, 2 ** -6, 2 ** -5]
