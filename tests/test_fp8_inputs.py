"""The E4M3 encoder of the input generator, checked against the format's
definition (the oracle's decoder is a separate implementation)."""

import numpy as np

from causal_attention_neox_amd import workloads as W
from oracle import neox_oracle as orc


def test_encoding_round_trips_every_finite_code():
    codes = np.r_[np.arange(127), np.arange(129, 255)]  # -0 (128) encodes as +0
    np.testing.assert_array_equal(W.e4m3_encode(orc.e4m3_decode(codes)), codes)


def test_encoding_rounds_to_nearest_with_ties_to_even():
    # midpoints between neighbouring codes go to the even code
    vals = orc.e4m3_decode(np.arange(127))
    mid = (vals[:-1] + vals[1:]) / 2
    codes = W.e4m3_encode(mid)
    lo = np.arange(126)
    np.testing.assert_array_equal(codes, np.where(lo % 2 == 0, lo, lo + 1))
    # just off the midpoint goes to the nearer code
    np.testing.assert_array_equal(W.e4m3_encode(mid * (1 - 1e-9)), lo)
    np.testing.assert_array_equal(W.e4m3_encode(mid * (1 + 1e-9)), lo + 1)


def test_encoding_saturates_and_keeps_sign():
    assert W.e4m3_encode(np.array([1e6]))[0] == 0x7E
    assert W.e4m3_encode(np.array([-1e6]))[0] == 0xFE
    assert W.e4m3_encode(np.array([-0.5]))[0] == 0xB0


def test_generated_fp8_inputs_use_the_full_range():
    wl = W.Fp8Workload("t", B=1, H=2, S=64, D=64, seed=3)
    inp = W.generate_fp8(wl)
    for codes, scale in zip((inp.q8, inp.k8, inp.v8), inp.scales):
        v = orc.e4m3_decode(codes)
        assert np.abs(v).max() == 448.0           # amax maps to the largest code
        assert np.all(np.isfinite(v)) and scale > 0


def test_encoding_matches_torch_float8_e4m3fn():
    """Independent check of the rounding: torch's float8_e4m3fn cast (the same
    OCP format) gives the same codes on 2e5 float32 samples across the whole
    finite range, subnormals included (|x| <= 448: torch's cast does not
    saturate)."""
    torch = __import__("pytest").importorskip("torch")
    rng = np.random.default_rng(2026)
    mag = np.exp2(rng.uniform(-12.0, np.log2(448.0), 200_000))
    x = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    x[:1000] = np.minimum(np.abs(x[:1000]), 448.0)  # some values at the top binade
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(W.e4m3_encode(x.astype(np.float64)), ref)
