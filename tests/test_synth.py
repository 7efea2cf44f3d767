"""Checks of the seeded input generator (shared by both sides)."""
import numpy as np

from synth import config_by_name, generate, bf16_bits_from_f32, f32_from_bf16_bits
from synth.inputs import apply_rope, rope_frequencies


def test_rope_expectation_form():
    # The MTraining review (page 1, section 三.1) writes the rotary logit of two
    # position-independent vectors as sum_i phi_i A_i + sum_i psi_i B_i with
    # phi_i = cos((n-m) theta_{i mod d/2}), psi_i = (-1)^[i >= d/2] sin(...).
    # With rotate-half RoPE the constants are A_i = a_i b_i, B_i = a_i b_{(i+d/2) mod d}.
    d = 16
    rng = np.random.default_rng(0)
    a, b = rng.standard_normal(d), rng.standard_normal(d)
    theta = rope_frequencies(d, 10000.0, 1.0, 1)
    pos = np.arange(40)
    qa = apply_rope(np.tile(a, (40, 1)), pos, theta)
    kb = apply_rope(np.tile(b, (40, 1)), pos, theta)
    A = a * b
    B = a * np.roll(b, -d // 2)
    for n in range(40):
        for m in range(40):
            i = np.arange(d)
            ang = (n - m) * theta[i % (d // 2)]
            expect = (np.cos(ang) * A).sum() + (np.where(i >= d // 2, -1.0, 1.0) * np.sin(ang) * B).sum()
            assert abs(qa[n] @ kb[m] - expect) < 1e-12


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.14159], dtype=np.float32)
    r = f32_from_bf16_bits(bf16_bits_from_f32(x))
    assert r[0] == 1.0 and r[1] == 1.0            # tie to even
    assert r[2] == np.float32(1.0 + 4 * 2 ** -8)  # tie to even (up)
    assert r[3] == -2.5
    assert abs(r[4] - 3.140625) < 1e-7


def test_generation_is_deterministic_and_sliceable():
    cfg = config_by_name("qwen32k", N=1024, Hq=4, Hkv=2, n_out=3)
    full = generate(cfg)
    part = generate(cfg, heads={"q": [3], "k": [1]}, rows=slice(512, 1024), tensors=("q", "k"))
    assert (part["q"][0] == full["q"][3, 512:]).all()
    assert (part["k"][0] == full["k"][1, 512:]).all()
    again = generate(cfg)
    assert all((again[t] == full[t]).all() for t in ("q", "k", "v", "do"))
    # bf16-exact values
    bits = bf16_bits_from_f32(full["q"])
    assert (f32_from_bf16_bits(bits) == full["q"]).all()
    # outlier rows of K carry the large norm
    norms = np.linalg.norm(full["k"][0].astype(np.float64), axis=1)
    assert norms[full["outliers"]].min() > np.median(norms) * 3
