"""The seeded input generators against the published definitions."""
import numpy as np

from synth import philox4x32_10, splitmix64, config_by_name, CONFIGS
from synth.philox import irwin_hall8_int
from synth.workload import f32_to_bf16_bits, bf16_bits_to_f32


def test_philox_known_answers():
    # known-answer vectors published with the Random123 library (Philox4x32-10)
    cases = [
        ((0, 0, 0, 0), (0, 0), (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
        ((0xffffffff,) * 4, (0xffffffff,) * 2, (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
        ((0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344), (0xa4093822, 0x299f31d0),
         (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
    ]
    for ctr, key, want in cases:
        got = tuple(int(v) for v in philox4x32_10(*ctr, *key))
        assert got == want


def test_splitmix64_known_answers():
    # first outputs of splitmix64 seeded with 1234567 (reference C implementation)
    x, out = 1234567, []
    for _ in range(3):
        out.append(splitmix64(x))
        x = (x + 0x9E3779B97F4A7C15) & ((1 << 64) - 1)
    assert out == [6457827717110365317, 3203168211198807973, 9817491932198370423]


def test_irwin_hall_moments():
    x = irwin_hall8_int((12345, 678), np.arange(20000), np.arange(16), 0).astype(np.float64)
    z = x * np.sqrt(1.5) / 65536
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01
    assert np.abs(x).max() <= 262140


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 1 + 2 ** -9], dtype=np.float32)
    y = bf16_bits_to_f32(f32_to_bf16_bits(x))
    assert list(y) == [1.0, 1.0, 1.0 + 2 ** -6, -2.5, 1.0]


def test_config_shapes():
    c4 = config_by_name("c4")
    assert c4.units == 288 and c4.n == 1 << 20
    s_log = config_by_name("c2").sigma(0, 0, 0)
    assert s_log.min() >= 0.1 and s_log.max() <= 4.0
    s_par = c4.sigma(0, 0, 5)
    assert s_par.min() >= 0.1 and s_par.max() <= 1000.0
    assert config_by_name("c5").capacity % 64 == 0
    r = config_by_name("c5").rotation(3, 2).astype(np.float64)
    assert np.allclose(r.T @ r, np.eye(128), atol=1e-5)
    assert [c.name for c in CONFIGS] == ["c1", "c2", "c3", "c4", "c5"]
