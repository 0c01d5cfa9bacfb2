"""The seeded input generator: Philox-4x32-10 known-answer vectors (Random123
kat_vectors, the published test set of the Philox paper's reference code), the
C build against its numpy twin, bf16 rounding, and the workload shapes."""
import numpy as np

from synth import philox
from synth.bf16 import bf16_bits_to_f32, f32_to_bf16_bits, round_to_bf16
from synth.configs import CONFIGS
from synth import params


def _kat(ctr, key):
    c = [np.array([x], dtype=np.uint64) for x in ctr]
    return [int(w[0]) for w in philox.philox4x32_10(*c, *key)]


def test_philox_known_answers():
    assert _kat([0, 0, 0, 0], [0, 0]) == [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]
    f = 0xFFFFFFFF
    assert _kat([f, f, f, f], [f, f]) == [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]
    assert _kat([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0]) == \
        [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]


def test_c_words_match_numpy_twin():
    for first in (0, 12345, (1 << 32) - 3):
        a = philox.philox_words(7, 300, first, 777, use_c=True)
        b = philox.philox_words(7, 300, first, 777, use_c=False)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_c_normals_match_numpy_twin():
    a = philox.normals_f32(0, 17, 20001, 0.02)
    b = philox.normals_reference(0, 17, 20001, 0.02)
    assert np.max(np.abs(a.view(np.int32) - b.view(np.int32))) <= 1
    assert abs(float(philox.normals_f32(0, 3, 400000).std()) - 1.0) < 0.01


def test_bf16_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.5, np.inf],
                 dtype=np.float32)
    r = round_to_bf16(x)
    # ties go to even mantissa; above-tie rounds up
    np.testing.assert_array_equal(r, np.array([1.0, 1.0, 1.0 + 4 * 2 ** -8, 1.0 + 2 * 2 ** -8,
                                               -2.5, np.inf], dtype=np.float32))
    bits = f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(bf16_bits_to_f32(bits)[0])


def test_workload_shapes():
    c = CONFIGS
    assert c["tiny_f32"].tokens == 16 and c["tiny_f32"].patch_dim == 16
    assert c["image_s_bf16"].tokens == 1024 and c["image_s_bf16"].patch_dim == 64
    assert c["wan1p3b_bf16"].tokens == 32760 and c["wan14b_bf16"].tokens == 32760
    assert c["image_l_bf16"].tokens == 4096
    for cfg in c.values():
        assert sum(cfg.rope) == cfg.head_dim and all(r % 2 == 0 for r in cfg.rope)
        assert cfg.heads * cfg.head_dim == cfg.hidden


def test_param_counts():
    def count(cfg):
        n = sum(int(np.prod(s)) for s in params.global_shapes(cfg).values())
        return n + cfg.num_blocks * sum(int(np.prod(s)) for s in params.block_shapes(cfg).values())
    assert abs(count(CONFIGS["image_s_bf16"]) / 1e9 - 0.118) < 0.002
    assert abs(count(CONFIGS["wan1p3b_bf16"]) / 1e9 - 1.416) < 0.01
    assert abs(count(CONFIGS["wan14b_bf16"]) / 1e9 - 14.26) < 0.05


def test_params_deterministic_and_bf16_exact():
    cfg = CONFIGS["tiny_f32"]
    a = params.make_params(cfg)
    b = params.make_params(cfg)
    assert np.array_equal(a["blocks"][0]["qkv_w"], b["blocks"][0]["qkv_w"])
    cfg2 = CONFIGS["image_s_bf16"]
    w = params.make_block_params(cfg2, 3)["o_w"]
    assert np.array_equal(round_to_bf16(w), w)
    assert abs(float(w.std()) - 0.02) < 1e-3
