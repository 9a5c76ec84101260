"""The seeded generators: reproducible, nested in T, and with the stated
shapes and value ranges."""
import numpy as np

from bit_adapters_amd import synth as S


def test_reproducible_and_nested():
    a = S.make_x(2, 4)
    b = S.make_x(2, 16)
    assert np.array_equal(a, b[:4])
    assert np.array_equal(S.make_x(2, 4), a)
    la, lb = S.make_layer(1), S.make_layer(1)
    for ta, tb in zip(la["terms"], lb["terms"]):
        for k in ta:
            assert np.array_equal(ta[k], tb[k])


def test_config1_shapes_and_ranges():
    L = S.make_layer(1)
    t = L["terms"][0]
    assert t["b1"].shape == (512, 256) and t["b2"].shape == (256, 512)
    assert set(np.unique(t["b1"])) == {-1, 1}
    for k in ("alpha", "beta", "gamma"):
        assert t[k].dtype == np.float16
        assert t[k].min() >= 0.5 and t[k].max() <= 1.5
    assert abs(float((t["b2"] > 0).mean()) - 0.5) < 0.01
    x = S.make_x(1, 1, "i8")
    assert x.dtype == np.int8 and x.min() >= -127


def test_decaying_scales():
    L = S.make_layer(4)
    assert len(L["terms"]) == 3
    means = [float(t["alpha"].astype(np.float64).mean()) for t in L["terms"]]
    assert means[0] > 1.8 * means[1] > 3.2 * means[2]


def test_bf16_rounding():
    v = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 0.0], dtype=np.float32)
    b = S.f32_to_bf16_bits(v)
    back = (b.astype(np.uint32) << 16).view(np.float32)
    assert back[0] == 1.0 and back[1] == 1.0  # tie to even
    assert back[2] == 1.0 + 2 ** -7 and back[3] == -2.5 and back[4] == 0.0


def test_adapter_layer():
    L = S.make_layer(3, R=16)
    assert L["w0"].shape == (4096, 4096) and L["w0"].dtype == np.uint16
    assert L["terms"][0]["b1"].shape == (4096, 16)
