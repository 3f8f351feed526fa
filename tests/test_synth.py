"""The seeded generator against SplitMix64's published outputs and its own
distribution contracts.  CPU only."""
import numpy as np

import synth


def test_splitmix64_published_vectors():
    # state 0 and state 1234567: first outputs of the reference SplitMix64
    assert int(synth.splitmix64(0, 0, 1)[0]) == 0xE220A8397B1DCDAF
    assert int(synth.splitmix64(1234567, 0, 1)[0]) == 6457827717110365317


def test_counter_form_slices_agree():
    a = synth.splitmix64(42, 0, 100)
    assert np.array_equal(a[37:60], synth.splitmix64(42, 37, 23))


def test_ranges_and_determinism():
    x = synth.uniform_int(7, (1000,), -127, 127, np.int8)
    assert x.min() >= -127 and x.max() <= 127 and x.min() < -120 and x.max() > 120
    assert np.array_equal(x, synth.uniform_int(7, (1000,), -127, 127, np.int8))
    y = synth.uniform_int(8, (4000,), -8, 7, np.int8)
    assert set(np.unique(y).tolist()) == set(range(-8, 8))
    f = synth.uniform_f32(9, (1000,), 0.002, 0.02)
    assert f.dtype == np.float32 and f.min() >= 0.002 and f.max() < 0.02
    z = synth.normal_f32(10, (20000,))
    assert abs(float(z.mean())) < 0.03 and abs(float(z.std()) - 1) < 0.03


def test_workload_shapes():
    d = synth.gemm_affine_per_tensor()
    assert d["A"].shape == (130, 129) and d["B"].shape == (129, 70) and d["bias"].shape == (70,)
    c = synth.conv3x3_nhwc()
    assert c["X"].shape == (1, 56, 56, 64) and c["W"].shape == (64, 64, 3, 3)
    g = synth.a8w4_gemv()
    assert g["X"].shape == (1, 4096) and g["W"].shape == (4096, 4096) and g["sw"].shape == (4096, 128)
