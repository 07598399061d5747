"""The seeded input generator: reproducible bits and the stated distributions."""
import hashlib
import math

import numpy as np

import synth


def test_counter_based_streams_are_addressable():
    k = synth.stream_key(5, synth.S_GATE)
    a = synth.raw64(k, 0, 1000)
    b = synth.raw64(k, 400, 600)
    assert np.array_equal(a[400:], b)
    assert not np.array_equal(synth.raw64(synth.stream_key(5, synth.S_UP), 0, 1000), a)
    assert not np.array_equal(synth.raw64(synth.stream_key(6, synth.S_GATE), 0, 1000), a)


def test_splitmix64_reference_values():
    # SplitMix64 with state 0: the first outputs of the published generator.
    state0 = synth.raw64(np.uint64(0), 0, 3)
    assert [int(v) for v in state0] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                        0x06C45D188009454F]


def test_normal_and_student_moments():
    k = synth.stream_key(1, 1)
    z = synth.normal(k, 0, 1 << 20)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1.0) < 5e-3
    assert abs((np.abs(z) > 1.6448536).mean() - 0.1) < 2e-3
    t = synth.student_t3(k, 0, 1 << 18)
    # Student-t(3): median 0, P(|t| > 3.182446) = 0.05
    assert abs(np.median(t)) < 1e-2
    assert abs((np.abs(t) > 3.182446).mean() - 0.05) < 3e-3


def test_recipes_shapes_and_determinism():
    x = synth.gelu_iid(4, 2048, seed=0)
    assert x.shape == (4, 4096) and x.dtype == np.uint16
    assert np.array_equal(x, synth.gelu_iid(4, 2048, seed=0))
    g = synth.bits_to_float(x[:, :2048], synth.BF16)
    assert abs(float(g.std()) - 1.0) < 0.05
    xl = synth.gelu_large(1, 16384)
    assert abs(float(synth.bits_to_float(xl[:, :16384], synth.BF16).std()) - 2.0) < 0.05
    xo = synth.gelu_offset_rows(8)
    assert xo.shape == (8, 16384)
    e = synth.edge_rows(7, 2000, synth.F16)
    ef = synth.bits_to_float(e[:, :2000], synth.F16)
    assert np.all(ef[2] == 0.0) and np.all(ef[3] == 100.0) and np.ptp(ef[1]) == 0
    assert abs(float(ef[0].mean()) - 100.0) < 0.01
    # bf16 rounds N(100, 0.01) to exactly 100: those rows are constant.
    eb = synth.bits_to_float(synth.edge_rows(1, 3000, synth.BF16)[:, :3000], synth.BF16)
    assert np.all(eb == 100.0)


def test_bf16_rounding_of_inputs_is_nearest_even():
    v = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 0.0])
    b = synth.to_bits(v, synth.BF16)
    assert [int(x) for x in b] == [0x3F80, 0x3F82, 0xC020, 0x0000]


def test_stable_digest_of_small_case():
    x = synth.gelu_iid(4, 2048, seed=0)
    h = hashlib.sha256(x.tobytes()).hexdigest()
    with open(__file__.replace("test_synth.py", "golden/gelu_T4_d2048_bf16_seed0.txt")) as f:
        want = [ln.split("=", 1)[1].strip() for ln in f if ln.startswith("input_sha256")][0]
    assert h == want
    assert math.isfinite(float(synth.bits_to_float(x, synth.BF16).sum()))


def test_fused_bf16_rows_match_numpy_rounding():
    k = synth.stream_key(9, 1)
    a = np.empty((37, 300), np.uint16)
    synth.normal_rows_into(a, k, scale=2.0, shift=0.5)
    b = synth.to_bits(synth.normal(k, 0, 37 * 300, 2.0, 0.5).reshape(37, 300), synth.BF16)
    assert np.array_equal(a, b)
    # strided destination (the gate half of a [rows, 2d] buffer)
    x = np.zeros((37, 600), np.uint16)
    synth.normal_rows_into(x[:, :300], k, scale=2.0, shift=0.5)
    assert np.array_equal(x[:, :300], b) and not x[:, 300:].any()


def test_c_core_matches_numpy_rederivation():
    k = synth.stream_key(3, 1)
    i = np.arange(1, 1001, dtype=np.uint64)
    with np.errstate(over="ignore"):
        r = synth._mix(np.uint64(k) + i * synth._GAMMA)
    assert np.array_equal(r, synth.raw64(k, 0, 1000))
    u = ((r >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
    assert np.array_equal(u, synth.uniform(k, 0, 1000))
    z = np.sqrt(-2 * np.log(u[0::2])) * np.cos(2 * np.pi * u[1::2])
    assert np.abs(z - synth.normal(k, 0, 500)).max() < 1e-14


def test_down_weight_recipe():
    w = synth.down_weight(64, 2048, seed=3)
    assert w.shape == (64, 2048) and w.dtype == np.uint16
    assert np.array_equal(w, synth.down_weight(64, 2048, seed=3))
    v = synth.bits_to_float(w, synth.BF16)
    assert abs(v.mean()) < 3e-4 and abs(v.std() * np.sqrt(2048) - 1.0) < 0.01
    # its own stream: not the gate or up values of the same seed
    x = synth.gelu_iid(64, 2048, seed=3)
    assert not np.array_equal(w, x[:, :2048])
    f = synth.down_weight(8, 256, seed=4, dtype=synth.F16)
    assert f.dtype == np.uint16 and np.isfinite(synth.bits_to_float(f, synth.F16)).all()
