"""Pins of the seeded input generator (synth/gen.c)."""
import numpy as np

import synth

MASK = (1 << 64) - 1


def _np_splitmix(x, k):
    """Numpy twin of SplitMix64's k-th output, from the published definition."""
    z = (np.uint64(x) + (k.astype(np.uint64) + np.uint64(1)) * np.uint64(0x9E3779B97F4A7C15))
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def test_splitmix64_published_outputs():
    # First outputs of SplitMix64 seeded with 0 (Steele, Lea, Flood 2014 reference code).
    assert synth.splitmix64(0, 0) == 0xE220A8397B1DCDAF
    assert synth.splitmix64(0, 1) == 0x6E789E6AA1B965F4
    assert synth.splitmix64(0, 2) == 0x06C45D188009454F


def test_numpy_twin_bit_identical():
    seed, tid, n = 3, 5, 20000
    key = synth.splitmix64((seed << 8) | tid, 0)
    with np.errstate(over="ignore"):
        k = np.arange(n, dtype=np.uint64)
        z0 = _np_splitmix(key, 2 * k)
        z1 = _np_splitmix(key, 2 * k + 1)
    u1 = ((z0 >> np.uint64(11)) + np.uint64(1)).astype(np.float64) * 2.0 ** -53
    u2 = (z1 >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
    ref = np.sqrt(-2.0 * np.log(u1)) * np.cos(2 * np.pi * u2)
    got = synth.normal_f64(seed, tid, n)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)
    # bf16 rounding of the same stream: compare to a numpy round-to-nearest-even
    bits = synth.normal_bf16(seed, tid, (n,))
    m, e = np.frexp(ref)
    q = e - 8
    r = np.ldexp(np.rint(np.ldexp(ref, -q)), q).astype(np.float32)
    assert np.array_equal(bits, (r.view(np.uint32) >> 16).astype(np.uint16))


def test_bf16_round_half_even():
    one = 1.0
    ulp = 2.0 ** -7
    assert synth.f64_to_bf16(one + ulp / 2) == 0x3F80          # tie -> even (1.0)
    assert synth.f64_to_bf16(one + 3 * ulp / 2) == 0x3F82      # tie -> even (1 + 2 ulp)
    assert synth.f64_to_bf16(one + ulp / 2 + 2.0 ** -40) == 0x3F81  # above the tie
    assert synth.f64_to_bf16(-2.0) == 0xC000
    assert synth.f64_to_bf16(0.0) == 0x0000
    assert synth.f64_to_bf16(2.0 ** -130) == 0x0008            # bf16 subnormal


def test_moments_and_counter_property():
    x = synth.normal_f64(1, 1, 400000)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    # counter-based: element n is the same whether drawn alone or in a block
    tail = synth.normal_f64(1, 1, 10, first=399990)
    assert np.array_equal(tail, x[-10:])
    # different tensor ids give different streams
    assert not np.array_equal(synth.normal_f64(1, 2, 100), x[:100])


def test_workload_recipe():
    wl = synth.WORKLOADS["batch_b8_t4096_h16"]
    lam = synth.lambdas(wl, 16, wl.seed)
    assert lam.dtype == np.float32 and lam.shape == (16,)
    assert np.all((lam >= 0.2) & (lam < 0.9))
    g = synth.normal_f32(1, 6, (2, 128), 1.0, 0.02)
    assert abs(float(g.mean()) - 1.0) < 0.01 and 0.01 < float(g.std()) < 0.03
