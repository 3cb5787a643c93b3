"""Pins of the probe's generator and inputs in the oracle (oracle/probe.py),
the kernel probe of the page's "Layer 3: the kernel probe"."""
import numpy as np

from oracle import probe


def test_splitmix64_published_outputs():
    """The first outputs of SplitMix64 seeded with 1234567, as published with
    the generator's reference implementation (Vigna's splitmix64.c; the same
    five values are the reference vector of the rand_xoshiro crate)."""
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    assert probe.splitmix64_py(1234567, 5) == want
    assert [int(z) for z in probe.splitmix64_np(1234567, 5)] == want


def test_splitmix64_counter_form():
    """Output k taken on its own (counter form) equals output k of the
    sequence, and numpy's mod-2^64 arithmetic equals Python's."""
    for seed in (0, 1, 2**64 - 1, 0x123456789ABCDEF0):
        seq = probe.splitmix64_py(seed, 40)
        for k in (0, 7, 39):
            assert probe.splitmix64_py(seed, 1, first=k) == [seq[k]]
        assert [int(z) for z in probe.splitmix64_np(seed, 30, first=10)] == seq[10:40]


def test_probe_values_exact_and_in_range():
    z = np.array([0, 2**64 - 1, 1 << 63, (1 << 63) - 1, 0x000000FFFFFFFFFF], dtype=np.uint64)
    v = probe.probe_values(z)
    assert v.dtype == np.float32
    assert v[0] == np.float32(-4.0)
    assert v[1] == np.float32((2**24 - 1 - 2**23) / 2**21)
    assert v[2] == np.float32(0.0)
    assert v[3] == np.float32(-1 / 2**21)
    assert v[4] == np.float32(-4.0)        # only the top 24 bits count
    # every value is k / 2^21 with k an integer in [-2^23, 2^23): exact in f32
    vals = probe.probe_values(probe.splitmix64_np(99, 4096))
    k = vals.astype(np.float64) * 2**21
    assert np.all(k == np.round(k)) and k.min() >= -2**23 and k.max() < 2**23


def test_probe_inputs_layout():
    """A takes outputs 0 .. MK-1 row-major, B the next KN outputs row-major."""
    M, N, K, seed = 3, 5, 4, 7
    A, B = probe.probe_inputs(seed, M, N, K)
    z = probe.splitmix64_py(seed, M * K + K * N)
    assert A.shape == (M, K) and B.shape == (K, N)
    assert A[2, 1] == probe.probe_values(np.array([z[2 * K + 1]], dtype=np.uint64))[0]
    assert B[3, 4] == probe.probe_values(np.array([z[M * K + 3 * N + 4]], dtype=np.uint64))[0]


def test_probe_hash_is_the_method_on_those_inputs():
    from oracle import hashref, ref
    A, B = probe.probe_inputs(5, 9, 11, 13)
    C = ref.blockscaled_gemm(A, B)[0]
    assert probe.probe_hash(5, 9, 11, 13) == hashref.output_hash(C)
    assert probe.probe_hash(5, 9, 11, 13) != probe.probe_hash(6, 9, 11, 13)
