"""The seeded input generator (shared by the GPU tests, the benchmark and the oracle tests)."""
import numpy as np

from negacyclic_ntt_amd import inputs, workloads


def test_splitmix64_published_sequence():
    # SplitMix64 from seed 1234567: the sequence commonly used to check ports of
    # the published generator (Steele, Lea, Flood 2014).
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423, 4593380528125082431,
            16408922859458223821]
    assert [int(x) for x in inputs.splitmix64(1234567, 0, 5)] == want
    # counter form: any window equals the corresponding slice of the stream
    assert np.array_equal(inputs.splitmix64(9, 3, 4), inputs.splitmix64(9, 0, 7)[3:])


def test_uniform_rows_are_sequential_rejection():
    q = (1 << 29) + 11  # about half of the draws are rejected at 30 bits
    st = inputs.Stream(77)
    row = st.uniform_row(q, 1000)
    raw = inputs.splitmix64(77, 0, st.pos) >> np.uint64(64 - q.bit_length())
    acc = raw[raw < np.uint64(q)]
    assert np.array_equal(acc, row) and raw[-1] < q
    assert row.max() < q and row.min() >= 0


def test_uniform_residues_layout():
    primes = [97, 193]
    x = inputs.uniform_residues((3, 2, 16), primes, 5)
    assert x.dtype == np.uint64 and x.shape == (3, 2, 16)
    assert (x[:, 0] < 97).all() and (x[:, 1] < 193).all()
    assert x[:, 1].max() >= 97  # the second limb really uses its own prime
    assert np.array_equal(x, inputs.uniform_residues((3, 2, 16), primes, 5))
    assert not np.array_equal(x, inputs.uniform_residues((3, 2, 16), primes, 6))


def test_small_signed_range():
    v = inputs.small_signed(10000, 1, 3)
    assert set(np.unique(v)) == {-1, 0, 1}


def test_galois_powers():
    g = workloads.galois_powers(65536)
    assert len(g) == 16 and g[0] == 5 and g[-2] == 65537 and g[-1] == 1
    assert g[:5] == (5, 25, 625, 128481, 28609)
