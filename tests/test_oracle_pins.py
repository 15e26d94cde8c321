"""Pins for the plain-C oracle: every oracle function is checked against something
other than itself -- hand-derived values, closed forms, brute force on tiny
inputs, invariants, or independent library routines (sympy's primality test,
root finder and CRT; Python's big integers; numpy's convolution).

These run on the CPU only.
"""
import random

import numpy as np
import pytest
import sympy
from sympy.ntheory.modular import crt as sympy_crt
from sympy.ntheory.residue_ntheory import nthroot_mod

import oracle as orc
from negacyclic_ntt_amd import inputs, workloads
from tests.golden import fixtures


def brv(x, bits):
    return int(format(x, f"0{bits}b")[::-1], 2) if bits else 0


@pytest.fixture(scope="module")
def primes():
    out = {}
    for w in workloads.ALL:
        out[w.name] = orc.find_primes(w.bits, 2 * w.n, w.prime_count)
    return out


# ---- P1: primes ----------------------------------------------------------------

def test_is_prime_vs_trial_division():
    def trial(n):
        if n < 2:
            return False
        i = 2
        while i * i <= n:
            if n % i == 0:
                return False
            i += 1
        return True

    for n in range(0, 5000):
        assert orc.is_prime(n) == trial(n), n
    rng = random.Random(7)
    for _ in range(300):
        n = rng.randrange(1 << 20, 1 << 32)
        assert orc.is_prime(n) == trial(n), n


def test_is_prime_vs_sympy_hard_cases():
    # Carmichael numbers, strong pseudoprimes to several small bases, squares of
    # primes, and large semiprimes: all composite; plus large known primes.
    composite = [561, 41041, 825265, 3215031751, 2152302898747, 3474749660383, 341550071728321,
                 3825123056546413051, 2147483649, 1000000007 * 998244353, 4294967291 ** 2]
    for n in composite:
        assert orc.is_prime(n) == sympy.isprime(n), n
    rng = random.Random(11)
    for _ in range(400):
        n = rng.randrange(1 << 40, 1 << 63) | 1
        assert orc.is_prime(n) == sympy.isprime(n), n
    for p in [(1 << 61) - 1, 1152921504606584833, 18446744073709551557]:
        assert orc.is_prime(p) == sympy.isprime(p)


@pytest.mark.parametrize("w", workloads.ALL, ids=lambda w: w.name)
def test_prime_lists_are_the_first_descending(w, primes):
    ps = primes[w.name]
    two_n = 2 * w.n
    assert len(ps) == w.prime_count and len(set(ps)) == len(ps)
    assert all(a > b for a, b in zip(ps, ps[1:]))
    assert all(p < (1 << w.bits) and p % two_n == 1 and sympy.isprime(p) for p in ps)
    # No prime of the form 1 mod 2n was skipped between 2^bits and the last one.
    listed = set(ps)
    c = ((1 << w.bits) - 2) // two_n * two_n + 1
    while c >= ps[-1]:
        assert (c in listed) == sympy.isprime(c), c
        c -= two_n


def test_prime_search_small_brute_force():
    """Every prime below 2^bits that is 1 mod 2n, largest first, by trial division,
    for widths where the largest candidate is itself prime (2^4: 13 = 3 * 4 + 1)."""
    def trial(n):
        return n >= 2 and all(n % d for d in range(2, int(n ** 0.5) + 1))

    for bits in range(3, 17):
        for two_n in (4, 8, 16, 32, 64):
            want = [c for c in range((1 << bits) - 1, 1, -1) if c % two_n == 1 and trial(c)]
            got = orc.find_primes(bits, two_n, len(want)) if want else []
            assert got == want, (bits, two_n)
    assert orc.find_primes(4, 4, 2) == [13, 5]


# ---- P2: psi --------------------------------------------------------------------

@pytest.mark.parametrize("w", workloads.ALL, ids=lambda w: w.name)
def test_psi_is_a_primitive_2n_th_root(w, primes):
    for q in primes[w.name][:6]:
        psi = orc.find_psi(q, w.n)
        assert pow(psi, w.n, q) == q - 1 and pow(psi, 2 * w.n, q) == 1


def test_psi_minimal_brute_force_30bit(primes):
    # Smallest x >= 2 with x^n = -1, by an ascending scan (brute force).
    n = 2048
    for q in primes[workloads.POLYMUL.name]:
        psi = orc.find_psi(q, n)
        x = 2
        while pow(x, n, q) != q - 1:
            x += 1
        assert x == psi


@pytest.mark.parametrize("w", [workloads.BATCH, workloads.RING, workloads.KEYSWITCH], ids=lambda w: w.name)
def test_psi_minimal_vs_sympy_roots(w, primes):
    for q in primes[w.name][:3] + primes[w.name][-2:]:
        roots = nthroot_mod(q - 1, w.n, q, all_roots=True)
        assert len(roots) == w.n
        assert min(roots) == orc.find_psi(q, w.n)


# ---- P3/P4: the transform ----------------------------------------------------------

def test_hand_worked_example():
    f = fixtures.load("ntt_q17_n4.txt")
    q, n = f["q"], f["n"]
    assert orc.find_psi(q, n) == f["psi"]
    psi = f["psi"]
    assert list(orc.ntt_forward(f["a"], q, psi)) == f["ntt_a"]
    assert list(orc.ntt_definition(f["a"], q, psi)) == f["ntt_a"]
    assert list(orc.ntt_forward(f["b"], q, psi)) == f["ntt_b"]
    assert list(orc.ntt_forward([0, 1, 0, 0], q, psi)) == f["ntt_x"]
    assert list(orc.schoolbook(f["a"], f["b"], q)) == f["ab"]
    prod = orc.ntt_inverse(f["ntt_a_times_ntt_b"], q, psi)
    assert list(prod) == f["ab"]
    assert list(orc.intt_definition(f["ntt_a_times_ntt_b"], q, psi)) == f["ab"]
    assert list(orc.automorph_coeff(f["a"], 3, q)) == f["sigma3_a"]
    assert list(orc.automorph_coeff(f["a"], 5, q)) == f["sigma5_a"]


def _test_primes(primes):
    return [primes[workloads.POLYMUL.name][0], primes[workloads.CHAIN.name][-1],
            primes[workloads.BATCH.name][0], primes[workloads.RING.name][-1],
            primes[workloads.KEYSWITCH.name][-1]]


def test_monomials_closed_form(primes):
    # NTT(X^j)[k] = psi^((2 brv(k) + 1) j); with linearity this fixes the whole map.
    for q in _test_primes(primes):
        for logn in (1, 2, 3, 5, 6):
            n = 1 << logn
            psi = orc.find_psi(q, n)
            for j in range(n):
                e = np.zeros(n, dtype=np.uint64)
                e[j] = 1
                got = orc.ntt_forward(e, q, psi)
                want = [pow(psi, (2 * brv(k, logn) + 1) * j, q) for k in range(n)]
                assert [int(v) for v in got] == want, (q, n, j)


def test_linearity_and_ones(primes):
    rng = np.random.default_rng(3)
    for q in _test_primes(primes):
        n = 256
        psi = orc.find_psi(q, n)
        a = inputs.uniform_residues((1, n), [q], 9)[0]
        b = inputs.uniform_residues((1, n), [q], 10)[0]
        c = int(rng.integers(1, 1 << 30))
        lhs = orc.ntt_forward([(int(x) * c + int(y)) % q for x, y in zip(a, b)], q, psi)
        fa, fb = orc.ntt_forward(a, q, psi), orc.ntt_forward(b, q, psi)
        assert [int(v) for v in lhs] == [(int(x) * c + int(y)) % q for x, y in zip(fa, fb)]
        one = np.zeros(n, dtype=np.uint64)
        one[0] = 1
        assert all(int(v) == 1 for v in orc.ntt_forward(one, q, psi))


@pytest.mark.parametrize("logn", list(range(1, 11)))
def test_fast_transform_equals_definition(logn, primes):
    n = 1 << logn
    for i, q in enumerate(_test_primes(primes)):
        psi = orc.find_psi(q, n)
        a = inputs.uniform_residues((1, n), [q], 1000 + 17 * logn + i)[0]
        assert np.array_equal(orc.ntt_forward(a, q, psi), orc.ntt_definition(a, q, psi))
        assert np.array_equal(orc.ntt_inverse(a, q, psi), orc.intt_definition(a, q, psi))


@pytest.mark.parametrize("w", workloads.ALL, ids=lambda w: w.name)
def test_round_trip_at_workload_size(w, primes):
    ps = primes[w.name][: w.limbs]
    x = inputs.uniform_residues((2, w.limbs, w.n) if w.n < 65536 else (1, 4, w.n),
                                ps if w.n < 65536 else ps[:4], 55)
    ps_used = ps if w.n < 65536 else ps[:4]
    f = orc.batch_ntt(x, ps_used)
    assert not np.array_equal(f, x)
    assert np.array_equal(orc.batch_ntt(f, ps_used, inverse=True), x)
    assert np.array_equal(orc.batch_ntt(orc.batch_ntt(x, ps_used, inverse=True), ps_used), x)


# ---- P5: schoolbook and the convolution theorem -------------------------------------

def test_schoolbook_vs_numpy_convolve(primes):
    for q in _test_primes(primes):
        for n in (1, 2, 8, 64, 256):
            a = inputs.uniform_residues((1, n), [q], 77 + n)[0]
            b = inputs.uniform_residues((1, n), [q], 78 + n)[0]
            full = np.convolve(a.astype(object), b.astype(object))
            want = [(int(full[i]) - (int(full[i + n]) if i + n < full.size else 0)) % q for i in range(n)]
            assert [int(v) for v in orc.schoolbook(a, b, q)] == want


def test_schoolbook_monomials():
    q, n = 1073692673, 16
    for i in range(n):
        for j in range(n):
            a = np.zeros(n, dtype=np.uint64)
            b = np.zeros(n, dtype=np.uint64)
            a[i] = 1
            b[j] = 1
            want = np.zeros(n, dtype=np.uint64)
            want[(i + j) % n] = 1 if i + j < n else q - 1
            assert np.array_equal(orc.schoolbook(a, b, q), want)


def test_convolution_theorem_polymul_workload(primes):
    w = workloads.POLYMUL
    ps = primes[w.name]
    a = inputs.uniform_residues(w.shape_a, ps, w.seed_a)
    b = inputs.uniform_residues(w.shape_a, ps, w.seed_b)
    prod = orc.batch_ntt(orc.batch_pointwise(orc.batch_ntt(a, ps), orc.batch_ntt(b, ps), ps), ps, inverse=True)
    for l, q in enumerate(ps):
        assert np.array_equal(prod[l], orc.schoolbook(a[l], b[l], q))


@pytest.mark.parametrize("w", [workloads.CHAIN, workloads.BATCH], ids=lambda w: w.name)
def test_convolution_theorem_sampled_limbs(w, primes):
    ps = primes[w.name][: w.limbs]
    sel = [0, w.limbs // 2, w.limbs - 1]
    sub = [ps[i] for i in sel]
    n = min(w.n, 4096)
    a = inputs.uniform_residues((len(sel), n), sub, 61)
    b = inputs.uniform_residues((len(sel), n), sub, 62)
    prod = orc.batch_ntt(orc.batch_pointwise(orc.batch_ntt(a, sub), orc.batch_ntt(b, sub), sub), sub, inverse=True)
    for t, q in enumerate(sub):
        assert np.array_equal(prod[t], orc.schoolbook(a[t], b[t], q))


# ---- P6: tensor product --------------------------------------------------------------

def test_tensor_karatsuba_and_schoolbook(primes):
    ps = primes[workloads.CHAIN.name][:3]
    n = 64
    a = inputs.uniform_residues((2, 2, 3, n), ps, 81)
    b = inputs.uniform_residues((2, 2, 3, n), ps, 82)
    d = orc.batch_tensor(a, b, ps)
    assert d.shape == (2, 3, 3, n)
    for bi in range(2):
        for l, q in enumerate(ps):
            a0, a1, b0, b1 = (int_(x) for x in (a[bi, 0, l], a[bi, 1, l], b[bi, 0, l], b[bi, 1, l]))
            d0, d1, d2 = (int_(x) for x in (d[bi, 0, l], d[bi, 1, l], d[bi, 2, l]))
            for e in range(n):
                s = (a0[e] + a1[e]) * (b0[e] + b1[e]) - d0[e] - d2[e]
                assert d1[e] == s % q and d0[e] == a0[e] * b0[e] % q and d2[e] == a1[e] * b1[e] % q
            # In the coefficient domain d1 is a0*b1 + a1*b0 as negacyclic products.
            psi = orc.find_psi(q, n)
            ca0, ca1, cb0, cb1 = (orc.ntt_inverse(x, q, psi) for x in (a[bi, 0, l], a[bi, 1, l], b[bi, 0, l], b[bi, 1, l]))
            want = (orc.schoolbook(ca0, cb1, q).astype(object) + orc.schoolbook(ca1, cb0, q).astype(object)) % q
            assert [int(v) for v in orc.ntt_inverse(d[bi, 1, l], q, psi)] == [int(v) for v in want]


def test_ct_tensor_coeff_is_the_negacyclic_product(primes):
    """The coefficient-domain ciphertext product: every output polynomial against the
    schoolbook negacyclic products, on 30- and 60-bit primes and two ring sizes."""
    for bits, n in ((30, 32), (60, 128)):
        ps = orc.find_primes(bits, 2 * n, 3)
        a = inputs.uniform_residues((2, 2, 3, n), ps, 91 + n)
        b = inputs.uniform_residues((2, 2, 3, n), ps, 92 + n)
        d = orc.ct_tensor_coeff(a, b, ps)
        assert d.shape == (2, 3, 3, n)
        for bi in range(2):
            for l, q in enumerate(ps):
                a0, a1, b0, b1 = a[bi, 0, l], a[bi, 1, l], b[bi, 0, l], b[bi, 1, l]
                assert np.array_equal(d[bi, 0, l], orc.schoolbook(a0, b0, q))
                want1 = (orc.schoolbook(a0, b1, q).astype(object) + orc.schoolbook(a1, b0, q).astype(object)) % q
                assert [int(v) for v in d[bi, 1, l]] == [int(v) for v in want1]
                assert np.array_equal(d[bi, 2, l], orc.schoolbook(a1, b1, q))


def int_(x):
    return [int(v) for v in x]


# ---- P7: automorphisms ----------------------------------------------------------------

def test_automorph_monomial_closed_form():
    q, n = 1073692673, 32
    for g in range(1, 2 * n, 2):
        for i in range(n):
            x = np.zeros(n, dtype=np.uint64)
            x[i] = 7
            e = i * g % (2 * n)
            want = np.zeros(n, dtype=np.uint64)
            if e < n:
                want[e] = 7
            else:
                want[e - n] = q - 7
            assert np.array_equal(orc.automorph_coeff(x, g, q), want), (g, i)


def test_automorph_identities(primes):
    q = primes[workloads.RING.name][0]
    n = 1 << 12
    a = inputs.uniform_residues((1, n), [q], 91)[0]
    b = inputs.uniform_residues((1, n), [q], 92)[0]
    assert np.array_equal(orc.automorph_coeff(a, 1, q), a)
    # sigma_{n+1} negates the odd coefficients
    s = orc.automorph_coeff(a, n + 1, q)
    want = a.copy()
    want[1::2] = np.where(a[1::2] == 0, 0, np.uint64(q) - a[1::2])
    assert np.array_equal(s, want)
    conj = orc.automorph_coeff(a, 2 * n - 1, q)
    assert np.array_equal(orc.automorph_coeff(conj, 2 * n - 1, q), a)
    for g, h in [(5, 25), (3, 2 * n - 5), (125, 7)]:
        lhs = orc.automorph_coeff(orc.automorph_coeff(a, h, q), g, q)
        assert np.array_equal(lhs, orc.automorph_coeff(a, g * h % (2 * n), q))
    # 5 has order n/2 modulo 2n: sigma_{5^(n/2)} = id
    assert pow(5, n // 2, 2 * n) == 1
    # ring homomorphism: sigma(a*b) = sigma(a) * sigma(b)
    m = 256
    a2, b2 = a[:m], b[:m]
    for g in (5, 3, 2 * m - 1):
        lhs = orc.automorph_coeff(orc.schoolbook(a2, b2, q), g, q)
        rhs = orc.schoolbook(orc.automorph_coeff(a2, g, q), orc.automorph_coeff(b2, g, q), q)
        assert np.array_equal(lhs, rhs)


def test_automorph_ntt_domain_commutes(primes):
    q = primes[workloads.RING.name][1]
    for logn in (3, 6, 10):
        n = 1 << logn
        psi = orc.find_psi(q, n)
        a = inputs.uniform_residues((1, n), [q], 93 + logn)[0]
        fa = orc.ntt_forward(a, q, psi)
        for g in list(workloads.galois_powers(n)) + [2 * n - 1, 3]:
            lhs = orc.ntt_forward(orc.automorph_coeff(a, g, q), q, psi)
            assert np.array_equal(lhs, orc.automorph_ntt(fa, g)), (n, g)


# ---- P8/P9: CRT, basis extension, ModDown -----------------------------------------------

@pytest.fixture(scope="module")
def ks_primes(primes):
    ps = primes[workloads.KEYSWITCH.name]
    return ps[:24], ps[24:]


def test_crt_words_vs_sympy(ks_primes):
    Q, P = ks_primes
    rng = random.Random(5)
    for basis in (Q[:8], P, Q + P, [17, 19, 23]):
        for _ in range(20):
            x = [rng.randrange(m) for m in basis]
            assert orc.crt_int(x, basis) == int(sympy_crt(basis, x)[0])


def test_basis_extend_vs_sympy_and_closed_forms(ks_primes):
    Q, P = ks_primes
    src = Q[8:16]
    dst = Q + P
    n = 64
    x = inputs.uniform_residues((8, n), src, 111)
    out = orc.basis_extend(x, src, dst)
    for e in range(n):
        D = int(sympy_crt(src, [int(v) for v in x[:, e]])[0])
        assert [int(v) for v in out[:, e]] == [D % p for p in dst]
    # restricting to the source primes returns the digit
    assert np.array_equal(out[8:16], x)
    # constant m < min(src) extends to m everywhere
    m = 123456789
    const = np.full((8, 4), m, dtype=np.uint64)
    assert np.all(orc.basis_extend(const, src, dst) == m)
    # all residues q-1 means D = Qj - 1
    top = np.array([[q - 1] * 3 for q in src], dtype=np.uint64)
    Qj = 1
    for q in src:
        Qj *= q
    assert [int(v) for v in orc.basis_extend(top, src, dst)[:, 0]] == [(Qj - 1) % p for p in dst]


def test_moddown_exact_floor(ks_primes):
    Q, P = ks_primes
    qp = Q + P
    Pm, Qm = 1, 1
    for p in P:
        Pm *= p
    for q in Q:
        Qm *= q
    rng = random.Random(13)
    n = 48
    ms = [rng.randrange(Qm) for _ in range(n)]
    rs = [rng.randrange(Pm) for _ in range(n)]
    rs[0], rs[1], ms[2] = 0, Pm - 1, Qm - 1
    X = [Pm * m + r for m, r in zip(ms, rs)]
    acc = np.array([[x % p for x in X] for p in qp], dtype=np.uint64)
    out = orc.moddown(acc, qp, len(Q))
    for l, q in enumerate(Q):
        assert [int(v) for v in out[l]] == [(x // Pm) % q for x in X]
    # ModDown(P * x) = x for x in [0, Q)
    acc2 = np.array([[Pm * m % p for m in ms] for p in qp], dtype=np.uint64)
    out2 = orc.moddown(acc2, qp, len(Q))
    for l, q in enumerate(Q):
        assert [int(v) for v in out2[l]] == [m % q for m in ms]


# ---- P10: key-switch -------------------------------------------------------------------

def _ks_setup(ks_primes, n, seed):
    Q, P = ks_primes
    qp = Q + P
    ct = inputs.uniform_residues((1, 2, 24, n), Q, seed)
    return Q, P, qp, ct


def test_keyswitch_zero_key_and_zero_c1(ks_primes):
    n = 256
    Q, P, qp, ct = _ks_setup(ks_primes, n, 120)
    ksk0 = np.zeros((3, 2, 32, n), dtype=np.uint64)
    g = 5
    sig = orc.batch_automorph(ct[0], g, 0, Q)
    out = orc.keyswitch(ct, ksk0, g, qp, 24, 3)
    assert np.array_equal(out[0, 0], sig[0]) and not out[0, 1].any()
    ksk = inputs.uniform_residues((3, 2, 32, n), qp, 121)
    ct1 = ct.copy()
    ct1[0, 1] = 0
    out = orc.keyswitch(ct1, ksk, g, qp, 24, 3)
    assert np.array_equal(out[0, 0], sig[0]) and not out[0, 1].any()


def _polymul_limbs(a, b, primes, n):
    """Negacyclic products per limb via the oracle's transform (a, b: [L, n])."""
    fa = orc.batch_ntt(a, primes)
    fb = orc.batch_ntt(b, primes)
    return orc.batch_ntt(orc.batch_pointwise(fa, fb, primes), primes, inverse=True)


def _to_limbs(v_signed, primes):
    return np.array([[int(x) % q for x in v_signed] for q in primes], dtype=np.uint64)


@pytest.mark.parametrize("g", [5, 25, 2 * 1024 - 1])
def test_keyswitch_semantic_small_ring(ks_primes, g):
    """Rotation key-switch with a real key at n = 1024: the switched ciphertext
    decrypts under s to what the rotated input decrypts to under sigma_g(s), up to
    a small error (key noise and the floor in ModDown)."""
    n = 1024
    Q, P = ks_primes
    qp = Q + P
    dnum, alpha = 3, 8
    s = inputs.small_signed(n, 1, 130)
    s_limbs = _to_limbs(s, qp)
    s_rot = orc.batch_automorph(s_limbs, g, 0, qp)   # sigma_g(s) on every limb
    Pm = 1
    for p in P:
        Pm *= p
    ksk = np.zeros((dnum, 2, 32, n), dtype=np.uint64)
    for j in range(dnum):
        a_j = inputs.uniform_residues((32, n), qp, 140 + j)
        e_j = _to_limbs(inputs.small_signed(n, 8, 150 + j), qp)
        as_ = _polymul_limbs(a_j, s_limbs, qp, n)
        # P * T_j * s' with T_j = 1 mod the primes of digit j, 0 mod the other Q primes
        pts = np.zeros((32, n), dtype=np.uint64)
        for l in range(j * alpha, (j + 1) * alpha):
            q = qp[l]
            pts[l] = (s_rot[l].astype(object) * (Pm % q) % q).astype(np.uint64)
        b_coef = np.array([[(int(e_j[l][i]) - int(as_[l][i]) + int(pts[l][i])) % qp[l] for i in range(n)]
                           for l in range(32)], dtype=np.uint64)
        ksk[j, 0] = orc.batch_ntt(b_coef, qp)
        ksk[j, 1] = orc.batch_ntt(a_j, qp)
    ct = inputs.uniform_residues((1, 2, 24, n), Q, 160)
    out = orc.keyswitch(ct, ksk, g, qp, 24, dnum)
    sQ = s_limbs[:24]
    lhs = (out[0, 0].astype(object) + _polymul_limbs(out[0, 1], sQ, Q, n).astype(object))
    c_rot = orc.batch_automorph(ct[0], g, 0, Q)
    rhs = (c_rot[0].astype(object) + _polymul_limbs(c_rot[1], s_rot[:24], Q, n).astype(object))
    diff = [[(int(lhs[l][i]) - int(rhs[l][i])) % Q[l] for i in range(n)] for l in range(24)]
    Qm = 1
    for q in Q:
        Qm *= q
    worst = 0
    for i in range(n):
        v = int(sympy_crt(Q, [diff[l][i] for l in range(24)])[0])
        if v > Qm // 2:
            v -= Qm
        worst = max(worst, abs(v))
    # bound: dnum * n * |e| * max(Qj)/P + 1 + n (floor terms) ~ 2^15; far below q
    assert worst < (1 << 20), worst


# ---- P11: rescale ------------------------------------------------------------------

def _residue_columns(values, primes):
    return np.array([[v % q for v in values] for q in primes], dtype=np.uint64)


@pytest.mark.parametrize("which", ["wide", "narrow", "mixed"])
def test_rescale_constructed_quotients(ks_primes, primes, which):
    """X = a q_k + r built from chosen quotient a and remainder r (r at the rounding
    boundaries and at random): truncation gives a, nearest gives a + [r > h] with
    h = floor(q_k / 2); for the negative X = Q - (a q_k + r) the centered results
    are -a - [r > 0] and -a - [r > h]."""
    Q, _ = ks_primes
    narrow = primes[workloads.POLYMUL.name]
    ps = {"wide": list(Q[:6]), "narrow": list(narrow[:4]), "mixed": [narrow[0], Q[1], narrow[1], Q[0]]}[which]
    qk = ps[-1]
    h = qk // 2
    Qm = 1
    for q in ps:
        Qm *= q
    amax = Qm // qk
    rng = random.Random(1100 + len(which))
    rs = [0, 1, h - 1, h, h + 1, qk - 1] + [rng.randrange(qk) for _ in range(10)]
    a_s = [rng.randrange(amax) for _ in rs]
    a_s[0] = 0
    a_s[1] = amax - 1
    pos = [a * qk + r for a, r in zip(a_s, rs)]
    neg = [Qm - x for x in pos if x]
    x = np.stack([_residue_columns(pos, ps)])
    t = orc.rescale(x, ps, 0)[0]
    nr = orc.rescale(x, ps, 1)[0]
    for l, q in enumerate(ps[:-1]):
        assert [int(v) for v in t[l]] == [a % q for a in a_s]
        assert [int(v) for v in nr[l]] == [(a + (r > h)) % q for a, r in zip(a_s, rs)]
    keep = [(a, r) for a, r in zip(a_s, rs) if a * qk + r]
    xn = np.stack([_residue_columns(neg, ps)])
    t = orc.rescale(xn, ps, 0)[0]
    nr = orc.rescale(xn, ps, 1)[0]
    for l, q in enumerate(ps[:-1]):
        assert [int(v) for v in t[l]] == [(-a - (r > 0)) % q for a, r in keep]
        assert [int(v) for v in nr[l]] == [(-a - (r > h)) % q for a, r in keep]


def test_rescale_twice_is_floor_by_the_product(ks_primes):
    """floor(floor(X / q1) / q2) = floor(X / (q1 q2)): two truncating rescales agree
    with one division by the product of the two dropped primes."""
    Q, _ = ks_primes
    ps = list(Q[:5])
    Qm = 1
    for q in ps:
        Qm *= q
    rng = random.Random(1111)
    xs = [rng.randrange(Qm) for _ in range(64)] + [0, Qm - 1]
    x = _residue_columns(xs, ps)[None]
    two = orc.rescale(orc.rescale(x, ps, 0), ps[:-1], 0)[0]
    d = ps[-1] * ps[-2]
    for l, q in enumerate(ps[:-2]):
        assert [int(v) for v in two[l]] == [(v // d) % q for v in xs]


def test_rescale_batch_layout(ks_primes):
    """Batch entries are independent: a [3][L][n] call equals three single calls."""
    Q, _ = ks_primes
    ps = list(Q[:4])
    x = inputs.uniform_residues((3, 4, 32), ps, 1120)
    both = orc.rescale(x, ps, 1)
    assert both.shape == (3, 3, 32)
    for b in range(3):
        assert np.array_equal(both[b], orc.rescale(x[b], ps, 1))


# ---- P12: relinearisation and the full ciphertext product ---------------------------

def test_relinearize_zero_key_and_zero_d2(ks_primes):
    Q, P = ks_primes
    qp = list(Q) + list(P)
    n = 128
    d = inputs.uniform_residues((1, 3, 24, n), Q, 1200)
    out = orc.relinearize(d, np.zeros((3, 2, 32, n), dtype=np.uint64), qp, 24, 3)
    assert np.array_equal(out[0, 0], d[0, 0]) and np.array_equal(out[0, 1], d[0, 1])
    d2 = d.copy()
    d2[0, 2] = 0
    rlk = inputs.uniform_residues((3, 2, 32, n), qp, 1201)
    out = orc.relinearize(d2, rlk, qp, 24, 3)
    assert np.array_equal(out[0, 0], d[0, 0]) and np.array_equal(out[0, 1], d[0, 1])


def _ciphertext(m_limbs, s, primes, seed):
    """(b, a) with b = -a s + m + e over the given primes (coefficient domain)."""
    from tests import keygen
    n = s.shape[1]
    a = inputs.uniform_residues((len(primes), n), list(primes), seed)
    e = keygen.to_limbs(inputs.small_signed(n, 8, seed + 1), primes)
    b = keygen.padd(keygen.psub(e, keygen.pmul(a, s, primes), primes), m_limbs, primes)
    return np.stack([b, a])


def test_relinearize_semantic_small_ring(ks_primes):
    """With a real s^2 -> s key at n = 1024, (c0, c1) = relin(d0, d1, d2) satisfies
    c0 + c1 s = d0 + d1 s + d2 s^2 up to a small error (key noise, floor ModDown)."""
    from tests import keygen
    Q, P = ks_primes
    qp = list(Q) + list(P)
    n = 1024
    s = keygen.to_limbs(inputs.small_signed(n, 1, 1210), qp)
    s2 = keygen.pmul(s, s, qp)
    rlk = keygen.switching_key(s2, s, qp, 24, 3, 1220)
    d = inputs.uniform_residues((1, 3, 24, n), Q, 1230)
    out = orc.relinearize(d, rlk, qp, 24, 3)
    sQ, s2Q = s[:24], s2[:24]
    lhs = keygen.padd(out[0, 0], keygen.pmul(out[0, 1], sQ, Q), Q)
    rhs = keygen.padd(keygen.padd(d[0, 0], keygen.pmul(d[0, 1], sQ, Q), Q), keygen.pmul(d[0, 2], s2Q, Q), Q)
    worst = keygen.centered_crt_max(keygen.psub(lhs, rhs, Q), Q, stride=5)
    assert worst < (1 << 20), worst


def test_ciphertext_product_decrypts_to_the_scaled_product(ks_primes):
    """Whole ct x ct multiply through the oracle: NTT, tensor, INTT, relinearise,
    rescale (nearest).  With m_i = Delta u_i, the result decrypts under s, modulo
    the remaining primes, to Delta^2 (u_1 * u_2) / q_last up to a small error;
    the signal is 2^20 per unit of u_1 * u_2."""
    from tests import keygen
    Q, P = ks_primes
    qp = list(Q) + list(P)
    n = 1024
    delta = 1 << 40
    s = keygen.to_limbs(inputs.small_signed(n, 1, 1240), qp)
    rlk = keygen.switching_key(keygen.pmul(s, s, qp), s, qp, 24, 3, 1250)
    u1 = [int(v) for v in inputs.small_signed(n, 3, 1260)]
    u2 = [int(v) for v in inputs.small_signed(n, 3, 1261)]
    sQ = s[:24]
    c1 = _ciphertext(keygen.to_limbs([delta * v for v in u1], Q), sQ, Q, 1270)
    c2 = _ciphertext(keygen.to_limbs([delta * v for v in u2], Q), sQ, Q, 1280)
    f1 = orc.batch_ntt(c1, Q)
    f2 = orc.batch_ntt(c2, Q)
    d = orc.batch_ntt(orc.batch_tensor(f1, f2, Q), Q, inverse=True)
    ct = orc.relinearize(d[None], rlk, qp, 24, 3)[0]
    r = orc.rescale(ct, Q, 1)
    Qr = Q[:-1]
    dec = keygen.padd(r[0], keygen.pmul(r[1], sQ[:-1], Qr), Qr)
    got = keygen.centered_values(dec, Qr)
    # integer negacyclic product u1 * u2
    uu = [0] * n
    for i, a in enumerate(u1):
        if a:
            for j, b in enumerate(u2):
                k = i + j
                if k < n:
                    uu[k] += a * b
                else:
                    uu[k - n] -= a * b
    scale = delta * delta
    worst = max(abs(g * Q[-1] - scale * v) for g, v in zip(got, uu)) / Q[-1]
    # rounding of (c0, c1) contributes at most (1 + ||s||_1) / 2 <= n / 2 + 1; key
    # and encryption noise are far below one unit after the division by q_last
    assert worst < n / 2 + 2, worst
    assert any(uu)


# ---- P13: hoisted rotations -----------------------------------------------------------

def test_hoisted_identity_rotation_equals_keyswitch(ks_primes):
    """With g = 1 there is no automorphism, so sharing the decomposition changes nothing."""
    Q, P = ks_primes
    qp = list(Q) + list(P)
    n = 256
    ct = inputs.uniform_residues((2, 2, 24, n), Q, 1300)
    ksk = inputs.uniform_residues((1, 3, 2, 32, n), qp, 1301)
    got = orc.keyswitch_hoisted(ct, ksk, [1], qp, 24, 3)
    assert np.array_equal(got[0], orc.keyswitch(ct, ksk[0], 1, qp, 24, 3))


def test_hoisted_matches_coefficient_domain_route(ks_primes):
    """The NTT-domain slot permutation of the shared digits equals the other route:
    lift each digit, apply sigma_g to the lifted integer polynomial in the
    coefficient domain (limb by limb over Q u P), then NTT; key product, INTT,
    ModDown and sigma_g(c0) as in the key-switch definition."""
    Q, P = ks_primes
    qp = list(Q) + list(P)
    n, dnum, alpha = 128, 3, 8
    gs = [5, 25, 2 * n - 1]
    ct = inputs.uniform_residues((1, 2, 24, n), Q, 1310)
    ksk = inputs.uniform_residues((len(gs), dnum, 2, 32, n), qp, 1311)
    got = orc.keyswitch_hoisted(ct, ksk, gs, qp, 24, dnum)
    lifted = [orc.basis_extend(ct[0, 1, j * alpha:(j + 1) * alpha], Q[j * alpha:(j + 1) * alpha], qp)
              for j in range(dnum)]
    for r, g in enumerate(gs):
        acc = np.zeros((2, 32, n), dtype=object)
        for j in range(dnum):
            dig = orc.batch_ntt(orc.batch_automorph(lifted[j], g, 0, qp), qp)
            for c in range(2):
                acc[c] += dig.astype(object) * ksk[r, j, c].astype(object)
        qcol = np.array(qp, dtype=object)[:, None]
        acc = (acc % qcol).astype(np.uint64)
        coef = orc.batch_ntt(acc, qp, inverse=True)
        c0r = orc.batch_automorph(ct[0, 0], g, 0, Q)
        want0 = (orc.moddown(coef[0], qp, 24).astype(object) + c0r.astype(object)) % np.array(Q, dtype=object)[:, None]
        assert np.array_equal(got[r, 0, 0], want0.astype(np.uint64)), g
        assert np.array_equal(got[r, 0, 1], orc.moddown(coef[1], qp, 24)), g


def test_hoisted_semantic_small_ring(ks_primes):
    """Real rotation keys (including the conjugation 2n - 1) at n = 1024: output r
    decrypts under s to what sigma_{g_r}(ct) decrypts to under sigma_{g_r}(s)."""
    from tests import keygen
    Q, P = ks_primes
    qp = list(Q) + list(P)
    n = 1024
    gs = [5, 2 * n - 1, 25]
    s = keygen.to_limbs(inputs.small_signed(n, 1, 1320), qp)
    keys = np.stack([keygen.switching_key(orc.batch_automorph(s, g, 0, qp), s, qp, 24, 3, 1330 + 10 * i)
                     for i, g in enumerate(gs)])
    ct = inputs.uniform_residues((1, 2, 24, n), Q, 1340)
    out = orc.keyswitch_hoisted(ct, keys, gs, qp, 24, 3)
    sQ = s[:24]
    for r, g in enumerate(gs):
        lhs = keygen.padd(out[r, 0, 0], keygen.pmul(out[r, 0, 1], sQ, Q), Q)
        c_rot = orc.batch_automorph(ct[0], g, 0, Q)
        rhs = keygen.padd(c_rot[0], keygen.pmul(c_rot[1], orc.batch_automorph(sQ, g, 0, Q), Q), Q)
        worst = keygen.centered_crt_max(keygen.psub(lhs, rhs, Q), Q, stride=7)
        assert worst < (1 << 20), (g, worst)


# ---- P14: modraise -------------------------------------------------------------------

def test_modraise_closed_form(ks_primes):
    """Columns with known integers X in [0, Q_from): every output limb is X mod q;
    the input limbs are kept."""
    Q, _ = ks_primes
    ps = list(Q[:10])
    frm = 3
    Qf = 1
    for q in ps[:frm]:
        Qf *= q
    rng = random.Random(1400)
    xs = [0, 1, Qf - 1, Qf // 2, Qf // 2 + 1] + [rng.randrange(Qf) for _ in range(59)]
    x = np.array([[v % q for v in xs] for q in ps[:frm]], dtype=np.uint64)[None]
    out = orc.modraise(x, ps, frm)[0]
    for t, q in enumerate(ps):
        assert [int(v) for v in out[t]] == [v % q for v in xs]


def test_modraise_decrypts_modulo_the_low_modulus(ks_primes):
    """A level-1 ciphertext raised to 24 primes decrypts to m + e + q_0 I with a
    small integer polynomial I (|I| <= ||s||_1 + 1); reducing that decryption
    modulo q_0 gives back exactly the level-1 decryption."""
    from tests import keygen
    Q, _ = ks_primes
    n = 256
    q0 = Q[0]
    s = keygen.to_limbs(inputs.small_signed(n, 1, 1410), Q)
    m = keygen.to_limbs([(1 << 40) * v for v in inputs.small_signed(n, 5, 1411)], Q[:1])
    ct = _ciphertext(m, s[:1], Q[:1], 1420)
    low = keygen.centered_values(keygen.padd(ct[0], keygen.pmul(ct[1], s[:1], Q[:1]), Q[:1]), Q[:1])
    up = orc.modraise(ct, Q, 1)
    full = keygen.centered_values(keygen.padd(up[0], keygen.pmul(up[1], s, Q), Q), Q)
    l1 = sum(abs(int(v)) for v in inputs.small_signed(n, 1, 1410))
    for a, b in zip(full, low):
        assert (a - b) % q0 == 0
        assert abs((a - b) // q0) <= l1 + 1


def test_a_planted_mistake_fails_a_pin():
    """The mutation driver (tests/oracle_mutations.py, all mutants on demand) on one
    representative: the forward butterfly's difference turned into a sum."""
    import tests.oracle_mutations as mut
    idx = [i for i, m in enumerate(mut.MUTANTS) if m[0].startswith("forward butterfly")][0]
    assert mut.run_mutant(idx).startswith("killed")
