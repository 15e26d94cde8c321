"""GPU parity: forward / inverse NTT through the C ABI, bit-exact against the oracle."""
import numpy as np
import pytest

import oracle as orc
from negacyclic_ntt_amd import workloads
from tests.helpers import announce, assert_bits_equal, dev, host, primes, require_gpu, residues

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    require_gpu()
    from negacyclic_ntt_amd import binding
    return binding


def _prime_set(bits):
    # 1 mod 2^17 so that every ring degree up to 2^16 can use them.
    return primes(bits, 1 << 17, 3)


@pytest.mark.parametrize("bits", [30, 31, 60, 62])
@pytest.mark.parametrize("logn", list(range(1, 17)))
def test_ntt_sweep(B, logn, bits):
    n = 1 << logn
    ps = _prime_set(bits)
    batch = 3 if logn <= 13 else 1
    announce("ntt_sweep", logn, bits)
    x = residues((batch, 3, n), ps, 7000 + 31 * logn + bits)
    plan = B.Plan(n, ps, 0)
    t = dev(x)
    B.ntt_forward(plan, t)
    want = orc.batch_ntt(x, ps)
    assert_bits_equal(host(t), want, f"forward n=2^{logn} {bits}-bit")
    B.ntt_inverse(plan, t)
    assert_bits_equal(host(t), x, f"round trip n=2^{logn} {bits}-bit")
    # inverse of an arbitrary residue vector
    t2 = dev(x)
    B.ntt_inverse(plan, t2)
    assert_bits_equal(host(t2), orc.batch_ntt(x, ps, inverse=True), f"inverse n=2^{logn} {bits}-bit")


@pytest.mark.parametrize("logn", [3, 6, 11, 14, 16])
def test_limb_subrange_and_ragged_batch(B, logn):
    n = 1 << logn
    ps = primes(60, 1 << 17, 5)
    plan = B.Plan(n, ps, 0)
    sub = ps[1:4]
    x = residues((5, 3, n), sub, 8100 + logn)  # 15 rows: ragged for every rows-per-workgroup
    announce("subrange", logn)
    t = dev(x)
    B.ntt_forward(plan, t, limb_begin=1)
    assert_bits_equal(host(t), orc.batch_ntt(x, sub), f"forward limbs 1..3 n=2^{logn}")
    B.ntt_inverse(plan, t, limb_begin=1)
    assert_bits_equal(host(t), x, "round trip")


@pytest.mark.parametrize("logn", [14, 16])
def test_forward_galois_limb_subrange(B, logn):
    # the two-pass split with the automorphism folded in, on plan limbs 2..4 of 6 and a
    # ragged batch, out of place and in place
    import torch
    n = 1 << logn
    ps = primes(60, 1 << 17, 6)
    plan = B.Plan(n, ps, 0)
    sub = ps[2:5]
    x = residues((3 if logn == 14 else 1, 3, n), sub, 8500 + logn)
    tx = dev(x)
    out = torch.empty_like(tx)
    announce("galois subrange", logn)
    B.ntt_forward_galois(plan, out, tx, 5, limb_begin=2)
    assert_bits_equal(host(out), orc.batch_ntt(orc.batch_automorph(x, 5, 0, sub), sub), "limbs 2..4, g = 5")
    B.ntt_forward_galois(plan, tx, tx, 2 * n - 1, limb_begin=2)
    assert_bits_equal(host(tx), orc.batch_ntt(orc.batch_automorph(x, 2 * n - 1, 0, sub), sub), "in place, g = 2n - 1")


def test_mixed_width_limb_range(B):
    # a 30-bit and a 60-bit prime in one call take the 64-bit path for both
    n = 1 << 11
    ps = [primes(30, 1 << 12, 1)[0], primes(60, 1 << 12, 1)[0]]
    plan = B.Plan(n, ps, 0)
    x = residues((4, 2, n), ps, 8200)
    t = dev(x)
    announce("mixed width")
    B.ntt_forward(plan, t)
    assert_bits_equal(host(t), orc.batch_ntt(x, ps), "mixed widths")


def test_zero_batch_is_a_noop(B):
    import torch
    ps = _prime_set(60)
    plan = B.Plan(1024, ps, 0)
    t = torch.zeros((0, 3, 1024), dtype=torch.int64, device="cuda:0")
    B.ntt_forward(plan, t)
    B.ntt_inverse(plan, t)


def test_special_values(B):
    n = 1 << 12
    ps = _prime_set(62)
    plan = B.Plan(n, ps, 0)
    x = np.zeros((4, 3, n), dtype=np.uint64)
    for l, q in enumerate(ps):
        x[1, l, :] = q - 1            # all maximal residues
        x[2, l, 0] = 1                # the constant 1 -> all ones
        x[3, l, 1] = 1                # X -> psi^(2 brv(k) + 1)
    t = dev(x)
    announce("special values")
    B.ntt_forward(plan, t)
    got = host(t)
    assert_bits_equal(got, orc.batch_ntt(x, ps), "special values")
    assert not got[0].any() and (got[2] == 1).all()


@pytest.mark.parametrize("w", [workloads.POLYMUL, workloads.CHAIN, workloads.BATCH, workloads.RING],
                         ids=lambda w: w.name)
def test_workload_round_trip(B, w):
    ps = primes(w.bits, 2 * w.n, w.limbs)
    announce("workload", w.name)
    x = residues(w.shape_a, ps, w.seed_a)
    plan = B.Plan(w.n, ps, 0)
    t = dev(x)
    B.ntt_forward(plan, t)
    assert_bits_equal(host(t), orc.batch_ntt(x, ps), f"{w.name} forward")
    B.ntt_inverse(plan, t)
    assert_bits_equal(host(t), x, f"{w.name} round trip")


def test_repeat_and_streams_bit_identical(B):
    import torch
    w = workloads.RING
    ps = primes(w.bits, 2 * w.n, w.limbs)
    plan = B.Plan(w.n, ps, 0)
    x = residues((2, w.limbs, w.n), ps, 8300)
    a, b = dev(x), dev(x)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    announce("two streams")
    with torch.cuda.stream(s1):
        B.ntt_forward(plan, a)
    with torch.cuda.stream(s2):
        B.ntt_forward(plan, b)
    torch.cuda.synchronize()
    assert_bits_equal(host(a), host(b), "same input on two streams")


# ---- forward NTT with the automorphism folded in -------------------------------------

def _galois_set(n):
    two_n = 2 * n
    return sorted({g % two_n for g in (1, 3, 5, 25, 2 * n - 1, n + 1, 5 ** 7)} | {1})


@pytest.mark.parametrize("logn", list(range(1, 17)))
def test_ntt_forward_galois_sweep(B, logn):
    import torch
    n = 1 << logn
    ps = _prime_set(60 if logn % 2 else 30)
    plan = B.Plan(n, ps, 0)
    x = residues((2 if logn < 15 else 1, 3, n), ps, 7700 + logn)
    tx = dev(x)
    out = torch.empty_like(tx)
    for g in _galois_set(n):
        if g % 2 == 0:
            continue
        announce("ntt_forward_galois", logn, g)
        B.ntt_forward_galois(plan, out, tx, g)
        want = orc.batch_ntt(orc.batch_automorph(x, g, 0, ps), ps)
        assert_bits_equal(host(out), want, f"NTT(sigma_{g}) n=2^{logn}")


@pytest.mark.parametrize("bits", [60, 62])
@pytest.mark.parametrize("logn", [13, 14])
def test_ntt_forward_galois_wide(B, logn, bits):
    # 64-bit residues where the transform changes shape (one row per workgroup at 2^13,
    # the two-pass split at 2^14), out of place and in place
    import torch
    n = 1 << logn
    ps = _prime_set(bits)
    plan = B.Plan(n, ps, 0)
    x = residues((3, 3, n), ps, 7800 + logn + bits)
    tx = dev(x)
    out = torch.empty_like(tx)
    for g in (3, 5, 2 * n - 1):
        announce("ntt_forward_galois wide", logn, bits, g)
        B.ntt_forward_galois(plan, out, tx, g)
        assert_bits_equal(host(out), orc.batch_ntt(orc.batch_automorph(x, g, 0, ps), ps), f"NTT(sigma_{g})")
    B.ntt_forward_galois(plan, tx, tx, 25)
    assert_bits_equal(host(tx), orc.batch_ntt(orc.batch_automorph(x, 25, 0, ps), ps), "in place")


@pytest.mark.parametrize("w", [workloads.CHAIN, workloads.RING], ids=lambda w: w.name)
def test_ntt_forward_galois_workload_in_place(B, w):
    ps = primes(w.bits, 2 * w.n, w.limbs)
    x = residues((1, 2, w.limbs, w.n), ps, w.seed_a)
    plan = B.Plan(w.n, ps, 0)
    for g in w.galois or workloads.galois_powers(w.n):
        tx = dev(x)
        announce("ntt_forward_galois in place", w.name, g)
        B.ntt_forward_galois(plan, tx, tx, g)
        want = orc.batch_automorph(orc.batch_ntt(x, ps), g, 1, ps)  # NTT-domain permutation of NTT(x)
        assert_bits_equal(host(tx), want, f"{w.name} g={g}")
