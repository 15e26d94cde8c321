"""GPU parity: pointwise product, tensor product and automorphisms vs the oracle;
device-side argument validation."""
import ctypes

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


def test_polymul_workload_vs_oracle_and_schoolbook(B):
    w = workloads.POLYMUL
    ps = primes(w.bits, 2 * w.n, w.limbs)
    a = residues(w.shape_a, ps, w.seed_a)
    b = residues(w.shape_a, ps, w.seed_b)
    plan = B.Plan(w.n, ps, 0)
    ta, tb = dev(a), dev(b)
    announce("polymul workload")
    B.ntt_forward(plan, ta)
    B.ntt_forward(plan, tb)
    tc = B.poly_mul_ntt(plan, ta.clone(), ta, tb)
    B.ntt_inverse(plan, tc)
    got = host(tc)
    for l, q in enumerate(ps):
        assert_bits_equal(got[l], orc.schoolbook(a[l], b[l], q), f"limb {l} vs schoolbook")


@pytest.mark.parametrize("bits,logn", [(30, 11), (60, 14), (62, 16), (31, 5)])
def test_pointwise_in_and_out_of_place(B, bits, logn):
    n = 1 << logn
    ps = primes(bits, 1 << 17, 3)
    plan = B.Plan(n, ps, 0)
    a = residues((5, 3, n), ps, 9000 + logn)
    b = residues((5, 3, n), ps, 9100 + logn)
    want = orc.batch_pointwise(a, b, ps)
    announce("pointwise", bits, logn)
    ta, tb = dev(a), dev(b)
    out = B.poly_mul_ntt(plan, dev(np.zeros_like(a)), ta, tb)
    assert_bits_equal(host(out), want, "out of place")
    B.poly_mul_ntt(plan, ta, ta, tb)
    assert_bits_equal(host(ta), want, "out == a")
    tb2 = dev(b)
    B.poly_mul_ntt(plan, tb2, dev(a), tb2)
    assert_bits_equal(host(tb2), want, "out == b")
    # extreme residues: (q-1)^2
    m = np.array([[[q - 1] * n for q in ps]], dtype=np.uint64)
    assert_bits_equal(host(B.poly_mul_ntt(plan, dev(m), dev(m), dev(m))), orc.batch_pointwise(m, m, ps), "q-1")


def test_batch_workload_pipeline(B):
    """n = 2^14 throughput batch: NTT(A), pointwise with B, inverse NTT."""
    w = workloads.BATCH
    ps = primes(w.bits, 2 * w.n, w.limbs)
    a = residues(w.shape_a, ps, w.seed_a)
    b = residues(w.shape_a, ps, w.seed_b)
    plan = B.Plan(w.n, ps, 0)
    announce("batch workload pipeline")
    ta = dev(a)
    B.ntt_forward(plan, ta)
    B.poly_mul_ntt(plan, ta, ta, dev(b))
    B.ntt_inverse(plan, ta)
    want = orc.batch_ntt(orc.batch_pointwise(orc.batch_ntt(a, ps), b, ps), ps, inverse=True)
    assert_bits_equal(host(ta), want, w.name)


def test_tensor_chain_workload(B):
    w = workloads.CHAIN
    ps = primes(w.bits, 2 * w.n, w.limbs)
    a = residues(w.shape_a, ps, w.seed_a)
    b = residues(w.shape_a, ps, w.seed_b)
    plan = B.Plan(w.n, ps, 0)
    announce("tensor chain workload")
    ta, tb = dev(a), dev(b)
    B.ntt_forward(plan, ta)
    B.ntt_forward(plan, tb)
    import torch
    d = torch.empty((4, 3, w.limbs, w.n), dtype=torch.int64, device="cuda:0")
    B.ct_tensor_ntt(plan, d, ta, tb)
    ah, bh = orc.batch_ntt(a, ps), orc.batch_ntt(b, ps)
    want = orc.batch_tensor(ah, bh, ps)
    assert_bits_equal(host(d), want, "tensor d0,d1,d2")
    # inverse of d (1344 limb-INTTs) back to the coefficient domain
    B.ntt_inverse(plan, d)
    assert_bits_equal(host(d), orc.batch_ntt(want, ps, inverse=True), "inverse of the tensor")


def test_tensor_limb_subrange(B):
    ps = primes(60, 1 << 13, 6)
    n = 4096
    plan = B.Plan(n, ps, 0)
    sub = ps[2:5]
    a = residues((3, 2, 3, n), sub, 9300)
    b = residues((3, 2, 3, n), sub, 9301)
    import torch
    d = torch.empty((3, 3, 3, n), dtype=torch.int64, device="cuda:0")
    announce("tensor subrange")
    B.ct_tensor_ntt(plan, d, dev(a), dev(b), limb_begin=2)
    assert_bits_equal(host(d), orc.batch_tensor(a, b, sub), "tensor limbs 2..4")


def test_ct_tensor_coeff_chain_workload(B):
    """The inner chain (n = 2048, 112 primes of 30 bits, 4 tokens x 2 components) as one
    coefficient-domain ciphertext product, against the oracle's NTT, tensor and INTT."""
    w = workloads.CHAIN
    ps = list(primes(w.bits, 2 * w.n, w.limbs))
    a = residues(w.shape_a, ps, w.seed_a)
    b = residues(w.shape_a, ps, w.seed_b)
    import torch
    out = torch.empty((w.shape_a[0], 3) + tuple(w.shape_a[2:]), dtype=torch.int64, device="cuda:0")
    announce("ct_tensor_coeff chain workload")
    B.ct_tensor_coeff(B.Plan(w.n, ps, 0), out, dev(a), dev(b))
    assert_bits_equal(host(out), orc.ct_tensor_coeff(a, b, ps), "ct_tensor_coeff chain")


@pytest.mark.parametrize("bits", [30, 60, 62])
def test_ct_tensor_coeff_sweep(B, bits):
    """Every supported ring (n = 2 .. 4096), a ragged batch of 3 ciphertexts."""
    import torch
    for logn in range(1, 13):
        n = 1 << logn
        ps = list(primes(bits, 1 << 17, 3))  # 1 mod 2^17 covers every n here
        a = residues((3, 2, 3, n), ps, 9300 + logn)
        b = residues((3, 2, 3, n), ps, 9350 + logn)
        out = torch.empty((3, 3, 3, n), dtype=torch.int64, device="cuda:0")
        announce("ct_tensor_coeff sweep", bits, logn)
        B.ct_tensor_coeff(B.Plan(n, ps, 0), out, dev(a), dev(b))
        assert_bits_equal(host(out), orc.ct_tensor_coeff(a, b, ps), f"ct_tensor_coeff bits={bits} logn={logn}")


def test_ct_tensor_coeff_subrange_and_validation(B):
    import ctypes
    import torch
    n = 1 << 11
    ps = list(primes(30, 2 * n, 4)) + list(primes(60, 2 * n, 4))
    plan = B.Plan(n, ps, 0)
    a = residues((2, 2, 3, n), ps[3:6], 9361)  # limbs 3..5: one 30-bit and two 60-bit primes
    b = residues((2, 2, 3, n), ps[3:6], 9362)
    out = torch.empty((2, 3, 3, n), dtype=torch.int64, device="cuda:0")
    announce("ct_tensor_coeff subrange")
    B.ct_tensor_coeff(plan, out, dev(a), dev(b), limb_begin=3)
    assert_bits_equal(host(out), orc.ct_tensor_coeff(a, b, ps[3:6]), "ct_tensor_coeff subrange")
    L, V = B.lib(), ctypes.c_void_p
    ta = dev(a)
    assert L.ct_tensor_coeff(plan.handle, V(ta.data_ptr()), V(ta.data_ptr()), V(ta.data_ptr()), 2, 3, 3,
                             None) == B.NTT_EOVERLAP
    assert L.ct_tensor_coeff(plan.handle, V(out.data_ptr() + 8), V(ta.data_ptr()), V(ta.data_ptr()), 2, 3, 3,
                             None) == B.NTT_EINVAL
    assert L.ct_tensor_coeff(plan.handle, V(out.data_ptr()), V(ta.data_ptr()), V(ta.data_ptr()), 2, 6, 3,
                             None) == B.NTT_EINVAL  # limbs beyond the plan
    big = B.Plan(1 << 13, list(primes(30, 1 << 14, 1)), 0)
    x = torch.zeros((1, 2, 1, 1 << 13), dtype=torch.int64, device="cuda:0")
    y = torch.zeros((1, 3, 1, 1 << 13), dtype=torch.int64, device="cuda:0")
    assert L.ct_tensor_coeff(big.handle, V(y.data_ptr()), V(x.data_ptr()), V(x.data_ptr()), 1, 0, 1,
                             None) == B.NTT_EUNSUPPORTED
    torch.cuda.synchronize()


@pytest.mark.parametrize("domain", [0, 1])
def test_automorph_ring_workload_all_galois(B, domain):
    w = workloads.RING
    ps = primes(w.bits, 2 * w.n, w.limbs)
    x = residues((1, 2, w.limbs, w.n), ps, w.seed_a)
    plan = B.Plan(w.n, ps, 0)
    tx = dev(x)
    import torch
    out = torch.empty_like(tx)
    for g in w.galois:
        announce("automorph", domain, g)
        B.automorph(plan, out, tx, g, domain)
        assert_bits_equal(host(out), orc.batch_automorph(x, g, domain, ps), f"automorph g={g} domain={domain}")


def test_automorph_full_batch_and_ntt_commutation(B):
    w = workloads.RING
    ps = primes(w.bits, 2 * w.n, w.limbs)
    x = residues(w.shape_a, ps, w.seed_a)
    plan = B.Plan(w.n, ps, 0)
    import torch
    tx = dev(x)
    out = torch.empty_like(tx)
    g = w.galois[0]
    announce("automorph full batch")
    B.automorph(plan, out, tx, g, 0)
    assert_bits_equal(host(out), orc.batch_automorph(x, g, 0, ps), "full batch")
    # NTT(sigma_g a) == automorph_ntt(NTT a) on the device
    B.ntt_forward(plan, out)
    fx = B.ntt_forward(plan, tx)
    out2 = torch.empty_like(fx)
    B.automorph(plan, out2, fx, g, 1)
    assert_bits_equal(host(out), host(out2), "NTT-domain automorph commutes with the NTT")


@pytest.mark.parametrize("logn", [1, 2, 5, 9, 10, 11, 13])
def test_automorph_small_rings(B, logn):
    n = 1 << logn
    ps = primes(30, 1 << 17, 2)
    plan = B.Plan(n, ps, 0)
    x = residues((3, 2, n), ps, 9400 + logn)
    tx = dev(x)
    import torch
    out = torch.empty_like(tx)
    for g in sorted({1, 3 % (2 * n) or 1, 5 % (2 * n) or 1, 2 * n - 1}):
        for domain in (0, 1):
            B.automorph(plan, out, tx, g, domain)
            assert_bits_equal(host(out), orc.batch_automorph(x, g, domain, ps), f"n={n} g={g} d={domain}")


def test_device_validation(B):
    import torch
    ps = primes(60, 1 << 12, 2)
    plan = B.Plan(2048, ps, 0)
    L = B.lib()
    t = torch.zeros((2, 2, 2048), dtype=torch.int64, device="cuda:0")
    p = ctypes.c_void_p(t.data_ptr())
    half = ctypes.c_void_p(t.data_ptr() + 8 * 2048)  # partial overlap with t
    mis = ctypes.c_void_p(t.data_ptr() + 8)           # 8-byte misaligned
    assert L.ntt_forward(plan.handle, mis, 1, 0, 2, None) == B.NTT_EINVAL
    assert L.ntt_forward(plan.handle, p, 1, 1, 2, None) == B.NTT_EINVAL       # limb range beyond the plan
    assert L.ntt_forward(plan.handle, p, 1, 0, 0, None) == B.NTT_EINVAL
    assert L.poly_mul_ntt(plan.handle, half, p, p, 1, 0, 2, None) == B.NTT_EOVERLAP
    assert L.automorph(plan.handle, p, p, 5, 0, 1, 0, 2, None) == B.NTT_EOVERLAP
    assert L.automorph(plan.handle, half, p, 4, 0, 1, 0, 2, None) == B.NTT_EINVAL   # even g
    assert L.automorph(plan.handle, half, p, 4097, 0, 1, 0, 2, None) == B.NTT_EINVAL  # g >= 2n
    assert L.automorph(plan.handle, half, p, 5, 2, 1, 0, 2, None) == B.NTT_EINVAL   # bad domain
    assert L.ct_tensor_ntt(plan.handle, p, p, p, 1, 0, 2, None) == B.NTT_EOVERLAP
    assert L.ntt_forward_galois(plan.handle, half, p, 5, 1, 0, 2, None) == B.NTT_EOVERLAP
    with pytest.raises(TypeError):
        B.ntt_forward(plan, t.to(torch.int32))
    with pytest.raises(ValueError):
        B.ntt_forward(plan, t[:, :, :1024])
    with pytest.raises(ValueError):
        B.ntt_forward(plan, t.transpose(0, 1))


def test_count_noncanonical_and_debug_checks():
    """The input check counts exactly the planted residues >= q (q itself, q + 5, 2^63 - 1);
    with debug checks on, entry points reject such inputs before launching and leave
    their outputs untouched; with checks off they run (result unspecified)."""
    require_gpu()
    import ctypes
    import torch
    from negacyclic_ntt_amd import binding as B
    n = 1 << 12
    ps = list(primes(60, 2 * n, 4))
    plan = B.Plan(n, ps, 0)
    x = residues((2, 4, n), ps, 9100)
    assert B.count_noncanonical(plan, dev(x)) == 0
    bad = x.copy()
    bad[0, 1, 7] = ps[1]
    bad[1, 3, 0] = ps[3] + 5
    bad[1, 0, n - 1] = (1 << 63) - 1
    tb = dev(bad)
    announce("count noncanonical")
    assert B.count_noncanonical(plan, tb) == 3
    assert B.count_noncanonical(plan, tb[:, 1:3].contiguous(), limb_begin=1) == 1
    L = B.lib()
    V = ctypes.c_void_p
    B.set_debug_checks(True)
    try:
        before = host(tb).copy()
        assert L.ntt_forward(plan.handle, V(tb.data_ptr()), 2, 0, 4, None) == B.NTT_EINVAL
        assert np.array_equal(host(tb), before)  # nothing ran
        good = dev(x)
        assert L.ntt_forward(plan.handle, V(good.data_ptr()), 2, 0, 4, None) == B.NTT_OK
        out = torch.zeros_like(good)
        assert L.poly_mul_ntt(plan.handle, V(out.data_ptr()), V(good.data_ptr()), V(tb.data_ptr()), 2, 0, 4,
                              None) == B.NTT_EINVAL
        assert not host(out).any()
        # key-switch: a non-canonical key is rejected
        ks_primes = list(primes(60, 1 << 17, 8))
        kplan = B.Plan(n, ks_primes, 0)
        ks = B.KeySwitchPlan(kplan, 6, 2, 3)
        ct = dev(residues((1, 2, 6, n), ks_primes[:6], 9101))
        key = residues((3, 2, 8, n), ks_primes, 9102)
        key[2, 1, 7, 5] = ks_primes[7]
        with pytest.raises(B.NttError):
            B.keyswitch(ks, torch.zeros_like(ct), ct, dev(key), 5)
    finally:
        B.set_debug_checks(False)
    assert L.ntt_forward(plan.handle, V(tb.data_ptr()), 2, 0, 4, None) == B.NTT_OK  # checks off: it runs
    torch.cuda.synchronize()


def _cap_case(B, logn):
    """Every one-dimensional launch is split into parts of whole polynomials (or
    ciphertexts) under a small launch cap; the results match the oracle, with a batch
    that leaves a ragged last part."""
    import torch
    n, L, batch = 1 << logn, 3, 7
    ps = primes(30 if logn < 8 else 60, 2 * n, L)
    plan = B.Plan(n, ps, 0)
    a = residues((batch, 2, L, n), ps, 9700 + logn)
    b = residues((batch, 2, L, n), ps, 9800 + logn)
    fa = orc.batch_ntt(a, ps)
    fb = orc.batch_ntt(b, ps)
    g = 5 % (2 * n)
    # n / 2 threads per limb and polynomial at most: a cap of L n threads admits two
    # polynomials (one ciphertext) per launch for n = 1024, five for n = 32
    B.set_max_launch_threads(max(256, L * n))
    try:
        ta = dev(a)
        B.ntt_forward(plan, ta)
        assert_bits_equal(host(ta), fa, "forward")
        tg = torch.empty_like(ta)
        B.ntt_forward_galois(plan, tg, dev(a), g)
        assert_bits_equal(host(tg), orc.batch_ntt(orc.batch_automorph(a, g, 0, ps), ps), "forward galois")
        tb = dev(fb)
        tc = B.poly_mul_ntt(plan, torch.empty_like(ta), ta, tb)
        assert_bits_equal(host(tc), orc.batch_pointwise(fa, fb, ps), "pointwise")
        td = torch.empty((batch, 3, L, n), dtype=torch.int64, device=ta.device)
        B.ct_tensor_ntt(plan, td, ta, tb)
        assert_bits_equal(host(td), orc.batch_tensor(fa, fb, ps), "tensor")
        tcc = torch.empty((batch, 3, L, n), dtype=torch.int64, device=ta.device)
        B.ct_tensor_coeff(plan, tcc, dev(a), dev(b))
        assert_bits_equal(host(tcc), orc.ct_tensor_coeff(a, b, ps), "coefficient-domain product")
        B.ntt_inverse(plan, ta)
        assert_bits_equal(host(ta), a, "inverse")
        for domain in (0, 1):
            src = a if domain == 0 else fa
            out = torch.empty_like(ta)
            B.automorph(plan, out, dev(src), g, domain)
            assert_bits_equal(host(out), orc.batch_automorph(src, g, domain, ps), f"automorph domain {domain}")
        assert B.count_noncanonical(plan, dev(a)) == 0
    finally:
        B.set_max_launch_threads(0)


@pytest.mark.parametrize("logn", [5, 10])
def test_launch_cap_splits_every_launch(B, logn):
    announce("launch cap", logn)
    _cap_case(B, logn)


def test_launch_cap_too_small_for_one_polynomial(B):
    import torch
    n, L = 1 << 12, 4
    ps = primes(60, 2 * n, L)
    plan = B.Plan(n, ps, 0)
    x = dev(residues((2, L, n), ps, 9900))
    B.set_max_launch_threads(256)  # one polynomial needs L n / 2 threads
    try:
        with pytest.raises(B.NttError) as ei:
            B.ntt_forward(plan, x)
        assert ei.value.status == B.NTT_EUNSUPPORTED
        with pytest.raises(B.NttError):
            B.poly_mul_ntt(plan, torch.empty_like(x), x, x)
    finally:
        B.set_max_launch_threads(0)
    B.ntt_forward(plan, x)  # the default cap is back
