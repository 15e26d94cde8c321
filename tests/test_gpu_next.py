"""GPU parity for the operations that complete a ciphertext product: rescale
(truncating and nearest) and relinearisation, each bit-exact against the oracle,
plus the whole product pipeline run on the GPU."""
import numpy as np
import pytest

import oracle as orc
from negacyclic_ntt_amd import inputs, workloads
from tests.helpers import announce, assert_bits_equal, dev, host, primes, require_gpu, residues

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    require_gpu()
    from negacyclic_ntt_amd import binding
    return binding


# ---- rescale ------------------------------------------------------------------------

def _rescale_gpu(B, plan, x, mode, limb_begin=0):
    out = dev(np.zeros(x.shape[:-2] + (x.shape[-2] - 1, x.shape[-1]), dtype=np.uint64))
    return host(B.rescale(plan, out, dev(x), mode, limb_begin))


@pytest.mark.parametrize("logn", [1, 2, 5, 9, 10, 12, 16])
@pytest.mark.parametrize("bits", [30, 60, 62])
def test_rescale_sweep(B, logn, bits):
    n = 1 << logn
    ps = list(primes(bits, 2 * n, 5))
    plan = B.Plan(n, ps, 0)
    x = residues((3, 5, n), ps, 7000 + logn + bits)
    for mode in (0, 1):
        announce("rescale", logn, bits, mode)
        assert_bits_equal(_rescale_gpu(B, plan, x, mode), orc.rescale(x, ps, mode), f"rescale {logn} {bits} {mode}")


def test_rescale_mixed_widths_and_subrange(B):
    """Narrow and wide primes in one plan (the dropped prime larger or smaller than
    the others) and limb ranges that do not start at 0."""
    n = 1 << 11
    narrow = list(primes(30, 2 * n, 3))
    wide = list(primes(62, 2 * n, 3))
    ps = [narrow[0], wide[0], narrow[1], wide[1], narrow[2], wide[2]]
    plan = B.Plan(n, ps, 0)
    for begin, count in [(0, 6), (0, 5), (1, 4), (2, 2), (4, 2), (3, 3)]:
        sub = ps[begin:begin + count]
        x = residues((2, count, n), sub, 7100 + 10 * begin + count)
        for mode in (0, 1):
            announce("rescale subrange", begin, count, mode)
            assert_bits_equal(_rescale_gpu(B, plan, x, mode, begin), orc.rescale(x, sub, mode),
                              f"rescale [{begin}, {begin + count}) mode {mode}")


def test_rescale_boundary_values(B):
    """Residues 0 and q - 1 everywhere, and columns whose last residue sits at the
    rounding boundary floor(q_k / 2) and next to it."""
    n = 1 << 10
    ps = list(primes(60, 2 * n, 4))
    plan = B.Plan(n, ps, 0)
    x = residues((1, 4, n), ps, 7200)
    x[0, :, :64] = 0
    for l, q in enumerate(ps):
        x[0, l, 64:128] = q - 1
    h = ps[-1] // 2
    x[0, 3, 128:192] = h
    x[0, 3, 192:256] = h + 1
    x[0, 3, 256:320] = h - 1
    for mode in (0, 1):
        announce("rescale boundary", mode)
        assert_bits_equal(_rescale_gpu(B, plan, x, mode), orc.rescale(x, ps, mode), f"rescale boundary {mode}")


def test_rescale_workload_full(B):
    """The large-ring batch [8][2][24][2^16], every output residue."""
    w = workloads.RING
    ps = list(primes(w.bits, 2 * w.n, w.prime_count))
    plan = B.Plan(w.n, ps, 0)
    x = residues(w.shape_a, ps, w.seed_a)
    for mode in (0, 1):
        announce("rescale workload", mode)
        assert_bits_equal(_rescale_gpu(B, plan, x, mode), orc.rescale(x, ps, mode), f"rescale workload mode {mode}")


def test_rescale_validation(B):
    import ctypes
    import torch
    n = 1 << 10
    ps = list(primes(60, 2 * n, 4))
    plan = B.Plan(n, ps, 0)
    L = B.lib()
    x = torch.zeros((2, 4, n), dtype=torch.int64, device="cuda:0")
    out = torch.zeros((2, 3, n), dtype=torch.int64, device="cuda:0")
    V = ctypes.c_void_p
    assert L.rescale(plan.handle, V(out.data_ptr()), V(x.data_ptr()), 2, 2, 0, 4, None) == B.NTT_EINVAL  # mode
    assert L.rescale(plan.handle, V(out.data_ptr()), V(x.data_ptr()), 0, 2, 0, 1, None) == B.NTT_EINVAL  # 1 limb
    assert L.rescale(plan.handle, V(out.data_ptr()), V(x.data_ptr()), 0, 2, 1, 4, None) == B.NTT_EINVAL  # range
    assert L.rescale(plan.handle, V(x.data_ptr()), V(x.data_ptr()), 0, 2, 0, 4, None) == B.NTT_EOVERLAP
    assert L.rescale(plan.handle, V(out.data_ptr() + 8), V(x.data_ptr()), 0, 2, 0, 4, None) == B.NTT_EINVAL
    assert L.rescale(plan.handle, V(out.data_ptr()), V(x.data_ptr()), 0, 0, 0, 4, None) == B.NTT_OK  # empty


# ---- relinearisation ------------------------------------------------------------------

def _ks_setup(B, n, nq=24, npr=8, dnum=3):
    qp = list(primes(60, 1 << 17, nq + npr))
    plan = B.Plan(n, qp, 0)
    return qp, plan, B.KeySwitchPlan(plan, nq, npr, dnum)


def _relin_gpu(B, ks, d, rlk):
    out = dev(np.zeros(d.shape[:-3] + (2,) + d.shape[-2:], dtype=np.uint64))
    return host(B.relinearize(ks, out, dev(d), dev(rlk)))


def test_relinearize_workload_vs_oracle(B):
    """The large-ring key-switch configuration (n = 2^16, 24 + 8 primes, dnum 3)."""
    w = workloads.KEYSWITCH
    qp, plan, ks = _ks_setup(B, w.n)
    d = residues((1, 3, 24, w.n), qp[:24], w.seed_a + 7)
    rlk = residues((3, 2, 32, w.n), qp, w.seed_b + 7)
    announce("relinearize workload")
    assert_bits_equal(_relin_gpu(B, ks, d, rlk), orc.relinearize(d, rlk, qp, 24, 3), "relinearize workload")


@pytest.mark.parametrize("logn,nq,npr,dnum,batch", [(10, 24, 8, 3, 2), (12, 6, 2, 2, 3), (11, 16, 16, 1, 1),
                                                    (3, 4, 3, 4, 2), (13, 12, 5, 3, 1)])
def test_relinearize_shapes_vs_oracle(B, logn, nq, npr, dnum, batch):
    n = 1 << logn
    qp, plan, ks = _ks_setup(B, n, nq, npr, dnum)
    d = residues((batch, 3, nq, n), qp[:nq], 7400 + logn)
    rlk = residues((dnum, 2, nq + npr, n), qp[: nq + npr], 7500 + logn)
    announce("relinearize shape", logn, nq, npr, dnum, batch)
    assert_bits_equal(_relin_gpu(B, ks, d, rlk), orc.relinearize(d, rlk, qp[: nq + npr], nq, dnum),
                      "relinearize shape")


def test_relinearize_two_pass_ring(B):
    """n = 2^15 (the 2^7 x 2^8 split with the key product inside the inverse transform), batch 2."""
    n = 1 << 15
    qp, plan, ks = _ks_setup(B, n, 12, 4, 3)
    d = residues((2, 3, 12, n), qp[:12], 7450)
    rlk = residues((3, 2, 16, n), qp[:16], 7451)
    announce("relinearize 2^15")
    assert_bits_equal(_relin_gpu(B, ks, d, rlk), orc.relinearize(d, rlk, qp[:16], 12, 3), "relinearize 2^15")


def test_relinearize_zero_key_and_zero_d2(B):
    n = 1 << 12
    qp, plan, ks = _ks_setup(B, n)
    d = residues((2, 3, 24, n), qp[:24], 7600)
    announce("relinearize zero key")
    out = _relin_gpu(B, ks, d, np.zeros((3, 2, 32, n), np.uint64))
    assert_bits_equal(out, d[:, :2], "rlk = 0 -> (d0, d1)")
    d[:, 2] = 0
    out = _relin_gpu(B, ks, d, residues((3, 2, 32, n), qp, 7601))
    assert_bits_equal(out, d[:, :2], "d2 = 0 -> (d0, d1)")


def test_relinearize_validation(B):
    import ctypes
    import torch
    n = 1 << 10
    qp, plan, ks = _ks_setup(B, n)
    L = B.lib()
    d = torch.zeros((1, 3, 24, n), dtype=torch.int64, device="cuda:0")
    out = torch.zeros((1, 2, 24, n), dtype=torch.int64, device="cuda:0")
    rlk = torch.zeros((3, 2, 32, n), dtype=torch.int64, device="cuda:0")
    ws = B.workspace(ks, 1)
    V = ctypes.c_void_p
    nb = ws.numel()
    args = (V(out.data_ptr()), V(d.data_ptr()), V(rlk.data_ptr()), 1)
    assert L.relinearize(ks.handle, *args, V(ws.data_ptr()), nb - 1, None) == B.NTT_EINVAL
    assert L.relinearize(ks.handle, V(d.data_ptr() + 16 * n * 8), V(d.data_ptr()), V(rlk.data_ptr()), 1,
                         V(ws.data_ptr()), nb, None) == B.NTT_EOVERLAP  # out inside d
    assert L.relinearize(ks.handle, *args, V(d.data_ptr()), nb, None) == B.NTT_EOVERLAP  # ws is d
    assert L.relinearize(ks.handle, *args[:3], 5000, V(ws.data_ptr()), nb, None) == B.NTT_EUNSUPPORTED
    assert L.relinearize(ks.handle, *args[:3], 0, V(ws.data_ptr()), nb, None) == B.NTT_OK


# ---- the whole ciphertext product on the GPU --------------------------------------------

def test_ciphertext_product_pipeline_vs_oracle(B):
    """NTT of both operands, tensor product, inverse NTT, relinearisation and a
    nearest rescale, all on the GPU, equal the same steps through the oracle (n =
    2^12, 24 + 8 primes, batch 2)."""
    n = 1 << 12
    qp, plan, ks = _ks_setup(B, n)
    Q = qp[:24]
    a = residues((2, 2, 24, n), Q, 7700)
    b = residues((2, 2, 24, n), Q, 7701)
    rlk = residues((3, 2, 32, n), qp, 7702)
    announce("ciphertext product pipeline")
    ta, tb = dev(a), dev(b)
    B.ntt_forward(plan, ta)
    B.ntt_forward(plan, tb)
    d = dev(np.zeros((2, 3, 24, n), np.uint64))
    B.ct_tensor_ntt(plan, d, ta, tb)
    B.ntt_inverse(plan, d)
    c = dev(np.zeros((2, 2, 24, n), np.uint64))
    B.relinearize(ks, c, d, dev(rlk))
    r = dev(np.zeros((2, 2, 23, n), np.uint64))
    got = host(B.rescale(plan, r, c, 1))
    fa, fb = orc.batch_ntt(a, Q), orc.batch_ntt(b, Q)
    dd = orc.batch_ntt(orc.batch_tensor(fa, fb, Q), Q, inverse=True)
    want = orc.rescale(orc.relinearize(dd, rlk, qp, 24, 3), Q, 1)
    assert_bits_equal(got, want, "ciphertext product pipeline")


# ---- hoisted rotations ------------------------------------------------------------------

def _hoisted_gpu(B, ks, ct, ksk, gs):
    R = len(gs)
    out = dev(np.zeros((R,) + ct.shape, dtype=np.uint64))
    return host(B.keyswitch_hoisted(ks, out, dev(ct), dev(ksk), gs))


def test_hoisted_workload_vs_oracle(B):
    """The large-ring key-switch configuration with four rotations sharing one
    decomposition: two powers of 5, the conjugation 2n - 1 and g = 1."""
    w = workloads.KEYSWITCH
    qp, plan, ks = _ks_setup(B, w.n)
    gs = [5, 25, 2 * w.n - 1, 1]
    ct = residues(w.shape_a, qp[:24], w.seed_a + 11)
    ksk = residues((len(gs), 3, 2, 32, w.n), qp, w.seed_b + 11)
    announce("hoisted workload", gs)
    assert_bits_equal(_hoisted_gpu(B, ks, ct, ksk, gs), orc.keyswitch_hoisted(ct, ksk, gs, qp, 24, 3),
                      "hoisted workload")


@pytest.mark.parametrize("logn,nq,npr,dnum,batch", [(1, 4, 2, 2, 1), (4, 4, 3, 4, 2), (9, 6, 2, 3, 2),
                                                    (10, 24, 8, 3, 2), (11, 16, 16, 16, 1), (12, 6, 2, 2, 3)])
def test_hoisted_shapes_vs_oracle(B, logn, nq, npr, dnum, batch):
    """Rings below, at and above the 512-slot segment, dnum up to the LDS limit of 16."""
    n = 1 << logn
    qp, plan, ks = _ks_setup(B, n, nq, npr, dnum)
    gs = sorted({1, 3 % (2 * n), 5 % (2 * n), (2 * n - 1), (2 * n - 3) % (2 * n) or 1})
    gs = [g for g in gs if g % 2 == 1]
    ct = residues((batch, 2, nq, n), qp[:nq], 7800 + logn)
    ksk = residues((len(gs), dnum, 2, nq + npr, n), qp[: nq + npr], 7900 + logn)
    announce("hoisted shape", logn, nq, npr, dnum, batch, gs)
    assert_bits_equal(_hoisted_gpu(B, ks, ct, ksk, gs),
                      orc.keyswitch_hoisted(ct, ksk, gs, qp[: nq + npr], nq, dnum), "hoisted shape")


@pytest.mark.parametrize("bits,nq,npr,dnum", [(60, 12, 4, 3), (60, 10, 2, 5), (62, 10, 3, 5), (62, 8, 4, 2),
                                               (62, 8, 4, 4)])
def test_hoisted_fused_product_paths(B, bits, nq, npr, dnum):
    """n = 2^15: the rotations' key products run inside the inverse transform's first
    pass (compile-time and runtime digit counts; 62-bit primes take several
    reductions per product sum).  P sigma_g(c0) joins the product sum while one more
    term fits its exact bound: 62-bit primes allow 4 terms per reduction, so dnum 2 folds
    it in and dnum 4, at the bound, adds it in ModDown."""
    n = 1 << 15
    qp = list(primes(bits, 2 * n, nq + npr))
    plan = B.Plan(n, qp, 0)
    ks = B.KeySwitchPlan(plan, nq, npr, dnum)
    gs = [5, 2 * n - 1, 25, 1]
    ct = residues((2, 2, nq, n), qp[:nq], 7850 + dnum + bits)
    ksk = residues((len(gs), dnum, 2, nq + npr, n), qp, 7860 + dnum + bits)
    announce("hoisted fused", bits, nq, npr, dnum)
    assert_bits_equal(_hoisted_gpu(B, ks, ct, ksk, gs), orc.keyswitch_hoisted(ct, ksk, gs, qp, nq, dnum),
                      "hoisted fused product")


def test_hoisted_identity_equals_keyswitch(B):
    n = 1 << 12
    qp, plan, ks = _ks_setup(B, n)
    ct = residues((2, 2, 24, n), qp[:24], 8000)
    ksk = residues((1, 3, 2, 32, n), qp, 8001)
    announce("hoisted identity")
    got = _hoisted_gpu(B, ks, ct, ksk, [1])
    ref = host(B.keyswitch(ks, dev(np.zeros_like(ct)), dev(ct), dev(ksk[0]), 1))
    assert_bits_equal(got[0], ref, "hoisted g=1 vs keyswitch")


def test_hoisted_validation(B):
    import ctypes
    import torch
    n = 1 << 10
    qp, plan, ks = _ks_setup(B, n)
    L = B.lib()
    ct = torch.zeros((1, 2, 24, n), dtype=torch.int64, device="cuda:0")
    out = torch.zeros((2, 1, 2, 24, n), dtype=torch.int64, device="cuda:0")
    ksk = torch.zeros((2, 3, 2, 32, n), dtype=torch.int64, device="cuda:0")
    ws = B.hoisted_workspace(ks, 2, 1)
    V = ctypes.c_void_p
    nb = ws.numel()

    def call(gs, R=None, o=out, w=ws, nbytes=nb):
        arr = np.asarray(gs, dtype=np.uint64)
        return L.keyswitch_hoisted(ks.handle, V(o.data_ptr()), V(ct.data_ptr()), V(ksk.data_ptr()),
                                   arr.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)), len(gs) if R is None else R,
                                   1, V(w.data_ptr()), nbytes, None)
    assert call([5, 25]) == B.NTT_OK
    assert call([5, 4]) == B.NTT_EINVAL          # even element
    assert call([5, 2 * n + 1]) == B.NTT_EINVAL  # beyond 2n
    assert call([5, 25], R=0) == B.NTT_EINVAL
    assert call([5] * 65) == B.NTT_EUNSUPPORTED
    assert call([5, 25], nbytes=nb - 1) == B.NTT_EINVAL
    assert call([5, 25], w=ct) == B.NTT_EOVERLAP
    torch.cuda.synchronize()


# ---- modraise ----------------------------------------------------------------------------

@pytest.mark.parametrize("logn,bits,frm,to,batch", [(1, 60, 1, 3, 2), (10, 60, 1, 24, 2), (12, 62, 3, 12, 3),
                                                    (16, 60, 1, 24, 2), (16, 60, 2, 24, 2), (11, 30, 4, 9, 1),
                                                    (13, 60, 16, 20, 1), (9, 62, 5, 6, 2)])
def test_modraise_vs_oracle(B, logn, bits, frm, to, batch):
    n = 1 << logn
    ps = list(primes(bits, 2 * n, to))
    plan = B.Plan(n, ps, 0)
    mr = B.ModRaisePlan(plan, frm, to)
    x = residues((batch, frm, n), ps[:frm], 8100 + logn + frm)
    announce("modraise", logn, bits, frm, to, batch)
    out = dev(np.zeros((batch, to, n), np.uint64))
    assert_bits_equal(host(B.modraise(mr, out, dev(x))), orc.modraise(x, ps, frm), "modraise")


def test_modraise_extremes(B):
    """Columns at 0 and at Q_from - 1 (all residues q_i - 1)."""
    n = 1 << 10
    ps = list(primes(60, 2 * n, 8))
    plan = B.Plan(n, ps, 0)
    mr = B.ModRaisePlan(plan, 3, 8)
    x = residues((1, 3, n), ps[:3], 8200)
    x[0, :, :100] = 0
    for i in range(3):
        x[0, i, 100:200] = ps[i] - 1
    announce("modraise extremes")
    out = dev(np.zeros((1, 8, n), np.uint64))
    assert_bits_equal(host(B.modraise(mr, out, dev(x))), orc.modraise(x, ps, 3), "modraise extremes")


def test_modraise_validation(B):
    import ctypes
    import torch
    n = 1 << 10
    ps = list(primes(60, 2 * n, 8))
    plan = B.Plan(n, ps, 0)
    L = B.lib()
    h = ctypes.c_void_p()
    assert L.modraise_plan_create(ctypes.byref(h), plan.handle, 0, 4) == B.NTT_EINVAL
    assert L.modraise_plan_create(ctypes.byref(h), plan.handle, 4, 4) == B.NTT_EINVAL
    assert L.modraise_plan_create(ctypes.byref(h), plan.handle, 2, 9) == B.NTT_EINVAL
    mr = B.ModRaisePlan(plan, 2, 8)
    x = torch.zeros((2, 2, n), dtype=torch.int64, device="cuda:0")
    out = torch.zeros((2, 8, n), dtype=torch.int64, device="cuda:0")
    V = ctypes.c_void_p
    assert L.modraise(mr.handle, V(out.data_ptr()), V(out.data_ptr()), 2, None) == B.NTT_EOVERLAP
    assert L.modraise(mr.handle, V(out.data_ptr() + 8), V(x.data_ptr()), 2, None) == B.NTT_EINVAL
    assert L.modraise(mr.handle, V(out.data_ptr()), V(x.data_ptr()), 0, None) == B.NTT_OK


# ---- launches larger than one grid dimension ------------------------------------------------

def test_keyswitch_batch_beyond_grid_y(B):
    """batch x digits = 4096 x 16 = 65536 exceeds the grid's y range: ModUp runs in
    chunks (n = 8, 16 one-prime digits, 2 special primes)."""
    n = 8
    qp = list(primes(60, 1 << 17, 18))
    plan = B.Plan(n, qp, 0)
    ks = B.KeySwitchPlan(plan, 16, 2, 16)
    ct = residues((4096, 2, 16, n), qp[:16], 9400)
    ksk = residues((16, 2, 18, n), qp, 9401)
    announce("keyswitch batch 4096 x dnum 16")
    out = host(B.keyswitch(ks, dev(np.zeros_like(ct)), dev(ct), dev(ksk), 3))
    # ciphertexts are independent: compare both ends, across the chunk boundary (4095 per chunk)
    pick = np.r_[0:32, 4064:4096]
    want = orc.keyswitch(np.ascontiguousarray(ct[pick]), ksk, 3, qp, 16, 16)
    assert_bits_equal(np.ascontiguousarray(out[pick]), want, "keyswitch grid-y chunks")


def test_rescale_and_modraise_batch_beyond_grid_y(B):
    """70000 polynomials (n = 2): the batch is split across launches."""
    n = 2
    ps = list(primes(60, 2 * n, 3))
    plan = B.Plan(n, ps, 0)
    x = residues((70000, 3, n), ps, 9410)
    announce("rescale batch 70000")
    got = host(B.rescale(plan, dev(np.zeros((70000, 2, n), np.uint64)), dev(x), 1))
    assert_bits_equal(got, orc.rescale(x, ps, 1), "rescale grid-y chunks")
    mr = B.ModRaisePlan(plan, 1, 3)
    lo = residues((70000, 1, n), ps[:1], 9411)
    announce("modraise batch 70000")
    up = host(B.modraise(mr, dev(np.zeros((70000, 3, n), np.uint64)), dev(lo)))
    assert_bits_equal(up, orc.modraise(lo, ps, 1), "modraise grid-y chunks")
