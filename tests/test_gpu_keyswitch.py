"""GPU parity: the rotation key-switch vs the oracle (bit-exact), plus its special
cases and the semantic check with a real key at a small ring."""
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


def _setup(B, n, nq=24, npr=8, dnum=3):
    qp = list(primes(60, 1 << 17, nq + npr))
    plan = B.Plan(n, qp, 0)
    ks = B.KeySwitchPlan(plan, nq, npr, dnum)
    return qp, plan, ks


@pytest.mark.parametrize("g", [5, 25, 65537, 1, 2 * 65536 - 1])
def test_keyswitch_workload_vs_oracle(B, g):
    w = workloads.KEYSWITCH
    qp, plan, ks = _setup(B, w.n)
    ct = residues(w.shape_a, qp[:24], w.seed_a)
    ksk = residues((3, 2, 32, w.n), qp, w.seed_b)
    announce("keyswitch workload", g)
    out = B.keyswitch(ks, dev(np.zeros_like(ct)), dev(ct), dev(ksk), g)
    want = orc.keyswitch(ct, ksk, g, qp, 24, 3)
    assert_bits_equal(host(out), want, f"keyswitch g={g}")


@pytest.mark.parametrize("logn,nq,npr,dnum", [(10, 24, 8, 3), (12, 6, 2, 2), (11, 16, 16, 1), (3, 4, 3, 4),
                                              (13, 12, 5, 3), (14, 9, 4, 3)])
def test_keyswitch_shapes_vs_oracle(B, logn, nq, npr, dnum):
    n = 1 << logn
    qp, plan, ks = _setup(B, n, nq, npr, dnum)
    ct = residues((2, 2, nq, n), qp[:nq], 9500 + logn)
    ksk = residues((dnum, 2, nq + npr, n), qp[: nq + npr], 9600 + logn)
    g = 5 % (2 * n)
    announce("keyswitch shape", logn, nq, npr, dnum)
    out = B.keyswitch(ks, dev(np.zeros_like(ct)), dev(ct), dev(ksk), g)
    assert_bits_equal(host(out), orc.keyswitch(ct, ksk, g, qp[: nq + npr], nq, dnum), "keyswitch shape")


@pytest.mark.parametrize("logn,bits,nq,npr,dnum", [(15, 60, 12, 4, 3), (15, 60, 10, 2, 5), (15, 62, 12, 4, 3),
                                                   (15, 62, 10, 3, 5), (16, 62, 8, 2, 4), (15, 30, 6, 2, 2),
                                                   (15, 60, 8, 4, 1), (16, 30, 6, 2, 3), (15, 30, 8, 3, 4)])
def test_keyswitch_fused_product_paths(B, logn, bits, nq, npr, dnum):
    """Two-pass ring sizes, where one kernel runs the forward row pass of every digit,
    the key product and the inverse row pass (dnum 1..4), or, for more digits, the key
    product rides on the inverse transform's row pass: both splits (2^15 = 2^7 x 2^8,
    2^16), every compile-time digit count and the runtime loop (dnum 5), 60-bit (one
    reduction) and 62-bit primes (four products per reduction, so five digits take
    two), and 30-bit primes."""
    n = 1 << logn
    qp = list(primes(bits, 2 * n, nq + npr))
    plan = B.Plan(n, qp, 0)
    ks = B.KeySwitchPlan(plan, nq, npr, dnum)
    ct = residues((2, 2, nq, n), qp[:nq], 9800 + logn + bits + dnum)
    ksk = residues((dnum, 2, nq + npr, n), qp, 9900 + logn + bits + dnum)
    g = 25
    announce("keyswitch fused product", logn, bits, nq, npr, dnum)
    out = B.keyswitch(ks, dev(np.zeros_like(ct)), dev(ct), dev(ksk), g)
    assert_bits_equal(host(out), orc.keyswitch(ct, ksk, g, qp, nq, dnum), "keyswitch fused product")


@pytest.mark.parametrize("logn,bits,nq,npr,dnum", [(10, 60, 4, 1, 2), (9, 62, 6, 1, 3), (8, 62, 8, 8, 1),
                                                   (12, 30, 8, 1, 8)])
def test_keyswitch_degenerate_bases(B, logn, bits, nq, npr, dnum):
    """One special prime (ModDown's Garner over P is the identity), one-prime digits,
    a single digit spanning Q, and 30- and 62-bit primes on the whole-limb path."""
    n = 1 << logn
    qp = list(primes(bits, 2 * n, nq + npr))
    plan = B.Plan(n, qp, 0)
    ks = B.KeySwitchPlan(plan, nq, npr, dnum)
    ct = residues((2, 2, nq, n), qp[:nq], 9700 + logn + bits)
    ksk = residues((dnum, 2, nq + npr, n), qp, 9750 + logn + bits)
    g = 2 * n - 1
    announce("keyswitch degenerate basis", logn, bits, nq, npr, dnum)
    out = B.keyswitch(ks, dev(np.zeros_like(ct)), dev(ct), dev(ksk), g)
    assert_bits_equal(host(out), orc.keyswitch(ct, ksk, g, qp, nq, dnum), "keyswitch degenerate basis")


def test_keyswitch_zero_key_and_zero_c1(B):
    n = 1 << 12
    qp, plan, ks = _setup(B, n)
    ct = residues((1, 2, 24, n), qp[:24], 9700)
    g = 25
    sig = orc.batch_automorph(ct[0], g, 0, qp[:24])
    announce("keyswitch zero key")
    out = host(B.keyswitch(ks, dev(np.zeros_like(ct)), dev(ct), dev(np.zeros((3, 2, 32, n), np.uint64)), g))
    assert_bits_equal(out[0, 0], sig[0], "ksk = 0 -> sigma(c0)")
    assert not out[0, 1].any()
    ct1 = ct.copy()
    ct1[0, 1] = 0
    ksk = residues((3, 2, 32, n), qp, 9701)
    out = host(B.keyswitch(ks, dev(np.zeros_like(ct)), dev(ct1), dev(ksk), g))
    assert_bits_equal(out[0, 0], sig[0], "c1 = 0 -> sigma(c0)")
    assert not out[0, 1].any()


def test_keyswitch_semantic_small_ring(B):
    """With a real key at n = 1024 the switched ciphertext decrypts, under s, to what
    sigma_g of the input decrypts to under sigma_g(s), up to a small error."""
    n, g, dnum, alpha = 1024, 5, 3, 8
    qp, plan, ks = _setup(B, n)
    Q, P = qp[:24], qp[24:]
    s = inputs.small_signed(n, 1, 130)
    s_limbs = np.array([[int(v) % q for v in s] for q in qp], dtype=np.uint64)
    s_rot = orc.batch_automorph(s_limbs, g, 0, qp)
    Pm = 1
    for p in P:
        Pm *= p

    def pmul(a, b, ps):
        return orc.batch_ntt(orc.batch_pointwise(orc.batch_ntt(a, ps), orc.batch_ntt(b, ps), ps), ps, inverse=True)

    ksk = np.zeros((dnum, 2, 32, n), dtype=np.uint64)
    for j in range(dnum):
        a_j = residues((32, n), qp, 140 + j)
        e = inputs.small_signed(n, 8, 150 + j)
        e_j = np.array([[int(v) % q for v in e] for q in qp], dtype=np.uint64)
        as_ = pmul(a_j, s_limbs, qp)
        b_coef = np.zeros((32, n), dtype=np.uint64)
        for l, q in enumerate(qp):
            pts = (s_rot[l].astype(object) * (Pm % q)) % q if j * alpha <= l < (j + 1) * alpha else 0
            b_coef[l] = ((e_j[l].astype(object) - as_[l].astype(object) + pts) % q).astype(np.uint64)
        ksk[j, 0] = orc.batch_ntt(b_coef, qp)
        ksk[j, 1] = orc.batch_ntt(a_j, qp)
    ct = residues((1, 2, 24, n), Q, 160)
    announce("keyswitch semantic")
    out = host(B.keyswitch(ks, dev(np.zeros_like(ct)), dev(ct), dev(ksk), g))
    assert_bits_equal(out, orc.keyswitch(ct, ksk, g, qp, 24, dnum), "semantic-key case vs oracle")
    lhs = out[0, 0].astype(object) + pmul(out[0, 1], s_limbs[:24], Q).astype(object)
    c_rot = orc.batch_automorph(ct[0], g, 0, Q)
    rhs = c_rot[0].astype(object) + pmul(c_rot[1], s_rot[:24], Q).astype(object)
    from sympy.ntheory.modular import crt
    Qm = 1
    for q in Q:
        Qm *= q
    worst = 0
    for i in range(0, n, 7):
        v = int(crt(Q, [int((lhs[l][i] - rhs[l][i]) % Q[l]) for l in range(24)])[0])
        v = v - Qm if v > Qm // 2 else v
        worst = max(worst, abs(v))
    assert worst < (1 << 20), worst


def test_keyswitch_validation(B):
    import ctypes
    import torch
    n = 1 << 10
    qp, plan, ks = _setup(B, n)
    L = B.lib()
    ct = torch.zeros((1, 2, 24, n), dtype=torch.int64, device="cuda:0")
    out = torch.zeros_like(ct)
    ksk = torch.zeros((3, 2, 32, n), dtype=torch.int64, device="cuda:0")
    ws = B.workspace(ks, 1)
    V = ctypes.c_void_p
    args = (V(out.data_ptr()), V(ct.data_ptr()), V(ksk.data_ptr()))
    nb = ws.numel()
    assert L.keyswitch(ks.handle, *args, 4, 1, V(ws.data_ptr()), nb, None) == B.NTT_EINVAL     # even g
    assert L.keyswitch(ks.handle, *args, 5, 1, V(ws.data_ptr()), nb - 1, None) == B.NTT_EINVAL  # small ws
    assert L.keyswitch(ks.handle, V(ct.data_ptr()), V(ct.data_ptr()), V(ksk.data_ptr()), 5, 1, V(ws.data_ptr()), nb,
                       None) == B.NTT_EOVERLAP
    assert L.keyswitch(ks.handle, *args, 5, 1, V(ct.data_ptr()), nb, None) == B.NTT_EOVERLAP
    h = V()
    assert L.keyswitch_plan_create(ctypes.byref(h), plan.handle, 24, 8, 5) == B.NTT_EINVAL  # 24 % 5
    assert L.keyswitch_plan_create(ctypes.byref(h), plan.handle, 24, 9, 3) == B.NTT_EINVAL  # beyond the plan
    assert L.keyswitch_plan_create(ctypes.byref(h), plan.handle, 24, 8, 1) == B.NTT_EUNSUPPORTED  # alpha 24


def test_graph_capture_replays_match_eager(B):
    """The entry points allocate nothing and launch on the caller's stream, so a HIP
    graph can hold them.  Capture: forward NTT (out of place, g = 1), pointwise
    product, inverse NTT, rotation key-switch; replay three times with eager work in
    between and compare every replay with the eager results."""
    import torch
    n = 1 << 12
    qp, plan, ks = _setup(B, n)
    x = dev(residues((2, 24, n), qp[:24], 9950))
    bb = dev(residues((2, 24, n), qp[:24], 9951))
    ct = dev(residues((1, 2, 24, n), qp[:24], 9952))
    ksk = dev(residues((3, 2, 32, n), qp, 9953))
    ws = B.workspace(ks, 1)
    f = torch.empty_like(x)
    c = torch.empty_like(x)
    ko = torch.empty_like(ct)

    def body():
        B.ntt_forward_galois(plan, f, x, 1)
        B.poly_mul_ntt(plan, c, f, bb)
        B.ntt_inverse(plan, c)
        B.keyswitch(ks, ko, ct, ksk, 25, ws)

    announce("graph capture eager")
    body()
    want_c, want_k = host(c).copy(), host(ko).copy()
    assert_bits_equal(want_c, orc.batch_ntt(orc.batch_pointwise(orc.batch_ntt(host(x), qp[:24]), host(bb), qp[:24]),
                                            qp[:24], inverse=True), "eager pipeline vs oracle")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()  # warm-up on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    announce("graph capture")
    with torch.cuda.graph(g):
        body()
    for rep in range(3):
        c.zero_()
        ko.zero_()
        torch.cuda.synchronize()
        announce("graph replay", rep)
        g.replay()
        torch.cuda.synchronize()
        assert_bits_equal(host(c), want_c, f"replay {rep} pipeline")
        assert_bits_equal(host(ko), want_k, f"replay {rep} keyswitch")
        B.ntt_forward(plan, dev(residues((2, 24, n), qp[:24], 9960 + rep)))  # eager work between replays


@pytest.mark.parametrize("as_int", [False, True])
def test_explicit_side_stream_without_workspace(B, as_int):
    """stream= names a stream other than torch's current one and no workspace is
    passed: the workspace the binding allocates, and the counter of
    count_noncanonical, are ordered on that stream.  Between calls the current stream
    allocates and fills tensors of the workspace's size, which would take over a
    workspace released to the current stream while the side stream still used it."""
    import torch
    n, nq, npr, dnum, g = 1 << 12, 6, 2, 3, 5
    qp, plan, ks = _setup(B, n, nq, npr, dnum)
    ct = residues((2, 2, nq, n), qp[:nq], 9401)
    ksk = residues((dnum, 2, nq + npr, n), qp[: nq + npr], 9402)
    want = orc.keyswitch(ct, ksk, g, qp[: nq + npr], nq, dnum)
    dct, dksk = dev(ct), dev(ksk)
    side = torch.cuda.Stream()
    stream = side.cuda_stream if as_int else side
    ws_elems = ks.workspace_bytes(2) // 8
    outs = []
    for rep in range(3):
        out = torch.zeros_like(dct)
        side.wait_stream(torch.cuda.current_stream())
        announce("keyswitch on a side stream, binding workspace", rep, as_int)
        B.keyswitch(ks, out, dct, dksk, g, stream=stream)
        out.record_stream(side)
        outs.append(out)
        torch.empty(ws_elems, dtype=torch.int64, device="cuda:0").fill_(-1)  # current stream
    side.synchronize()
    torch.cuda.synchronize()
    for rep, out in enumerate(outs):
        assert_bits_equal(host(out), want, f"side-stream keyswitch {rep}")
    bad = ct.copy()
    bad[0, 1, 2, 7] = qp[2]          # exactly q: not canonical
    bad[1, 0, 5, 100] = qp[5] + 3
    dbad = dev(bad)
    torch.cuda.synchronize()
    announce("count_noncanonical on a side stream", as_int)
    assert B.count_noncanonical(plan, dbad.view(-1, nq, n), stream=stream) == 2
    assert B.count_noncanonical(plan, dct.view(-1, nq, n), stream=stream) == 0


def test_keyswitch_middle_split_under_launch_cap(B):
    """Under a launch cap that admits one ciphertext's transforms per launch, the fused
    middle of a 2^15 key-switch (forward column pass, fused row kernel, inverse column
    pass) runs in parts: three ciphertexts against the oracle."""
    n, nq, npr, dnum, g = 1 << 15, 4, 2, 2, 5
    qp = list(primes(60, 2 * n, nq + npr))
    plan = B.Plan(n, qp, 0)
    ks = B.KeySwitchPlan(plan, nq, npr, dnum)
    ct = residues((3, 2, nq, n), qp[:nq], 9420)
    ksk = residues((dnum, 2, nq + npr, n), qp, 9421)
    # the largest of the three launches is a column pass over dnum x 6 limbs: 16 blocks
    # of 256 threads per limb
    B.set_max_launch_threads(dnum * (nq + npr) * 16 * 256)
    try:
        announce("keyswitch middle under a launch cap")
        out = host(B.keyswitch(ks, dev(np.zeros_like(ct)), dev(ct), dev(ksk), g))
    finally:
        B.set_max_launch_threads(0)
    assert_bits_equal(out, orc.keyswitch(ct, ksk, g, qp, nq, dnum), "keyswitch middle in parts")
